"""GPU parity of the prefill path against the CPU oracle, through the C ABI.

Every test compares every output element (and the lse) with the oracle: small
shapes (several tiles, ragged tails, GQA, causal bottom-right with Sq < Skv and
Sq > Skv), and the full-size workloads -- non-causal MHA 4x16x2048x64, and
causal GQA as 32 microbatches of 512 queries over 16384 tokens in the launch
configuration the bench times, one test per microbatch.
"""
import os

import numpy as np
import pytest

import fa_inputs as fi
import oracle
from helpers import assert_lse, assert_parity, log, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import flashattention_forward_amd as fa
    return fa


def _dtype_torch(name):
    import torch
    return {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}[name]


def run(fa, inp, *, lse=True, allow_split=True, q=None, k=None, v=None):
    import torch
    q = to_dev(inp.q, inp.in_dtype) if q is None else q
    k = to_dev(inp.k, inp.in_dtype) if k is None else k
    v = to_dev(inp.v, inp.in_dtype) if v is None else v
    res = fa.prefill(q, k, v, causal=inp.causal, scale=inp.scale,
                     out_dtype=_dtype_torch(inp.out_dtype), return_lse=lse,
                     allow_split=allow_split)
    torch.cuda.synchronize()
    return res


SMALL = [
    # B, Hq, Hkv, Sq, Skv, D, causal, in, out
    (2, 4, 2, 200, 333, 64, True, "bf16", "bf16"),
    (2, 4, 2, 200, 333, 128, False, "bf16", "bf16"),
    (1, 8, 2, 77, 77, 128, True, "fp16", "fp16"),
    (1, 2, 1, 300, 100, 64, True, "bf16", "fp32"),   # Sq > Skv: leading rows see no key
    (1, 2, 2, 1, 1000, 128, True, "bf16", "bf16"),   # one query
    (3, 2, 1, 130, 1, 64, False, "bf16", "bf16"),    # one key
    (1, 6, 3, 129, 700, 128, True, "bf16", "bf16"),
    (1, 16, 1, 64, 64, 64, False, "fp16", "fp32"),   # G = 16
    (2, 3, 3, 255, 255, 128, True, "fp16", "bf16"),
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "x".join(map(str, s)))
def test_prefill_small_parity(fa, shape):
    B, Hq, Hkv, Sq, Skv, D, causal, it, ot = shape
    log(f"prefill small {shape}")
    inp = fi.prefill_inputs(20, B, Hq, Hkv, Sq, Skv, D, causal, it, ot)
    o, lse = run(fa, inp)
    ref, ref_lse = oracle.prefill(inp)
    assert_parity(to_f64(o), ref, it, f"prefill {shape}")
    assert_lse(to_f64(lse), ref_lse, f"prefill {shape}", dtype=it)
    if causal and Sq > Skv:
        assert np.all(to_f64(o)[:, :Sq - Skv] == 0.0)


def test_tiny_causal_fp16_fp32_out(fa):
    """Workload 1 in full: B=1, 4 heads, 128 tokens, D=64, fp16 in, fp32 out."""
    inp = fi.workload(1)
    log("workload 1 tiny causal")
    o, lse = run(fa, inp)
    ref, ref_lse = oracle.prefill(inp)
    assert o.dtype.itemsize == 4
    assert_parity(to_f64(o), ref, "fp16", "workload 1")
    assert_lse(to_f64(lse), ref_lse, "workload 1", dtype="fp16")


@pytest.mark.parametrize("splits", ["none", "1", "2", "4", "8", "auto"])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_split_sweep(fa, splits, causal, monkeypatch):
    """Every key-split count gives the oracle's result (the p4 practice of
    checking every value of a tuning knob)."""
    inp = fi.prefill_inputs(21, 1, 4, 2, 256, 2000, 128, causal, "bf16", "bf16")
    if splits not in ("none", "auto"):
        monkeypatch.setenv("FA_PREFILL_SPLITS", splits)
    log(f"prefill split sweep splits={splits} causal={causal}")
    o, lse = run(fa, inp, allow_split=splits != "none")
    ref, ref_lse = oracle.prefill(inp)
    assert_parity(to_f64(o), ref, "bf16", f"splits={splits}")
    assert_lse(to_f64(lse), ref_lse, f"splits={splits}")


WAVE_SHAPES = [s for s in SMALL if s[5] == 128] + [
    (1, 4, 2, 600, 2000, 128, True, "bf16", "bf16"),
    # fp32 output: rows (and fp32 split partials) stored directly, not through LDS
    (1, 4, 2, 333, 900, 128, True, "bf16", "fp32"),
]


@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("splits", ["1", "4"])
@pytest.mark.parametrize("shape", WAVE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_waves(fa, shape, waves, splits, monkeypatch):
    """Head size 128 runs 4- or 8-wave workgroups (128 or 256 query rows); both
    give the oracle's result, with and without key splits."""
    B, Hq, Hkv, Sq, Skv, D, causal, it, ot = shape
    monkeypatch.setenv("FA_PREFILL_WAVES", waves)
    monkeypatch.setenv("FA_PREFILL_SPLITS", splits)
    log(f"prefill waves={waves} splits={splits} {shape}")
    inp = fi.prefill_inputs(22, B, Hq, Hkv, Sq, Skv, D, causal, it, ot)
    o, lse = run(fa, inp)
    ref, ref_lse = oracle.prefill(inp)
    assert_parity(to_f64(o), ref, it, f"waves={waves} splits={splits} {shape}")
    assert_lse(to_f64(lse), ref_lse, f"waves={waves} splits={splits} {shape}")


@pytest.mark.parametrize("splits", ["1", "4"])
@pytest.mark.parametrize("shape", WAVE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_pingpong(fa, shape, splits, monkeypatch):
    """The two-group ping-pong schedule of the 8-wave kernel gives the oracle's
    result too."""
    B, Hq, Hkv, Sq, Skv, D, causal, it, ot = shape
    monkeypatch.setenv("FA_PREFILL_WAVES", "8")
    monkeypatch.setenv("FA_PREFILL_PINGPONG", "1")
    monkeypatch.setenv("FA_PREFILL_SPLITS", splits)
    log(f"prefill ping-pong splits={splits} {shape}")
    inp = fi.prefill_inputs(23, B, Hq, Hkv, Sq, Skv, D, causal, it, ot)
    o, lse = run(fa, inp)
    ref, ref_lse = oracle.prefill(inp)
    assert_parity(to_f64(o), ref, it, f"ping-pong splits={splits} {shape}")
    assert_lse(to_f64(lse), ref_lse, f"ping-pong splits={splits} {shape}")


SCALES = [None, -0.07, 0.0, 0.69, 1.0, -2.0]  # None: 1/sqrt(D)
SCALE_SHAPES = [
    (1, 4, 2, 200, 333, 64, True, "bf16", "bf16"),
    (1, 4, 2, 333, 900, 128, True, "bf16", "bf16"),
    (1, 8, 2, 77, 300, 128, False, "fp16", "fp16"),
    (1, 2, 2, 129, 129, 64, True, "fp16", "fp32"),
]


@pytest.mark.parametrize("splits", ["1", "3"])
@pytest.mark.parametrize("scale", SCALES, ids=lambda s: f"scale={s}")
@pytest.mark.parametrize("shape", SCALE_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_scales(fa, shape, scale, splits, monkeypatch):
    """The unmasked kernel over negative, zero and large scales (a large scale
    makes the softmax peaked, where the rounding of each score matters most),
    with and without key splits. With splits and a 16-bit output the partial
    rows are 16-bit too, and the gate allows their one extra rounding."""
    B, Hq, Hkv, Sq, Skv, D, causal, it, ot = shape
    monkeypatch.setenv("FA_PREFILL_SPLITS", splits)
    inp = fi.prefill_inputs(24, B, Hq, Hkv, Sq, Skv, D, causal, it, ot)
    if scale is not None:
        inp.scale = fi.f32(scale)
    what = f"scale={inp.scale} splits={splits} {shape}"
    log(f"prefill {what}")
    o, lse = run(fa, inp)
    ref, ref_lse = oracle.prefill(inp)
    assert_parity(to_f64(o), ref, it, what, partial_dtype=ot if splits != "1" else None)
    assert_lse(to_f64(lse), ref_lse, what, dtype=it)


def test_prefill_no_keys(fa):
    import torch
    q = torch.randn(1, 40, 2, 64, device="cuda").to(torch.bfloat16)
    k = torch.empty(1, 0, 2, 64, device="cuda", dtype=torch.bfloat16)
    o, lse = fa.prefill(q, k, k.clone(), causal=False, scale=0.125, return_lse=True)
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(lse))


def test_causal_first_query_is_v0_exact(fa):
    """Causal with Sq = Skv: row 0 sees only key 0, with weight exactly 1."""
    inp = fi.prefill_inputs(22, 2, 4, 2, 150, 150, 128, True, "bf16", "bf16")
    o, _ = run(fa, inp)
    got = o[:, 0].view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)
    G = inp.Hq // inp.Hkv
    want = np.repeat(inp.v[:, 0], G, axis=1)
    np.testing.assert_array_equal(got, want)


def test_mha_full_size(fa):
    """Workload 2 in full (non-causal MHA B=4, 16 heads, 2048 tokens, D=64):
    every output element and every lse against the oracle."""
    inp = fi.workload(2)
    log("workload 2 full size")
    o, lse = run(fa, inp)
    ref, ref_lse = oracle.prefill(inp)
    assert_parity(to_f64(o), ref, "bf16", "workload 2")
    assert_lse(to_f64(lse), ref_lse, "workload 2")


@pytest.fixture(scope="module")
def ubatch_run(fa):
    """Workload 3 as the bench runs it: 32 microbatch calls of fa_prefill_ex
    (queries [512u, 512u+512) against keys [0, 512(u+1)), causal bottom-right,
    planner-chosen waves and splits, one workspace), once without lse as the
    bench times it and once with lse; returns (inputs, o, lse) on the host."""
    import torch
    inp = fi.workload(3)
    UB = fi.UBATCH
    q = to_dev(inp.q, "bf16")
    k = to_dev(inp.k, "bf16")
    v = to_dev(inp.v, "bf16")
    n_ub = inp.Sq // UB
    ws_bytes = max(fa.fa_prefill_workspace_size(1, inp.Hq, inp.Hkv, UB, UB * (u + 1), inp.D, 1,
                                                fa.FA_BF16) for u in range(n_ub))
    ws = torch.empty(max(ws_bytes, 16) // 4 + 4, dtype=torch.float32, device="cuda")
    outs = []
    for with_lse in (False, True):
        o = torch.empty_like(q)
        lse = torch.empty((n_ub, 1, inp.Hq, UB), dtype=torch.float32, device="cuda")
        for u in range(n_ub):
            Skv = UB * (u + 1)
            log(f"workload 3 microbatch {u} lse={with_lse}")
            fa.fa_prefill_ex(q[:, UB * u:UB * (u + 1)], k[:, :Skv], v[:, :Skv],
                             o[:, UB * u:UB * (u + 1)], lse[u] if with_lse else None, 1, inp.Hq,
                             inp.Hkv, UB, Skv, inp.D, 1, inp.scale, fa.FA_BF16, fa.FA_BF16, ws,
                             ws_bytes)
        torch.cuda.synchronize()
        outs.append((o, lse))
    # The lse output changes no other result.
    assert torch.equal(outs[0][0], outs[1][0])
    return inp, to_f64(outs[0][0]), to_f64(outs[1][1])


@pytest.mark.parametrize("u", range(32))
def test_gqa_ubatch_full_size(ubatch_run, u):
    """Workload 3 in full, microbatch u: all 512 x 32 output rows and their lse
    against the oracle's causal attention over the whole 16384-token sequence
    (rows 512u .. 512u + 511; under the bottom-right reading microbatch u
    computes exactly those rows)."""
    inp, o, lse = ubatch_run
    UB = fi.UBATCH
    rows = np.array([(0, h, i) for i in range(UB * u, UB * (u + 1)) for h in range(inp.Hq)])
    ref, ref_lse = oracle.prefill_rows(inp, rows)
    got = o[0, UB * u:UB * (u + 1)].reshape(-1, inp.D)  # rows in (i, h) order, as `rows`
    assert_parity(got, ref, "bf16", f"workload 3 microbatch {u}")
    got_lse = lse[u, 0].T.reshape(-1)  # [Hq, 512] -> (i, h) order
    assert_lse(got_lse, ref_lse, f"workload 3 microbatch {u}")


# --------------------------------------------------------------------------
# explicit additive mask (fa_prefill_mask)
# --------------------------------------------------------------------------

def run_masked(fa, inp, *, stride_pad=0):
    """Runs fa.prefill with inp.mask (bits [Bm, Sq, W]); W is the mask's own
    row stride (Skv rounded up to 8 plus padding, NaN-poisoned past Skv)."""
    import torch
    q, k, v = (to_dev(x, inp.in_dtype) for x in (inp.q, inp.k, inp.v))
    m = to_dev(inp.mask, inp.in_dtype)
    if m.shape[0] == 1:
        m = m[0]
    res = fa.prefill(q, k, v, causal=inp.causal, scale=inp.scale,
                     out_dtype=_dtype_torch(inp.out_dtype), return_lse=True, mask=m)
    torch.cuda.synchronize()
    return res


def _mask_inputs(c, shape, kind, batched=False, pad=0):
    B, Hq, Hkv, Sq, Skv, D, causal, it, ot = shape
    inp = fi.prefill_inputs(c, B, Hq, Hkv, Sq, Skv, D, causal, it, ot)
    stride = (Skv + 7) // 8 * 8 + pad
    return fi.with_mask(inp, c, kind, batched=batched, stride=stride)


MASK_SHAPES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, in, out
    (1, 4, 2, 200, 333, 128, False, "bf16", "bf16"),
    (1, 4, 2, 200, 333, 128, True, "bf16", "bf16"),
    (2, 4, 4, 130, 67, 64, False, "fp16", "fp16"),
    (1, 2, 1, 96, 250, 64, True, "bf16", "fp32"),
    (1, 32, 8, 512, 1536, 128, True, "bf16", "bf16"),  # 8-wave workgroups, split keys
]


@pytest.mark.parametrize("kind", ["normal", "packed", "bias", "rows"])
@pytest.mark.parametrize("shape", MASK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_mask_parity(fa, shape, kind):
    """softmax(scale Q K^T + M) V for random, packed-sequence, distance-bias and
    hidden-row masks (one shared [Sq, W] matrix, W padded with NaN past Skv)."""
    log(f"prefill mask {kind} {shape}")
    inp = _mask_inputs(60, shape, kind, pad=8)
    o, lse = run_masked(fa, inp)
    ref, ref_lse = oracle.prefill(inp)
    assert_parity(to_f64(o), ref, shape[7], f"mask {kind} {shape}")
    assert_lse(to_f64(lse), ref_lse, f"mask {kind} {shape}", dtype=shape[7])
    if kind == "rows":  # fully hidden rows give exactly 0 and -inf
        hidden = np.isneginf(ref_lse)
        assert hidden.any() and np.all(to_f64(o).transpose(0, 2, 1, 3)[hidden] == 0)


def test_prefill_mask_batched_and_scales(fa):
    """One mask per batch entry; scale 0 (softmax of the mask alone) and a
    negative scale."""
    shape = (3, 4, 2, 100, 150, 128, False, "bf16", "bf16")
    for scale in (None, 0.0, -0.07):
        inp = _mask_inputs(61, shape, "normal", batched=True)
        if scale is not None:
            inp.scale = fi.f32(scale)
        log(f"prefill batched mask scale={inp.scale}")
        o, lse = run_masked(fa, inp)
        ref, ref_lse = oracle.prefill(inp)
        assert_parity(to_f64(o), ref, "bf16", f"batched mask scale={inp.scale}")
        assert_lse(to_f64(lse), ref_lse, f"batched mask scale={inp.scale}")


@pytest.mark.parametrize("waves,splits", [("4", "1"), ("4", "4"), ("8", "1"), ("8", "3")])
def test_prefill_mask_waves_and_splits(fa, waves, splits, monkeypatch):
    """Both workgroup shapes and forced split counts with a mask (the split
    partials carry base-2 maxima through the lse)."""
    monkeypatch.setenv("FA_PREFILL_WAVES", waves)
    monkeypatch.setenv("FA_PREFILL_SPLITS", splits)
    shape = (1, 4, 2, 600, 2000, 128, True, "bf16", "bf16")
    inp = _mask_inputs(62, shape, "bias")
    log(f"prefill mask waves={waves} splits={splits}")
    o, lse = run_masked(fa, inp)
    ref, ref_lse = oracle.prefill(inp)
    assert_parity(to_f64(o), ref, "bf16", f"mask waves={waves} splits={splits}")
    assert_lse(to_f64(lse), ref_lse, f"mask waves={waves} splits={splits}")


def test_prefill_zero_mask_equals_unmasked(fa):
    """An all-zero mask gives the unmasked kernel's result up to the one extra
    rounding of the exponent argument."""
    import torch
    shape = (1, 8, 2, 300, 700, 128, True, "bf16", "bf16")
    inp = fi.prefill_inputs(63, *shape)
    q, k, v = (to_dev(x, "bf16") for x in (inp.q, inp.k, inp.v))
    zero = torch.zeros((300, 704), dtype=torch.bfloat16, device=q.device)  # rows of 8k
    o0 = fa.prefill(q, k, v, causal=True, scale=inp.scale)
    o1 = fa.prefill(q, k, v, causal=True, scale=inp.scale, mask=zero)
    torch.cuda.synchronize()
    assert_parity(to_f64(o1), to_f64(o0).astype(np.float64), "bf16", "zero mask vs none")


# --------------------------------------------------------------------------
# head packs: a workgroup takes PK query heads of one K/V head
# --------------------------------------------------------------------------

PACK_SHAPES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, in, out
    (1, 8, 2, 200, 333, 128, True, "bf16", "bf16"),     # G = 4, ragged
    (2, 16, 2, 130, 700, 128, False, "bf16", "bf16"),   # G = 8
    (1, 6, 3, 129, 400, 64, True, "fp16", "fp32"),      # G = 2, head size 64
    (1, 32, 8, 512, 1536, 128, True, "bf16", "bf16"),   # a workload-3 microbatch
    (1, 4, 1, 40, 30, 128, True, "bf16", "bf16"),       # Sq > Skv: leading rows see nothing
]


@pytest.mark.parametrize("masked", [False, True], ids=["nomask", "mask"])
@pytest.mark.parametrize("splits", ["auto", "3"])
@pytest.mark.parametrize("pack", ["1", "2", "4", "8"])
@pytest.mark.parametrize("waves", ["4", "8"])
@pytest.mark.parametrize("shape", PACK_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_head_pack(fa, shape, waves, pack, splits, masked, monkeypatch):
    """Every head pack the shape allows (PK query heads of one K/V head per
    workgroup, the mask tile copied once for them into a shared ring), with
    and without an additive mask, both workgroup shapes and split counts, gives
    the oracle's result. A pack the shape does not allow falls back to the
    planner's."""
    monkeypatch.setenv("FA_PREFILL_WAVES", waves)
    monkeypatch.setenv("FA_PREFILL_PACK", pack)
    if splits != "auto":
        monkeypatch.setenv("FA_PREFILL_SPLITS", splits)
    B, Hq, Hkv, Sq, Skv, D, causal, it, ot = shape
    log(f"prefill pack={pack} waves={waves} splits={splits} mask={masked} {shape}")
    if masked:
        inp = _mask_inputs(64, shape, "bias", pad=8)
        o, lse = run_masked(fa, inp)
    else:
        inp = fi.prefill_inputs(64, *shape)
        o, lse = run(fa, inp)
    ref, ref_lse = oracle.prefill(inp)
    what = f"pack={pack} waves={waves} splits={splits} mask={masked} {shape}"
    assert_parity(to_f64(o), ref, it, what)
    assert_lse(to_f64(lse), ref_lse, what, dtype=it)
