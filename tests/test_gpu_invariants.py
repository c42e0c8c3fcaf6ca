"""GPU checks of properties the attention forward pass has whatever the inputs,
independent of the oracle (through the C ABI):

- every value row equal to one vector v: each output row is v (the softmax
  weights sum to one), up to one rounding of the 16-bit output;
- one key whose score exceeds every other by far: the output row is that
  key's value row, up to one rounding;
- without a mask the keys may be permuted (with their value rows): the output
  changes only by rounding order;
- paged decode with constant value rows: the same as the first, through the
  page table, with and without key splits.

The bound "one rounding of the output" is one ulp of v: |o - v| <= 2^-7 |v|
for bf16 and 2^-10 |v| for fp16. (The fp32 weights and their sum differ only
by summation order, a relative 1e-6, so in practice o rounds back to v
exactly.)
"""
import dataclasses

import numpy as np
import pytest

import fa_inputs as fi
from helpers import i32_dev, log, metrics, to_dev, to_f64

pytestmark = pytest.mark.gpu

REL = {"bf16": 2.0 ** -7, "fp16": 2.0 ** -10}  # one ulp, for the final rounding


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import flashattention_forward_amd as fa
    return fa


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return bits.view(np.float16).astype(np.float64)


def prefill(fa, inp):
    import torch
    o, lse = fa.prefill(to_dev(inp.q, inp.in_dtype), to_dev(inp.k, inp.in_dtype),
                        to_dev(inp.v, inp.in_dtype), causal=inp.causal, scale=inp.scale,
                        return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


def assert_rows_equal(got, want, dtype, what):
    err = np.abs(got - want)
    bound = REL[dtype] * np.abs(want) + 1e-30
    worst = float((err / bound).max())
    log(f"{what}: worst error / one ulp = {worst:.3f}")
    assert np.isfinite(got).all(), what
    assert (err <= bound).all(), f"{what}: error beyond one output rounding ({worst:.3f} ulp)"


CONST_SHAPES = [
    # B, Hq, Hkv, Sq, Skv, D, causal, dtype
    (2, 8, 2, 200, 700, 128, True, "bf16"),
    (1, 4, 4, 333, 333, 64, False, "bf16"),
    (1, 32, 8, 512, 4096, 128, True, "bf16"),  # a late-microbatch shape (key splits)
    (2, 6, 3, 97, 150, 128, False, "fp16"),
]


@pytest.mark.parametrize("shape", CONST_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_prefill_constant_value_rows(fa, shape):
    B, Hq, Hkv, Sq, Skv, D, causal, dt = shape
    log(f"constant value rows {shape}")
    inp = fi.prefill_inputs(60, B, Hq, Hkv, Sq, Skv, D, causal, dt, dt)
    vstar = fi.normal_bits((B, 1, Hkv, D), dt, fi.rng_for(60, 99))
    inp = dataclasses.replace(inp, v=np.ascontiguousarray(np.broadcast_to(vstar, inp.v.shape)))
    o, _ = prefill(fa, inp)
    want = np.repeat(bits_to_f64(vstar, dt), Hq // Hkv, axis=2)  # [B, 1, Hq, D]
    assert_rows_equal(o, np.broadcast_to(want, o.shape), dt, f"constant V {shape}")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_one_dominant_key(fa, D):
    """q = 16 k_j for a chosen key j per query row: its score (2 |k_j|^2 at
    D = 64) exceeds every other by more than 30, so the other keys carry less
    than e^-30 of the weight and o = v_j."""
    B, Hq, Hkv, Sq, Skv = 2, 8, 2, 150, 333
    inp = fi.prefill_inputs(61, B, Hq, Hkv, Sq, Skv, D, False)
    r = np.random.default_rng(61)
    j = r.integers(0, Skv, size=(B, Sq, Hq))
    G = Hq // Hkv
    bi = np.arange(B)[:, None, None]
    gi = (np.arange(Hq) // G)[None, None, :]
    kf = bits_to_f64(inp.k, "bf16")
    q = fi.round_bits((16.0 * kf[bi, j, gi]).astype(np.float32), "bf16")  # exact: a power of 2
    inp = dataclasses.replace(inp, q=q)
    o, _ = prefill(fa, inp)
    want = bits_to_f64(inp.v, "bf16")[bi, j, gi]
    assert_rows_equal(o, want, "bf16", f"one dominant key D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_prefill_key_permutation(fa, D):
    """Non-causal: permuting the keys together with their value rows leaves
    the output unchanged up to rounding order."""
    B, Hq, Hkv, Sq, Skv = 2, 8, 2, 300, 1000
    inp = fi.prefill_inputs(62, B, Hq, Hkv, Sq, Skv, D, False)
    perm = np.random.default_rng(62).permutation(Skv)
    inp_p = dataclasses.replace(inp, k=np.ascontiguousarray(inp.k[:, perm]),
                                v=np.ascontiguousarray(inp.v[:, perm]))
    o, lse = prefill(fa, inp)
    o_p, lse_p = prefill(fa, inp_p)
    m = metrics(o_p, o)
    log(f"key permutation D={D}: {m}")
    assert m["max_abs"] <= 8e-3 and m["mean_abs"] <= 2e-4, m
    assert np.abs(lse_p - lse).max() <= 5e-3


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_decode_constant_value_rows(fa, splits):
    """GQA paged decode (page size 16, ragged lengths): every value row of K/V
    head g is one vector v_g, so every output row of a non-empty sequence is
    v_g of its group."""
    import torch
    Hq, Hkv, D = 32, 8, 128
    lens = [1500, 1, 333, 0, 4096]
    inp = fi.split_decode_inputs(63, len(lens), Hq, Hkv, D, lens, 16)
    vstar = fi.normal_bits((Hkv, D), "bf16", fi.rng_for(63, 99))
    pool = inp.pool.copy()
    pool[:, 1] = vstar[None, :, None, :]  # [P, 2 (K, V), Hkv, page, D]
    o, lse = fa.decode_paged(to_dev(inp.q, "bf16"), to_dev(pool, "bf16"),
                             i32_dev(inp.page_table), i32_dev(inp.seq_lens),
                             layout=fa.FA_KV_SPLIT, scale=inp.scale,
                             max_seq_len=inp.max_seq_len, page_size=16, num_splits=splits,
                             return_lse=True)
    torch.cuda.synchronize()
    o = to_f64(o)
    want = np.repeat(bits_to_f64(vstar, "bf16"), Hq // Hkv, axis=0)  # [Hq, D]
    live = np.array(lens) > 0
    assert_rows_equal(o[live], np.broadcast_to(want, o[live].shape), "bf16",
                      f"decode constant V splits={splits}")
    assert np.all(o[~live] == 0)
