"""LDS-race debug build against the fast build, bit for bit.

libfa_ldsdebug.so is compiled from the same sources with -DFA_LDS_DEBUG=1:
every LDS hand-off also waits for all outstanding memory operations
(global-to-LDS copies included), partial vmcnt waits wait for everything, and
the loops over workgroup-shared K/V stages end each step with a full barrier.
The arithmetic and its order are the same, so outputs and log-sum-exps must be
identical to the fast library's. A stage read before its copy landed, or
overwritten while another wave still reads it, shows up as a difference (and,
run to run, as nondeterminism, which the second fast call checks).

Both libraries are called through the same Python wrappers: the test points
the binding's library handle at the debug build for the second call.
"""
import ctypes
import os

import numpy as np
import pytest

import fa_inputs as fi
from helpers import i32_dev, log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def libs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import flashattention_forward_amd as fa
    path = os.path.join(os.path.dirname(fa.LIB_PATH), "libfa_ldsdebug.so")
    assert os.path.exists(path), f"{path} is not built (flashattention_forward_amd/build.py)"
    dbg = ctypes.CDLL(path)
    for name in ("fa_prefill_ex", "fa_prefill_mask", "fa_prefill_workspace_size",
                 "fa_decode_paged", "fa_decode_paged_multi", "fa_decode_workspace_size",
                 "fa_decode_multi_workspace_size", "fa_strerror"):
        fast_fn, dbg_fn = getattr(fa._lib, name), getattr(dbg, name)
        dbg_fn.argtypes, dbg_fn.restype = fast_fn.argtypes, fast_fn.restype
    return fa, dbg


def _bits(t):
    import torch
    torch.cuda.synchronize()
    x = t.detach().cpu()
    if x.dtype == torch.float32:
        return x.view(torch.int32).numpy().copy()
    return x.view(torch.int16).numpy().copy()


def three_runs(libs, monkeypatch, call, what):
    """fast, debug, fast again: all three bit-identical."""
    fa, dbg = libs
    fast = fa._lib
    outs = []
    for lib in (fast, dbg, fast):
        monkeypatch.setattr(fa, "_lib", lib)
        res = call(fa)
        outs.append([_bits(r) for r in res if r is not None])
    monkeypatch.setattr(fa, "_lib", fast)
    names = ["o", "lse"]
    for i, (a, b, c) in enumerate(zip(*outs)):
        assert np.array_equal(a, c), f"{what}: fast build not deterministic ({names[i]})"
        diff = int((a != b).sum())
        log(f"{what}: {names[i]} {a.size} values, {diff} differ from the LDS debug build")
        assert diff == 0, f"{what}: LDS debug build differs in {diff} of {a.size} {names[i]} values"


PREFILL_CASES = [
    # (B, Hq, Hkv, Sq, Skv, D, causal, in, out, mask kind, env)
    (1, 32, 8, 512, 4196, 128, True, "bf16", "bf16", None, {}),
    (2, 16, 16, 300, 777, 64, False, "bf16", "bf16", None, {}),
    (1, 4, 4, 128, 128, 64, True, "fp16", "fp32", None, {}),
    (2, 16, 4, 200, 900, 128, True, "bf16", "bf16", "normal", {}),
    (2, 16, 4, 200, 900, 128, True, "bf16", "bf16", "normal", {"FA_PREFILL_PACK": "1"}),
    (1, 8, 2, 333, 2000, 128, False, "bf16", "fp32", "bias", {"FA_PREFILL_WAVES": "4"}),
    (1, 8, 8, 512, 1500, 128, True, "bf16", "bf16", None,
     {"FA_PREFILL_PINGPONG": "1", "FA_PREFILL_WAVES": "8"}),
    (1, 8, 8, 512, 1500, 128, True, "bf16", "bf16", None, {"FA_PREFILL_SPLITS": "5"}),
]


@pytest.mark.parametrize("case", PREFILL_CASES,
                         ids=lambda c: "x".join(map(str, c[:6])) + f"-c{int(c[6])}-{c[7]}-{c[8]}"
                         f"-{c[9]}-" + ",".join(f"{k[3:]}={v}" for k, v in c[10].items()))
def test_prefill_lds_debug_bitwise(libs, monkeypatch, case):
    import torch
    B, Hq, Hkv, Sq, Skv, D, causal, ind, outd, mkind, env = case
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    log(f"lds debug prefill {case}")
    inp = fi.prefill_inputs(71, B, Hq, Hkv, Sq, Skv, D, causal, ind, outd)
    q, k, v = (to_dev(x, ind) for x in (inp.q, inp.k, inp.v))
    mask = None
    if mkind:
        stride = (Skv + 7) // 8 * 8
        mask = to_dev(fi.additive_mask(72, B, Sq, Skv, mkind, ind, stride), ind)
    out_t = torch.float32 if outd == "fp32" else q.dtype

    def call(fa):
        return fa.prefill(q, k, v, causal=causal, scale=inp.scale, out_dtype=out_t,
                          return_lse=True, mask=mask)

    three_runs(libs, monkeypatch, call, f"prefill {case[:10]}")


DECODE_CASES = [
    # (layout, B, Sq, Hq, Hkv, lens or seq_len, page_size, num_splits, env)
    ("split", 4, 1, 32, 8, [1500, 1, 333, 4096], 16, 0, {}),
    ("split", 4, 1, 32, 8, [1500, 1, 333, 4096], 16, 1, {}),
    ("split", 3, 4, 32, 8, [700, 64, 2500], 5, 0, {}),
    ("mla", 8, 1, 64, 1, 1024, 1, 0, {}),
    ("mla", 8, 1, 64, 1, 1024, 16, 3, {}),
    ("mla", 8, 1, 64, 1, 1024, 1, 0, {"FA_MLA_HEADS": "32"}),
    ("mla", 4, 2, 64, 1, 640, 1, 0, {}),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: "-".join(
    str(x) if not isinstance(x, (list, dict)) else
    ("L" + str(len(x)) if isinstance(x, list) else ",".join(f"{k[3:]}={v}" for k, v in x.items()))
    for x in c))
def test_decode_lds_debug_bitwise(libs, monkeypatch, case):
    layout, B, Sq, Hq, Hkv, lens, ps, ns, env = case
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    fa = libs[0]
    log(f"lds debug decode {case}")
    if layout == "mla":
        inp = fi.mla_decode_inputs(73, B, Hq, lens, page_size=ps, Sq=Sq)
        lay = fa.FA_KV_MLA_SHARED
    else:
        inp = fi.split_decode_inputs(74, B, Hq, Hkv, 128, lens, ps, Sq=Sq)
        lay = fa.FA_KV_SPLIT
    q, pool = to_dev(inp.q, "bf16"), to_dev(inp.pool, "bf16")
    pt, sl = i32_dev(inp.page_table), i32_dev(inp.seq_lens)

    def call(fa):
        return fa.decode_paged(q, pool, pt, sl, layout=lay, scale=inp.scale,
                               max_seq_len=inp.max_seq_len, page_size=ps, num_splits=ns,
                               return_lse=True)

    three_runs(libs, monkeypatch, call, f"decode {case[:8]}")
