"""The decode entry point that allocates nothing (fa_decode_paged_noalloc),
through the C ABI: its output equals fa_decode_paged's with a caller workspace
bit for bit, and the oracle's within the parity bar, on calls in a row whose
later inputs are smaller (the library's static scratch keeps the previous
call's contents); a plan too large for the scratch is refused on the host."""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from helpers import assert_lse, assert_parity, i32_dev, log, to_dev, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import flashattention_forward_amd as fa
    return fa


def _both(fa, inp):
    """(noalloc o, lse), (fa_decode_paged o, lse) on the same device inputs."""
    import torch
    mla = inp.layout == "mla"
    layout = fa.FA_KV_MLA_SHARED if mla else fa.FA_KV_SPLIT
    Hkv, D_qk, D_v = (1, 576, 512) if mla else (inp.Hkv, 128, 128)
    q, pool = to_dev(inp.q, inp.dtype), to_dev(inp.pool, inp.dtype)
    pt, sl = i32_dev(inp.page_table), i32_dev(inp.seq_lens)
    dt = fa.FA_BF16 if inp.dtype == "bf16" else fa.FA_FP16
    outs = []
    for noalloc in (True, False):
        o = torch.full((inp.B, inp.Hq, D_v), float("nan"), dtype=q.dtype, device=q.device)
        lse = torch.full((inp.B, inp.Hq), float("nan"), dtype=torch.float32, device=q.device)
        args = (q, pool, pt, sl, pool.shape[0], o, lse, inp.B, inp.Hq, Hkv, D_qk, D_v,
                inp.page_size, pt.shape[1], inp.max_seq_len, layout, inp.scale, 0, dt)
        if noalloc:
            fa.fa_decode_paged_noalloc(*args)
        else:
            nbytes = fa.fa_decode_workspace_size(inp.B, inp.Hq, Hkv, D_qk, D_v, inp.page_size,
                                                 inp.max_seq_len, layout, 0)
            ws = torch.empty(max(nbytes, 16) // 4 + 4, dtype=torch.float32, device=q.device)
            fa.fa_decode_paged(*args, ws, nbytes)
        torch.cuda.synchronize()
        outs.append((o, lse))
    return outs


def _check(fa, inp, what):
    import torch
    (o1, l1), (o2, l2) = _both(fa, inp)
    assert torch.equal(o1, o2), f"{what}: noalloc output differs from fa_decode_paged"
    assert torch.equal(l1.isneginf(), l2.isneginf())
    fin = ~l2.isneginf()
    assert torch.equal(l1[fin], l2[fin]), f"{what}: noalloc lse differs"
    ref, ref_lse = oracle.decode_paged(inp)
    assert_parity(to_f64(o1), ref, inp.dtype, what)
    assert_lse(to_f64(l1), ref_lse, what, dtype=inp.dtype)


def test_noalloc_matches_workspace_entry_point(fa):
    """Three calls in a row: MLA at full size (batch 128 x 64 heads x 2048
    tokens, two splits: 16.8 MB of the scratch), then a smaller ragged MLA
    batch (the scratch still holds the first call's partials), then a small
    grouped-query batch."""
    big = fi.workload(4)
    assert fa.fa_decode_num_splits(128, 64, 1, 576, 512, 1, 2048, fa.FA_KV_MLA_SHARED) > 1
    log("noalloc: MLA workload 4")
    _check(fa, big, "noalloc MLA 128 x 2048")
    small = fi.mla_decode_inputs(90, 6, 64, 320, page_size=1)
    small.seq_lens = np.array([320, 1, 77, 0, 250, 299], dtype=np.int32)
    log("noalloc: small ragged MLA batch")
    _check(fa, small, "noalloc MLA small ragged")
    gqa = fi.split_decode_inputs(91, 3, 16, 4, 128, [1500, 33, 700], 16)
    log("noalloc: small GQA batch")
    _check(fa, gqa, "noalloc GQA small")


def test_noalloc_refuses_plan_beyond_scratch(fa):
    """A split plan whose partials exceed the static scratch is refused before
    anything is enqueued (the pointers are never dereferenced)."""
    A = 1 << 20
    need = fa.fa_decode_workspace_size(2048, 64, 1, 576, 512, 1, 8192, fa.FA_KV_MLA_SHARED, 16)
    assert need > (32 << 20)
    with pytest.raises(fa.FaError) as e:
        fa.fa_decode_paged_noalloc(A, A, A, A, 10, A, None, 2048, 64, 1, 576, 512, 1, 8192, 8192,
                                   fa.FA_KV_MLA_SHARED, 0.1, 16, fa.FA_BF16, stream=0)
    assert e.value.status == -7
