"""GPU parity of paged decode (grouped-query split pool and MLA shared pool)
against the CPU oracle, through the C ABI. Covers ragged and empty sequences,
page sizes 1 / 16 / odd, NaN-poisoned unused slots, every split count, and the
two full-size workloads (MLA batch 128 x 2048 tokens; GQA batch 4 with lengths
U[1024, 32768]) in the bench's launch configuration, every sequence and every
output element."""
import dataclasses

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


def run(fa, inp, num_splits=0, dev=None):
    import torch
    if dev is None:
        dev = (to_dev(inp.q, inp.dtype), to_dev(inp.pool, inp.dtype), i32_dev(inp.page_table),
               i32_dev(inp.seq_lens))
    q, pool, pt, sl = dev
    layout = fa.FA_KV_MLA_SHARED if inp.layout == "mla" else fa.FA_KV_SPLIT
    o, lse = fa.decode_paged(q, pool, pt, sl, layout=layout, scale=inp.scale,
                             max_seq_len=inp.max_seq_len, page_size=inp.page_size, D_v=inp.D_v,
                             num_splits=num_splits, return_lse=True)
    torch.cuda.synchronize()
    return to_f64(o), to_f64(lse)


def check(fa, inp, what, num_splits=0, batches=None):
    o, lse = run(fa, inp, num_splits)
    ref, ref_lse = oracle.decode_paged(inp, batches)
    sel = slice(None) if batches is None else list(batches)
    assert_parity(o[sel], ref, inp.dtype, what)
    assert_lse(lse[sel], ref_lse, what, dtype=inp.dtype)
    return o, lse


# --------------------------------------------------------------------------
# grouped-query decode, split K/V pool
# --------------------------------------------------------------------------

@pytest.mark.parametrize("page_size", [16, 1, 5])
@pytest.mark.parametrize("G", [4, 1, 16, 20])
def test_gqa_decode_small(fa, page_size, G):
    Hkv = 2
    lens = [1, 50, 333, 31]
    inp = fi.split_decode_inputs(30 + G, 4, G * Hkv, Hkv, 128, lens, page_size)
    log(f"gqa decode page={page_size} G={G}")
    check(fa, inp, f"gqa page={page_size} G={G}")


@pytest.mark.parametrize("splits", [1, 5, 0])
@pytest.mark.parametrize("Hkv,G,page_size", [(3, 2, 16), (5, 4, 5), (7, 1, 16)])
def test_gqa_decode_odd_kv_heads(fa, Hkv, G, page_size, splits):
    """K/V head counts that do not divide a workgroup's 8 waves: a workgroup
    then holds units of several key ranges and sequences (units are numbered
    with the K/V head fastest), and the last one is partly empty."""
    lens = [777, 1, 1500, 96, 0]
    inp = fi.split_decode_inputs(48 + Hkv, 5, G * Hkv, Hkv, 128, lens, page_size)
    log(f"gqa decode Hkv={Hkv} G={G} page={page_size} splits={splits}")
    check(fa, inp, f"gqa Hkv={Hkv} G={G} page={page_size} splits={splits}", num_splits=splits)


@pytest.mark.parametrize("splits", [1, 2, 3, 8, 24, 0])
def test_gqa_decode_split_sweep(fa, splits):
    inp = fi.split_decode_inputs(40, 3, 8, 2, 128, [1500, 700, 64], 16)
    log(f"gqa decode splits={splits}")
    check(fa, inp, f"gqa splits={splits}", num_splits=splits)


@pytest.mark.parametrize("splits", [1, 4])
def test_gqa_decode_scale_zero(fa, splits):
    """scale 0: every visible token has the same weight, and masked slots (past
    a split's end) must still weigh 0, not NaN."""
    inp = dataclasses.replace(fi.split_decode_inputs(44, 3, 8, 2, 128, [1500, 700, 64], 16),
                              scale=0.0)
    log(f"gqa decode scale 0 splits={splits}")
    check(fa, inp, f"gqa scale 0 splits={splits}", num_splits=splits)


@pytest.mark.parametrize("Sq", [1, 2])
def test_mla_decode_scale_zero(fa, Sq):
    inp = dataclasses.replace(fi.mla_decode_inputs(45, 3, 16, 1000, Sq=Sq), scale=0.0)
    log(f"mla decode scale 0 Sq={Sq}")
    check(fa, inp, f"mla scale 0 Sq={Sq}")


def test_gqa_decode_fp16(fa):
    inp = fi.split_decode_inputs(41, 2, 16, 4, 128, [1000, 129], 16, dtype="fp16")
    check(fa, inp, "gqa fp16")


def test_gqa_decode_empty_sequence(fa):
    inp = fi.split_decode_inputs(42, 3, 8, 2, 128, [0, 40, 0], 16)
    o, lse = check(fa, inp, "gqa empty")
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


def test_gqa_decode_page_permutation_bit_exact(fa):
    """Moving pages to other physical slots (same logical order) changes nothing."""
    inp = fi.split_decode_inputs(43, 2, 8, 2, 128, [900, 400], 16, poison=False)
    o1, l1 = run(fa, inp)
    perm = np.random.default_rng(1).permutation(inp.pool.shape[0])
    inv = np.argsort(perm)
    inp2 = fi.DecodeInputs(**{**inp.__dict__})
    inp2.pool = inp.pool[perm]  # new slot j holds old page perm[j]
    inp2.page_table = np.where(inp.page_table >= 0, inv[np.maximum(inp.page_table, 0)], -1)
    inp2.page_table = inp2.page_table.astype(np.int32)
    o2, l2 = run(fa, inp2)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("page_size", [16, 5])
def test_gqa_decode_pool_beyond_4gib(fa, page_size):
    """Page offsets past 4 GiB: the sequences' pages sit at the top of a pool of
    about 4.6 GB (8 K/V heads; pages of 64 KB at page size 16), so a row's byte
    offset needs more than 32 bits. The oracle reads the same pages from a
    compact host copy."""
    import torch
    lens = [300, 700]
    inp = fi.split_decode_inputs(46, 2, 32, 8, 128, lens, page_size, spare_pages=0)
    n_used = inp.pool.shape[0]
    page_bytes = inp.pool[0].nbytes
    n_total = (4 << 30) // page_bytes + 4096  # the top pages start past 4 GiB
    base = n_total - n_used
    log(f"pool of {n_total} pages x {page_bytes} B = {n_total * page_bytes / 1e9:.2f} GB, "
        f"used pages from {base}")
    big = torch.empty((n_total,) + inp.pool.shape[1:], dtype=torch.bfloat16, device="cuda")
    big[base:] = to_dev(inp.pool, "bf16")
    pt = np.where(inp.page_table >= 0, inp.page_table + base, -1).astype(np.int32)
    o, lse = fa.decode_paged(to_dev(inp.q, "bf16"), big, i32_dev(pt), i32_dev(inp.seq_lens),
                             layout=fa.FA_KV_SPLIT, scale=inp.scale, max_seq_len=inp.max_seq_len,
                             page_size=page_size, return_lse=True)
    torch.cuda.synchronize()
    del big
    ref, ref_lse = oracle.decode_paged(inp)
    assert_parity(to_f64(o), ref, "bf16", f"pool beyond 4 GiB, page {page_size}")
    assert_lse(to_f64(lse), ref_lse, "pool beyond 4 GiB")


def test_gqa_decode_full_size(fa):
    """Workload 5 in full: batch 4, 32 query / 8 K/V heads, lengths U[1024, 32768],
    page_size 16, NaN in every unused slot; planner-chosen split count."""
    inp = fi.workload(5)
    log(f"workload 5 lens={inp.seq_lens.tolist()}")
    check(fa, inp, "workload 5")


# --------------------------------------------------------------------------
# several new tokens per sequence (fa_decode_paged_multi)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("Sq,G,page_size", [(2, 4, 16), (4, 1, 16), (7, 8, 5), (16, 4, 1),
                                            (64, 2, 16), (5, 16, 16)])
def test_gqa_decode_multi_token(fa, Sq, G, page_size):
    """Sq new tokens packed with the group's heads into the MFMA rows; lengths
    include one shorter than Sq (its first rows see no key) and a ragged tail."""
    Hkv = 2
    lens = [333, 3, 1200, 40]
    inp = fi.split_decode_inputs(70 + Sq, 4, G * Hkv, Hkv, 128, lens, page_size, Sq=Sq)
    log(f"gqa decode multi Sq={Sq} G={G} page={page_size}")
    o, lse = check(fa, inp, f"gqa multi Sq={Sq} G={G} page={page_size}")
    if Sq > 3:
        assert np.all(o[1, :Sq - 3] == 0) and np.all(np.isneginf(lse[1, :, :Sq - 3]))


@pytest.mark.parametrize("splits", [1, 3, 0])
def test_gqa_decode_multi_token_splits(fa, splits):
    inp = fi.split_decode_inputs(77, 2, 16, 4, 128, [2000, 777], 16, Sq=4, dtype="fp16")
    log(f"gqa decode multi splits={splits}")
    check(fa, inp, f"gqa multi splits={splits}", num_splits=splits)


# --------------------------------------------------------------------------
# MLA decode, shared [ckv | kpe] pool
# --------------------------------------------------------------------------

def _mla_ragged(c, B, Hq, max_len, page_size, lens, dtype="bf16"):
    inp = fi.mla_decode_inputs(c, B, Hq, max_len, page_size=page_size, dtype=dtype)
    inp.seq_lens = np.asarray(lens, dtype=np.int32)
    return inp


@pytest.mark.parametrize("Hq", [64, 16, 128, 48])
def test_mla_decode_small(fa, Hq):
    inp = _mla_ragged(50, 3, Hq, 320, 1, [320, 33, 1])
    log(f"mla decode Hq={Hq}")
    check(fa, inp, f"mla Hq={Hq}")


@pytest.mark.parametrize("page_size", [16, 5])
def test_mla_decode_page_sizes(fa, page_size):
    inp = _mla_ragged(51, 2, 64, 640, page_size, [640, 411])
    check(fa, inp, f"mla page={page_size}")


@pytest.mark.parametrize("splits", [1, 2, 4, 7, 16, 0])
def test_mla_decode_split_sweep(fa, splits):
    inp = _mla_ragged(52, 2, 64, 1024, 1, [1024, 999])
    log(f"mla splits={splits}")
    check(fa, inp, f"mla splits={splits}", num_splits=splits)


@pytest.mark.parametrize("heads", ["32", "64"])
@pytest.mark.parametrize("case", [(64, 1, 1, "bf16"), (48, 5, 3, "bf16"), (128, 16, 2, "fp16"),
                                  (16, 1, 1, "bf16")])
def test_mla_decode_heads_per_workgroup(fa, heads, case, monkeypatch):
    """Both workgroup shapes (64 heads sharing each tile, or 32 heads taking the
    two tiles of a 64-token step and merging at the end) on ragged lengths,
    partial head blocks, page sizes 1 / 5 / 16 and split counts 1-3."""
    Hq, page_size, splits, dtype = case
    monkeypatch.setenv("FA_MLA_HEADS", heads)
    inp = _mla_ragged(56, 3, Hq, 720, page_size, [720, 63, 97], dtype=dtype)
    log(f"mla heads/wg={heads} Hq={Hq} page={page_size} splits={splits} {dtype}")
    check(fa, inp, f"mla heads/wg={heads} Hq={Hq}", num_splits=splits)


@pytest.mark.parametrize("heads", ["32", "64"])
def test_mla_decode_long_single_split(fa, heads, monkeypatch):
    """5000 tokens (157 tiles, ragged tail) with one split requested: 32 heads per
    workgroup read the page table per step and take it in one split; 64 heads
    hold a split's row ids in LDS, at most 2048 tokens, so the planner uses 3."""
    monkeypatch.setenv("FA_MLA_HEADS", heads)
    inp = _mla_ragged(57, 1, 64, 5000, 1, [5000])
    log(f"mla long single split heads/wg={heads}")
    check(fa, inp, f"mla long heads/wg={heads}", num_splits=1)


def test_mla_decode_long_without_workspace(fa):
    """64 heads over 5000 tokens with no workspace: the planner takes 32-head
    workgroups, which need no key split, instead of failing for want of one."""
    import torch
    inp = _mla_ragged(58, 2, 64, 5000, 1, [5000, 2500])
    q, pool = to_dev(inp.q, "bf16"), to_dev(inp.pool, "bf16")
    pt, sl = i32_dev(inp.page_table), i32_dev(inp.seq_lens)
    o = torch.empty((inp.B, inp.Hq, 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((inp.B, inp.Hq), dtype=torch.float32, device=q.device)
    fa.fa_decode_paged(q, pool, pt, sl, pool.shape[0], o, lse, inp.B, inp.Hq, 1, 576, 512, 1,
                       pt.shape[1], inp.max_seq_len, fa.FA_KV_MLA_SHARED, inp.scale, 0,
                       fa.FA_BF16, None, 0, None)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.decode_paged(inp)
    assert_parity(to_f64(o), ref, "bf16", "mla long, no workspace")
    assert_lse(to_f64(lse), ref_lse, "mla long, no workspace")


@pytest.mark.parametrize("heads", ["32", "64"])
@pytest.mark.parametrize("Sq,Hq,splits", [(2, 64, 0), (3, 16, 1), (4, 128, 2), (2, 48, 3)])
def test_mla_decode_multi_token(fa, heads, Sq, Hq, splits, monkeypatch):
    """Several new tokens per sequence with the shared MLA pool: rows are
    (token, head) pairs of the workgroup; lengths shorter than Sq included."""
    monkeypatch.setenv("FA_MLA_HEADS", heads)
    inp = _mla_ragged(80 + Sq, 3, Hq, 400, 1, [400, 2, 129])
    inp.q = fi.normal_bits((3, Sq, Hq, 576), "bf16", fi.rng_for(80 + Sq, fi.T_Q))
    inp.Sq = Sq
    log(f"mla decode multi heads/wg={heads} Sq={Sq} Hq={Hq} splits={splits}")
    o, lse = check(fa, inp, f"mla multi Sq={Sq} Hq={Hq}", num_splits=splits)
    if Sq > 2:
        assert np.all(o[1, :Sq - 2] == 0) and np.all(np.isneginf(lse[1, :, :Sq - 2]))


@pytest.mark.parametrize("heads", ["32", "64"])
def test_mla_decode_pool_beyond_4gib(fa, heads, monkeypatch):
    """MLA rows past 4 GiB: the sequences' pages sit at the top of a pool of
    about 4.3 GB (1152-byte rows, page size 1); the oracle reads the same rows
    from a compact host copy."""
    import torch
    monkeypatch.setenv("FA_MLA_HEADS", heads)
    inp = fi.mla_decode_inputs(47, 2, 64, 384)
    n_used = inp.pool.shape[0]
    n_total = (4 << 30) // inp.pool[0].nbytes + 4096
    base = n_total - n_used
    log(f"MLA pool of {n_total} rows, used rows from {base}, {heads} heads per workgroup")
    big = torch.empty((n_total,) + inp.pool.shape[1:], dtype=torch.bfloat16, device="cuda")
    big[base:] = to_dev(inp.pool, "bf16")
    o, lse = fa.decode_paged(to_dev(inp.q, "bf16"), big, i32_dev(inp.page_table + base),
                             i32_dev(inp.seq_lens), layout=fa.FA_KV_MLA_SHARED, scale=inp.scale,
                             max_seq_len=inp.max_seq_len, page_size=1, return_lse=True)
    torch.cuda.synchronize()
    del big
    ref, ref_lse = oracle.decode_paged(inp)
    assert_parity(to_f64(o), ref, "bf16", f"MLA pool beyond 4 GiB ({heads} heads)")
    assert_lse(to_f64(lse), ref_lse, "MLA pool beyond 4 GiB")


def test_mla_decode_fp16_and_empty(fa):
    inp = _mla_ragged(53, 3, 64, 256, 1, [256, 0, 100], dtype="fp16")
    o, lse = check(fa, inp, "mla fp16")
    assert np.all(o[1] == 0) and np.all(np.isneginf(lse[1]))


def test_mla_equals_gqa_with_materialised_kv(fa):
    """MLA decode equals plain attention with one K/V head, K = [ckv | kpe] and
    V = ckv materialised from the pool (the oracle's contiguous path, not its
    paged gather)."""
    inp = _mla_ragged(54, 2, 64, 200, 1, [200, 77])
    o, _ = run(fa, inp)
    pool = oracle.widen(inp.pool, "bf16")
    q = oracle.widen(inp.q, "bf16")
    for b in range(inp.B):
        n = int(inp.seq_lens[b])
        rows = pool[inp.page_table[b, :n], 0]  # [n, 576]
        K = rows[None, :, None, :]
        V = rows[None, :, None, :512]
        ref, _ = oracle.attention(q[b][None, None], K, V, False, inp.scale)
        assert_parity(o[b], ref[0, 0], "bf16", f"mla materialised b={b}")


def test_mla_decode_full_size(fa):
    """Workload 4 in full: batch 128 x 64 heads x 2048 tokens, page_size 1 with a
    random page permutation, scale 1/sqrt(192), in the bench's configuration
    (planner: 64 heads per workgroup, two key splits and the combine); every
    sequence against the oracle."""
    inp = fi.workload(4)
    log("workload 4 full size")
    o, lse = run(fa, inp)
    ref, ref_lse = oracle.decode_paged(inp)
    assert_parity(o, ref, "bf16", "workload 4")
    assert_lse(lse, ref_lse, "workload 4")


def test_mla_decode_full_size_32_heads(fa, monkeypatch):
    """Workload 4 with the other workgroup shape (32 heads per workgroup, two
    workgroups per sequence), every sequence."""
    monkeypatch.setenv("FA_MLA_HEADS", "32")
    inp = fi.workload(4)
    log("workload 4 full size, 32 heads per workgroup")
    o, lse = run(fa, inp)
    ref, ref_lse = oracle.decode_paged(inp)
    assert_parity(o, ref, "bf16", "workload 4, 32 heads")
    assert_lse(lse, ref_lse, "workload 4, 32 heads")
