"""The C-ABI library loads, exports every symbol its header declares, and
rejects bad arguments on the host before any launch (CPU only: no call here
reaches a kernel)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


@pytest.fixture(scope="module")
def fa():
    import flashattention_forward_amd as fa
    return fa


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ["fa_prefill", "fa_prefill_ex", "fa_prefill_mask", "fa_decode_paged",
              "fa_decode_paged_multi", "fa_decode_multi_workspace_size",
              "fa_prefill_workspace_size", "fa_decode_workspace_size", "fa_strerror"]:
        assert n in names


def declared_params(name):
    """Parameter names of one declaration in fa.h, in order."""
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    m = re.search(r"\b" + name + r"\s*\(([^)]*)\)\s*;", text)
    assert m, f"{name} not declared"
    return [re.findall(r"(\w+)\s*$", p.strip())[0] for p in m.group(1).split(",")]


def test_specified_argument_order():
    """The two calls the path is specified by keep their argument lists:
    fa_prefill(q,k,v,o,B,Hq,Hkv,Sq,Skv,D,causal,scale,stream) exactly, and
    fa_decode_paged(q,kv_pool,page_table,seq_lens,...,stream)."""
    assert declared_params("fa_prefill") == ["q", "k", "v", "o", "B", "Hq", "Hkv", "Sq", "Skv",
                                             "D", "causal", "scale", "stream"]
    for name in ("fa_decode_paged", "fa_decode_paged_multi"):
        ps = declared_params(name)
        assert ps[:4] == ["q", "kv_pool", "page_table", "seq_lens"], (name, ps)
        assert ps[-1] == "stream"


def test_binding_argument_counts(fa):
    """The ctypes binding passes as many arguments as the header declares."""
    import flashattention_forward_amd as pkg
    for name in declared_functions():
        fn = getattr(pkg._lib, name)
        n = len(declared_params(name))
        if declared_params(name) == ["void"]:
            n = 0
        assert len(fn.argtypes) == n, f"{name}: binding {len(fn.argtypes)} vs header {n}"


@pytest.mark.parametrize("lib_name", ["libfa.so", "libfa_ldsdebug.so"])
def test_library_exports_every_declared_symbol(fa, lib_name):
    """Both builds (the library and its LDS-race debug build) load and export
    every function fa.h declares."""
    path = os.path.join(os.path.dirname(fa.LIB_PATH), lib_name)
    assert os.path.exists(path), f"{path} is not built"
    lib = ctypes.CDLL(path)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in fa.h but not exported by {lib_name}"


def test_strerror_and_version(fa):
    assert fa.fa_strerror(0) == "ok"
    assert "workspace" in fa.fa_strerror(-5)
    assert fa.fa_strerror(12345) == "unknown status"
    assert re.match(r"\d+\.\d+\.\d+", fa.fa_version())


def _err(fn, *a, **k):
    import flashattention_forward_amd as fa
    with pytest.raises(fa.FaError) as e:
        fn(*a, **k)
    return e.value.status


A = 1 << 20  # a 16-byte aligned fake address: never dereferenced by these calls


def test_prefill_mask_validation(fa):
    def call(mask=A, stride=16, bstride=0, Skv=13):
        return fa.fa_prefill_mask(A, A, A, mask, stride, bstride, A, None, 1, 4, 2, 8, Skv, 64, 0,
                                  0.1, fa.FA_BF16, fa.FA_BF16, None, 0, stream=0)

    assert _err(call, mask=None) == -1
    assert _err(call, mask=A + 8) == -4  # mask rows are copied 16 bytes at a time
    assert _err(call, stride=20) == -4
    assert _err(call, bstride=12) == -4
    assert _err(call, stride=8) == -2  # Skv = 13 needs rows of >= 16 elements
    assert _err(call, bstride=-8) == -2
    assert _err(call, stride=1 << 28) == -2  # Sq (8) x stride > 2^30: 32-bit row offsets


def test_decode_multi_validation(fa):
    def call(Sq=4, layout=None, Dqk=128, Dv=128, Hkv=2):
        lay = fa.FA_KV_SPLIT if layout is None else layout
        return fa.fa_decode_paged_multi(A, A, A, A, 8, A, None, 2, Sq, 8, Hkv, Dqk, Dv, 16, 4, 64,
                                        lay, 0.1, 0, fa.FA_BF16, None, 0, stream=0)

    assert _err(call, Sq=0) == -2
    assert _err(call, Sq=65) == -2
    # MLA: 128 sequences x 2 new tokens x 64 heads fill 256 64-row workgroups unsplit
    mla = fa.FA_KV_MLA_SHARED
    assert fa.fa_decode_multi_workspace_size(128, 2, 64, 1, 576, 512, 1, 2048, mla, 0) == 0
    assert (fa.fa_decode_multi_workspace_size(128, 2, 64, 1, 576, 512, 1, 2048, mla, 2)
            == 2 * 128 * 2 * 64 * (512 * 2 + 4))
    # rows = new tokens x heads: 4 sequences x 4 tokens x 32 heads of 16-bit partials + fp32 lse
    ws = fa.fa_decode_multi_workspace_size(4, 4, 32, 8, 128, 128, 16, 32768, fa.FA_KV_SPLIT, 3)
    assert ws == 3 * 4 * 4 * 32 * (128 * 2 + 4)
    assert fa.fa_decode_multi_workspace_size(4, 1, 32, 8, 128, 128, 16, 32768, fa.FA_KV_SPLIT,
                                             3) == \
        fa.fa_decode_workspace_size(4, 32, 8, 128, 128, 16, 32768, fa.FA_KV_SPLIT, 3)


def test_prefill_validation(fa):
    f = fa.fa_prefill_ex
    args = dict(B=1, Hq=4, Hkv=2, Sq=16, Skv=16, D=64, causal=1, scale=0.1, in_dtype=fa.FA_BF16,
                out_dtype=fa.FA_BF16)

    def call(q=A, k=A, v=A, o=A, lse=None, ws=None, ws_bytes=0, **kw):
        a = dict(args)
        a.update(kw)
        return f(q, k, v, o, lse, a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Skv"], a["D"],
                 a["causal"], a["scale"], a["in_dtype"], a["out_dtype"], ws, ws_bytes, stream=0)

    assert _err(call, q=None) == -1
    assert _err(call, v=None) == -1
    assert _err(call, Hkv=3) == -2
    assert _err(call, B=0) == -2
    assert _err(call, Sq=-1) == -2
    assert _err(call, D=96) == -3
    assert _err(call, in_dtype=fa.FA_FP32) == -3
    assert _err(call, out_dtype=7) == -3
    assert _err(call, q=A + 8) == -4
    assert _err(call, lse=A + 2) == -4
    assert _err(call, ws=A + 4) == -4
    # a plan that splits the keys needs the full workspace
    big = dict(B=1, Hq=4, Hkv=4, Sq=128, Skv=8192, D=128)
    need = fa.fa_prefill_workspace_size(1, 4, 4, 128, 8192, 128, 0, fa.FA_BF16)
    assert need > 0
    assert _err(call, ws=A, ws_bytes=need - 4, **big) == -5
    # nothing to do: returns before any launch
    call(Sq=0)
    assert fa.fa_prefill(None, None, None, None, 1, 1, 1, 0, 0, 64, 0, 1.0, stream=0) is None


def test_prefill_workspace_size_rules(fa):
    # short keys: no split
    assert fa.fa_prefill_workspace_size(1, 32, 8, 512, 512, 128, 1, fa.FA_BF16) == 0
    rows = 512 * 32
    # per split: partial rows in the output type and an fp32 lse per row
    for dt, per_row in ((fa.FA_BF16, 128 * 2 + 4), (fa.FA_FP16, 128 * 2 + 4),
                        (fa.FA_FP32, 128 * 4 + 4)):
        ws = fa.fa_prefill_workspace_size(1, 32, 8, 512, 16384, 128, 1, dt)
        assert ws % (rows * per_row) == 0 and ws // (rows * per_row) in (2, 4, 8, 16)
    assert fa.fa_prefill_workspace_size(0, 1, 1, 1, 1, 64, 0, fa.FA_BF16) == 0
    assert fa.fa_prefill_workspace_size(1, 32, 8, 512, 16384, 128, 1, 7) == 0  # bad type


def test_decode_validation(fa):
    f = fa.fa_decode_paged

    def call(q=A, pool=A, npages=10, pt=A, sl=A, o=A, lse=None, B=2, Hq=8, Hkv=2, Dqk=128,
             Dv=128, ps=16, maxp=4, maxlen=64, layout=fa.FA_KV_SPLIT, splits=0,
             dtype=fa.FA_BF16, ws=None, wsb=0):
        return f(q, pool, pt, sl, npages, o, lse, B, Hq, Hkv, Dqk, Dv, ps, maxp, maxlen, layout,
                 0.1, splits, dtype, ws, wsb, stream=0)

    assert _err(call, pool=None) == -1
    assert _err(call, sl=None) == -1
    assert _err(call, Hkv=3) == -2
    assert _err(call, ps=0) == -2
    assert _err(call, maxp=3, maxlen=64) == -2  # 3 pages of 16 < 64 tokens
    assert _err(call, npages=0) == -2
    # A page of the split pool (K and V of every K/V head) must stay below 2 GiB:
    # 2 * 64 heads * 65536 slots * 256 bytes is exactly 2 GiB.
    assert _err(call, Hq=64, Hkv=64, ps=65536, maxp=1, maxlen=64) == -2
    call(Hq=64, Hkv=64, ps=65535, maxp=1, maxlen=64, B=0)  # just below: accepted
    assert _err(call, Dqk=64, Dv=64) == -3
    assert _err(call, layout=fa.FA_KV_MLA_SHARED) == -3  # needs (576, 512)
    assert _err(call, layout=fa.FA_KV_MLA_SHARED, Dqk=576, Dv=512, Hkv=2) == -2
    assert _err(call, layout=5) == -3
    assert _err(call, dtype=fa.FA_FP32) == -3
    assert _err(call, o=A + 2) == -4
    assert _err(call, pt=A + 1) == -4
    need = fa.fa_decode_workspace_size(2, 8, 2, 128, 128, 16, 4096, fa.FA_KV_SPLIT, 4)
    assert need == 4 * 2 * 8 * (128 * 2 + 4)  # 16-bit partials + fp32 lse per split
    assert _err(call, maxp=256, maxlen=4096, splits=4, ws=A, wsb=need - 16) == -5
    call(B=0)  # empty batch: nothing enqueued


def test_decode_split_planning(fa, monkeypatch):
    mla = fa.FA_KV_MLA_SHARED
    # MLA, 128 sequences of 2048 tokens, 64 heads per workgroup: 2 splits fill 256 CUs
    assert fa.fa_decode_num_splits(128, 64, 1, 576, 512, 1, 2048, mla) == 2
    # (16-bit partial outputs and fp32 lse per split)
    assert (fa.fa_decode_workspace_size(128, 64, 1, 576, 512, 1, 2048, mla, 0)
            == 2 * 128 * 64 * (512 * 2 + 4))
    assert fa.fa_decode_num_splits(256, 64, 1, 576, 512, 1, 2048, mla) == 1
    # 32 heads per workgroup: 128 sequences x 32 heads still split twice, 64 x 128 heads not
    assert fa.fa_decode_num_splits(128, 32, 1, 576, 512, 1, 2048, mla) == 2
    monkeypatch.setenv("FA_MLA_HEADS", "32")
    assert fa.fa_decode_num_splits(64, 128, 1, 576, 512, 1, 2048, mla) == 1
    assert fa.fa_decode_workspace_size(64, 128, 1, 576, 512, 1, 2048, mla, 0) == 0
    monkeypatch.delenv("FA_MLA_HEADS")
    # GQA, 4 sequences x 8 K/V heads: four waves per SIMD over 32 units wants 128
    # splits, capped at chunks of 8 tiles (256 tokens), rounded down to whole tiles
    assert fa.fa_decode_num_splits(4, 32, 8, 128, 128, 16, 32768, fa.FA_KV_SPLIT) == 128
    assert fa.fa_decode_num_splits(4, 32, 8, 128, 128, 16, 23450, fa.FA_KV_SPLIT) == 92
    # many sequences: few splits (4096 tokens, 32 x 8 units wants 16)
    assert fa.fa_decode_num_splits(32, 32, 8, 128, 128, 16, 4096, fa.FA_KV_SPLIT) == 16
    # explicit request is honoured (clamped to the 32-token tiles available)
    assert fa.fa_decode_num_splits(4, 32, 8, 128, 128, 16, 32768, fa.FA_KV_SPLIT, 3) == 3
    assert fa.fa_decode_num_splits(4, 32, 8, 128, 128, 16, 40, fa.FA_KV_SPLIT, 8) == 2
    assert fa.fa_decode_num_splits(4, 32, 8, 128, 128, 16, 0, fa.FA_KV_SPLIT) == 1
    assert fa.fa_decode_workspace_size(4, 32, 8, 128, 128, 16, 100, fa.FA_KV_SPLIT, 1) == 0


def test_decode_noalloc_validation(fa):
    """The entry point that allocates nothing checks its arguments like
    fa_decode_paged, and refuses a split plan larger than its static scratch
    before touching the device."""
    def call(B=2, splits=0, maxlen=64, layout=fa.FA_KV_SPLIT, Dqk=128, Dv=128, pool=A):
        return fa.fa_decode_paged_noalloc(A, pool, A, A, 10, A, None, B, 8, 2 if Dqk == 128 else 1,
                                          Dqk, Dv, 1, maxlen, maxlen, layout, 0.1, splits,
                                          fa.FA_BF16, stream=0)
    assert _err(call, pool=None) == -1
    assert _err(call, Dqk=64, Dv=64) == -3
    mla = fa.FA_KV_MLA_SHARED
    # 2048 sequences x 8 heads x 16 splits of 512-column partials: 136 MB > 32 MiB
    assert _err(call, B=2048, splits=16, maxlen=8192, layout=mla, Dqk=576, Dv=512) == -7
    assert "scratch" in fa.fa_strerror(-7)
    call(B=0)  # empty batch: nothing enqueued


def test_binding_rejects_host_tensors(fa):
    import torch
    x = torch.zeros(16, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_prefill(x, x, x, x, 1, 1, 1, 1, 1, 64, 0, 1.0, stream=0)
