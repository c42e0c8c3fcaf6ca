"""Fused attention forward for AMD MI355X (gfx950): Python binding of libfa.so.

The functions named like the C entry points (``fa_prefill``, ``fa_prefill_ex``,
``fa_prefill_mask``, ``fa_decode_paged``, ``fa_decode_paged_multi``, the
workspace-size queries, ``fa_strerror``) marshal their arguments and call the
library; every step of the computation runs in the HIP
kernels. torch is used only for device memory and streams. ``prefill`` and
``decode_paged`` are conveniences that allocate outputs and workspace with torch
and then call the same entry points.

There is no fallback: if ``libfa.so`` has not been built, importing this package
raises ImportError (build it with ``python flashattention_forward_amd/build.py``),
and so does a library older than this binding (a missing entry point).
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

__all__ = [
    "FA_BF16", "FA_FP16", "FA_FP32", "FA_KV_SPLIT", "FA_KV_MLA_SHARED", "FaError",
    "fa_prefill", "fa_prefill_ex", "fa_prefill_mask", "fa_prefill_workspace_size",
    "fa_decode_paged", "fa_decode_paged_multi", "fa_decode_multi_workspace_size",
    "fa_decode_workspace_size", "fa_decode_num_splits", "fa_decode_paged_noalloc",
    "fa_strerror", "fa_version",
    "prefill", "decode_paged", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_BF16, FA_FP16, FA_FP32 = 0, 1, 2
FA_KV_SPLIT, FA_KV_MLA_SHARED = 0, 1

_BUILD_HINT = "run `python flashattention_forward_amd/build.py`"
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; {_BUILD_HINT}")

_lib = ctypes.CDLL(LIB_PATH)
for _name in ("fa_prefill", "fa_prefill_ex", "fa_prefill_mask", "fa_prefill_workspace_size",
              "fa_decode_paged", "fa_decode_paged_multi", "fa_decode_multi_workspace_size",
              "fa_decode_workspace_size", "fa_decode_num_splits", "fa_decode_paged_noalloc",
              "fa_strerror", "fa_version"):
    if not hasattr(_lib, _name):
        raise ImportError(f"{LIB_PATH} lacks {_name} (older than its sources); {_BUILD_HINT}")
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t

_lib.fa_prefill.argtypes = [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]
_lib.fa_prefill.restype = _I
_lib.fa_prefill_ex.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P,
                               _Z, _P]
_lib.fa_prefill_ex.restype = _I
_L = ctypes.c_int64
_lib.fa_prefill_mask.argtypes = [_P, _P, _P, _P, _L, _L, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F,
                                 _I, _I, _P, _Z, _P]
_lib.fa_prefill_mask.restype = _I
_lib.fa_prefill_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I]
_lib.fa_prefill_workspace_size.restype = _Z
_lib.fa_decode_paged.argtypes = [_P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _I, _F,
                                 _I, _I, _P, _Z, _P]
_lib.fa_decode_paged.restype = _I
_lib.fa_decode_paged_multi.argtypes = [_P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                       _I, _I, _I, _F, _I, _I, _P, _Z, _P]
_lib.fa_decode_paged_multi.restype = _I
_lib.fa_decode_multi_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _I, _I]
_lib.fa_decode_multi_workspace_size.restype = _Z
_lib.fa_decode_workspace_size.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _I]
_lib.fa_decode_workspace_size.restype = _Z
_lib.fa_decode_num_splits.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, _I]
_lib.fa_decode_num_splits.restype = _I
_lib.fa_decode_paged_noalloc.argtypes = [_P, _P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                         _I, _I, _F, _I, _I, _P]
_lib.fa_decode_paged_noalloc.restype = _I
_lib.fa_strerror.argtypes = [_I]
_lib.fa_strerror.restype = ctypes.c_char_p
_lib.fa_version.argtypes = []
_lib.fa_version.restype = ctypes.c_char_p


class FaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {fa_strerror(status)} (status {status})")
        self.status = status


def fa_strerror(status: int) -> str:
    return _lib.fa_strerror(int(status)).decode()


def fa_version() -> str:
    return _lib.fa_version().decode()


def _ptr(x) -> Optional[int]:
    """Device address of a tensor (must live on a GPU), an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not getattr(x, "is_cuda", False):
        raise ValueError("tensor arguments must be device (GPU) tensors")
    if x.numel() > 0 and not x.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return x.data_ptr() if x.numel() > 0 else None


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != 0:
        raise FaError(status, where)


def fa_prefill(q, k, v, o, B, Hq, Hkv, Sq, Skv, D, causal, scale, stream=None) -> None:
    _check(_lib.fa_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(o), B, Hq, Hkv, Sq, Skv, D,
                           int(bool(causal)), float(scale), _stream(stream)), "fa_prefill")


def fa_prefill_ex(q, k, v, o, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale, in_dtype, out_dtype,
                  workspace=None, workspace_bytes=0, stream=None) -> None:
    if workspace is not None and not isinstance(workspace, int) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.fa_prefill_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq,
                              Skv, D, int(bool(causal)), float(scale), int(in_dtype),
                              int(out_dtype), _ptr(workspace), int(workspace_bytes),
                              _stream(stream)), "fa_prefill_ex")


def fa_prefill_mask(q, k, v, mask, mask_stride, mask_batch_stride, o, lse, B, Hq, Hkv, Sq, Skv,
                    D, causal, scale, in_dtype, out_dtype, workspace=None, workspace_bytes=0,
                    stream=None) -> None:
    if workspace is not None and not isinstance(workspace, int) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.fa_prefill_mask(_ptr(q), _ptr(k), _ptr(v), _ptr(mask), int(mask_stride),
                                int(mask_batch_stride), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq, Skv,
                                D, int(bool(causal)), float(scale), int(in_dtype),
                                int(out_dtype), _ptr(workspace), int(workspace_bytes),
                                _stream(stream)), "fa_prefill_mask")


def fa_prefill_workspace_size(B, Hq, Hkv, Sq, Skv, D, causal, out_dtype) -> int:
    return int(_lib.fa_prefill_workspace_size(B, Hq, Hkv, Sq, Skv, D, int(bool(causal)),
                                              int(out_dtype)))


def fa_decode_paged(q, kv_pool, page_table, seq_lens, num_pages, o, lse, B, Hq, Hkv, D_qk, D_v,
                    page_size, max_pages_per_seq, max_seq_len, layout, scale, num_splits, dtype,
                    workspace=None, workspace_bytes=0, stream=None) -> None:
    if workspace is not None and not isinstance(workspace, int) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.fa_decode_paged(_ptr(q), _ptr(kv_pool), _ptr(page_table), _ptr(seq_lens),
                                int(num_pages), _ptr(o), _ptr(lse), B, Hq, Hkv, D_qk, D_v,
                                page_size,
                                max_pages_per_seq, max_seq_len, int(layout), float(scale),
                                int(num_splits), int(dtype), _ptr(workspace),
                                int(workspace_bytes), _stream(stream)), "fa_decode_paged")


def fa_decode_paged_multi(q, kv_pool, page_table, seq_lens, num_pages, o, lse, B, Sq, Hq, Hkv,
                          D_qk, D_v, page_size, max_pages_per_seq, max_seq_len, layout, scale,
                          num_splits, dtype, workspace=None, workspace_bytes=0,
                          stream=None) -> None:
    if workspace is not None and not isinstance(workspace, int) and not workspace_bytes:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check(_lib.fa_decode_paged_multi(_ptr(q), _ptr(kv_pool), _ptr(page_table), _ptr(seq_lens),
                                      int(num_pages), _ptr(o), _ptr(lse), B, Sq, Hq, Hkv, D_qk,
                                      D_v, page_size, max_pages_per_seq, max_seq_len,
                                      int(layout), float(scale), int(num_splits), int(dtype),
                                      _ptr(workspace), int(workspace_bytes), _stream(stream)),
           "fa_decode_paged_multi")


def fa_decode_paged_noalloc(q, kv_pool, page_table, seq_lens, num_pages, o, lse, B, Hq, Hkv,
                            D_qk, D_v, page_size, max_pages_per_seq, max_seq_len, layout, scale,
                            num_splits, dtype, stream=None) -> None:
    _check(_lib.fa_decode_paged_noalloc(_ptr(q), _ptr(kv_pool), _ptr(page_table),
                                        _ptr(seq_lens), int(num_pages), _ptr(o), _ptr(lse), B,
                                        Hq, Hkv, D_qk, D_v, page_size, max_pages_per_seq,
                                        max_seq_len, int(layout), float(scale), int(num_splits),
                                        int(dtype), _stream(stream)), "fa_decode_paged_noalloc")


def fa_decode_multi_workspace_size(B, Sq, Hq, Hkv, D_qk, D_v, page_size, max_seq_len, layout,
                                   num_splits=0) -> int:
    return int(_lib.fa_decode_multi_workspace_size(B, Sq, Hq, Hkv, D_qk, D_v, page_size,
                                                   max_seq_len, int(layout), int(num_splits)))


def fa_decode_workspace_size(B, Hq, Hkv, D_qk, D_v, page_size, max_seq_len, layout,
                             num_splits=0) -> int:
    return int(_lib.fa_decode_workspace_size(B, Hq, Hkv, D_qk, D_v, page_size, max_seq_len,
                                             int(layout), int(num_splits)))


def fa_decode_num_splits(B, Hq, Hkv, D_qk, D_v, page_size, max_seq_len, layout,
                         num_splits=0) -> int:
    return int(_lib.fa_decode_num_splits(B, Hq, Hkv, D_qk, D_v, page_size, max_seq_len,
                                         int(layout), int(num_splits)))


# ---------------------------------------------------------------------------
# conveniences over torch tensors
# ---------------------------------------------------------------------------

def _fa_dtype(t) -> int:
    import torch
    m = {torch.bfloat16: FA_BF16, torch.float16: FA_FP16, torch.float32: FA_FP32}
    if t not in m:
        raise ValueError(f"unsupported dtype {t}")
    return m[t]


def _workspace(nbytes: int, device):
    import torch
    if nbytes <= 0:
        return None
    return torch.empty((nbytes + 15) // 16 * 4, dtype=torch.float32, device=device)


def prefill(q, k, v, *, causal: bool, scale: Optional[float] = None, out=None, out_dtype=None,
            return_lse: bool = False, allow_split: bool = True, mask=None, stream=None):
    """Attention prefill on torch tensors q [B, Sq, Hq, D], k/v [B, Skv, Hkv, D]
    (bf16 or fp16, contiguous, on the GPU). ``mask`` is None or an additive mask
    of q's dtype, [Sq, W] or [B, Sq, W] with W >= Skv rounded up to 8 and a
    multiple of 8 (contiguous, 16-byte aligned). Returns o [B, Sq, Hq, D] (and lse [B, Hq, Sq]
    fp32 if asked)."""
    import torch
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Skv, Hkv, D] like q")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must share one dtype")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, Sq, Hq, D), dtype=out_dtype or q.dtype, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    ws = _workspace(fa_prefill_workspace_size(B, Hq, Hkv, Sq, Skv, D, causal,
                                              _fa_dtype(out.dtype)), q.device) \
        if allow_split else None
    wsb = 0 if ws is None else ws.numel() * 4
    if mask is None:
        fa_prefill_ex(q, k, v, out, lse, B, Hq, Hkv, Sq, Skv, D, causal, scale,
                      _fa_dtype(q.dtype), _fa_dtype(out.dtype), ws, wsb, stream)
    else:
        if mask.dtype != q.dtype or not mask.is_contiguous() or mask.shape[-2] != Sq:
            raise ValueError("mask must be a contiguous [Sq, W] or [B, Sq, W] tensor of q's dtype")
        bstride = 0 if mask.dim() == 2 else mask.stride(0)
        if mask.dim() == 3 and mask.shape[0] != B:
            raise ValueError("a batched mask needs one matrix per batch entry")
        fa_prefill_mask(q, k, v, mask, mask.shape[-1], bstride, out, lse, B, Hq, Hkv, Sq, Skv, D,
                        causal, scale, _fa_dtype(q.dtype), _fa_dtype(out.dtype), ws, wsb, stream)
    return (out, lse) if return_lse else out


def decode_paged(q, kv_pool, page_table, seq_lens, *, layout: int, scale: float,
                 max_seq_len: int, page_size: int, D_v: Optional[int] = None,
                 num_splits: int = 0, out=None, return_lse: bool = False, workspace=None,
                 stream=None):
    """Paged decode on torch tensors. q [B, Hq, D_qk], or [B, Sq, Hq, D_qk] for
    Sq new tokens per sequence (causal, bottom-right);
    kv_pool per layout; page_table [B, max_pages] int32; seq_lens [B] int32
    (device). o has q's leading shape; lse is [B, Hq] or [B, Hq, Sq]."""
    import torch
    if q.dim() == 4:
        return _decode_multi(q, kv_pool, page_table, seq_lens, layout=layout, scale=scale,
                             max_seq_len=max_seq_len, page_size=page_size, D_v=D_v,
                             num_splits=num_splits, out=out, return_lse=return_lse,
                             workspace=workspace, stream=stream)
    B, Hq, D_qk = q.shape
    if layout == FA_KV_MLA_SHARED:
        Hkv = 1
        D_v = 512 if D_v is None else D_v
    else:
        Hkv = kv_pool.shape[2]
        D_v = D_qk if D_v is None else D_v
    if out is None:
        out = torch.empty((B, Hq, D_v), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        workspace = _workspace(fa_decode_workspace_size(B, Hq, Hkv, D_qk, D_v, page_size,
                                                        max_seq_len, layout, num_splits),
                               q.device)
    fa_decode_paged(q, kv_pool, page_table, seq_lens, kv_pool.shape[0], out, lse, B, Hq, Hkv,
                    D_qk, D_v, page_size,
                    page_table.shape[1], max_seq_len, layout, scale, num_splits,
                    _fa_dtype(q.dtype), workspace,
                    0 if workspace is None else workspace.numel() * workspace.element_size(),
                    stream)
    return (out, lse) if return_lse else out


def _decode_multi(q, kv_pool, page_table, seq_lens, *, layout, scale, max_seq_len, page_size,
                  D_v, num_splits, out, return_lse, workspace, stream):
    import torch
    B, Sq, Hq, D_qk = q.shape
    if layout == FA_KV_MLA_SHARED:
        Hkv = 1
        D_v = 512 if D_v is None else D_v
    else:
        Hkv = kv_pool.shape[2]
        D_v = D_qk if D_v is None else D_v
    if out is None:
        out = torch.empty((B, Sq, Hq, D_v), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if return_lse else None
    if workspace is None:
        workspace = _workspace(fa_decode_multi_workspace_size(B, Sq, Hq, Hkv, D_qk, D_v, page_size,
                                                              max_seq_len, layout, num_splits),
                               q.device)
    fa_decode_paged_multi(q, kv_pool, page_table, seq_lens, kv_pool.shape[0], out, lse, B, Sq, Hq,
                          Hkv, D_qk, D_v, page_size, page_table.shape[1], max_seq_len, layout,
                          scale, num_splits, _fa_dtype(q.dtype), workspace,
                          0 if workspace is None else workspace.numel() * workspace.element_size(),
                          stream)
    return (out, lse) if return_lse else out
