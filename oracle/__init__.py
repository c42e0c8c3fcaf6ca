"""CPU oracle for the attention forward pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package. The library never does, and nothing here imports the library:
the two share no code. The arithmetic lives in ``attention.c`` (plain C, fp64,
full-row two-pass softmax); this wrapper only widens the input bits to double,
gathers paged K/V rows into contiguous arrays, and calls it.

Definitions followed (the pages name the operation but print no formula):

* attention: ``O = softmax(scale * Q K^T + mask) V`` with ``mask`` causal aligned
  bottom-right or none, plus optionally an explicit additive mask ``M[i][j]``
  (finite or -inf) added to the scaled scores; grouped-query head
  ``g = h // (Hq // Hkv)``; output 0 and log-sum-exp -inf for a row with no
  visible key.
* paged decode: token t of sequence b lives in physical page
  ``page_table[b][t // page_size]`` at slot ``t % page_size`` (the page-table
  gather of "perf: FlashAttention-3 style MLA PageAttention", section
  "Results", page_size = 1 and larger pages).
* MLA: K and V are the same compressed-KV rows; the score uses all ``D_qk``
  columns ``[ckv | kpe]``, the output the first ``D_v`` columns (``ckv``) --
  change list item 4 of the same page.

Parity pins for every function are in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (IEEE arithmetic: no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-pthread", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        f = lib.oracle_attention_rows
        P = ctypes.c_void_p
        I = ctypes.c_int64
        f.argtypes = [P, P, P, P, I, P, P, I, I, I, I, I, I, I, ctypes.c_int, ctypes.c_double,
                      P, I, I, P, P, ctypes.c_int]
        f.restype = ctypes.c_int
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of bf16 / fp16 bit patterns (uint16) to float64."""
    bits = np.asarray(bits)
    if dtype == "bf16":
        with np.errstate(invalid="ignore"):  # NaN poison widens to NaN
            return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    if dtype in ("fp32", "fp64"):
        return np.asarray(bits, dtype=np.float64)
    raise ValueError(dtype)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def attention_rows(q_rows, rb, rh, ri, k, v, Hq, Sq, causal, scale, nthreads=None, mask=None):
    """Attention for the listed query rows.

    q_rows [n, Dqk] float64; rb/rh/ri [n] batch, query-head and query index;
    k [B, Skv, Hkv, Dqk] and v [B, Skv, Hkv, Dv] float64. ``scale`` is used as a
    double exactly as given. ``mask`` is None or a float64 additive mask
    [Bm, Sq, stride] (Bm 1: shared by the batch; stride >= Skv; -inf hides a
    key). Returns (o_rows [n, Dv], lse_rows [n]).
    """
    q_rows = np.ascontiguousarray(q_rows, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    rb = np.ascontiguousarray(rb, dtype=np.int64)
    rh = np.ascontiguousarray(rh, dtype=np.int64)
    ri = np.ascontiguousarray(ri, dtype=np.int64)
    n = int(rb.shape[0])
    B, Skv, Hkv, Dqk = k.shape
    Dv = v.shape[3]
    assert v.shape[:3] == (B, Skv, Hkv) and q_rows.shape == (n, Dqk)
    o = np.zeros((n, Dv), dtype=np.float64)
    lse = np.zeros((n,), dtype=np.float64)
    mptr, mb, ms = None, 0, 0
    if mask is not None:
        mask = np.ascontiguousarray(mask, dtype=np.float64)
        assert mask.ndim == 3 and mask.shape[1] == Sq and mask.shape[2] >= Skv
        assert mask.shape[0] in (1, B)
        mptr, ms = _ptr(mask), mask.shape[2]
        mb = 0 if mask.shape[0] == 1 else Sq * ms
    rc = _load().oracle_attention_rows(
        _ptr(q_rows), _ptr(rb), _ptr(rh), _ptr(ri), n, _ptr(k), _ptr(v), B, Hq, Hkv, Sq, Skv,
        Dqk, Dv, int(bool(causal)), float(scale), mptr, mb, ms, _ptr(o), _ptr(lse),
        int(nthreads or default_threads()))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_rows failed ({rc})")
    return o, lse


def attention(q, k, v, causal, scale, nthreads=None, mask=None):
    """Full attention. q [B, Sq, Hq, Dqk], k [B, Skv, Hkv, Dqk], v [B, Skv, Hkv, Dv]
    (float arrays), optional additive ``mask`` as in ``attention_rows``.
    Returns (o [B, Sq, Hq, Dv], lse [B, Hq, Sq])."""
    q = np.asarray(q, dtype=np.float64)
    B, Sq, Hq, Dqk = q.shape
    bb, ii, hh = np.meshgrid(np.arange(B), np.arange(Sq), np.arange(Hq), indexing="ij")
    o, lse = attention_rows(q.reshape(-1, Dqk), bb.ravel(), hh.ravel(), ii.ravel(), k, v, Hq,
                            Sq, causal, scale, nthreads, mask)
    Dv = o.shape[1]
    return o.reshape(B, Sq, Hq, Dv), lse.reshape(B, Sq, Hq).transpose(0, 2, 1).copy()


def prefill_rows(inp, rows, nthreads=None):
    """Oracle rows of a prefill input set (an object with the bit arrays q/k/v,
    dtype ``in_dtype`` and the shape fields); ``rows`` is an int array [n, 3] of
    (b, h, i). Returns (o_rows [n, D], lse_rows [n])."""
    rows = np.asarray(rows, dtype=np.int64).reshape(-1, 3)
    qb = inp.q[rows[:, 0], rows[:, 2], rows[:, 1], :]
    return attention_rows(widen(qb, inp.in_dtype), rows[:, 0], rows[:, 1], rows[:, 2],
                          widen(inp.k, inp.in_dtype), widen(inp.v, inp.in_dtype), inp.Hq, inp.Sq,
                          inp.causal, float(inp.scale), nthreads, _mask_of(inp))


def _mask_of(inp):
    m = getattr(inp, "mask", None)
    return None if m is None else widen(m, inp.in_dtype)


def prefill(inp, nthreads=None):
    """Full oracle output of a prefill input set: (o [B,Sq,Hq,D], lse [B,Hq,Sq])."""
    return attention(widen(inp.q, inp.in_dtype), widen(inp.k, inp.in_dtype),
                     widen(inp.v, inp.in_dtype), inp.causal, float(inp.scale), nthreads,
                     _mask_of(inp))


def gather_paged(pool, page_table, seq_len, page_size, layout, b, Hkv, D_qk, D_v):
    """K_b [1, n, Hkv, D_qk] and V_b [1, n, Hkv, D_v] of sequence b, gathered token by
    token through the page table (pool already widened to float64)."""
    n = int(seq_len)
    t = np.arange(n)
    page = np.asarray(page_table)[b, t // page_size].astype(np.int64)
    slot = t % page_size
    if layout == "split":  # pool [P, 2, Hkv, page, D]
        K = pool[page, 0, :, slot, :]  # [n, Hkv, D]
        V = pool[page, 1, :, slot, :]
    elif layout == "mla":  # pool [P, page, D_qk]; one row is both K and V
        rows = pool[page, slot, :]  # [n, D_qk]
        K = rows[:, None, :D_qk]
        V = rows[:, None, :D_v]
    else:
        raise ValueError(layout)
    return K[None].copy(), V[None].copy()


def decode_paged(inp, batches=None, nthreads=None):
    """Oracle of paged decode.

    ``inp`` has q bits, pool bits, page_table, seq_lens, page_size, layout
    ("split" or "mla"), Hkv, D_qk, D_v, scale, dtype and Sq. With Sq = 1, q is
    [B, Hq, D_qk], one query token per sequence seeing all its cached tokens,
    and the result is (o [nb, Hq, D_v], lse [nb, Hq]). With Sq > 1, q is
    [B, Sq, Hq, D_qk]: the queries are the sequence's last Sq tokens, token i
    at position seq_len - Sq + i, each seeing the tokens up to its own position
    (the bottom-right causal rule of the prefill reading); the result is
    (o [nb, Sq, Hq, D_v], lse [nb, Hq, Sq]). Listed batches, all by default.
    """
    if batches is None:
        batches = range(inp.B)
    batches = list(batches)
    pool = widen(inp.pool, inp.dtype)
    q = widen(inp.q, inp.dtype)
    outs, lses = [], []
    for b in batches:
        K, V = gather_paged(pool, inp.page_table, inp.seq_lens[b], inp.page_size, inp.layout, b,
                            inp.Hkv, inp.D_qk, inp.D_v)
        if getattr(inp, "Sq", 1) > 1:
            o, lse = attention(q[b][None], K, V, True, float(inp.scale), nthreads)
            outs.append(o[0])
            lses.append(lse[0])
        else:
            o, lse = attention(q[b][None, None], K, V, False, float(inp.scale), nthreads)
            outs.append(o[0, 0])
            lses.append(lse[0, :, 0])
    return np.stack(outs), np.stack(lses)
