"""Seeded synthetic inputs for the attention forward pass.

This module is the only code shared by the CPU oracle's tests and the GPU path's
tests and bench. It produces raw input bytes (bf16 / fp16 bit patterns as numpy
``uint16`` arrays, int32 page tables and sequence lengths) and holds none of the
attention arithmetic: no products, no softmax, no masking.

Workloads follow the shapes of the pages:

* "CUDA: fix FA occupancy, optimize tile kernel" (llama.cpp), table "Performance
  changes": prompt processing of 16384 tokens split into microbatches, for an
  8B-class Llama layer (32 query heads sharing 8 K/V heads, head size 128).
* "perf: FlashAttention-3 style MLA PageAttention" (FlashInfer), section
  "Results": batch x seq_len x 64 heads with page_size = 1, and the MLA property
  that K and V are one compressed-KV matrix (item 4 of the change list).

Recipe (every tensor): ``numpy.random.default_rng([1000 + c, tensor_id])`` with
``c`` the workload number below and tensor ids q = 0, k = 1 (or the paged pool),
v = 2, page permutation = 3, sequence lengths = 4, additive mask = 5; values are
float32 ``standard_normal`` rounded once to bf16 / fp16 with round-to-nearest-even.

Additive masks (``additive_mask``) take the shapes of the KQ mask that the
llama.cpp page's opening paragraph counts as memory traffic: one [Sq, Skv]
matrix (optionally one per batch entry), padded rows, -inf for hidden keys.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

BF16 = "bf16"
FP16 = "fp16"
FP32 = "fp32"

# Tensor ids of the seeding recipe.
T_Q, T_K, T_V, T_POOL, T_PERM, T_LENS, T_MASK = 0, 1, 2, 1, 3, 4, 5

# NaN bit patterns used to poison pool slots that no valid token owns.
NAN_BITS = {BF16: 0x7FC0, FP16: 0x7E00}
NEG_INF_BITS = {BF16: 0xFF80, FP16: 0xFC00}


def rng_for(c: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([1000 + c, tensor_id])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 with round-to-nearest-even; returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = NAN_BITS[BF16]
    return r


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to IEEE half (numpy's conversion is round-to-nearest-even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return f32_to_bf16_bits(x)
    if dtype == FP16:
        return f32_to_fp16_bits(x)
    raise ValueError(f"unsupported input dtype {dtype}")


def normal_bits(shape, dtype: str, rng: np.random.Generator) -> np.ndarray:
    """N(0,1) float32 samples rounded to ``dtype``; returns uint16 bits of ``shape``."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return round_bits(x, dtype)


@dataclasses.dataclass
class PrefillInputs:
    q: np.ndarray  # uint16 bits [B, Sq, Hq, D]
    k: np.ndarray  # uint16 bits [B, Skv, Hkv, D]
    v: np.ndarray  # uint16 bits [B, Skv, Hkv, D]
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Skv: int
    D: int
    causal: bool
    scale: float  # the float32 value handed to the kernel
    in_dtype: str
    out_dtype: str
    mask: Optional[np.ndarray] = None  # uint16 bits [Bm, Sq, stride] (Bm 1 or B), or None


@dataclasses.dataclass
class DecodeInputs:
    q: np.ndarray  # uint16 bits [B, Hq, D_qk], or [B, Sq, Hq, D_qk] when Sq > 1
    pool: np.ndarray  # uint16 bits, layout depends on ``layout``
    page_table: np.ndarray  # int32 [B, max_pages]
    seq_lens: np.ndarray  # int32 [B]
    B: int
    Hq: int
    Hkv: int
    D_qk: int
    D_v: int
    page_size: int
    max_seq_len: int
    layout: str  # "split": [P, 2, Hkv, page, D]; "mla": [P, page, D_qk]
    scale: float
    dtype: str
    Sq: int = 1  # new tokens per sequence (the last Sq of each sequence)

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])


def f32(x: float) -> float:
    """The float32 value nearest to ``x`` (what the C boundary receives)."""
    return float(np.float32(x))


def prefill_inputs(c: int, B: int, Hq: int, Hkv: int, Sq: int, Skv: int, D: int,
                   causal: bool, in_dtype: str = BF16, out_dtype: Optional[str] = None,
                   scale: Optional[float] = None) -> PrefillInputs:
    q = normal_bits((B, Sq, Hq, D), in_dtype, rng_for(c, T_Q))
    k = normal_bits((B, Skv, Hkv, D), in_dtype, rng_for(c, T_K))
    v = normal_bits((B, Skv, Hkv, D), in_dtype, rng_for(c, T_V))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return PrefillInputs(q, k, v, B, Hq, Hkv, Sq, Skv, D, bool(causal), f32(scale),
                         in_dtype, out_dtype or in_dtype)


def additive_mask(c: int, Bm: int, Sq: int, Skv: int, kind: str, dtype: str = BF16,
                  stride: Optional[int] = None) -> np.ndarray:
    """uint16 bits [Bm, Sq, stride] of an additive mask (stride >= Skv; columns
    >= Skv hold NaN, which no key may read). Query i sits at key position
    p_i = Skv - Sq + i. Kinds:

    * ``normal``: N(0,1) values with about one entry in eight -inf;
    * ``packed``: several sequences packed into one microbatch at seeded cut
      points of the key positions: key j is visible (0) to query i only inside
      p_i's sequence and for j <= p_i, else -inf;
    * ``bias``: a distance bias -2^-e (p_i - j) for j <= p_i and -inf beyond,
      with a seeded e in 0..3 per batch entry;
    * ``rows``: ``normal`` with every key of a few seeded rows -inf.
    """
    stride = Skv if stride is None else stride
    assert stride >= Skv
    rng = rng_for(c, T_MASK)
    pos = (Skv - Sq + np.arange(Sq))[:, None]
    key = np.arange(Skv)[None, :]
    vals = np.empty((Bm, Sq, Skv), dtype=np.float32)
    for b in range(Bm):
        if kind in ("normal", "rows"):
            x = rng.standard_normal(size=(Sq, Skv), dtype=np.float32)
            x[rng.random(size=(Sq, Skv)) < 0.125] = -np.inf
            if kind == "rows":
                x[rng.choice(Sq, size=max(1, Sq // 16), replace=False)] = -np.inf
        elif kind == "packed":
            n_cut = int(rng.integers(1, 5))
            cuts = np.sort(rng.choice(np.arange(1, max(Skv, 2)), size=min(n_cut, max(Skv - 1, 1)),
                                      replace=False))
            seq = np.searchsorted(cuts, np.arange(Skv), side="right")
            same = seq[np.clip(pos[:, 0], 0, Skv - 1)][:, None] == seq[None, :]
            x = np.where(same & (key <= pos), np.float32(0), np.float32(-np.inf))
        elif kind == "bias":
            slope = np.float32(2.0 ** -int(rng.integers(0, 4)))
            x = np.where(key <= pos, -slope * (pos - key).astype(np.float32), np.float32(-np.inf))
        else:
            raise ValueError(kind)
        vals[b] = x
    bits = np.full((Bm, Sq, stride), NAN_BITS[dtype], dtype=np.uint16)
    r = round_bits(vals, dtype)
    r[np.isneginf(vals)] = NEG_INF_BITS[dtype]
    bits[:, :, :Skv] = r
    return bits


def bias_mask(Sq: int, Skv: int, e: int, dtype: str = BF16, stride: Optional[int] = None,
              block: int = 512) -> np.ndarray:
    """uint16 bits [Sq, stride] of the ``bias`` kind of ``additive_mask`` with a
    given exponent e (value -2^-e (p_i - j) for j <= p_i, -inf beyond; NaN past
    Skv), built a block of rows at a time so that large masks stay cheap."""
    stride = Skv if stride is None else stride
    assert stride >= Skv
    out = np.full((Sq, stride), NAN_BITS[dtype], dtype=np.uint16)
    slope = np.float32(2.0 ** -e)
    key = np.arange(Skv, dtype=np.int64)[None, :]
    for r0 in range(0, Sq, block):
        pos = (Skv - Sq + np.arange(r0, min(r0 + block, Sq), dtype=np.int64))[:, None]
        d = (pos - key).astype(np.float32)
        x = np.where(d >= 0, -slope * d, np.float32(-np.inf))  # -inf rounds to -inf
        out[r0:r0 + len(pos), :Skv] = round_bits(x, dtype)
    return out


def with_mask(inp: PrefillInputs, c: int, kind: str, batched: bool = False,
              stride: Optional[int] = None) -> PrefillInputs:
    """The same inputs with an additive mask attached (one per batch entry if
    ``batched``)."""
    inp.mask = additive_mask(c, inp.B if batched else 1, inp.Sq, inp.Skv, kind, inp.in_dtype,
                             stride)
    return inp


def mla_decode_inputs(c: int, B: int, Hq: int, seq_len: int, D_qk: int = 576, D_v: int = 512,
                      page_size: int = 1, dtype: str = BF16,
                      scale: Optional[float] = None, Sq: int = 1) -> DecodeInputs:
    """Paged MLA decode: every sequence holds ``seq_len`` tokens; the pool has
    exactly B * seq_len / page_size pages, assigned by one seeded permutation.
    With Sq > 1 the queries are each sequence's last Sq tokens, q [B, Sq, Hq, D_qk]."""
    assert seq_len % page_size == 0
    n_pages = B * seq_len // page_size
    q = normal_bits((B, Sq, Hq, D_qk) if Sq > 1 else (B, Hq, D_qk), dtype, rng_for(c, T_Q))
    pool = normal_bits((n_pages, page_size, D_qk), dtype, rng_for(c, T_POOL))
    perm = rng_for(c, T_PERM).permutation(n_pages).astype(np.int32)
    page_table = np.ascontiguousarray(perm.reshape(B, seq_len // page_size))
    seq_lens = np.full((B,), seq_len, dtype=np.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(192.0)
    return DecodeInputs(q, pool, page_table, seq_lens, B, Hq, 1, D_qk, D_v, page_size,
                        seq_len, "mla", f32(scale), dtype, Sq)


def split_decode_inputs(c: int, B: int, Hq: int, Hkv: int, D: int, lens, page_size: int,
                        dtype: str = BF16, spare_pages: int = 64,
                        scale: Optional[float] = None, poison: bool = True,
                        Sq: int = 1) -> DecodeInputs:
    """Paged decode with separate K and V per (page, head); with Sq > 1 the
    queries are the last Sq tokens of each sequence, q [B, Sq, Hq, D].

    Pool layout ``[num_pages, 2 (K, V), Hkv, page_size, D]``. Sequence b owns
    ceil(len_b / page_size) pages drawn from a seeded permutation of the pool;
    page-table entries past a sequence's last page are -1. Slots past a
    sequence's length in its last page, and every spare page, hold NaN.
    """
    lens = np.asarray(lens, dtype=np.int64)
    assert lens.shape == (B,)
    pages_per = [(int(n) + page_size - 1) // page_size for n in lens]
    n_pages = int(sum(pages_per)) + spare_pages
    max_len = int(lens.max()) if B else 0
    max_pages = max(1, (max_len + page_size - 1) // page_size)
    q = normal_bits((B, Sq, Hq, D) if Sq > 1 else (B, Hq, D), dtype, rng_for(c, T_Q))
    pool = normal_bits((n_pages, 2, Hkv, page_size, D), dtype, rng_for(c, T_POOL))
    perm = rng_for(c, T_PERM).permutation(n_pages).astype(np.int32)
    page_table = np.full((B, max_pages), -1, dtype=np.int32)
    used = np.zeros(n_pages, dtype=bool)
    at = 0
    for b in range(B):
        n = pages_per[b]
        page_table[b, :n] = perm[at:at + n]
        used[perm[at:at + n]] = True
        at += n
        if poison and n and lens[b] % page_size:
            tail = int(lens[b] % page_size)
            pool[perm[at - 1], :, :, tail:, :] = NAN_BITS[dtype]
    if poison:
        pool[~used] = NAN_BITS[dtype]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return DecodeInputs(q, pool, page_table, lens.astype(np.int32), B, Hq, Hkv, D, D,
                        page_size, max_len, "split", f32(scale), dtype, Sq)


def random_lens(c: int, B: int, lo: int, hi: int) -> np.ndarray:
    """Per-sequence lengths uniform over the closed range [lo, hi]."""
    return rng_for(c, T_LENS).integers(lo, hi, size=B, endpoint=True).astype(np.int32)


# ---------------------------------------------------------------------------
# The five workloads. Numbering is the ``c`` of the seeding recipe.
# ---------------------------------------------------------------------------

WORKLOADS = {
    1: "tiny causal attention: B=1 Hq=Hkv=4 S=128 D=64 fp16 in, fp32 out, scale 1/8",
    2: "non-causal MHA prefill: B=4 Hq=Hkv=16 S=2048 D=64 bf16, scale 1/8",
    3: "causal GQA prefill: B=1 Hq=32 Hkv=8 S=16384 D=128 bf16 as 32 ubatches of 512 queries",
    4: "paged MLA decode: batch 128, 64 heads, D_qk 576 (512 latent + 64 rope), D_v 512, "
       "seq_len 2048, page_size 1, random page permutation, scale 1/sqrt(192)",
    5: "small-batch GQA decode: batch 4, Hq 32, Hkv 8, D 128, lengths U[1024, 32768], page_size 16",
}

UBATCH = 512  # queries per microbatch of workload 3


def workload(c: int):
    if c == 1:
        return prefill_inputs(1, 1, 4, 4, 128, 128, 64, True, FP16, FP32, scale=0.125)
    if c == 2:
        return prefill_inputs(2, 4, 16, 16, 2048, 2048, 64, False, BF16, BF16, scale=0.125)
    if c == 3:
        return prefill_inputs(3, 1, 32, 8, 16384, 16384, 128, True, BF16, BF16)
    if c == 4:
        return mla_decode_inputs(4, 128, 64, 2048)
    if c == 5:
        return split_decode_inputs(5, 4, 32, 8, 128, random_lens(5, 4, 1024, 32768), 16)
    raise KeyError(c)


def bits_view(a: np.ndarray, dtype: str) -> np.ndarray:
    """Reinterpret uint16 bits as numpy float16 (fp16 only; bf16 has no numpy type)."""
    if dtype != FP16:
        raise ValueError("only fp16 has a numpy view")
    return a.view(np.float16)
