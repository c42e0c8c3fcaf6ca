// Paged-KV decode attention for gfx950, grouped-query variant: one query token
// per sequence against every cached token of the sequence, read through a page
// table from a pool with separate K and V blocks per (page, K/V head). The
// query heads that share a K/V head are packed into one MFMA operand, the GQA
// idea of "CUDA: fix FA occupancy, optimize tile kernel" (opening paragraph), so
// each K/V row is read once per group. (The MLA variant is decode_mla.hip.)
//
// The kernel uses v_mfma_f32_16x16x32 with the scores transposed
// (S^T = K Q^T: A = 16 keys, B = 16 query heads of the group held in
// registers). A lane then holds one head and 4 keys of each 16-key block; the
// head's max and sum need two cross-lane steps. The probabilities are rounded to
// 16 bits in registers and become the B operand of O^T += V^T P^T, whose A
// operand is read from a row-major V tile in LDS with the transpose read
// (ds_read_b64_tr_b16); the contraction index is relabelled so that each lane's
// 8 keys match its probability registers.
//
// Several new tokens per sequence (Sq > 1: speculative or chunked decode) are
// packed into the MFMA rows with the heads: row r = i * G + h is token i (at
// position seq_len - Sq + i, so it sees keys up to that position: causal,
// bottom-right) and head h of the group, and all rows of a unit share each
// K/V row it loads.
//
// Sequences too short to fill the chip are split over several key ranges
// (split-KV); each split writes a normalised partial O and its log-sum-exp for
// the combine kernel. Tokens past seq_len, including page slots that hold
// garbage or NaN, are never loaded: their K and V registers are zero and their
// scores -infinity.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// ---------------------------------------------------------------------------
// Grouped-query decode over the split K/V pool [P, 2, Hkv, page, 128].
// One wave is one work unit (sequence b, K/V head g, block of up to 16 query
// heads of the group, key split); a workgroup holds 8 independent units.
// ---------------------------------------------------------------------------
constexpr int DS_D = 128;
constexpr int DS_VS = DS_D + 16;  // V row stride in LDS (elements)

template <typename TI, int PS>
__global__ __launch_bounds__(512) void decode_split_kernel(DecodeSplitParams p) {
  using T = in_traits<TI>;
  constexpr int D = DS_D;
  __shared__ __attribute__((aligned(16))) char smem[8][DEC_TILE * DS_VS * 2];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // unit indices stay scalar
  int unit = blockIdx.x * 8 + w;
  if (unit >= p.n_units) return;  // whole wave leaves; the kernel has no barriers
  char* vlds = smem[w];

  // Units are numbered with the K/V head fastest: the waves of a workgroup take
  // neighbouring head slices of the same pages (the same key range of one
  // sequence; with 8 K/V heads the 8 waves read each 16-token page of K and V
  // whole, 2 x 32 KB contiguous, at about the same time), and the units of a
  // split past its sequence's end fill whole workgroups that leave at once.
  // Workload 5: 48.0 us with split-fastest numbering in 4-wave workgroups,
  // 47.0 with head-fastest, 45.2 with 8-wave workgroups (one process each).
  const int S = p.n_splits;
  const int g = unit % p.Hkv;
  unit /= p.Hkv;
  const int hb = unit % p.n_hblk;
  unit /= p.n_hblk;
  const int split = unit % S;
  const int b = unit / S;
  const int G = p.Hq / p.Hkv;
  const int c16 = lane & 15, gq = lane >> 4;
  const int rig = hb * 16 + c16;  // row inside the group: token rig / G, head rig % G
  const bool hvalid = rig < G * p.Sq;
  const int tok = hvalid ? rig / G : 0;
  const int hq = g * G + (hvalid ? rig % G : 0);

  const int seq_len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int t0 = split * p.chunk;
  const int t1 = min(t0 + p.chunk, seq_len);
  const int lim = seq_len - p.Sq + tok;  // last key this row sees
  const int lim_lo = seq_len - p.Sq;     // the smallest such key over the rows

  u32x4 qf[D / 32];
  {
    const char* qrow = (const char*)p.q + (((int64_t)b * p.Sq + tok) * p.Hq + hq) * D * 2;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[s] = hvalid ? ldg16(qrow + (32 * s + 8 * gq) * 2) : u32x4{0, 0, 0, 0};
  }
  const int32_t* ptab = p.page_table + (int64_t)b * p.max_pages;
  // Bytes per page and from a page's K block to its V block (a page is below
  // 2 GiB: checked on the host).
  const unsigned page_stride = 2u * (unsigned)p.Hkv * (unsigned)p.page_size * D * 2;
  const unsigned kv_stride = (unsigned)p.Hkv * (unsigned)p.page_size * D * 2;
  const char* pool_g = (const char*)p.pool + (int64_t)g * p.page_size * D * 2;

  // Each lane touches 10 token rows of a 32-token tile: 2 as key rows of the
  // MFMA A operand (tokens 16*kb + c16) and 8 as value rows copied to LDS
  // (tokens gq + 4*r). With a page size that is a multiple of 16 every 16-token
  // half of a tile lies in one page, so a lane needs the page ids of the two
  // halves only (HALVES); otherwise it needs one per row. The ids are fetched
  // two tiles ahead, so no row load waits on a page-table load; the table is
  // read at keys clamped to max_seq_len - 1 (inside the table, whose rows cover
  // max_seq_len tokens), so the first fetch does not wait for the sequence's
  // length: the length, the first page ids and the queries are three loads in
  // flight together, and the first rows follow one round trip later. Invalid
  // rows (past the split, or with an out-of-range page id) load the pool's
  // first row and are zeroed by a select. Key and
  // slot arithmetic is unsigned (keys are never negative), and a page's bytes
  // fit in 32 bits (checked on the host), so a row's offset is one 32 x 32 ->
  // 64-bit multiply-add.
  constexpr bool HALVES = PS > 0 && PS % 16 == 0;
  constexpr int NPG = HALVES ? 2 : 10;
  const unsigned last_key = (unsigned)max(p.max_seq_len - 1, 0);
  const unsigned psize = PS > 0 ? (unsigned)PS : (unsigned)p.page_size;
  auto row_key = [&](int r, int tt) { return tt + (r < 2 ? 16 * r + c16 : gq + 4 * (r - 2)); };
  auto fetch_pages = [&](int (&pg)[NPG], int tt) {
#pragma unroll
    for (int i = 0; i < NPG; ++i) {
      const int key = HALVES ? tt + 16 * i : row_key(i, tt);
      const unsigned kc = min((unsigned)key, last_key);
      pg[i] = ptab[kc / psize];  // (row_off rejects keys past the split)
    }
  };
  auto row_off = [&](const int (&pg)[NPG], int r, int tt, bool& ok) -> uint64_t {
    const int key = row_key(r, tt);
    const int id = HALVES ? pg[r < 2 ? r : (r - 2) / 4] : pg[r];
    const unsigned slot = (unsigned)key % psize;
    ok = key < t1 && (unsigned)id < (unsigned)p.num_pages;
    const uint64_t o = (uint64_t)(unsigned)id * page_stride + slot * (unsigned)(D * 2);
    return ok ? o : 0;
  };

  // One tile in flight: K of tile t + 1 is loaded into the registers that K
  // of tile t has just fed to the score MFMAs, and V of tile t + 1 into the
  // staging registers once V of tile t is in LDS. (Two tiles in flight, with
  // the loads issued on every path, measured no faster on the small-batch
  // workload, 50.5 against 47.7 us: the waves are not waiting on a single
  // tile's latency.)
  u32x4 kr[2][D / 32], vr[8];
  bool kok[2], vok[8];
  auto load_k = [&](const int (&pg)[NPG], int tt) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint64_t o = row_off(pg, kb, tt, kok[kb]);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) kr[kb][s] = ldg16(pool_g + o + (32 * s + 8 * gq) * 2);
    }
  };
  auto load_v = [&](const int (&pg)[NPG], int tt) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const uint64_t o = row_off(pg, 2 + r, tt, vok[r]);
      vr[r] = ldg16(pool_g + o + kv_stride + c16 * 16);
    }
  };
  // Rows outside the split (or with a page id out of range) are zeroed only
  // in a tile that has one: the last tile of a split.
  auto store_v = [&]() {
    bool all = true;
#pragma unroll
    for (int r = 0; r < 8; ++r) all = all && vok[r];
    if (__ballot(!all)) {
#pragma unroll
      for (int r = 0; r < 8; ++r)
        *(u32x4*)(vlds + ((gq + 4 * r) * DS_VS + c16 * 8) * 2) = vok[r] ? vr[r] : u32x4{0, 0, 0, 0};
    } else {
#pragma unroll
      for (int r = 0; r < 8; ++r) *(u32x4*)(vlds + ((gq + 4 * r) * DS_VS + c16 * 8) * 2) = vr[r];
    }
  };

  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  // pg holds the page ids of the tile whose loads are issued next.
  int pg[NPG];
  fetch_pages(pg, t0);
  if (t0 < t1) {
    load_k(pg, t0);
    load_v(pg, t0);
    fetch_pages(pg, t0 + DEC_TILE);
  }
  // A negative scale runs as -Q with |scale|; the sign is applied after the
  // first tile's loads are issued, so the query loads overlap the page-table
  // and row loads instead of being waited for first.
  if (p.q_neg) {
#pragma unroll
    for (int s = 0; s < D / 32; ++s) qf[s] = neg16x8(qf[s]);
  }
  for (int tt = t0; tt < t1; tt += DEC_TILE) {
    const bool more = tt + DEC_TILE < t1;
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
    if (__ballot(!(kok[0] && kok[1]))) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < D / 32; ++s)
          if (!kok[kb]) kr[kb][s] = u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int s = 0; s < D / 32; ++s) sacc[kb] = T::mma16(kr[kb][s], qf[s], sacc[kb]);
    }
    if (more) load_k(pg, tt + DEC_TILE);
    wave_lds_sync();  // the previous tile's V reads are done
    store_v();
    if (more) {
      load_v(pg, tt + DEC_TILE);
      fetch_pages(pg, tt + 2 * DEC_TILE);
    }
    wave_lds_sync();
    const bool tail = tt + DEC_TILE > t1;
    if (tail) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tt + 16 * kb + 4 * gq + i >= t1) sacc[kb][i] = -INFINITY;
    }
    if (tt + DEC_TILE - 1 > lim_lo) {  // keys past an earlier new token's position
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tt + 16 * kb + 4 * gq + i > lim) sacc[kb][i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                     fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    const bool grow = mx > m_run && (m_run == -INFINITY || (mx - m_run) * sl2 > RESCALE_LOG2);
    if (__ballot(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * sl2);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float nb = m_run == -INFINITY ? 0.f : -m_run * sl2;
    float pv[2][4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) pv[kb][i] = fast_exp2(fmaf(sacc[kb][i], sl2, nb));
    const u32x4 pb{T::pack2(pv[0][0], pv[0][1]), T::pack2(pv[0][2], pv[0][3]),
                   T::pack2(pv[1][0], pv[1][1]), T::pack2(pv[1][2], pv[1][3])};
    // The row sum is taken over the 16-bit probabilities the P V product uses,
    // so the output's weights are exactly the ones it is normalised by.
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) l_run = T::sum2(pb[q4], l_run);
    const int j = c16;
    const char* va = vlds + ((4 * gq + (j >> 2)) * DS_VS + 4 * (j & 3)) * 2;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const u32x2 r0 = lds_read_tr16(va + 16 * db * 2);
      const u32x2 r1 = lds_read_tr16(va + (16 * DS_VS + 16 * db) * 2);
      oacc[db] = T::mma16(u32x4{r0[0], r0[1], r1[0], r1[1]}, pb, oacc[db]);
    }
  }

  float l_tot = l_run + xor16(l_run);
  l_tot += xor32(l_tot);
  if (!hvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_run * p.scale + __logf(l_tot) : -INFINITY;
  // The output row ([B, Sq, Hq] order), or with several splits this split's
  // partial row (same 16-bit type; the combine weighs the partials by their
  // lse and writes lse as [B, Hq, Sq]).
  const int64_t row = ((int64_t)b * p.Sq + tok) * p.Hq + hq;
  const int64_t prow = S == 1 ? row : (int64_t)split * p.B * p.Sq * p.Hq + row;
  char* orow = (char*)(S == 1 ? p.o : p.part_o) + prow * D * 2;
#pragma unroll
  for (int db = 0; db < D / 16; ++db) {
    const int d = 16 * db + 4 * gq;
    const u32x2 v{T::pack2(oacc[db][0] * inv, oacc[db][1] * inv),
                  T::pack2(oacc[db][2] * inv, oacc[db][3] * inv)};
    *(u32x2*)(orow + d * 2) = v;
  }
  if (gq == 0) {
    if (S > 1)
      p.part_lse[prow] = lse;
    else if (p.lse)
      p.lse[((int64_t)b * p.Hq + hq) * p.Sq + tok] = lse;
  }
}

template <typename TI>
static hipError_t split_dispatch(const DecodeSplitParams& p, hipStream_t stream) {
  const int blocks = (p.n_units + 7) / 8;
  if (p.page_size == 16)
    hipLaunchKernelGGL((decode_split_kernel<TI, 16>), dim3(blocks), dim3(512), 0, stream, p);
  else if (p.page_size == 1)
    hipLaunchKernelGGL((decode_split_kernel<TI, 1>), dim3(blocks), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<TI, 0>), dim3(blocks), dim3(512), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeSplitParams& p, InType it, hipStream_t stream) {
  return it == InType::bf16 ? split_dispatch<bf16_t>(p, stream) : split_dispatch<f16_t>(p, stream);
}

}  // namespace fa
