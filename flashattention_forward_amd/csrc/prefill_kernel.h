// Fused attention prefill kernel for gfx950 (a template, instantiated per head size
// and input type by prefill.hip, prefill_f16.hip and prefill_d64.hip): O = softmax(scale * Q K^T + mask) V with an
// online softmax, one pass over the keys.
//
// The tile-FA idea of "CUDA: fix FA occupancy, optimize tile kernel" (llama.cpp,
// opening paragraph) -- stage K/V tiles on chip with 16-byte copies, keep the
// score tile in registers and compress it to 16 bits before the second product,
// size tiles to the chip's shared memory -- rebuilt for CDNA4 matrix cores:
//
//  * each wave owns 32 query rows of one head; a workgroup of 4 or 8 waves
//    (chosen by the host) shares every K/V tile of 64 keys in LDS. It takes
//    128 or 256 rows of one query head, or (a head pack, the grouped-query
//    packing) the same 32 NW / PK rows of PK query heads that share one K/V
//    head. With 8 waves a tile copied into LDS serves twice the rows, halving
//    the L2-to-CU traffic per flop;
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16 (A = K
//    rows from LDS, B = the wave's Q rows held in registers for the whole pass).
//    Each lane then owns one query column and 16 keys of each 32-key block, so
//    the row max is in-lane plus one v_permlane32_swap;
//  * the probabilities are rounded to 16 bits in registers and fed straight back
//    as the B operand of O^T += V^T P^T. The contraction index of that product
//    is relabelled to match the accumulator layout; the V^T operand comes from
//    the row-major V tile through the LDS transpose read (ds_read_b64_tr_b16);
//  * K and V tiles go from global memory straight into LDS (global_load_lds,
//    no register staging), each into a 2-stage ring, and barriers wait on LDS
//    traffic only;
//  * the steps are software-pipelined as in the FlashAttention-3 schedule that
//    "perf: FlashAttention-3 style MLA PageAttention" (FlashInfer, change list
//    item 3) adopts: the MFMAs of S(t+1) = K(t+1) Q^T are issued before the
//    softmax of tile t, so the exp-heavy vector work of one tile overlaps the
//    matrix-core work of the next. Each step is one straight-line block written
//    out in issue order (K reads four MFMAs ahead, six vector ops of the
//    softmax under each score MFMA, the transpose reads ahead of the PV MFMAs,
//    the next tile's row max under them) and fenced with sched_barrier;
//  * tiles are stored in 8 x 8 blocks of 16-byte chunks (blk_slot): a copy
//    instruction moves 8 key rows x 128 contiguous bytes, and the K reads (16
//    rows of one chunk) and the transposed V reads (4 rows x 4 chunks) each
//    touch 64 distinct banks;
//  * causal (bottom-right aligned) blocks stop at their last visible tile and
//    only tiles crossing the diagonal or the end of the keys are masked (a tile
//    above a wave's diagonal runs through the same block with probability 0);
//  * the exponent uses exp2 with scale * log2(e) folded into one FMA, and the
//    running max moves only when it grows by more than 2^8, so the O
//    accumulators are rarely rescaled;
//  * a workgroup may process one of several key splits; it then writes its
//    normalised partial O and log-sum-exp for a separate combine kernel;
//  * with an explicit additive mask (the KQ mask that the same llama.cpp page
//    counts as memory traffic) the mask of the workgroup's query rows for the
//    next tile is copied into LDS with the same direct copies as K and V (8
//    rows x 128 bytes per instruction) -- once per head pack, so with PK heads
//    per workgroup each mask tile is read from memory once for PK heads, the
//    page's grouped-query optimisation of the mask I/O; every lane then reads the
//    16 values of its row per 32-key block from LDS, and the scores are taken
//    to the softmax's natural-log domain as fma(s, scale, mask) (one op after
//    unpacking the 16-bit value) before the row max; the running max, rescale
//    and exponent then work unchanged with an exponent scale of log2 e.
#pragma once

#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <int D, int NW_> struct PfCfg {
  static constexpr int NCH = D / 8;           // 16-byte chunks per key row
  static constexpr int NCB = NCH / 8;         // 8-chunk blocks per key row
  static constexpr int TILE = PF_BN * D * 2;  // bytes of one K (or V) tile
  static constexpr int LDS = 4 * TILE;        // 2 K stages + 2 V stages
  // LDS reserved per workgroup. Head size 64 with 4 waves needs only 32 KB
  // and 164 VGPRs, so three workgroups would share a CU; the schedule is built
  // for two waves per SIMD, and a third made the 1024-workgroup grid of the
  // 4 x 16 x 2048 x 64 MHA run as 1 1/3 rounds (102.8 us against 93.2 us with
  // 56 KB reserved, which leaves room for two).
  static constexpr int LDS_RESERVE = (D == 64 && NW_ == 4) ? 56 * 1024 : LDS;
  static constexpr int NW = NW_;              // waves per workgroup
  static constexpr int BPW = 8 * NCB / NW;    // 1 KB blocks of a tile each wave copies
  // With an additive mask the K/V stages are followed by 4 KB of mask tile
  // per wave (32 rows x 64 keys): one stage of each wave's own rows, or, with a
  // head pack, two stages of the workgroup's shared rows; 4 waves of head size
  // 128 then take 80 KB, so two workgroups still share a CU.
  static constexpr int MASK_LDS = NW * 4096;
  static constexpr int LDS_MASKED = LDS + MASK_LDS > LDS_RESERVE ? LDS + MASK_LDS : LDS_RESERVE;
};

// AM: 0 no additive mask; 1 mask added at each step's start (one head per
// workgroup); 2 mask added one tile ahead under the P V MFMAs (head packs).
template <int D, int NW, typename TI, typename TO, bool CAUSAL, int AM>
__global__ __launch_bounds__(64 * NW, 2) void prefill_kernel(PrefillParams p) {
  constexpr bool AMASK = AM != 0;
  using C = PfCfg<D, NW>;
  using T = in_traits<TI>;
  __shared__ __attribute__((aligned(16))) char smem[AMASK ? C::LDS_MASKED : C::LDS_RESERVE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c = lane & 31, h = lane >> 5;

  // Logical block: (b, kv head g, query tile, head pack, split), with the
  // blocks that share one K/V head kept on one XCD (its L2). A head pack is
  // PK of the G query heads that share K/V head g: the workgroup's waves are
  // PK groups of WPH = NW / PK waves, group j taking query head hp PK + j and
  // the same BMq = 32 WPH query rows. With PK > 1 every K/V tile and every
  // mask tile copied into LDS serves PK heads (the grouped-query packing: the
  // mask is read once per head pack instead of once per head). (A split-major
  // order, which puts the workgroups that share a mask tile on fewer XCDs,
  // measured the same.)
  int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int S = p.n_splits;
  const int split = blk % S;
  blk /= S;
  const int G = p.Hq / p.Hkv;
  const int PK = p.pack;
  const int WPH = NW / PK;  // waves per head
  const int hp = blk % (G / PK);
  blk /= G / PK;
  int qt = blk % p.n_qtiles;
  blk /= p.n_qtiles;
  const int g = blk % p.Hkv;
  const int b = blk / p.Hkv;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // longest rows first
  const int hq = g * G + hp * PK + w / WPH;
  const int off = p.Skv - p.Sq;  // bottom-right alignment
  const int BMq = 32 * WPH;      // query rows of the workgroup
  const int q0 = qt * BMq;

  int kv_end = p.Skv;
  if (CAUSAL) kv_end = min(kv_end, min(q0 + BMq, p.Sq) + off);
  const int n_tiles = kv_end > 0 ? (kv_end + PF_BN - 1) / PF_BN : 0;
  const int tps = (n_tiles + S - 1) / S;
  const int t_begin = min(split * tps, n_tiles);
  const int t_end = min(t_begin + tps, n_tiles);

  const int row_bytes = p.Hkv * D * 2;
  const char* kbase = (const char*)p.k + ((int64_t)b * p.Skv * p.Hkv + g) * D * 2;
  const char* vbase = (const char*)p.v + ((int64_t)b * p.Skv * p.Hkv + g) * D * 2;

  // This lane's query row and its Q fragment (B operand, 16 dims per MFMA step).
  const int qw0 = q0 + 32 * (w % WPH);  // first row of this wave
  const int qi = qw0 + c;
  const bool q_ok = qi < p.Sq;
  u32x4 qf[D / 16];
  {
    const char* qrow = (const char*)p.q + (((int64_t)b * p.Sq + qi) * p.Hq + hq) * D * 2;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 v = q_ok ? ldg16(qrow + (16 * s + 8 * h) * 2) : u32x4{0, 0, 0, 0};
      qf[s] = p.q_neg ? neg16x8(v) : v;
    }
  }

  // Copies. K and V have separate 2-stage rings: K tile t lives in K stage
  // (t - t_begin) & 1, V tile t in V stage (t - t_begin) & 1. Each tile is
  // 8 * NCB blocks of 1 KB (8 key rows x 8 chunks); wave w copies blocks
  // n = BPW w + i (i < BPW). In block n (row block RB = n / NCB, chunk block
  // CB = n % NCB) lane l copies chunk 8 CB + ((l >> 3) ^ (RB & 1)) of key row
  // 8 RB + ((l & 7) ^ 4 * ((l >> 4) & 1)) (the inverse of blk_slot), so a
  // copy instruction moves 8 rows x 128 contiguous bytes. The per-lane byte
  // offsets are fixed; a tile only moves the wave-uniform base. In the last
  // tile, keys past the end are clamped to the last key: their scores are
  // masked and their probabilities are 0.
  const uint32_t smem_lds = __builtin_amdgcn_readfirstlane(lds_addr(smem));
  const int dma_rho = (lane & 7) ^ (4 * ((lane >> 4) & 1));
  uint32_t voff[C::BPW];
  int vrow[C::BPW];
#pragma unroll
  for (int i = 0; i < C::BPW; ++i) {
    const int n = C::BPW * w + i, RB = n / C::NCB, cb = n % C::NCB, rb_odd = RB & 1;
    vrow[i] = 8 * RB + dma_rho;
    voff[i] = (uint32_t)(vrow[i] * row_bytes + (8 * cb + ((lane >> 3) ^ rb_odd)) * 16);
  }
  auto issue = [&](const char* base, uint32_t st, int t) {
    const int k0 = t * PF_BN;
    const char* src = base + (int64_t)k0 * row_bytes;
    const uint32_t dst = st + C::BPW * w * 1024;
    if (k0 + PF_BN <= p.Skv) {
#pragma unroll
      for (int i = 0; i < C::BPW; ++i) dma16s(src, voff[i], dst + i * 1024);
    } else {
      const int last = p.Skv - 1 - k0;
#pragma unroll
      for (int i = 0; i < C::BPW; ++i) {
        const int over = vrow[i] - last;
        dma16s(src, over > 0 ? voff[i] - (uint32_t)(over * row_bytes) : voff[i], dst + i * 1024);
      }
    }
  };
  auto k_stage = [&](int t) { return ((t - t_begin) & 1) * C::TILE; };
  auto v_stage = [&](int t) { return (2 + ((t - t_begin) & 1)) * C::TILE; };
  auto issue_k = [&](int t) { issue(kbase, smem_lds + k_stage(t), t); };
  auto issue_v = [&](int t) { issue(vbase, smem_lds + v_stage(t), t); };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  // The row sum is kept as four partial sums (dot product r of a step feeds
  // sum r % 4), so accumulating dot products that issue close together are
  // independent and need no wait states between them.
  float m_run = -INFINITY, l_run[4] = {0.f, 0.f, 0.f, 0.f};
  // With a mask the scores are already scaled (natural-log domain).
  const float sl2 = AMASK ? 1.4426950408889634f : p.scale_log2;

  // Mask tiles in LDS. The workgroup's BMq x 64 mask tile is held in 1 KB
  // blocks of 8 query rows (block RB: rows q0 + 8 RB .. + 7 and all 8 chunks of
  // 8 keys), row r and chunk k in 16-byte slot 8 (k ^ (RB & 1)) + r, so that
  // one copy instruction moves 8 rows x 128 contiguous bytes and a read of one
  // chunk by a wave's 32 rows spreads over the banks. With one head per
  // workgroup (PK = 1) each wave copies the 4 blocks of its own rows into its
  // own one-stage buffer; with a head pack the tile is copied once for the PK
  // heads into a shared 2-stage ring (tile t in stage (t - t_begin) & 1; the
  // step's barrier orders copies and reads), the copies spread over the waves.
  // Each wave reads the 4 blocks of its 32 rows. Rows past the end of the
  // queries copy the last row; in the last tile a chunk at or past the end of
  // the keys copies chunk 0 instead (those keys are masked anyway, and the rest
  // of the chunk holding the end lies inside the mask's row stride).
  // Lane (c, h) needs keys 8 m + 4 h .. + 3 of chunk m, i.e. the four scores
  // 4 (m & 3) .. + 3 of score block m >> 2.
  u32x2 mk[8];
  const char* mbase = nullptr;
  uint32_t moff[4] = {};
  int mchunk[4] = {};
  // Blocks this wave copies: mblk0 .. mblk0 + n_mblk - 1.
  const int nbw = PK >= 4 ? 1 : 4 / PK;
  const int n_mblk = (w / WPH) * nbw < 4 ? nbw : 0;
  const int mblk0 = 4 * (w % WPH) + (w / WPH) * nbw;
  constexpr int MSTAGE = C::MASK_LDS / 2;  // bytes of a ring stage (PK > 1)
  const uint32_t mlds = smem_lds + C::LDS + 1024 * mblk0;
  const char* mread = smem + C::LDS + 4096 * (w % WPH) + 1024 * (c >> 3) + 16 * (c & 7) + 8 * h;
  const int mflip = ((c >> 3) & 1) ? 128 : 0;
  if constexpr (AMASK) {
    mbase = (const char*)p.mask + (int64_t)b * p.mask_bstride * 2;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = min(q0 + 8 * (mblk0 + i) + (lane & 7), p.Sq - 1);
      mchunk[i] = (lane >> 3) ^ ((mblk0 + i) & 1);
      moff[i] = (uint32_t)row * (uint32_t)(p.mask_stride * 2) + 16 * mchunk[i];
    }
  }
  auto m_stage = [&](int t) { return PK > 1 ? ((t - t_begin) & 1) * MSTAGE : 0; };
  auto issue_mask = [&](int t) {
    const int k0 = t * PF_BN;
    const char* src = mbase + (int64_t)k0 * 2;
    const uint32_t dst = mlds + m_stage(t);
    if (k0 + PF_BN <= p.Skv) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < n_mblk) dma16s(src, moff[i], dst + 1024 * i);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (i < n_mblk)
          dma16s(src, k0 + 8 * mchunk[i] < p.Skv ? moff[i] : moff[i] - 16 * mchunk[i],
                 dst + 1024 * i);
    }
  };
  // Chunk m is at slot 8 (m ^ (RB & 1)) + r: 128 m, moved by -128 or +128 for
  // odd row blocks.
  auto read_mask = [&](int t) {
    const char* mr = mread + m_stage(t);
#pragma unroll
    for (int m = 0; m < 8; ++m)
      mk[m] = *(const u32x2*)(mr + 128 * m + ((m & 1) ? -mflip : mflip));
  };
  // Scores of the tile into the natural-log domain: s * scale + mask.
  auto add_mask = [&](f32x16 (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t w2 = mk[4 * kb + (i >> 2)][(i >> 1) & 1];
        const uint16_t bits = (i & 1) ? (uint16_t)(w2 >> 16) : (uint16_t)w2;
        float mv;
        if constexpr (std::is_same<TI, bf16_t>::value)
          mv = __uint_as_float((uint32_t)bits << 16);
        else
          mv = (float)__builtin_bit_cast(_Float16, bits);
        sacc[kb][i] = fmaf(sacc[kb][i], p.scale, mv);
      }
  };

  // Per-lane LDS offsets (blk_slot written out). K (A operand): row 32 kb + c,
  // chunk 2s + h; the offset alternates with the parity of s.
  const int kbase_off = 1024 * C::NCB * (c >> 3) + 128 * (h ^ ((c >> 3) & 1));
  const int koffE = kbase_off + 16 * (c & 7), koffO = kbase_off + 16 * ((c & 7) ^ 4);
  // V^T (A operand) by transpose reads: lane j = lane & 15 of 16-lane group gb
  // = (lane >> 4) & 1 reads rows 16 jj + 4h + j/4 (read A) and + 8 (read B) of
  // chunk 4 db + 2 gb + e, e = (j & 3) >> 1, byte 8 * (j & 1).
  const int j = lane & 15, gb = (lane >> 4) & 1, e = (j & 3) >> 1;
  const int voffA = 256 * gb + 128 * e + 64 * (h ^ gb) + 16 * (j >> 2) + 8 * (j & 1);
  const int voffB = voffA + 1024 * C::NCB + 128 * (1 - 2 * e);

  // S^T of one tile: 2 * D / 16 MFMAs from the K stage.
  auto qk = [&](f32x16 (&sacc)[2], const char* Ks) {
    sacc[0] = f32x16{};
    sacc[1] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const u32x4 a = lds16(Ks + ((s & 1) ? koffO : koffE) + 256 * s + 4096 * C::NCB * kb);
        sacc[kb] = T::mma32(a, qf[s], sacc[kb]);
      }
    }
  };

  // Last key this lane's query row may see.
  const int lim = CAUSAL ? min(p.Skv - 1, qi + off) : p.Skv - 1;

  // Row max of one tile's scores (both lane halves combined).
  auto tile_max = [&](const f32x16 (&sacc)[2]) {
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
    return max_xor32(mx);
  };
  // Masked tiles: keys beyond `lim` (per lane) get score -inf, and the max is
  // taken again over what is left.
  auto apply_mask = [&](f32x16 (&sacc)[2], int k0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
        if (key > lim) sacc[kb][i] = -INFINITY;
      }
    return tile_max(sacc);
  };
  // Lazy rescale: the running max moves only when it grows by > 2^8; returns
  // the exponent offset -m * scale * log2(e).
  auto rescale = [&](float mx) {
    const bool grow = mx > m_run && (m_run == -INFINITY || (mx - m_run) * sl2 > RESCALE_LOG2);
    if (__ballot(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * sl2);
#pragma unroll
      for (int i = 0; i < 4; ++i) l_run[i] *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    return m_run == -INFINITY ? 0.f : -m_run * sl2;
  };

  // One straight-line block, written out in issue order and fenced slot by
  // slot so that the compiler keeps the interleave:
  //   slots 0 .. NQK-1: one MFMA of S(t+1) = K(t+1) Q^T, the K read PD MFMAs
  //     ahead;
  //   slots NQK .. NQK+NPV-1: one MFMA of O^T += V^T(t) P^T(t), its transpose
  //     reads PD MFMAs ahead;
  //   and under every MFMA VPS vector ops of the step's vector work, in order:
  //     E: for each 8 of tile t's 32 probabilities per lane, 8 (fma, exp2)
  //        pairs and 4 packs to 16 bits (done before the first P V MFMA that
  //        reads them);
  //     R: the 16 row-sum dot products over the packed probabilities, into
  //        four partial sums;
  //     M: the row max of S(t+1), four chains of max3 (they start once the
  //        score MFMAs have drained; returned in mx_next).
  //   (Accumulating ops of one chain that issue within two instructions of
  //   each other need a wait state between them; four chains avoid it.)
  //   Spread over both halves of the step the vector work stays near four ops
  //   per MFMA, which the SIMD co-issues with the matrix core; packed under
  //   the score MFMAs alone it was six, and the vector unit set the pace.
  //   Each op's result is pinned in its slot (an empty asm that takes and
  //   returns the value), since instruction selection would otherwise sink
  //   the row-sum and max chains to the end of the block.
  //   Masked scores are -inf already, and exp2(-inf * sl2 + nb) = 0 because
  //   sl2 > 0 (a zero scale is passed as the smallest positive one).
  auto body = [&](f32x16 (&cur)[2], f32x16 (&nxt)[2], const char* Ks, const char* Vs, float nb,
                  float& mx_next, auto ahead_tag, const char* mnext, auto&& copy_k, auto&& copy_v) {
    // ahead: add the additive mask of tile t + 1 (read from LDS at mnext) to
    // S(t+1) in the M part, under the P V MFMAs, instead of at the next step's
    // start: each M unit is then two (unpack, fma) pairs and a max3.
    constexpr bool AHEAD = decltype(ahead_tag)::value;
    constexpr int NQK = D / 8, NPV = D / 8, NDB = D / 32, PD = 4;
    constexpr int MW = AHEAD ? 5 : 1;  // op slots per M unit
    constexpr int NE = 4 * 20, NR = 16, NM = 16 * MW;
    constexpr int NOPS = NE + NR + NM;
    constexpr int NSLOT = NQK + NPV;
    // Head size 128: the step's K and V copies go out under the score MFMAs
    // of slots CPK and CPV instead of in one burst before the block (workload
    // 3 -0.3 to -0.9%, masked -0.6 to -1.5%, two boxes); head size 64 keeps the
    // burst (its block is half as long).
    constexpr int CPK = D == 128 ? 2 : -1, CPV = D == 128 ? 6 : -1;
    constexpr int VPS = (NOPS + NSLOT - 1) / NSLOT;
    // E(jj) ends before the first P V MFMA of jj; M starts after the last
    // score MFMA (two slots after it when that costs no extra slot).
    static_assert((NE - 1) / VPS < NQK + 3 * NDB, "probabilities late for P V");
    static_assert((NE / 4 * 3 - 1) / VPS < NQK + 2 * NDB, "probabilities late for P V");
    static_assert((NE + NR) / VPS >= NQK + (AHEAD ? 0 : 2), "row max before the scores drain");
    float pv[32];
    u32x4 pb[4];
    // Four independent max chains (unit u feeds chain u % 4).
    float mxc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    auto pin = [](float& x) { asm volatile("" : "+v"(x)); };
    // Masked score of S(t+1) element (kb, i): scale s + M (natural-log domain).
    auto masked = [&](int kb, int i) {
      const uint32_t w2 = mk[4 * kb + (i >> 2)][(i >> 1) & 1];
      const uint16_t bits = (i & 1) ? (uint16_t)(w2 >> 16) : (uint16_t)w2;
      float mv;
      if constexpr (std::is_same<TI, bf16_t>::value)
        mv = __uint_as_float((uint32_t)bits << 16);
      else
        mv = (float)__builtin_bit_cast(_Float16, bits);
      return fmaf(nxt[kb][i], p.scale, mv);
    };
    auto valu = [&](auto kc) {
      constexpr int k = decltype(kc)::value;
      if constexpr (k < NE) {
        constexpr int jj = k / 20, r = k % 20, kb = jj >> 1, base = 8 * (jj & 1);
        if constexpr (r < 16) {
          constexpr int ee = r >> 1, x = 8 * jj + ee;
          if constexpr ((r & 1) == 0) {
            pv[x] = fmaf(cur[kb][base + ee], sl2, nb);
          } else {
            pv[x] = fast_exp2(pv[x]);
            pin(pv[x]);
          }
        } else {
          constexpr int q4 = r - 16;
          pb[jj][q4] = T::pack2(pv[8 * jj + 2 * q4], pv[8 * jj + 2 * q4 + 1]);
        }
      } else if constexpr (k < NE + NR) {
        constexpr int r = k - NE;
        l_run[r & 3] = T::sum2(pb[r >> 2][r & 3], l_run[r & 3]);
        pin(l_run[r & 3]);
      } else {
        constexpr int u = (k - NE - NR) / MW, sub = (k - NE - NR) % MW;
        constexpr int kb = u & 1, i = 2 * (u >> 1);
        float& m = mxc[u & 3];
        if constexpr (AHEAD) {
          if constexpr (sub == 0 || sub == 2) {
            float x = masked(kb, i + sub / 2);
            pin(x);
            nxt[kb][i + sub / 2] = x;
          } else if constexpr (sub == 4) {
            m = fmaxf(fmaxf(m, nxt[kb][i]), nxt[kb][i + 1]);
            pin(m);
          }
        } else {
          m = fmaxf(fmaxf(m, nxt[kb][i]), nxt[kb][i + 1]);
          pin(m);
        }
      }
    };
    u32x4 kf[NQK];
    u32x2 va[NPV], vb[NPV];
    auto kread = [&](int i) {
      const int s = i >> 1, kb = i & 1;
      kf[i] = lds16(Ks + ((s & 1) ? koffO : koffE) + 256 * s + 4096 * C::NCB * kb);
    };
    auto vread = [&](int i) {
      const int jj = i / NDB, db = i % NDB;
      va[i] = lds_read_tr16(Vs + voffA + 2048 * C::NCB * jj + 512 * db);
      vb[i] = lds_read_tr16(Vs + voffB + 2048 * C::NCB * jj + 512 * db);
    };
    if constexpr (CPK < 0) copy_k();
    if constexpr (CPV < 0) copy_v();
#pragma unroll
    for (int i = 0; i < PD; ++i) kread(i);
    static_for<0, NSLOT>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (i == CPK) copy_k();
      if constexpr (i == CPV) copy_v();
      if constexpr (i < NQK) {
        if constexpr (i + PD < NQK) kread(i + PD);
        else vread(i + PD - NQK);
        constexpr int s = i >> 1, kb = i & 1;
        nxt[kb] = T::mma32(kf[i], qf[s], s == 0 ? f32x16{} : nxt[kb]);
      } else {
        constexpr int j = i - NQK;
        if constexpr (j + PD < NPV) vread(j + PD);
        constexpr int jj = j / NDB, db = j % NDB;
        oacc[db] = T::mma32(u32x4{va[j][0], va[j][1], vb[j][0], vb[j][1]}, pb[jj], oacc[db]);
      }
      if constexpr (AHEAD) {
        // The next tile's mask values, 8 bytes per read, each issued three
        // slots before the first M unit that uses it (fragment m first serves
        // unit 4 (m % 4) + m / 4), so few of them are live at a time.
        static_for<0, 8>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          constexpr int need = (NE + NR + MW * (4 * (m % 4) + m / 4)) / VPS;
          if constexpr ((need >= 3 ? need - 3 : 0) == i)
            mk[m] = *(const u32x2*)(mnext + 128 * m + ((m & 1) ? -mflip : mflip));
        });
      }
      static_for<0, VPS>([&](auto vc) {
        constexpr int k = i * VPS + decltype(vc)::value;
        if constexpr (k < NOPS) valu(std::integral_constant<int, k>{});
      });
    });
    __builtin_amdgcn_sched_barrier(0);
    mx_next = max_xor32(fmaxf(fmaxf(mxc[0], mxc[1]), fmaxf(mxc[2], mxc[3])));
  };

  // Tiles [t_begin, t_mask) are visible to every row of the workgroup and lie
  // inside the keys; the rest (the causal diagonal, the key tail) are masked.
  int t_mask = p.Skv / PF_BN;
  if (CAUSAL)
    t_mask = min(t_mask, q0 + off - (PF_BN - 1) >= 0 ? (q0 + off - (PF_BN - 1)) / PF_BN + 1 : 0);
  t_mask = max(t_begin, min(t_mask, t_end));

  // Software pipeline (the scores of tile t+1 are computed on the matrix cores
  // while the softmax of tile t runs on the vector ALUs):
  //   prologue: copy K(t0), V(t0), K(t0+1); wait; S(t0) = QK(t0)
  //   step t:   wait for K(t+1), V(t); copy K(t+2), V(t+1);
  //             S(t+1) = QK(t+1); softmax(S(t)); O += P V(t)
  // One barrier per step also guarantees that the stages being refilled
  // (K(t), V(t-1)) have been read by every wave.
  // The scores alternate between two register sets (the unmasked loop is
  // unrolled by two so that no copies are needed). mx_pend is the row max of
  // the scores held for the next step, before any mask.
  f32x16 sA[2], sB[2];
  float mx_pend = -INFINITY;
  if (t_begin < t_end) {
    // All first copies (K(t0), V(t0), K(t0+1)) go out together with the query
    // loads: the prologue waits for memory once, and the first step's wait
    // finds them done.
    if constexpr (AMASK) {
      issue_mask(t_begin);
      if (AM == 2 && t_begin + 1 < t_end) issue_mask(t_begin + 1);
    }
    issue_k(t_begin);
    issue_v(t_begin);
    if (t_begin + 1 < t_end) issue_k(t_begin + 1);
    wait_vmcnt<0>();
    lds_barrier();
    qk(sA, smem + k_stage(t_begin));
    if constexpr (AM == 2) {  // (with AM == 1 the step adds the mask)
      read_mask(t_begin);
      add_mask(sA);
    }
    mx_pend = tile_max(sA);
  }
  constexpr std::integral_constant<bool, false> kNow{};
  constexpr std::integral_constant<bool, true> kAhead{};
  // Additive mask: with one head per workgroup each wave's one-stage buffer
  // holds tile t's mask, read and added to S(t) at the start of step t (the
  // buffer is refilled with tile t + 1 once the reads have returned). With a
  // head pack the shared 2-stage ring holds tiles t + 1 and t + 2 during step
  // t: the body adds tile t + 1's mask to S(t+1) under the P V MFMAs, and
  // tile t + 2 is copied into the stage tile t used (every wave's reads of it
  // completed before this step's barrier).
  auto step = [&](auto mask_tag, int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    constexpr bool MASK = decltype(mask_tag)::value;
    wait_vmcnt<0>();
    lds_barrier();
    constexpr bool ahead = AM == 2;
    if constexpr (AMASK && !ahead) read_mask(t);
    auto copy_k = [&] {
      if (t + 2 < t_end) issue_k(t + 2);
    };
    auto copy_v = [&] {
      if (t + 1 < t_end) issue_v(t + 1);
    };
    if constexpr (AMASK) {
      if constexpr (ahead) {
        if (t + 2 < t_end) issue_mask(t + 2);
      } else {
        wave_lds_sync();
        if (t + 1 < t_end) issue_mask(t + 1);
        add_mask(cur);
      }
    }
    // After the last tile the block still computes scores from a stale K stage
    // (in bounds, never used): that keeps the block free of branches.
    // A tile wholly above this wave's causal diagonal is masked out entirely
    // (every probability 0); it runs through the same block.
    const float mx = MASK ? apply_mask(cur, t * PF_BN) : (AMASK && !ahead) ? tile_max(cur) : mx_pend;
    const float nb = rescale(mx);
    if constexpr (ahead)
      body(cur, nxt, smem + k_stage(t + 1), smem + v_stage(t), nb, mx_pend, kAhead,
           mread + m_stage(t + 1), copy_k, copy_v);
    else
      body(cur, nxt, smem + k_stage(t + 1), smem + v_stage(t), nb, mx_pend, kNow, nullptr, copy_k,
           copy_v);
    debug_step_barrier();
  };
  constexpr std::integral_constant<bool, false> kFull{};
  constexpr std::integral_constant<bool, true> kMasked{};
  int t = t_begin;
  for (; t + 1 < t_mask; t += 2) {
    step(kFull, t, sA, sB);
    step(kFull, t + 1, sB, sA);
  }
  if (t < t_mask) {
    step(kFull, t, sA, sB);
    ++t;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sA[kb] = sB[kb];
  }
  for (; t + 1 < t_end; t += 2) {
    step(kMasked, t, sA, sB);
    step(kMasked, t + 1, sB, sA);
  }
  if (t < t_end) step(kMasked, t, sA, sB);

  // Epilogue: both lane halves hold parts of the row sum.
  const float l_tot = sum_xor32((l_run[0] + l_run[1]) + (l_run[2] + l_run[3]));
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // (With a mask m_run is already scaled.)
  const float lse = l_tot > 0.f ? (AMASK ? m_run : m_run * p.scale) + __logf(l_tot) : -INFINITY;
  // The output rows, or with several splits this split's partial rows (in the
  // output's type; the combine weighs the partials by their lse). Query row i
  // of head hq is row (b * Sq + i) * Hq + hq of the output.
  constexpr int OB = out_size<TO>::bytes;
  char* obase = (char*)(S == 1 ? p.o : p.part_o) +
                (S == 1 ? 0 : (int64_t)split * p.B * p.Sq * p.Hq * D * OB);
  auto out_row = [&](int i) { return obase + (((int64_t)b * p.Sq + i) * p.Hq + hq) * D * OB; };
  // A 16-bit output goes through LDS: each lane holds 4 columns of one row per
  // store, so direct stores would touch the 32 rows of the wave (32 cache
  // lines) per instruction. Instead every wave writes its 32 rows into its own
  // slice of the (now idle) K/V stages, 16-byte chunk q of row r at chunk
  // q ^ (r % NCO), and stores them back a few whole rows per instruction.
  constexpr int RB = D * 2;     // bytes per row
  constexpr int NCO = RB / 16;  // 16-byte chunks per row
  constexpr bool LDS_EPI = OB == 2 && NW * 32 * RB <= C::LDS;
  if constexpr (LDS_EPI) {
    lds_barrier();  // every wave has finished reading the K/V stages
    char* ot = smem + w * 32 * RB;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        store4(TO{}, ot + c * RB + 16 * ((4 * db + i4) ^ (c % NCO)) + 8 * h,
               oacc[db][4 * i4] * inv, oacc[db][4 * i4 + 1] * inv,
               oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv);
    wave_lds_sync();
    constexpr int RPI = 64 / NCO;  // rows per store instruction
    const int rr = lane / NCO, ch = lane % NCO;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + rr;
      const u32x4 v = lds16(ot + r * RB + 16 * (ch ^ (r % NCO)));
      if (qw0 + r < p.Sq) *(u32x4*)(out_row(qw0 + r) + 16 * ch) = v;
    }
  } else if (q_ok) {
    char* orow = out_row(qi);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * h;
        store4(TO{}, orow + d * OB, oacc[db][4 * i4] * inv, oacc[db][4 * i4 + 1] * inv,
               oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv);
      }
  }
  if (q_ok && h == 0) {
    if (S == 1) {
      if (p.lse) p.lse[((int64_t)b * p.Hq + hq) * p.Sq + qi] = lse;
    } else {
      p.part_lse[(int64_t)split * p.B * p.Sq * p.Hq + ((int64_t)b * p.Sq + qi) * p.Hq + hq] = lse;
    }
  }
}

template <int D, int NW, typename TI, typename TO>
inline hipError_t launch4(const PrefillParams& p, bool causal, hipStream_t stream) {
  const int n = p.B * (p.Hq / p.pack) * p.n_qtiles * p.n_splits;
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, dim3(n), dim3(64 * NW), 0, stream, p); };
  if (p.mask && p.pack > 1)
    causal ? go(prefill_kernel<D, NW, TI, TO, true, 2>)
           : go(prefill_kernel<D, NW, TI, TO, false, 2>);
  else if (p.mask)
    causal ? go(prefill_kernel<D, NW, TI, TO, true, 1>)
           : go(prefill_kernel<D, NW, TI, TO, false, 1>);
  else
    causal ? go(prefill_kernel<D, NW, TI, TO, true, 0>)
           : go(prefill_kernel<D, NW, TI, TO, false, 0>);
  return hipGetLastError();
}

template <int D, typename TI, typename TO>
inline hipError_t launch3(const PrefillParams& p, bool causal, hipStream_t stream) {
  if constexpr (D == 128) {
    if (p.waves == 8) return launch4<D, 8, TI, TO>(p, causal, stream);
  }
  return launch4<D, 4, TI, TO>(p, causal, stream);
}

template <int D, typename TI>
inline hipError_t launch2(const PrefillParams& p, OutType ot, bool causal, hipStream_t stream) {
  switch (ot) {
    case OutType::bf16: return launch3<D, TI, out_bf16>(p, causal, stream);
    case OutType::f16: return launch3<D, TI, out_f16>(p, causal, stream);
    default: return launch3<D, TI, out_f32>(p, causal, stream);
  }
}

}  // namespace fa
