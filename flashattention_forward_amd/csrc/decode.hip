// Paged-KV decode attention for gfx950: one query token per sequence against
// every cached token of the sequence, read through a page table.
//
// Workloads: "perf: FlashAttention-3 style MLA PageAttention" (FlashInfer) --
// batch x seq_len x 64 heads at page_size = 1 ("Results"), and MLA, where one
// compressed-KV row per token is both the key and the value (change list item
// 4: one KV stream instead of two, so one load must serve both products). The
// grouped-query variant packs the query heads that share a K/V head, the GQA
// idea of "CUDA: fix FA occupancy, optimize tile kernel" (opening paragraph), so
// each K/V row is read once per group.
//
// Both kernels use v_mfma_f32_16x16x32 with the scores transposed
// (S^T = K Q^T: A = 16 keys, B = 16 query heads of the group held in
// registers). A lane then holds one head and 4 keys of each 16-key block; the
// head's max and sum need two cross-lane steps. The probabilities are rounded to
// 16 bits in registers and become the B operand of O^T += V^T P^T, whose A
// operand is read from a row-major V tile in LDS with the transpose read
// (ds_read_b64_tr_b16); the contraction index is relabelled so that each lane's
// 8 keys match its probability registers.
//
// Sequences too short to fill the chip are split over several key ranges
// (split-KV); each split writes a normalised partial O and its log-sum-exp for
// the combine kernel. Tokens past seq_len, including page slots that hold
// garbage or NaN, are never loaded: their K and V registers are zero and their
// scores -infinity.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <int PS>
__device__ __forceinline__ void page_of(int key, int ps, int& page_idx, int& slot) {
  if (PS > 0) {
    page_idx = key / PS;
    slot = key % PS;
  } else {
    page_idx = key / ps;
    slot = key - page_idx * ps;
  }
}

// ---------------------------------------------------------------------------
// Grouped-query decode over the split K/V pool [P, 2, Hkv, page, 128].
// One wave is one work unit (sequence b, K/V head g, block of up to 16 query
// heads of the group, key split); a workgroup holds 4 independent units.
// ---------------------------------------------------------------------------
constexpr int DS_D = 128;
constexpr int DS_VS = DS_D + 16;  // V row stride in LDS (elements)

template <typename TI, int PS>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeSplitParams p) {
  using T = in_traits<TI>;
  constexpr int D = DS_D;
  __shared__ __attribute__((aligned(16))) char smem[4][DEC_TILE * DS_VS * 2];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int unit = blockIdx.x * 4 + w;
  if (unit >= p.n_units) return;  // whole wave leaves; the kernel has no barriers
  char* vlds = smem[w];

  const int S = p.n_splits;
  const int split = unit % S;
  unit /= S;
  const int hb = unit % p.n_hblk;
  unit /= p.n_hblk;
  const int g = unit % p.Hkv;
  const int b = unit / p.Hkv;
  const int G = p.Hq / p.Hkv;
  const int c16 = lane & 15, gq = lane >> 4;
  const int hig = hb * 16 + c16;  // head index inside the group
  const bool hvalid = hig < G;
  const int hq = g * G + (hvalid ? hig : 0);

  const int seq_len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int t0 = split * p.chunk;
  const int t1 = min(t0 + p.chunk, seq_len);

  u32x4 qf[D / 32];
  {
    const char* qrow = (const char*)p.q + ((int64_t)b * p.Hq + hq) * D * 2;
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
      qf[s] = hvalid ? ldg16(qrow + (32 * s + 8 * gq) * 2) : u32x4{0, 0, 0, 0};
  }
  const int32_t* ptab = p.page_table + (int64_t)b * p.max_pages;
  const int64_t page_stride = (int64_t)2 * p.Hkv * p.page_size * D * 2;  // bytes per page
  const int64_t kv_stride = (int64_t)p.Hkv * p.page_size * D * 2;       // K -> V bytes
  const char* pool_g = (const char*)p.pool + (int64_t)g * p.page_size * D * 2;
  // Address of token `key`'s K row, or null when its page id is out of range.
  auto row_ptr = [&](int key) -> const char* {
    int pi, slot;
    page_of<PS>(key, p.page_size, pi, slot);
    const int page = ptab[pi];
    if ((unsigned)page >= (unsigned)p.num_pages) return nullptr;
    return pool_g + (int64_t)page * page_stride + (int64_t)slot * D * 2;
  };

  u32x4 kcur[2][D / 32], knext[2][D / 32], vnext[8];
  auto load_k = [&](u32x4 (&kr)[2][D / 32], int tt) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int key = tt + 16 * kb + c16;
      const char* rp = key < t1 ? row_ptr(key) : nullptr;
#pragma unroll
      for (int s = 0; s < D / 32; ++s)
        kr[kb][s] = rp ? ldg16(rp + (32 * s + 8 * gq) * 2) : u32x4{0, 0, 0, 0};
    }
  };
  auto load_v = [&](int tt) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int key = tt + gq + 4 * r;
      const char* rp = key < t1 ? row_ptr(key) : nullptr;
      vnext[r] = rp ? ldg16(rp + kv_stride + c16 * 16) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_v = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) *(u32x4*)(vlds + ((gq + 4 * r) * DS_VS + c16 * 8) * 2) = vnext[r];
  };

  f32x4 oacc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) oacc[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  if (t0 < t1) {
    load_k(kcur, t0);
    load_v(t0);
    store_v();
    wave_lds_sync();
  }
  for (int tt = t0; tt < t1; tt += DEC_TILE) {
    const bool more = tt + DEC_TILE < t1;
    if (more) {
      load_k(knext, tt + DEC_TILE);
      load_v(tt + DEC_TILE);
    }
    f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < D / 32; ++s) sacc[kb] = T::mma16(kcur[kb][s], qf[s], sacc[kb]);
    if (tt + DEC_TILE > t1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (tt + 16 * kb + 4 * gq + i >= t1) sacc[kb][i] = -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                     fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
    mx = fmaxf(mx, xor16(mx));
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2((m_run - m_use) * sl2);
    const float nb = -m_use * sl2;
    float pv[2][4];
    float rs = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[kb][i] = fast_exp2(fmaf(sacc[kb][i], sl2, nb));
        rs += pv[kb][i];
      }
    const u32x4 pb{T::pack2(pv[0][0], pv[0][1]), T::pack2(pv[0][2], pv[0][3]),
                   T::pack2(pv[1][0], pv[1][1]), T::pack2(pv[1][2], pv[1][3])};
    l_run = l_run * alpha + rs;
    m_run = m_new;
    const int j = c16;
    const char* va = vlds + ((4 * gq + (j >> 2)) * DS_VS + 4 * (j & 3)) * 2;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const u32x2 r0 = lds_read_tr16(va + 16 * db * 2);
      const u32x2 r1 = lds_read_tr16(va + (16 * DS_VS + 16 * db) * 2);
      oacc[db] = T::mma16(u32x4{r0[0], r0[1], r1[0], r1[1]}, pb, oacc[db] * alpha);
    }
    if (more) {
      wave_lds_sync();
      store_v();
      wave_lds_sync();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < D / 32; ++s) kcur[kb][s] = knext[kb][s];
    }
  }

  float l_tot = l_run + xor16(l_run);
  l_tot += xor32(l_tot);
  if (!hvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_run * p.scale + __logf(l_tot) : -INFINITY;
  const int64_t row = (int64_t)b * p.Hq + hq;
  if (S == 1) {
    char* orow = (char*)p.o + row * D * 2;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int d = 16 * db + 4 * gq;
      const u32x2 v{T::pack2(oacc[db][0] * inv, oacc[db][1] * inv),
                    T::pack2(oacc[db][2] * inv, oacc[db][3] * inv)};
      *(u32x2*)(orow + d * 2) = v;
    }
    if (p.lse && gq == 0) p.lse[row] = lse;
  } else {
    const int64_t rows = (int64_t)p.B * p.Hq;
    float* orow = p.part_o + ((int64_t)split * rows + row) * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *(f32x4*)(orow + 16 * db + 4 * gq) = oacc[db] * inv;
    if (gq == 0) p.part_lse[split * rows + row] = lse;
  }
}

// ---------------------------------------------------------------------------
// MLA decode over the shared pool [P, page, 576]: the 576-column row of a token
// is the key ([ckv | kpe]) and its first 512 columns are the value. A workgroup
// of 4 waves handles one sequence, 64 query heads (16 per wave) and one key
// split; each row is loaded from HBM once into LDS and read by both products.
// ---------------------------------------------------------------------------
constexpr int MLA_DQ = 576;
constexpr int MLA_DV = 512;
constexpr int MLA_RS = MLA_DQ + 16;  // LDS row stride (elements)
constexpr int MLA_TILE_BYTES = DEC_TILE * MLA_RS * 2;
constexpr int MLA_CPR = MLA_DQ / 8;                    // 16-byte chunks per row (72)
constexpr int MLA_NLD = DEC_TILE * MLA_CPR / 256;      // chunks per thread per tile (9)

template <typename TI, int PS>
__global__ __launch_bounds__(256, 1) void decode_mla_kernel(DecodeMlaParams p) {
  using T = in_traits<TI>;
  __shared__ __attribute__((aligned(16))) char smem[2 * MLA_TILE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c16 = lane & 15, gq = lane >> 4;

  int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int S = p.n_splits;
  const int split = blk % S;
  blk /= S;
  const int hb = blk % p.n_hblk;
  const int b = blk / p.n_hblk;
  const int head = hb * MLA_HEADS_PER_WG + 16 * w + c16;
  const bool hvalid = head < p.Hq;
  const bool wave_active = hb * MLA_HEADS_PER_WG + 16 * w < p.Hq;

  const int seq_len = min(max(p.seq_lens[b], 0), p.max_seq_len);
  const int t0 = split * p.chunk;
  const int t1 = min(t0 + p.chunk, seq_len);

  u32x4 qf[MLA_DQ / 32];
  {
    const char* qrow = (const char*)p.q + ((int64_t)b * p.Hq + (hvalid ? head : 0)) * MLA_DQ * 2;
#pragma unroll
    for (int s = 0; s < MLA_DQ / 32; ++s)
      qf[s] = hvalid ? ldg16(qrow + (32 * s + 8 * gq) * 2) : u32x4{0, 0, 0, 0};
  }
  const int32_t* ptab = p.page_table + (int64_t)b * p.max_pages;
  const char* pool = (const char*)p.pool;

  u32x4 regs[MLA_NLD];
  auto load_tile = [&](int tt) {
#pragma unroll
    for (int r = 0; r < MLA_NLD; ++r) {
      const int id = tid + 256 * r;
      const int row = id / MLA_CPR, col = id % MLA_CPR;
      const int key = tt + row;
      regs[r] = u32x4{0, 0, 0, 0};
      if (key < t1) {
        int pi, slot;
        page_of<PS>(key, p.page_size, pi, slot);
        const int page = ptab[pi];
        if ((unsigned)page < (unsigned)p.num_pages)
          regs[r] = ldg16(pool + ((int64_t)page * p.page_size + slot) * (MLA_DQ * 2) + col * 16);
      }
    }
  };
  auto store_tile = [&](char* st) {
#pragma unroll
    for (int r = 0; r < MLA_NLD; ++r) {
      const int id = tid + 256 * r;
      const int row = id / MLA_CPR, col = id % MLA_CPR;
      *(u32x4*)(st + (row * MLA_RS + col * 8) * 2) = regs[r];
    }
  };

  f32x4 oacc[MLA_DV / 16];
#pragma unroll
  for (int db = 0; db < MLA_DV / 16; ++db) oacc[db] = f32x4{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  if (t0 < t1) {
    load_tile(t0);
    store_tile(smem);
  }
  __syncthreads();
  for (int tt = t0; tt < t1; tt += DEC_TILE) {
    const int st = ((tt - t0) / DEC_TILE) & 1;
    const bool more = tt + DEC_TILE < t1;
    if (more) load_tile(tt + DEC_TILE);
    if (wave_active) {
      const char* tile = smem + st * MLA_TILE_BYTES;
      f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
      for (int s = 0; s < MLA_DQ / 32; ++s)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 a = *(const u32x4*)(tile + ((16 * kb + c16) * MLA_RS + 32 * s + 8 * gq) * 2);
          sacc[kb] = T::mma16(a, qf[s], sacc[kb]);
        }
      if (tt + DEC_TILE > t1) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (tt + 16 * kb + 4 * gq + i >= t1) sacc[kb][i] = -INFINITY;
      }
      float mx = fmaxf(fmaxf(fmaxf(sacc[0][0], sacc[0][1]), fmaxf(sacc[0][2], sacc[0][3])),
                       fmaxf(fmaxf(sacc[1][0], sacc[1][1]), fmaxf(sacc[1][2], sacc[1][3])));
      mx = fmaxf(mx, xor16(mx));
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * sl2);
      const float nb = -m_use * sl2;
      float pv[2][4];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pv[kb][i] = fast_exp2(fmaf(sacc[kb][i], sl2, nb));
          rs += pv[kb][i];
        }
      const u32x4 pb{T::pack2(pv[0][0], pv[0][1]), T::pack2(pv[0][2], pv[0][3]),
                     T::pack2(pv[1][0], pv[1][1]), T::pack2(pv[1][2], pv[1][3])};
      l_run = l_run * alpha + rs;
      m_run = m_new;
      const int j = c16;
      const char* va = tile + ((4 * gq + (j >> 2)) * MLA_RS + 4 * (j & 3)) * 2;
#pragma unroll
      for (int db = 0; db < MLA_DV / 16; ++db) {
        const u32x2 r0 = lds_read_tr16(va + 16 * db * 2);
        const u32x2 r1 = lds_read_tr16(va + (16 * MLA_RS + 16 * db) * 2);
        oacc[db] = T::mma16(u32x4{r0[0], r0[1], r1[0], r1[1]}, pb, oacc[db] * alpha);
      }
    }
    if (more) store_tile(smem + (st ^ 1) * MLA_TILE_BYTES);
    __syncthreads();
  }

  float l_tot = l_run + xor16(l_run);
  l_tot += xor32(l_tot);
  if (!hvalid) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_run * p.scale + __logf(l_tot) : -INFINITY;
  const int64_t row = (int64_t)b * p.Hq + head;
  if (S == 1) {
    char* orow = (char*)p.o + row * MLA_DV * 2;
#pragma unroll
    for (int db = 0; db < MLA_DV / 16; ++db) {
      const u32x2 v{T::pack2(oacc[db][0] * inv, oacc[db][1] * inv),
                    T::pack2(oacc[db][2] * inv, oacc[db][3] * inv)};
      *(u32x2*)(orow + (16 * db + 4 * gq) * 2) = v;
    }
    if (p.lse && gq == 0) p.lse[row] = lse;
  } else {
    const int64_t rows = (int64_t)p.B * p.Hq;
    float* orow = p.part_o + ((int64_t)split * rows + row) * MLA_DV;
#pragma unroll
    for (int db = 0; db < MLA_DV / 16; ++db)
      *(f32x4*)(orow + 16 * db + 4 * gq) = oacc[db] * inv;
    if (gq == 0) p.part_lse[split * rows + row] = lse;
  }
}

template <typename TI>
static hipError_t split_dispatch(const DecodeSplitParams& p, hipStream_t stream) {
  const int blocks = (p.n_units + 3) / 4;
  if (p.page_size == 16)
    hipLaunchKernelGGL((decode_split_kernel<TI, 16>), dim3(blocks), dim3(256), 0, stream, p);
  else if (p.page_size == 1)
    hipLaunchKernelGGL((decode_split_kernel<TI, 1>), dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_split_kernel<TI, 0>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename TI>
static hipError_t mla_dispatch(const DecodeMlaParams& p, hipStream_t stream) {
  const int blocks = p.B * p.n_hblk * p.n_splits;
  if (p.page_size == 1)
    hipLaunchKernelGGL((decode_mla_kernel<TI, 1>), dim3(blocks), dim3(256), 0, stream, p);
  else if (p.page_size == 16)
    hipLaunchKernelGGL((decode_mla_kernel<TI, 16>), dim3(blocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_mla_kernel<TI, 0>), dim3(blocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeSplitParams& p, InType it, hipStream_t stream) {
  return it == InType::bf16 ? split_dispatch<bf16_t>(p, stream) : split_dispatch<f16_t>(p, stream);
}

hipError_t launch_decode_mla(const DecodeMlaParams& p, InType it, hipStream_t stream) {
  return it == InType::bf16 ? mla_dispatch<bf16_t>(p, stream) : mla_dispatch<f16_t>(p, stream);
}

}  // namespace fa
