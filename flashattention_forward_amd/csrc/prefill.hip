// Fused attention prefill for gfx950: O = softmax(scale * Q K^T + mask) V with an
// online softmax, one pass over the keys.
//
// The tile-FA idea of "CUDA: fix FA occupancy, optimize tile kernel" (llama.cpp,
// opening paragraph) -- stage K/V tiles on chip with 16-byte copies, keep the
// score tile in registers and compress it to 16 bits before the second product,
// size tiles to the chip's shared memory -- rebuilt for CDNA4 matrix cores:
//
//  * a workgroup is 4 waves; each wave owns 32 query rows of one head, so a
//    workgroup covers 128 rows and shares every K/V tile of 64 keys in LDS;
//  * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16 (A = K
//    rows from LDS, B = the wave's Q rows held in registers for the whole pass).
//    Each lane then owns one query column and 16 keys of each 32-key block, so
//    the row max is in-lane plus one exchange with lane l ^ 32;
//  * the probabilities are rounded to 16 bits in registers and fed straight back
//    as the B operand of O^T += V^T P^T. The contraction index of that product
//    is relabelled to match the accumulator layout, and V is written to LDS
//    transposed in that relabelled key order, so every MFMA operand read is one
//    conflict-free 16-byte LDS load;
//  * K/V tiles are double-buffered: global loads of tile t+1 are issued before
//    the math of tile t and written to the other LDS buffer after it, one
//    workgroup barrier per tile;
//  * causal (bottom-right aligned) blocks stop at their last visible tile, waves
//    skip tiles that none of their rows can see, and only tiles crossing the
//    diagonal or the end of the keys are masked;
//  * the exponent uses exp2 with scale * log2(e) folded into one FMA;
//  * a workgroup may process one of several key splits; it then writes its
//    normalised partial O and log-sum-exp for a separate combine kernel.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

constexpr int PF_KPAD = 8;  // bf16 elements of padding per K row in LDS
constexpr int PF_VPAD = 8;  // per transposed-V row

template <int D> struct PfLds {
  static constexpr int KS = D + PF_KPAD;      // K row stride (elements)
  static constexpr int VS = PF_BN + PF_VPAD;  // V^T row stride (elements)
  static constexpr int K_BYTES = PF_BN * KS * 2;
  static constexpr int V_BYTES = D * VS * 2;
  static constexpr int STAGE = K_BYTES + V_BYTES;
  static constexpr int NK = PF_BN * D / 8 / 256;  // 16-byte K chunks per thread
  static constexpr int NV_UNITS = 16 * (D / 8);   // (4 keys x 8 dims) V units per tile
};

// Position of key `kg * 4` (kg = 4-key group 0..15 in a 64-key tile) in the
// relabelled order of the P V contraction: within each 16 keys, swap bits 2, 3.
__device__ __forceinline__ int vt_pos(int kg) {
  return 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1);
}

template <int D, typename TI>
struct TileRegs {
  u32x4 k[PfLds<D>::NK];
  u32x4 v[4];
};

template <int D, typename TI>
__device__ __forceinline__ void load_tile(TileRegs<D, TI>& r, const char* kbase,
                                          const char* vbase, int k0, int Skv, int row_bytes,
                                          int tid) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < PfLds<D>::NK; ++i) {
    const int id = tid + 256 * i;
    const int row = id / CPR, col = id % CPR;
    const int key = k0 + row;
    r.k[i] = key < Skv ? ldg16(kbase + (int64_t)key * row_bytes + col * 16) : u32x4{0, 0, 0, 0};
  }
  if (tid < PfLds<D>::NV_UNITS) {
    const int kg = tid / CPR, dc = tid % CPR;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int key = k0 + 4 * kg + j;
      r.v[j] = key < Skv ? ldg16(vbase + (int64_t)key * row_bytes + dc * 16) : u32x4{0, 0, 0, 0};
    }
  }
}

template <int D, typename TI>
__device__ __forceinline__ void store_tile(const TileRegs<D, TI>& r, char* stage, int tid) {
  using L = PfLds<D>;
  constexpr int CPR = D / 8;
#pragma unroll
  for (int i = 0; i < L::NK; ++i) {
    const int id = tid + 256 * i;
    const int row = id / CPR, col = id % CPR;
    *(u32x4*)(stage + (row * L::KS + col * 8) * 2) = r.k[i];
  }
  if (tid < L::NV_UNITS) {
    const int kg = tid / CPR, dc = tid % CPR;
    char* vt = stage + L::K_BYTES + vt_pos(kg) * 2;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int d0 = dc * 8 + 2 * e;
      *(u32x2*)(vt + d0 * L::VS * 2) =
          u32x2{pack_lo(r.v[0][e], r.v[1][e]), pack_lo(r.v[2][e], r.v[3][e])};
      *(u32x2*)(vt + (d0 + 1) * L::VS * 2) =
          u32x2{pack_hi(r.v[0][e], r.v[1][e]), pack_hi(r.v[2][e], r.v[3][e])};
    }
  }
}

template <int D, typename TI, typename TO, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  using L = PfLds<D>;
  using T = in_traits<TI>;
  __shared__ __attribute__((aligned(16))) char smem[2 * L::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int c = lane & 31, h = lane >> 5;

  // Logical block: (b, kv head g, query tile, head in group, split), with the
  // blocks that share one K/V head kept on one XCD.
  int blk = xcd_remap(blockIdx.x, gridDim.x);
  const int S = p.n_splits;
  const int split = blk % S;
  blk /= S;
  const int G = p.Hq / p.Hkv;
  const int hh = blk % G;
  blk /= G;
  int qt = blk % p.n_qtiles;
  blk /= p.n_qtiles;
  const int g = blk % p.Hkv;
  const int b = blk / p.Hkv;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // longest rows first
  const int hq = g * G + hh;
  const int off = p.Skv - p.Sq;  // bottom-right alignment
  const int q0 = qt * PF_BM;

  int kv_end = p.Skv;
  if (CAUSAL) kv_end = min(kv_end, min(q0 + PF_BM, p.Sq) + off);
  const int n_tiles = kv_end > 0 ? (kv_end + PF_BN - 1) / PF_BN : 0;
  const int tps = (n_tiles + S - 1) / S;
  const int t_begin = min(split * tps, n_tiles);
  const int t_end = min(t_begin + tps, n_tiles);

  const int row_bytes = p.Hkv * D * 2;
  const char* kbase = (const char*)p.k + ((int64_t)b * p.Skv * p.Hkv + g) * D * 2;
  const char* vbase = (const char*)p.v + ((int64_t)b * p.Skv * p.Hkv + g) * D * 2;

  // This lane's query row and its Q fragment (B operand, 16 dims per MFMA step).
  const int qw0 = q0 + 32 * w;  // first row of this wave
  const int qi = qw0 + c;
  const bool q_ok = qi < p.Sq;
  u32x4 qf[D / 16];
  {
    const char* qrow = (const char*)p.q + (((int64_t)b * p.Sq + qi) * p.Hq + hq) * D * 2;
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      qf[s] = q_ok ? ldg16(qrow + (16 * s + 8 * h) * 2) : u32x4{0, 0, 0, 0};
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;
  const int q_last_wave = min(qw0 + 31, p.Sq - 1);

  TileRegs<D, TI> regs;
  if (t_begin < t_end) {
    load_tile<D, TI>(regs, kbase, vbase, t_begin * PF_BN, p.Skv, row_bytes, tid);
    store_tile<D, TI>(regs, smem, tid);
  }
  __syncthreads();

  for (int t = t_begin; t < t_end; ++t) {
    const int st = (t - t_begin) & 1;
    const bool more = t + 1 < t_end;
    if (more) load_tile<D, TI>(regs, kbase, vbase, (t + 1) * PF_BN, p.Skv, row_bytes, tid);

    const int k0 = t * PF_BN;
    const bool active = !CAUSAL || k0 <= q_last_wave + off;
    if (active) {
      const char* Ks = smem + st * L::STAGE;
      const char* Vt = Ks + L::K_BYTES;
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 a = *(const u32x4*)(Ks + ((32 * kb + c) * L::KS + 16 * s + 8 * h) * 2);
          sacc[kb] = T::mma32(a, qf[s], sacc[kb]);
        }
      }
      const bool need_mask = (k0 + PF_BN > p.Skv) || (CAUSAL && k0 + PF_BN - 1 > qw0 + off);
      if (need_mask) {
        const int lim = CAUSAL ? min(p.Skv - 1, qi + off) : p.Skv - 1;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
            if (key > lim) sacc[kb][i] = -INFINITY;
          }
      }
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[kb][i]);
      mx = fmaxf(mx, xor32(mx));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2((m_run - m_use) * sl2);
      const float nb = -m_use * sl2;
      float rs = 0.f;
      u32x4 pb[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int kb = jj >> 1, base = 8 * (jj & 1);
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = fast_exp2(fmaf(sacc[kb][base + e], sl2, nb));
          rs += pv[e];
        }
        pb[jj] = u32x4{T::pack2(pv[0], pv[1]), T::pack2(pv[2], pv[3]), T::pack2(pv[4], pv[5]),
                       T::pack2(pv[6], pv[7])};
      }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const u32x4 a = *(const u32x4*)(Vt + ((32 * db + c) * L::VS + 16 * jj + 8 * h) * 2);
          oacc[db] = T::mma32(a, pb[jj], oacc[db]);
        }
      }
    }
    if (more) store_tile<D, TI>(regs, smem + (st ^ 1) * L::STAGE, tid);
    __syncthreads();
  }

  // Epilogue: both lane halves hold parts of the row sum.
  const float l_tot = l_run + xor32(l_run);
  if (!q_ok) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_run * p.scale + __logf(l_tot) : -INFINITY;
  const int64_t row = ((int64_t)b * p.Sq + qi) * p.Hq + hq;
  if (S == 1) {
    char* orow = (char*)p.o + row * D * out_size<TO>::bytes;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * h;
        store4(TO{}, orow + d * out_size<TO>::bytes, oacc[db][4 * i4] * inv,
               oacc[db][4 * i4 + 1] * inv, oacc[db][4 * i4 + 2] * inv,
               oacc[db][4 * i4 + 3] * inv);
      }
    if (p.lse && h == 0) p.lse[((int64_t)b * p.Hq + hq) * p.Sq + qi] = lse;
  } else {
    const int64_t rows = (int64_t)p.B * p.Sq * p.Hq;
    float* orow = p.part_o + ((int64_t)split * rows + row) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * db + 8 * i4 + 4 * h;
        store4(out_f32{}, orow + d, oacc[db][4 * i4] * inv, oacc[db][4 * i4 + 1] * inv,
               oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv);
      }
    if (h == 0) p.part_lse[split * rows + row] = lse;
  }
}

template <int D, typename TI, typename TO>
static hipError_t launch3(const PrefillParams& p, bool causal, hipStream_t stream) {
  const int n = p.B * p.Hq * p.n_qtiles * p.n_splits;
  if (causal)
    hipLaunchKernelGGL((prefill_kernel<D, TI, TO, true>), dim3(n), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<D, TI, TO, false>), dim3(n), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int D, typename TI>
static hipError_t launch2(const PrefillParams& p, OutType ot, bool causal, hipStream_t stream) {
  switch (ot) {
    case OutType::bf16: return launch3<D, TI, out_bf16>(p, causal, stream);
    case OutType::f16: return launch3<D, TI, out_f16>(p, causal, stream);
    default: return launch3<D, TI, out_f32>(p, causal, stream);
  }
}

hipError_t launch_prefill(const PrefillParams& p, int D, InType it, OutType ot, bool causal,
                          hipStream_t stream) {
  if (D == 64)
    return it == InType::bf16 ? launch2<64, bf16_t>(p, ot, causal, stream)
                              : launch2<64, f16_t>(p, ot, causal, stream);
  return it == InType::bf16 ? launch2<128, bf16_t>(p, ot, causal, stream)
                            : launch2<128, f16_t>(p, ot, causal, stream);
}

}  // namespace fa
