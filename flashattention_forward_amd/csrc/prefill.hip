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
//    is relabelled to match the accumulator layout; the V^T operand comes from
//    the row-major V tile through the LDS transpose read (ds_read_b64_tr_b16);
//  * K and V tiles go from global memory straight into LDS (global_load_lds,
//    no register staging) into a ring of stages: the copy of tile t+1 is in
//    flight while tile t is computed, and barriers wait on LDS traffic only;
//  * tiles are stored in 8 x 8 blocks of 16-byte chunks (blk_slot): a copy
//    instruction moves 8 key rows x 128 contiguous bytes, and the K reads (16
//    rows of one chunk) and the transposed V reads (4 rows x 4 chunks) each
//    touch 64 distinct banks;
//  * causal (bottom-right aligned) blocks stop at their last visible tile, waves
//    skip tiles that none of their rows can see, and only tiles crossing the
//    diagonal or the end of the keys are masked;
//  * the exponent uses exp2 with scale * log2(e) folded into one FMA, and the
//    running max moves only when it grows by more than 2^8, so the O
//    accumulators are rarely rescaled;
//  * a workgroup may process one of several key splits; it then writes its
//    normalised partial O and log-sum-exp for a separate combine kernel.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <int D> struct PfCfg {
  static constexpr int NCH = D / 8;                 // 16-byte chunks per key row
  static constexpr int NCB = NCH / 8;               // 8-chunk blocks per key row
  static constexpr int TILE = PF_BN * D * 2;        // bytes of one K (or V) tile
  static constexpr int STAGE = 2 * TILE;            // K tile then V tile
  static constexpr int NST = D == 64 ? 4 : 2;       // stages in the LDS ring
  static constexpr int CPW = NCH / 4;               // chunk columns per wave (K and V each)
  static constexpr int IPW = 2 * CPW;               // copy instructions per wave and tile
};

template <int D, typename TI, typename TO, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void prefill_kernel(PrefillParams p) {
  using C = PfCfg<D>;
  using T = in_traits<TI>;
  __shared__ __attribute__((aligned(16))) char smem[C::NST * C::STAGE];

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
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 v = q_ok ? ldg16(qrow + (16 * s + 8 * h) * 2) : u32x4{0, 0, 0, 0};
      qf[s] = p.q_neg ? neg16x8(v) : v;
    }
  }

  // Copies of tile t into stage (t - t_begin) % NST: the K and the V tile are
  // each 8 * NCB blocks; wave w copies blocks n = 2 NCB w + i (i < 2 NCB) of
  // both, i.e. key rows 16w .. 16w + 15. Lane l copies chunk
  // 8 CB + ((l >> 3) ^ (RB & 1)) of key row 8 RB + ((l & 7) ^ 4 * ((l >> 4) & 1))
  // (the inverse of blk_slot). Keys past the end are clamped to the last key:
  // their scores are masked and their probabilities are 0.
  const uint32_t smem_lds = lds_addr(smem);
  const int dma_rho = (lane & 7) ^ (4 * ((lane >> 4) & 1));
  auto issue = [&](int t) {
    const uint32_t st = smem_lds + ((t - t_begin) % C::NST) * C::STAGE;
    const int k0 = t * PF_BN;
#pragma unroll
    for (int i = 0; i < 2 * C::NCB; ++i) {
      const int n = 2 * C::NCB * w + i;
      const int rb_odd = (i / C::NCB) & 1, cb = i % C::NCB;
      const int key = min(k0 + 16 * w + 8 * rb_odd + dma_rho, p.Skv - 1);
      const int chunk = 8 * cb + ((lane >> 3) ^ rb_odd);
      const int64_t off = (int64_t)key * row_bytes + chunk * 16;
      dma16(kbase + off, st + n * 1024);
      dma16(vbase + off, st + C::TILE + n * 1024);
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;
  const int q_last_wave = min(qw0 + 31, p.Sq - 1);

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

  for (int t = t_begin; t < min(t_end, t_begin + C::NST - 1); ++t) issue(t);

  for (int t = t_begin; t < t_end; ++t) {
    // Wait for this wave's copies of tile t (later tiles may stay in flight).
    if (C::NST >= 4 && t + 2 < t_end)
      wait_vmcnt<2 * C::IPW>();
    else if (C::NST >= 3 && t + 1 < t_end)
      wait_vmcnt<C::IPW>();
    else
      wait_vmcnt<0>();
    lds_barrier();
    if (t + C::NST - 1 < t_end) issue(t + C::NST - 1);

    const int k0 = t * PF_BN;
    const bool active = !CAUSAL || k0 <= q_last_wave + off;
    if (active) {
      const char* Ks = smem + ((t - t_begin) % C::NST) * C::STAGE;
      const char* Vs = Ks + C::TILE;
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 a = lds16(Ks + ((s & 1) ? koffO : koffE) + 256 * s + 4096 * C::NCB * kb);
          sacc[kb] = T::mma32(a, qf[s], sacc[kb]);
        }
      }
      const bool need_mask = (k0 + PF_BN > p.Skv) || (CAUSAL && k0 + PF_BN - 1 > qw0 + off);
      // Masked keys: -inf for the max, probability forced to 0 below.
      const int lim = !need_mask ? k0 + PF_BN : (CAUSAL ? min(p.Skv - 1, qi + off) : p.Skv - 1);
      if (need_mask) {
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
      // Lazy rescale: move the running max only when it grows by > 2^8.
      const bool grow =
          mx > m_run && (m_run == -INFINITY || (mx - m_run) * sl2 > RESCALE_LOG2);
      if (__ballot(grow)) {
        const float m_new = grow ? mx : m_run;
        const float alpha = m_run == -INFINITY ? 0.f : fast_exp2((m_run - m_new) * sl2);
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        m_run = m_new;
      }
      const float nb = m_run == -INFINITY ? 0.f : -m_run * sl2;
      u32x4 pb[4];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int kb = jj >> 1, base = 8 * (jj & 1);
        float pv[8];
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) {
          pv[ee] = fast_exp2(fmaf(sacc[kb][base + ee], sl2, nb));
          if (need_mask) {
            const int i = base + ee;
            const int key = k0 + 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
            if (key > lim) pv[ee] = 0.f;
          }
          l_run += pv[ee];
        }
        pb[jj] = u32x4{T::pack2(pv[0], pv[1]), T::pack2(pv[2], pv[3]), T::pack2(pv[4], pv[5]),
                       T::pack2(pv[6], pv[7])};
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const u32x2 ra = lds_read_tr16(Vs + voffA + 2048 * C::NCB * jj + 512 * db);
          const u32x2 rb = lds_read_tr16(Vs + voffB + 2048 * C::NCB * jj + 512 * db);
          oacc[db] = T::mma32(u32x4{ra[0], ra[1], rb[0], rb[1]}, pb[jj], oacc[db]);
        }
      }
    }
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
