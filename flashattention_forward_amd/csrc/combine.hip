// Split-KV combine: merges the partial results of S key ranges of one query row.
// Each split s holds a normalised partial output O_s (in the output's type:
// a 16-bit output halves the partials' traffic against fp32) and its
// log-sum-exp lse_s (fp32).
// With L = log sum_s exp(lse_s) the row's output is sum_s exp(lse_s - L) O_s and
// its log-sum-exp is L (a split with lse_s = -inf contributes nothing; a row
// whose splits are all empty gets O = 0, lse = -inf).
//
// Split-reduction as in the dk-split of "perf(kernels): speed up
// linear-attention prefill ~2.6x" (hip-ep, Summary), here over key ranges.
// A row is handled by D/4 lanes (4 consecutive output columns each; 8 with
// 16-bit partials), and the loads of up to four splits are issued together.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// Four partial-output columns as fp32, stored as fp32 or as the output's
// 16-bit type.
template <typename TO, bool P16> __device__ __forceinline__ f32x4 load_part4(const void* base, int64_t i) {
  if constexpr (!P16) {
    return *(const f32x4*)((const float*)base + i);
  } else {
    const u32x2 v = *(const u32x2*)((const uint16_t*)base + i);
    if constexpr (__is_same(TO, out_bf16)) {
      return f32x4{__uint_as_float(v[0] << 16), __uint_as_float(v[0] & 0xffff0000u),
                   __uint_as_float(v[1] << 16), __uint_as_float(v[1] & 0xffff0000u)};
    } else {
      // (Scalar halves: a bit-cast of each dword to a 2-vector of _Float16
      // lost the second dword in this compiler.)
      auto h = [](uint32_t x) { return (float)__builtin_bit_cast(_Float16, (uint16_t)x); };
      return f32x4{h(v[0]), h(v[0] >> 16), h(v[1]), h(v[1] >> 16)};
    }
  }
}

// CPT consecutive partial-output columns (16 bytes: 4 fp32 or 8 16-bit values) as fp32.
template <typename TO, bool P16>
__device__ __forceinline__ void load_part16B(const void* base, int64_t i, float* v) {
  if constexpr (!P16) {
    const f32x4 x = *(const f32x4*)((const float*)base + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = x[k];
  } else {
    const u32x4 x = *(const u32x4*)((const uint16_t*)base + i);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (__is_same(TO, out_bf16)) {
        v[2 * k] = __uint_as_float(x[k] << 16);
        v[2 * k + 1] = __uint_as_float(x[k] & 0xffff0000u);
      } else {
        v[2 * k] = (float)__builtin_bit_cast(_Float16, (uint16_t)x[k]);
        v[2 * k + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(x[k] >> 16));
      }
    }
  }
}

// Row-parallel combine: TPR threads per row, each with CPT = D / TPR columns
// (one 16-byte load per split). Splits are taken NB at a time with all of a
// batch's loads issued together (splits past the last re-read it and get
// weight 0); the running maximum of lse rescales the sums as it grows, so a
// row needs no separate pass over its lse values.
template <typename TO, int TPR, int NB, bool P16>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int RPB = 256 / TPR;
  constexpr int CPT = P16 ? 8 : 4;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int d = CPT * (threadIdx.x % TPR);
  if (row >= p.rows) return;
  const int S = p.n_splits;
  const int64_t rows = p.rows;
  const float* lse_p = p.part_lse + row;
  const int64_t o_i = (int64_t)row * p.D + d;
  const int64_t o_stride = rows * p.D;
  float acc[CPT] = {};
  float m = -INFINITY, sum = 0.f;
  for (int s0 = 0; s0 < S; s0 += NB) {
    float l[NB], o[NB][CPT];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int s = min(s0 + u, S - 1);
      l[u] = s0 + u < S ? lse_p[s * rows] : -INFINITY;
      load_part16B<TO, P16>(p.part_o, o_i + s * o_stride, o[u]);
    }
    float m_new = m;
#pragma unroll
    for (int u = 0; u < NB; ++u) m_new = fmaxf(m_new, l[u]);
    // Reference point 0 while every split so far is empty (lse -inf); no
    // branch, so that no load is moved behind one.
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float r = __expf(m - m_ref);  // 0 while m is -inf
    sum *= r;
#pragma unroll
    for (int k = 0; k < CPT; ++k) acc[k] *= r;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const float wgt = __expf(l[u] - m_ref);  // 0 for an empty split
      sum += wgt;
#pragma unroll
      for (int k = 0; k < CPT; ++k) acc[k] = wgt != 0.f ? fmaf(wgt, o[u][k], acc[k]) : acc[k];
    }
    m = m_new;
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  char* dst = (char*)p.o + ((int64_t)row * p.D + d) * out_size<TO>::bytes;
  if constexpr (CPT == 8) {
    store4(TO{}, dst, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    store4(TO{}, dst + 4 * out_size<TO>::bytes, acc[4] * inv, acc[5] * inv, acc[6] * inv,
           acc[7] * inv);
  } else {
    store4(TO{}, dst, acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  }
  if (p.lse && d == 0) {
    const int h = row % p.Hq;
    const int i = (row / p.Hq) % p.Sq;
    const int b = row / (p.Hq * p.Sq);
    p.lse[((int64_t)b * p.Hq + h) * p.Sq + i] = sum > 0.f ? m + __logf(sum) : -INFINITY;
  }
}

// Few rows, many splits (decode of a small batch): one 256-thread block per
// row. Thread (sg, col) handles output columns 4 col .. 4 col + 3 for the
// splits s = sg, sg + SG, ..., eight at a time with all of a batch's loads
// issued together and a running maximum of lse (as in combine_one); the SG
// split groups' (max, sum, columns) are then merged through LDS.
template <typename TO, int TPR, bool P16>
__global__ __launch_bounds__(256) void combine_row_kernel(CombineParams p) {
  constexpr int SG = 256 / TPR;
  constexpr int NB = 8;
  __shared__ f32x4 racc[SG][TPR];
  __shared__ float rsum[SG][TPR], rmax[SG][TPR];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int sg = tid / TPR, col = tid % TPR, d = 4 * col;
  const int S = p.n_splits;
  const int64_t rows = p.rows;
  const float* lse_p = p.part_lse + row;
  const int64_t o_i = (int64_t)row * p.D + d;
  const int64_t o_stride = rows * p.D;
  f32x4 acc = f32x4{};
  float m = -INFINITY, sum = 0.f;
  for (int s0 = sg; s0 < S; s0 += NB * SG) {
    float l[NB];
    f32x4 o[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int s = min(s0 + u * SG, S - 1);
      l[u] = s0 + u * SG < S ? lse_p[s * rows] : -INFINITY;
      o[u] = load_part4<TO, P16>(p.part_o, o_i + s * o_stride);
    }
    float m_new = m;
#pragma unroll
    for (int u = 0; u < NB; ++u) m_new = fmaxf(m_new, l[u]);
    // Reference point 0 while every split so far is empty (lse -inf).
    const float m_ref = m_new == -INFINITY ? 0.f : m_new;
    const float r = __expf(m - m_ref);  // 0 while m is -inf
    sum *= r;
    acc *= r;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const float wgt = __expf(l[u] - m_ref);  // 0 for an empty split
      sum += wgt;
      if (wgt != 0.f) acc += wgt * o[u];
    }
    m = m_new;
  }
  racc[sg][col] = acc;
  rsum[sg][col] = sum;
  rmax[sg][col] = m;
  __syncthreads();
  if (sg != 0) return;
  float mx = m;
  for (int k = 1; k < SG; ++k) mx = fmaxf(mx, rmax[k][col]);
  const float mx_ref = mx == -INFINITY ? 0.f : mx;
  const float w0 = __expf(m - mx_ref);  // each group's sums are relative to its own max
  acc *= w0;
  sum *= w0;
  for (int k = 1; k < SG; ++k) {
    const float wk = __expf(rmax[k][col] - mx_ref);
    acc += wk * racc[k][col];
    sum += wk * rsum[k][col];
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  acc *= inv;
  store4(TO{}, (char*)p.o + ((int64_t)row * p.D + d) * out_size<TO>::bytes, acc[0], acc[1], acc[2],
         acc[3]);
  if (p.lse && d == 0) {
    const int h = row % p.Hq;
    const int i = (row / p.Hq) % p.Sq;
    const int b = row / (p.Hq * p.Sq);
    p.lse[((int64_t)b * p.Hq + h) * p.Sq + i] = sum > 0.f ? mx + __logf(sum) : -INFINITY;
  }
}

template <typename TO, bool P16>
hipError_t launch_combine_t(const CombineParams& p, hipStream_t stream) {
  // Row-parallel unless that leaves the chip mostly idle and there are
  // enough splits to spread over a block.
  const int tpr = p.D / 4;
  const int64_t blocks_rowpar = ((int64_t)p.rows * tpr + 255) / 256;
  if (blocks_rowpar < 256 && p.n_splits >= 8) {
    auto go = [&](auto kern) {
      hipLaunchKernelGGL(kern, dim3(p.rows), dim3(256), 0, stream, p);
    };
    switch (p.D) {
      case 64: go(combine_row_kernel<TO, 16, P16>); break;
      case 128: go(combine_row_kernel<TO, 32, P16>); break;
      case 256: go(combine_row_kernel<TO, 64, P16>); break;
      case 512: go(combine_row_kernel<TO, 128, P16>); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  constexpr int CPT = P16 ? 8 : 4;
  auto go = [&](auto k2, auto k4) {
    const int rpb = 256 / (p.D / CPT);
    const dim3 grid((p.rows + rpb - 1) / rpb);
    if (p.n_splits <= 2)
      hipLaunchKernelGGL(k2, grid, dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL(k4, grid, dim3(256), 0, stream, p);
  };
  switch (p.D) {
    case 64: go(combine_kernel<TO, 64 / CPT, 2, P16>, combine_kernel<TO, 64 / CPT, 4, P16>); break;
    case 128: go(combine_kernel<TO, 128 / CPT, 2, P16>, combine_kernel<TO, 128 / CPT, 4, P16>); break;
    case 256: go(combine_kernel<TO, 256 / CPT, 2, P16>, combine_kernel<TO, 256 / CPT, 4, P16>); break;
    case 512: go(combine_kernel<TO, 512 / CPT, 2, P16>, combine_kernel<TO, 512 / CPT, 4, P16>); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, OutType ot, hipStream_t stream) {
  if (p.part16 && ot == OutType::f32) return hipErrorInvalidValue;
  switch (ot) {
    case OutType::bf16:
      return p.part16 ? launch_combine_t<out_bf16, true>(p, stream)
                      : launch_combine_t<out_bf16, false>(p, stream);
    case OutType::f16:
      return p.part16 ? launch_combine_t<out_f16, true>(p, stream)
                      : launch_combine_t<out_f16, false>(p, stream);
    default: return launch_combine_t<out_f32, false>(p, stream);
  }
}

}  // namespace fa
