// Split-KV combine: merges the partial results of S key ranges of one query row.
// Each split s holds a normalised partial output O_s and its log-sum-exp lse_s.
// With L = log sum_s exp(lse_s) the row's output is sum_s exp(lse_s - L) O_s and
// its log-sum-exp is L (a split with lse_s = -inf contributes nothing; a row
// whose splits are all empty gets O = 0, lse = -inf).
//
// Split-reduction as in the dk-split of "perf(kernels): speed up
// linear-attention prefill ~2.6x" (hip-ep, Summary), here over key ranges.
// A row is handled by D/4 lanes (4 consecutive output columns each), so a
// 256-thread block covers 1024/D rows; the loads of four splits are issued
// together.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <typename TO, int TPR>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  constexpr int RPB = 256 / TPR;
  const int row = blockIdx.x * RPB + threadIdx.x / TPR;
  const int d = 4 * (threadIdx.x % TPR);
  if (row >= p.rows) return;
  const int S = p.n_splits;
  const int64_t rows = p.rows;
  const float* lse_p = p.part_lse + row;
  const float* o_p = p.part_o + (int64_t)row * p.D + d;
  const int64_t o_stride = rows * p.D;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, lse_p[s * rows]);
  f32x4 acc = f32x4{};
  float sum = 0.f;
  if (mx != -INFINITY) {
    for (int s0 = 0; s0 < S; s0 += 4) {
      float l[4];
      f32x4 o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool ok = s0 + u < S;
        l[u] = ok ? lse_p[(s0 + u) * rows] : -INFINITY;
        o[u] = ok ? *(const f32x4*)(o_p + (s0 + u) * o_stride) : f32x4{};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wgt = __expf(l[u] - mx);  // 0 for an empty split (lse -inf)
        sum += wgt;
        if (wgt != 0.f) acc += wgt * o[u];
      }
    }
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

// Few rows, many splits (decode of a small batch): one 256-thread block per
// row. Thread (sg, col) handles output columns 4 col .. 4 col + 3 for the
// splits s = sg, sg + SG, ...; the per-thread partial sums are then added up
// over the SG split groups through LDS.
template <typename TO, int TPR>
__global__ __launch_bounds__(256) void combine_row_kernel(CombineParams p) {
  constexpr int SG = 256 / TPR;
  __shared__ float red[256];
  __shared__ f32x4 racc[SG][TPR];
  __shared__ float rsum[SG][TPR];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int sg = tid / TPR, col = tid % TPR, d = 4 * col;
  const int S = p.n_splits;
  const int64_t rows = p.rows;
  const float* lse_p = p.part_lse + row;
  float m = -INFINITY;
  for (int s = tid; s < S; s += 256) m = fmaxf(m, lse_p[s * rows]);
  red[tid] = m;
  __syncthreads();
  for (int k = 128; k > 0; k >>= 1) {
    if (tid < k) red[tid] = fmaxf(red[tid], red[tid + k]);
    __syncthreads();
  }
  const float mx = red[0];
  f32x4 acc = f32x4{};
  float sum = 0.f;
  if (mx != -INFINITY) {
    const float* o_p = p.part_o + (int64_t)row * p.D + d;
    const int64_t o_stride = rows * p.D;
    for (int s0 = sg; s0 < S; s0 += 4 * SG) {
      float l[4];
      f32x4 o[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = s0 + u * SG;
        const bool ok = s < S;
        l[u] = ok ? lse_p[s * rows] : -INFINITY;
        o[u] = ok ? *(const f32x4*)(o_p + s * o_stride) : f32x4{};
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wgt = __expf(l[u] - mx);  // 0 for an empty split (lse -inf)
        sum += wgt;
        if (wgt != 0.f) acc += wgt * o[u];
      }
    }
  }
  racc[sg][col] = acc;
  rsum[sg][col] = sum;
  __syncthreads();
  if (sg != 0) return;
  for (int k = 1; k < SG; ++k) {
    acc += racc[k][col];
    sum += rsum[k][col];
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

template <typename TO>
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
      case 64: go(combine_row_kernel<TO, 16>); break;
      case 128: go(combine_row_kernel<TO, 32>); break;
      case 256: go(combine_row_kernel<TO, 64>); break;
      case 512: go(combine_row_kernel<TO, 128>); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  auto go = [&](auto kern, int tpr) {
    const int rpb = 256 / tpr;
    hipLaunchKernelGGL(kern, dim3((p.rows + rpb - 1) / rpb), dim3(256), 0, stream, p);
  };
  switch (p.D) {
    case 64: go(combine_kernel<TO, 16>, 16); break;
    case 128: go(combine_kernel<TO, 32>, 32); break;
    case 256: go(combine_kernel<TO, 64>, 64); break;
    case 512: go(combine_kernel<TO, 128>, 128); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineParams& p, OutType ot, hipStream_t stream) {
  switch (ot) {
    case OutType::bf16: return launch_combine_t<out_bf16>(p, stream);
    case OutType::f16: return launch_combine_t<out_f16>(p, stream);
    default: return launch_combine_t<out_f32>(p, stream);
  }
}

}  // namespace fa
