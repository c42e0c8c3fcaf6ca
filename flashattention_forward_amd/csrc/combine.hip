// Split-KV combine: merges the partial results of S key ranges of one query row.
// Each split s holds a normalised partial output O_s and its log-sum-exp lse_s.
// With L = log sum_s exp(lse_s) the row's output is sum_s exp(lse_s - L) O_s and
// its log-sum-exp is L (a split with lse_s = -inf contributes nothing; a row
// whose splits are all empty gets O = 0, lse = -inf).
//
// Split-reduction as in the dk-split of "perf(kernels): speed up
// linear-attention prefill ~2.6x" (hip-ep, Summary), here over key ranges.
// One wave per row; each lane owns 4 consecutive output columns.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <typename TO>
__global__ __launch_bounds__(256) void combine_kernel(CombineParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int S = p.n_splits;
  const int64_t rows = p.rows;
  float mx = -INFINITY;
  for (int s = 0; s < S; ++s) mx = fmaxf(mx, p.part_lse[s * rows + row]);
  float sum = 0.f;
  if (mx != -INFINITY)
    for (int s = 0; s < S; ++s) sum += __expf(p.part_lse[s * rows + row] - mx);
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  for (int d = 4 * lane; d < p.D; d += 256) {
    f32x4 acc = f32x4{};
    if (mx != -INFINITY)
      for (int s = 0; s < S; ++s) {
        const float wgt = __expf(p.part_lse[s * rows + row] - mx) * inv;
        if (wgt != 0.f) acc += wgt * *(const f32x4*)(p.part_o + (s * rows + row) * p.D + d);
      }
    store4(TO{}, (char*)p.o + ((int64_t)row * p.D + d) * out_size<TO>::bytes, acc[0], acc[1],
           acc[2], acc[3]);
  }
  if (p.lse && lane == 0) {
    const int h = row % p.Hq;
    const int i = (row / p.Hq) % p.Sq;
    const int b = row / (p.Hq * p.Sq);
    p.lse[((int64_t)b * p.Hq + h) * p.Sq + i] = sum > 0.f ? mx + __logf(sum) : -INFINITY;
  }
}

hipError_t launch_combine(const CombineParams& p, OutType ot, hipStream_t stream) {
  const int blocks = (p.rows + 3) / 4;
  switch (ot) {
    case OutType::bf16:
      hipLaunchKernelGGL(combine_kernel<out_bf16>, dim3(blocks), dim3(256), 0, stream, p);
      break;
    case OutType::f16:
      hipLaunchKernelGGL(combine_kernel<out_f16>, dim3(blocks), dim3(256), 0, stream, p);
      break;
    default:
      hipLaunchKernelGGL(combine_kernel<out_f32>, dim3(blocks), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace fa
