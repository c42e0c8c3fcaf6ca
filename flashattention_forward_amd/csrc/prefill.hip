// Prefill launch dispatch and the instantiations for head size 128 with bf16
// inputs (the other head size / input type pairs are compiled in
// prefill_f16.hip and prefill_d64.hip, in parallel).
#include "prefill_kernel.h"

namespace fa {

hipError_t launch_prefill_128_bf16(const PrefillParams& p, OutType ot, bool causal,
                                   hipStream_t stream) {
  return launch2<128, bf16_t>(p, ot, causal, stream);
}

hipError_t launch_prefill(const PrefillParams& p, int D, InType it, OutType ot, bool causal,
                          hipStream_t stream) {
  if (D == 128 && p.waves == 8 && p.pingpong && !p.mask)
    return launch_prefill_pp(p, it, ot, causal, stream);
  if (D == 64)
    return it == InType::bf16 ? launch_prefill_64_bf16(p, ot, causal, stream)
                              : launch_prefill_64_f16(p, ot, causal, stream);
  return it == InType::bf16 ? launch_prefill_128_bf16(p, ot, causal, stream)
                            : launch_prefill_128_f16(p, ot, causal, stream);
}

}  // namespace fa
