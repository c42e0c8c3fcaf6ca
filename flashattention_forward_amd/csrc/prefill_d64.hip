// Prefill instantiations for head size 64 (bf16 and fp16 inputs).
#include "prefill_kernel.h"

namespace fa {

hipError_t launch_prefill_64_bf16(const PrefillParams& p, OutType ot, bool causal,
                                  hipStream_t stream) {
  return launch2<64, bf16_t>(p, ot, causal, stream);
}

hipError_t launch_prefill_64_f16(const PrefillParams& p, OutType ot, bool causal,
                                 hipStream_t stream) {
  return launch2<64, f16_t>(p, ot, causal, stream);
}

}  // namespace fa
