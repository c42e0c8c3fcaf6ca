// Prefill instantiations for head size 128 with fp16 inputs.
#include "prefill_kernel.h"

namespace fa {

hipError_t launch_prefill_128_f16(const PrefillParams& p, OutType ot, bool causal,
                                  hipStream_t stream) {
  return launch2<128, f16_t>(p, ot, causal, stream);
}

}  // namespace fa
