// Fused kernel instantiations for bf16 tensors with head size 64.
#include "mta_fused_impl.h"

namespace mta {
hipError_t launch_fused_bf16_d64(const Problem& p, hipStream_t stream) {
  return fused::launch_d<__bf16, 64>(p, stream);
}
}  // namespace mta
