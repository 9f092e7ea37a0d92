// Fused kernel instantiations for bf16 tensors with head size 128.
#include "mta_fused_impl.h"

namespace mta {
hipError_t launch_fused_bf16_d128(const Problem& p, hipStream_t stream) {
  return fused::launch_d<__bf16, 128>(p, stream);
}
}  // namespace mta
