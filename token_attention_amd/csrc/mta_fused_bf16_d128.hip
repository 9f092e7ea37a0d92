// Fused kernel instantiations for bf16 tensors with head size 128 (key-major schedule):
// placements without a convolution after softmax.
#include "mta_kmajor_impl.h"

namespace mta {
hipError_t launch_fused_bf16_d128(const Problem& p, hipStream_t stream) {
  return kmajor::launch_d<128, false, false>(p, stream);
}
}  // namespace mta
