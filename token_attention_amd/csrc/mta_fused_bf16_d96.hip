// Fused kernel instantiations for bf16 tensors with head size 96 (key-major schedule):
// placements without a convolution after softmax.
#include "mta_kmajor_impl.h"

namespace mta {
hipError_t launch_fused_bf16_d96(const Problem& p, hipStream_t stream) {
  return kmajor::launch_d<96, false, false>(p, stream);
}
}  // namespace mta
