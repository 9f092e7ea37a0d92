// Fused kernel instantiations for bf16 tensors with head size 32 (key-major schedule):
// placements without a convolution after softmax, in the instantiations that cover one
// chunk of a split key range.
#include "mta_kmajor_impl.h"

namespace mta {
hipError_t launch_fused_bf16_d32_split(const Problem& p, hipStream_t stream) {
  return kmajor::launch_d<32, false, true>(p, stream);
}
}  // namespace mta
