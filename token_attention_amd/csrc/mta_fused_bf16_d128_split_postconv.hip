// Fused kernel instantiations for bf16 tensors with head size 128 (key-major schedule):
// placements with the key-query convolution after softmax (two-phase schedule), in the
// instantiations that cover one chunk of a split key range.
#include "mta_kmajor_impl.h"

namespace mta {
hipError_t launch_fused_bf16_d128_split_postconv(const Problem& p, hipStream_t stream) {
  return kmajor::launch_d<128, true, true>(p, stream);
}
}  // namespace mta
