// Fused kernel instantiations for fp32 tensors with head size 32 (row-major schedule).
#include "mta_fused_impl.h"

namespace mta {
hipError_t launch_fused_f32_d32(const Problem& p, hipStream_t stream) {
  return fused::launch_d<float, 32>(p, stream);
}
}  // namespace mta
