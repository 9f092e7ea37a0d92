// Internal interface of the backward pass (mta_backward.hip).
#pragma once

#include "mta_internal.h"

namespace mta {

// Gradient buffers of one backward call (device memory; unused ones may be null).
struct BwdGrads {
  const void* dout;  // [B,T,M,d] input dtype: gradient of the layer output
  void* dq;          // [B,T,M,d] input dtype
  void* dk;
  void* dv;
  float* dtheta;  // shape of theta_kq
  float* dw;      // shape of w_mix
  float* dgamma;  // [M*d]
  float* dbeta;   // [M*d]
  float* dlambda;  // [1]
};

size_t backward_workspace_bytes(const Problem& p);
bool backward_supported(const Problem& p);
hipError_t launch_backward(const Problem& p, const BwdGrads& g, void* workspace, hipStream_t stream,
                           bool* unsupported);

// Fused backward (mta_bwd_fused.hip): no T x T map in memory. lse [B,T,M] and o32 [B,T,M,d]
// (needed with GroupNorm) come from the forward (Problem::lse, Problem::o32).
size_t backward_fused_workspace_bytes(const Problem& p);
bool backward_fused_supported(const Problem& p);
hipError_t launch_backward_fused(const Problem& p, const BwdGrads& g, const float* lse, const float* o32,
                                 void* workspace, hipStream_t stream, bool* unsupported);

}  // namespace mta
