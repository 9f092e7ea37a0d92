// Unfused Multi-Token Attention forward: one kernel per step, fp32 [B, M, T, T] maps
// in HBM. This is the implementation style whose memory and runtime cost the page
// "Multi-Token Attention | Summary" reports for MTA (Appendix F, complexity table);
// it is kept as a comparison path for the fused kernel.
//
// Chain (X and Y are the two workspace maps; every map kernel touches all T x T
// entries, writing the masked value above the diagonal):
//   logits      X = Q K^T / sqrt(d)                                   (§2)
//   [mix pre]   X_u <- sum_u' w[u][u'] X_u'  (in place)               (§3.2)
//   [kq pre]    Y = Mask_-inf(Conv2d_theta(Mask_0(X)))                (§3.1)
//   softmax     causal row softmax, in place, zeros above the diagonal (§2)
//   [kq post]   Y = Mask_0(Conv2d_theta(A))                           (§3.1)
//   [mix post]  in place                                              (§3.2)
//   AV + GroupNorm + gate -> out                                      (§2, §3.3)
// The map kernels are in mta_map_kernels.h (shared with the backward pass).
#include "mta_map_kernels.h"

namespace mta {
namespace {

template <typename T, int D>
hipError_t run_chain(const Problem& p, float* X, float* Y, hipStream_t st) {
  const T* q = reinterpret_cast<const T*>(p.q);
  const T* k = reinterpret_cast<const T*>(p.k);
  hipError_t e;
  const float scale = (float)(1.0 / __builtin_sqrt((double)p.d));
  hipLaunchKernelGGL((logits_kernel<T, D>), dim3((p.T + 127) / 128, (p.T + 127) / 128, p.B * p.M),
                     dim3(MT_THREADS), 0, st, q, k, X, p.T, p.M, scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  float* cur = X;
  float* other = Y;
  if ((p.mix & MIX_PRE) && (e = launch_mix(cur, p.w_pre, p, st)) != hipSuccess) return e;
  if (p.kq & KQ_PRE) {
    if ((e = launch_conv(true, cur, other, p, st)) != hipSuccess) return e;
    float* t = cur;
    cur = other;
    other = t;
  }
  if ((e = launch_softmax(cur, p, st)) != hipSuccess) return e;
  if (p.kq & KQ_POST) {
    if ((e = launch_conv(false, cur, other, p, st)) != hipSuccess) return e;
    float* t = cur;
    cur = other;
    other = t;
  }
  if ((p.mix & MIX_POST) && (e = launch_mix(cur, p.w_post, p, st)) != hipSuccess) return e;
  return launch_av<T, D>(cur, p, st);
}

}  // namespace

size_t materialized_workspace_bytes(int B, int T, int M) {
  if (B <= 0 || T <= 0 || M <= 0) return 0;
  return 2 * (size_t)B * M * T * map_ld(T) * sizeof(float);
}

bool materialized_supported(const Problem& p) {
  if (p.mix && !(p.c_h == 1 || p.c_h == 2 || p.c_h == 4)) return false;
  if (p.kq && (p.c_q < 1 || p.c_q > 8 || p.c_k < 1 || p.c_k > 17 || p.c_k % 2 == 0)) return false;
  if (p.fp32) return p.d == 16 || p.d == 32 || p.d == 64;
  return p.d == 32 || p.d == 64 || p.d == 96 || p.d == 128;
}

hipError_t launch_materialized(const Problem& p, void* workspace, hipStream_t st, bool* unsupported) {
  *unsupported = false;
  if (!materialized_supported(p)) {
    *unsupported = true;
    return hipSuccess;
  }
  float* X = reinterpret_cast<float*>(workspace);
  float* Y = X + (size_t)p.B * p.M * p.T * map_ld(p.T);
  if (p.fp32) {
    switch (p.d) {
      case 16: return run_chain<float, 16>(p, X, Y, st);
      case 32: return run_chain<float, 32>(p, X, Y, st);
      case 64: return run_chain<float, 64>(p, X, Y, st);
    }
  } else {
    switch (p.d) {
      case 32: return run_chain<__bf16, 32>(p, X, Y, st);
      case 64: return run_chain<__bf16, 64>(p, X, Y, st);
      case 96: return run_chain<__bf16, 96>(p, X, Y, st);
      case 128: return run_chain<__bf16, 128>(p, X, Y, st);
    }
  }
  *unsupported = true;
  return hipSuccess;
}

}  // namespace mta
