// C ABI of libmta: argument validation, dispatch to the kernel files, error reporting.
// Declarations and the contract of every entry point are in include/mta.h.
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/mta.h"
#include "mta_backward.h"
#include "mta_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return MTA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr unsigned kKnownFlags = MTA_KQ_PRE | MTA_KQ_POST | MTA_MIX_PRE | MTA_MIX_POST | MTA_GN | MTA_FP32;

// Validates the arguments and fills *pr. Host-only: never touches the GPU.
int validate(const void* q, const void* k, const void* v, const float* theta, const float* w,
             const float* gamma, const float* beta, float lambda, const void* out, int B, int T, int M,
             int d, int c_q, int c_k, int c_h, unsigned flags, mta::Problem* pr) {
  if (flags & ~kKnownFlags) return fail(MTA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags & ~kKnownFlags);
  if (B <= 0 || T <= 0 || M <= 0 || d <= 0)
    return fail(MTA_ERR_INVALID_ARG, "sizes must be positive (B=%d T=%d M=%d d=%d)", B, T, M, d);
  if (!q || !k || !v || !out) return fail(MTA_ERR_INVALID_ARG, "q, k, v and out must not be NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(MTA_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  const bool kq = flags & (MTA_KQ_PRE | MTA_KQ_POST);
  const bool mix = flags & (MTA_MIX_PRE | MTA_MIX_POST);
  if (kq) {
    if (!theta) return fail(MTA_ERR_INVALID_ARG, "theta_kq is required with a KQ flag");
    if (c_q <= 0 || c_k <= 0) return fail(MTA_ERR_INVALID_ARG, "c_q and c_k must be positive (c_q=%d c_k=%d)", c_q, c_k);
    if (c_k % 2 == 0) return fail(MTA_ERR_UNSUPPORTED, "c_k must be odd (centred key taps), got %d", c_k);
    if (c_q > 8 || c_k > 17) return fail(MTA_ERR_UNSUPPORTED, "kernel %dx%d exceeds the supported 8x17", c_q, c_k);
  }
  if (mix) {
    if (!w) return fail(MTA_ERR_INVALID_ARG, "w_mix is required with a MIX flag");
    if (c_h <= 0 || M % c_h != 0) return fail(MTA_ERR_INVALID_ARG, "M=%d must be a multiple of c_h=%d", M, c_h);
    if (c_h != 1 && c_h != 2 && c_h != 4) return fail(MTA_ERR_UNSUPPORTED, "c_h=%d not in {1, 2, 4}", c_h);
  }
  if ((flags & MTA_GN) && (!gamma || !beta))
    return fail(MTA_ERR_INVALID_ARG, "gn_gamma and gn_beta are required with MTA_GN");
  // the GroupNorm epilogue reads gamma and beta four floats at a time
  if ((flags & MTA_GN) && (!aligned16(gamma) || !aligned16(beta)))
    return fail(MTA_ERR_INVALID_ARG, "gn_gamma and gn_beta must be 16-byte aligned");
  const bool fp32 = flags & MTA_FP32;
  if (fp32 ? !(d == 16 || d == 32 || d == 64) : !(d == 32 || d == 64 || d == 96 || d == 128))
    return fail(MTA_ERR_UNSUPPORTED, "head size d=%d is not built for %s", d, fp32 ? "fp32" : "bf16");
  if ((long long)B * T * M * d > (1LL << 40)) return fail(MTA_ERR_INVALID_ARG, "tensor too large");
  // the kernels address one batch of q, k, v or out with 32-bit byte offsets
  if ((long long)T * M * d * (fp32 ? 4 : 2) >= (1LL << 31))
    return fail(MTA_ERR_UNSUPPORTED, "one batch of a tensor (T*M*d elements) must be below 2 GiB");
  if (out == q || out == k || out == v) return fail(MTA_ERR_INVALID_ARG, "out may not alias an input");
  mta::Problem p;
  p.q = q;
  p.k = k;
  p.v = v;
  // with both sides the parameters before softmax come first, then those after
  const bool kq_both = (flags & MTA_KQ_PRE) && (flags & MTA_KQ_POST);
  const bool mix_both = (flags & MTA_MIX_PRE) && (flags & MTA_MIX_POST);
  p.theta_pre = (flags & MTA_KQ_PRE) ? theta : nullptr;
  p.theta_post = (flags & MTA_KQ_POST) ? theta + (kq_both ? (size_t)M * c_q * c_k : 0) : nullptr;
  p.w_pre = (flags & MTA_MIX_PRE) ? w : nullptr;
  p.w_post = (flags & MTA_MIX_POST) ? w + (mix_both ? (size_t)M * c_h : 0) : nullptr;
  p.gamma = (flags & MTA_GN) ? gamma : nullptr;
  p.beta = (flags & MTA_GN) ? beta : nullptr;
  p.lambda = lambda;
  p.out = const_cast<void*>(out);
  p.B = B;
  p.T = T;
  p.M = M;
  p.d = d;
  p.c_q = kq ? c_q : 1;
  p.c_k = kq ? c_k : 1;
  p.c_h = mix ? c_h : 1;
  p.kq = ((flags & MTA_KQ_PRE) ? mta::KQ_PRE : 0) | ((flags & MTA_KQ_POST) ? mta::KQ_POST : 0);
  p.mix = ((flags & MTA_MIX_PRE) ? mta::MIX_PRE : 0) | ((flags & MTA_MIX_POST) ? mta::MIX_POST : 0);
  p.gn = (flags & MTA_GN) ? 1 : 0;
  p.fp32 = fp32 ? 1 : 0;
  *pr = p;
  return MTA_OK;
}

// The size and placement fields of a problem (no pointers), for workspace-size queries;
// false for sizes that no call would accept.
bool sizes_problem(int B, int T, int M, int d, int c_q, int c_k, int c_h, unsigned flags, mta::Problem* p) {
  if (B <= 0 || T <= 0 || M <= 0 || d <= 0 || (flags & ~kKnownFlags)) return false;
  const bool kq = flags & (MTA_KQ_PRE | MTA_KQ_POST);
  const bool mix = flags & (MTA_MIX_PRE | MTA_MIX_POST);
  if ((kq && (c_q <= 0 || c_k <= 0)) || (mix && (c_h <= 0 || M % c_h != 0))) return false;
  p->B = B;
  p->T = T;
  p->M = M;
  p->d = d;
  p->c_q = kq ? c_q : 1;
  p->c_k = kq ? c_k : 1;
  p->c_h = mix ? c_h : 1;
  p->kq = ((flags & MTA_KQ_PRE) ? mta::KQ_PRE : 0) | ((flags & MTA_KQ_POST) ? mta::KQ_POST : 0);
  p->mix = ((flags & MTA_MIX_PRE) ? mta::MIX_PRE : 0) | ((flags & MTA_MIX_POST) ? mta::MIX_POST : 0);
  p->gn = (flags & MTA_GN) ? 1 : 0;
  p->fp32 = (flags & MTA_FP32) ? 1 : 0;
  return true;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(MTA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int mta_check_args(const void* q, const void* k, const void* v, const float* theta_kq, const float* w_mix,
                   const float* gn_gamma, const float* gn_beta, const void* out, int B, int T, int M, int d,
                   int c_q, int c_k, int c_h, unsigned flags) {
  mta::Problem p;
  const int st = validate(q, k, v, theta_kq, w_mix, gn_gamma, gn_beta, 1.0f, out, B, T, M, d, c_q, c_k, c_h,
                          flags, &p);
  return st == MTA_OK ? ok() : st;
}

int mta_forward(const void* q, const void* k, const void* v, const float* theta_kq, const float* w_mix,
                const float* gn_gamma, const float* gn_beta, float lambda, void* out, int B, int T, int M,
                int d, int c_q, int c_k, int c_h, unsigned flags, void* stream) {
  mta::Problem p;
  const int st = validate(q, k, v, theta_kq, w_mix, gn_gamma, gn_beta, lambda, out, B, T, M, d, c_q, c_k, c_h,
                          flags, &p);
  if (st != MTA_OK) return st;
  bool unsupported = false;
  const hipError_t e = mta::launch_fused(p, reinterpret_cast<hipStream_t>(stream), &unsupported);
  if (unsupported) return fail(MTA_ERR_UNSUPPORTED, "no fused kernel for this shape");
  return hip_status(e, "mta_forward launch");
}

int mta_forward_rows(const void* q, const void* k, const void* v, const float* theta_kq, const float* w_mix,
                     const float* gn_gamma, const float* gn_beta, float lambda, void* out, int B, int T, int M,
                     int d, int c_q, int c_k, int c_h, int row_begin, unsigned flags, void* stream) {
  mta::Problem p;
  const int st = validate(q, k, v, theta_kq, w_mix, gn_gamma, gn_beta, lambda, out, B, T, M, d, c_q, c_k, c_h,
                          flags, &p);
  if (st != MTA_OK) return st;
  if (row_begin < 0 || row_begin >= T)
    return fail(MTA_ERR_INVALID_ARG, "row_begin=%d must lie in [0, T=%d)", row_begin, T);
  p.row_begin = row_begin;
  bool unsupported = false;
  const hipError_t e = mta::launch_fused(p, reinterpret_cast<hipStream_t>(stream), &unsupported);
  if (unsupported) return fail(MTA_ERR_UNSUPPORTED, "no fused kernel for this shape");
  return hip_status(e, "mta_forward_rows launch");
}

size_t mta_forward_rows_split_workspace_bytes(int B, int T, int M, int d, int c_q, int c_k, int c_h, int row_begin,
                                              unsigned flags) {
  mta::Problem p{};
  if (!sizes_problem(B, T, M, d, c_q, c_k, c_h, flags, &p) || row_begin < 0 || row_begin >= T) return 0;
  p.row_begin = row_begin;
  return mta::rows_split_workspace_bytes(p);
}

int mta_forward_rows_split(const void* q, const void* k, const void* v, const float* theta_kq, const float* w_mix,
                           const float* gn_gamma, const float* gn_beta, float lambda, void* out, int B, int T, int M,
                           int d, int c_q, int c_k, int c_h, int row_begin, unsigned flags, void* workspace,
                           size_t workspace_bytes, void* stream) {
  mta::Problem p;
  const int st = validate(q, k, v, theta_kq, w_mix, gn_gamma, gn_beta, lambda, out, B, T, M, d, c_q, c_k, c_h,
                          flags, &p);
  if (st != MTA_OK) return st;
  if (row_begin < 0 || row_begin >= T)
    return fail(MTA_ERR_INVALID_ARG, "row_begin=%d must lie in [0, T=%d)", row_begin, T);
  p.row_begin = row_begin;
  const size_t need = mta::rows_split_workspace_bytes(p);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MTA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (need > 0 && !aligned16(workspace)) return fail(MTA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  bool unsupported = false;
  const hipError_t e = mta::launch_rows_split(p, workspace, reinterpret_cast<hipStream_t>(stream), &unsupported);
  if (unsupported) return fail(MTA_ERR_UNSUPPORTED, "no fused kernel for this shape");
  return hip_status(e, "mta_forward_rows_split launch");
}

int mta_forward_rows_split_plan(int B, int T, int M, int d, int c_q, int c_k, int c_h, int row_begin, unsigned flags,
                                int compute_units, int* n_chunks, int* chunk_keys) {
  mta::Problem p{};
  if (!n_chunks || !chunk_keys) return fail(MTA_ERR_INVALID_ARG, "n_chunks and chunk_keys must not be NULL");
  if (!sizes_problem(B, T, M, d, c_q, c_k, c_h, flags, &p))
    return fail(MTA_ERR_INVALID_ARG, "invalid sizes or flags");
  if (row_begin < 0 || row_begin >= T)
    return fail(MTA_ERR_INVALID_ARG, "row_begin=%d must lie in [0, T=%d)", row_begin, T);
  if (compute_units < 0) return fail(MTA_ERR_INVALID_ARG, "compute_units must be >= 0");
  p.row_begin = row_begin;
  const mta::SplitPlan plan = mta::split_plan(p, compute_units ? compute_units : mta::device_compute_units());
  *n_chunks = plan.n;
  *chunk_keys = plan.n > 1 ? plan.keys : T;
  return ok();
}

// ---- split row ranges without a caller workspace ---------------------------------------------
// For callers that cannot allocate: the partial results of mta_forward_rows_split_noalloc live
// in `scratch`, a file-scope device array of MTA_NOALLOC_SCRATCH_BYTES. Each device that runs
// the library holds its own copy until the process ends. Host code never passes the array's
// name to a kernel (on the host it is only a stand-in for the device symbol): the device
// address is looked up once per device with hipGetSymbolAddress, with that device current, and
// only that address reaches the kernels.
namespace {

static __device__ __align__(256) unsigned char scratch[MTA_NOALLOC_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchDevices];

// Device address of the current device's scratch array; MTA_OK or an error status.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kScratchDevices)
    return fail(MTA_ERR_UNSUPPORTED, "device %d: scratch is kept for devices 0..%d", dev, kScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MTA_OK;
}

}  // namespace

int mta_forward_rows_split_noalloc(const void* q, const void* k, const void* v, const float* theta_kq,
                                   const float* w_mix, const float* gn_gamma, const float* gn_beta, float lambda,
                                   void* out, int B, int T, int M, int d, int c_q, int c_k, int c_h, int row_begin,
                                   unsigned flags, void* stream) {
  mta::Problem p;
  int st = validate(q, k, v, theta_kq, w_mix, gn_gamma, gn_beta, lambda, out, B, T, M, d, c_q, c_k, c_h, flags, &p);
  if (st != MTA_OK) return st;
  if (row_begin < 0 || row_begin >= T)
    return fail(MTA_ERR_INVALID_ARG, "row_begin=%d must lie in [0, T=%d)", row_begin, T);
  p.row_begin = row_begin;
  const size_t need = mta::rows_split_workspace_bytes(p);
  if (need > (size_t)MTA_NOALLOC_SCRATCH_BYTES)
    return fail(MTA_ERR_WORKSPACE, "this row range needs %zu bytes of partial results; the library's scratch holds %zu",
                need, (size_t)MTA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0 && (st = scratch_address(&ws)) != MTA_OK) return st;
  bool unsupported = false;
  const hipError_t e = mta::launch_rows_split(p, ws, reinterpret_cast<hipStream_t>(stream), &unsupported);
  if (unsupported) return fail(MTA_ERR_UNSUPPORTED, "no fused kernel for this shape");
  return hip_status(e, "mta_forward_rows_split_noalloc launch");
}

size_t mta_materialized_workspace_bytes(int B, int T, int M, unsigned flags) {
  (void)flags;
  return mta::materialized_workspace_bytes(B, T, M);
}

int mta_forward_materialized(const void* q, const void* k, const void* v, const float* theta_kq,
                             const float* w_mix, const float* gn_gamma, const float* gn_beta, float lambda,
                             void* out, int B, int T, int M, int d, int c_q, int c_k, int c_h, unsigned flags,
                             void* workspace, size_t workspace_bytes, void* stream) {
  mta::Problem p;
  const int st = validate(q, k, v, theta_kq, w_mix, gn_gamma, gn_beta, lambda, out, B, T, M, d, c_q, c_k, c_h,
                          flags, &p);
  if (st != MTA_OK) return st;
  const size_t need = mta::materialized_workspace_bytes(B, T, M);
  if (!workspace || workspace_bytes < need)
    return fail(MTA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (!aligned16(workspace)) return fail(MTA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  bool unsupported = false;
  const hipError_t e = mta::launch_materialized(p, workspace, reinterpret_cast<hipStream_t>(stream), &unsupported);
  if (unsupported) return fail(MTA_ERR_UNSUPPORTED, "no materialized kernel for this shape");
  return hip_status(e, "mta_forward_materialized launch");
}

size_t mta_backward_workspace_bytes(int B, int T, int M, int d, int c_q, int c_k, int c_h, unsigned flags) {
  mta::Problem p{};
  if (!sizes_problem(B, T, M, d, c_q, c_k, c_h, flags, &p)) return 0;
  return mta::backward_workspace_bytes(p);
}

int mta_backward_materialized(const void* q, const void* k, const void* v, const float* theta_kq, const float* w_mix,
                              const float* gn_gamma, const float* gn_beta, float lambda, const void* dout, void* dq,
                              void* dk, void* dv, float* dtheta_kq, float* dw_mix, float* dgn_gamma, float* dgn_beta,
                              float* dlambda, int B, int T, int M, int d, int c_q, int c_k, int c_h, unsigned flags,
                              void* workspace, size_t workspace_bytes, void* stream) {
  mta::Problem p;
  const int st = validate(q, k, v, theta_kq, w_mix, gn_gamma, gn_beta, lambda, dq, B, T, M, d, c_q, c_k, c_h, flags,
                          &p);
  if (st != MTA_OK) return st;
  if (!dout || !dk || !dv) return fail(MTA_ERR_INVALID_ARG, "dout, dq, dk and dv must not be NULL");
  if (!aligned16(dout) || !aligned16(dk) || !aligned16(dv))
    return fail(MTA_ERR_INVALID_ARG, "dout, dq, dk and dv must be 16-byte aligned");
  const void* ins[4] = {q, k, v, dout};
  void* outs[3] = {dq, dk, dv};
  for (void* o : outs)
    for (const void* in : ins)
      if (o == in) return fail(MTA_ERR_INVALID_ARG, "dq, dk and dv may not alias q, k, v or dout");
  if (dq == dk || dq == dv || dk == dv) return fail(MTA_ERR_INVALID_ARG, "dq, dk and dv must be distinct");
  if (p.kq && !dtheta_kq) return fail(MTA_ERR_INVALID_ARG, "dtheta_kq is required with a KQ flag");
  if (p.mix && !dw_mix) return fail(MTA_ERR_INVALID_ARG, "dw_mix is required with a MIX flag");
  if (p.gn && (!dgn_gamma || !dgn_beta || !dlambda))
    return fail(MTA_ERR_INVALID_ARG, "dgn_gamma, dgn_beta and dlambda are required with MTA_GN");
  const size_t need = mta::backward_workspace_bytes(p);
  if (!workspace || workspace_bytes < need)
    return fail(MTA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (!aligned16(workspace)) return fail(MTA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  mta::BwdGrads g{dout, dq, dk, dv, dtheta_kq, dw_mix, dgn_gamma, dgn_beta, dlambda};
  bool unsupported = false;
  const hipError_t e = mta::launch_backward(p, g, workspace, reinterpret_cast<hipStream_t>(stream), &unsupported);
  if (unsupported) return fail(MTA_ERR_UNSUPPORTED, "no backward kernels for this shape");
  return hip_status(e, "mta_backward_materialized launch");
}

int mta_forward_train(const void* q, const void* k, const void* v, const float* theta_kq, const float* w_mix,
                      const float* gn_gamma, const float* gn_beta, float lambda, void* out, float* lse,
                      float* out_pre_gn, int B, int T, int M, int d, int c_q, int c_k, int c_h, unsigned flags,
                      void* stream) {
  mta::Problem p;
  const int st = validate(q, k, v, theta_kq, w_mix, gn_gamma, gn_beta, lambda, out, B, T, M, d, c_q, c_k, c_h,
                          flags, &p);
  if (st != MTA_OK) return st;
  if (p.fp32) return fail(MTA_ERR_UNSUPPORTED, "mta_forward_train is built for bf16 tensors");
  if (!lse) return fail(MTA_ERR_INVALID_ARG, "lse must not be NULL");
  if (!aligned16(lse) || (out_pre_gn && !aligned16(out_pre_gn)))
    return fail(MTA_ERR_INVALID_ARG, "lse and out_pre_gn must be 16-byte aligned");
  p.lse = lse;
  p.o32 = out_pre_gn;
  bool unsupported = false;
  const hipError_t e = mta::launch_fused(p, reinterpret_cast<hipStream_t>(stream), &unsupported);
  if (unsupported) return fail(MTA_ERR_UNSUPPORTED, "no fused kernel for this shape");
  return hip_status(e, "mta_forward_train launch");
}

size_t mta_backward_fused_workspace_bytes(int B, int T, int M, int d, int c_q, int c_k, int c_h, unsigned flags) {
  mta::Problem p{};
  if (!sizes_problem(B, T, M, d, c_q, c_k, c_h, flags, &p)) return 0;
  return mta::backward_fused_workspace_bytes(p);
}

int mta_backward_fused(const void* q, const void* k, const void* v, const float* theta_kq, const float* w_mix,
                       const float* gn_gamma, const float* gn_beta, float lambda, const float* lse,
                       const float* out_pre_gn, const void* dout, void* dq, void* dk, void* dv, float* dtheta_kq,
                       float* dw_mix, float* dgn_gamma, float* dgn_beta, float* dlambda, int B, int T, int M, int d,
                       int c_q, int c_k, int c_h, unsigned flags, void* workspace, size_t workspace_bytes,
                       void* stream) {
  mta::Problem p;
  const int st = validate(q, k, v, theta_kq, w_mix, gn_gamma, gn_beta, lambda, dq, B, T, M, d, c_q, c_k, c_h, flags,
                          &p);
  if (st != MTA_OK) return st;
  if (p.fp32) return fail(MTA_ERR_UNSUPPORTED, "mta_backward_fused is built for bf16 tensors");
  if (!dout || !dk || !dv) return fail(MTA_ERR_INVALID_ARG, "dout, dq, dk and dv must not be NULL");
  if (!aligned16(dout) || !aligned16(dk) || !aligned16(dv))
    return fail(MTA_ERR_INVALID_ARG, "dout, dq, dk and dv must be 16-byte aligned");
  const void* ins[4] = {q, k, v, dout};
  void* outs[3] = {dq, dk, dv};
  for (void* o : outs)
    for (const void* in : ins)
      if (o == in) return fail(MTA_ERR_INVALID_ARG, "dq, dk and dv may not alias q, k, v or dout");
  if (dq == dk || dq == dv || dk == dv) return fail(MTA_ERR_INVALID_ARG, "dq, dk and dv must be distinct");
  if (!lse) return fail(MTA_ERR_INVALID_ARG, "lse (from mta_forward_train) must not be NULL");
  if (p.gn && !out_pre_gn) return fail(MTA_ERR_INVALID_ARG, "out_pre_gn (from mta_forward_train) is required with MTA_GN");
  if (p.gn && !aligned16(out_pre_gn)) return fail(MTA_ERR_INVALID_ARG, "out_pre_gn must be 16-byte aligned");
  if (p.kq && !dtheta_kq) return fail(MTA_ERR_INVALID_ARG, "dtheta_kq is required with a KQ flag");
  if (p.mix && !dw_mix) return fail(MTA_ERR_INVALID_ARG, "dw_mix is required with a MIX flag");
  if (p.gn && (!dgn_gamma || !dgn_beta || !dlambda))
    return fail(MTA_ERR_INVALID_ARG, "dgn_gamma, dgn_beta and dlambda are required with MTA_GN");
  if (!mta::backward_fused_supported(p))
    return fail(MTA_ERR_UNSUPPORTED, "the fused backward's tiles of this placement do not fit in LDS");
  const size_t need = mta::backward_fused_workspace_bytes(p);
  if (!workspace || workspace_bytes < need)
    return fail(MTA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, workspace ? workspace_bytes : 0);
  if (!aligned16(workspace)) return fail(MTA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  mta::BwdGrads g{dout, dq, dk, dv, dtheta_kq, dw_mix, dgn_gamma, dgn_beta, dlambda};
  bool unsupported = false;
  const hipError_t e = mta::launch_backward_fused(p, g, lse, out_pre_gn, workspace,
                                                  reinterpret_cast<hipStream_t>(stream), &unsupported);
  if (unsupported) return fail(MTA_ERR_UNSUPPORTED, "no fused backward for this shape");
  return hip_status(e, "mta_backward_fused launch");
}

int mta_attention_plain(const void* q, const void* k, const void* v, void* out, int B, int T, int M, int d,
                        unsigned flags, void* stream) {
  if (flags & ~MTA_FP32) return fail(MTA_ERR_INVALID_ARG, "mta_attention_plain accepts only MTA_FP32");
  return mta_forward(q, k, v, nullptr, nullptr, nullptr, nullptr, 1.0f, out, B, T, M, d, 1, 1, 1, flags, stream);
}

const char* mta_status_string(int status) {
  switch (status) {
    case MTA_OK: return "ok";
    case MTA_ERR_INVALID_ARG: return "invalid argument";
    case MTA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MTA_ERR_HIP: return "HIP runtime error";
    case MTA_ERR_WORKSPACE: return "workspace missing or too small";
  }
  return "unknown status";
}

const char* mta_last_error(void) { return g_last_error.c_str(); }

int mta_version(void) { return 100; }

}  // extern "C"
