// Fused backward: region and LDS planning of the tile kernels (mta_bwd_tile.h), the
// GroupNorm backward, the two tile passes, and the fixed-order sums of the partial results.
#include <algorithm>

#include "mta_backward.h"
#include "mta_bwd_common.h"
#include "mta_bwd_tile.h"

namespace mta {

hipError_t launch_bwd_tiles_d32(const bwt::BwArgs& a, int ch, int mode, int spec, size_t lds, unsigned grid,
                                 hipStream_t st);
hipError_t launch_bwd_tiles_d64(const bwt::BwArgs& a, int ch, int mode, int spec, size_t lds, unsigned grid,
                                 hipStream_t st);
hipError_t launch_bwd_tiles_d96(const bwt::BwArgs& a, int ch, int mode, int spec, size_t lds, unsigned grid,
                                 hipStream_t st);
hipError_t launch_bwd_tiles_d128(const bwt::BwArgs& a, int ch, int mode, int spec, size_t lds, unsigned grid,
                                 hipStream_t st);

namespace {

constexpr size_t LDS_LIMIT = 160 * 1024;

// The placement bits of a problem as the plan takes them: 1 before softmax, 2 after.
int kq_bits(const Problem& p) { return ((p.kq & KQ_PRE) ? 1 : 0) | ((p.kq & KQ_POST) ? 2 : 0); }
int mix_bits(const Problem& p) { return ((p.mix & MIX_PRE) ? 1 : 0) | ((p.mix & MIX_POST) ? 2 : 0); }

// The specialised kernel of this shape, 0 for the generic one.
int spec_of(const Problem& p) {
  for (int s = 1; s < bwt::NSPEC; ++s) {
    const bwt::SpecShape sh = bwt::spec_shape(s);
    if (sh.kq == kq_bits(p) && sh.mix == mix_bits(p) && sh.cq == p.c_q && sh.ck == p.c_k &&
        bwt::spec_built(s, p.c_h, p.d))
      return s;
  }
  return 0;
}

// The plan of one pass (mta_bwd_tile.h): a specialised kernel's own, else the generic kernel's,
// which it reads from its arguments; returns the LDS bytes, 0 if the tiles do not fit.
size_t plan_tiles(const Problem& p, int mode, bwt::BwArgs& a) {
  const int spec = spec_of(p);
  a.P = spec ? bwt::spec_plan(mode, spec, p.c_h, p.d)
             : bwt::make_plan(mode, kq_bits(p), mix_bits(p), p.c_q, p.c_k, p.c_h, p.d);
  const size_t bytes = (size_t)a.P.lds_floats * sizeof(float);
  return bytes <= LDS_LIMIT ? bytes : 0;
}

__global__ void fill_zero_kernel(float4* __restrict__ p, size_t n4) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n4) p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

// dq = bf16(scale * acc), four elements per thread
__global__ void dq_convert_kernel(const float4* __restrict__ acc, uint2* __restrict__ dq, float scale, size_t n4) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n4) return;
  const float4 x = acc[i];
  __bf16 h[4] = {(__bf16)(x.x * scale), (__bf16)(x.y * scale), (__bf16)(x.z * scale), (__bf16)(x.w * scale)};
  dq[i] = *reinterpret_cast<const uint2*>(h);
}

struct FusedLayout {
  size_t dO, dq, dvec, lse_c, thpre, thpost, wpre, wpost, gn, total;
};

FusedLayout fused_layout(const Problem& p) {
  FusedLayout l{};
  const size_t tens = (size_t)p.B * p.T * p.M * p.d;
  const size_t nt = (size_t)(p.T + bwt::TB - 1) / bwt::TB;
  const size_t nch = (size_t)(p.T + GN_RB - 1) / GN_RB;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  l.dO = take(p.gn ? tens * 2 : 0);
  l.dq = take(tens * sizeof(float));
  l.dvec = take((size_t)p.B * p.T * p.M * sizeof(float));
  l.lse_c = take((size_t)p.B * p.T * p.M * sizeof(float));
  const size_t th = (size_t)p.B * nt * p.M * p.c_q * p.c_k * sizeof(float);
  const size_t w = (size_t)p.B * nt * p.M * p.c_h * sizeof(float);
  l.thpre = take((p.kq & KQ_PRE) ? th : 0);
  l.thpost = take((p.kq & KQ_POST) ? th : 0);
  l.wpre = take((p.mix & MIX_PRE) ? w : 0);
  l.wpost = take((p.mix & MIX_POST) ? w : 0);
  l.gn = take(p.gn ? (2 * p.B * nch * p.M * p.d + p.B * nch * p.M) * sizeof(float) : 0);
  l.total = off;
  return l;
}

hipError_t launch_tiles(const Problem& p, const bwt::BwArgs& a, int mode, size_t lds, hipStream_t st) {
  const unsigned grid = (unsigned)((size_t)p.B * (p.M / p.c_h) * a.n_tiles);
  const int spec = spec_of(p);
  switch (p.d) {
    case 32: return launch_bwd_tiles_d32(a, p.c_h, mode, spec, lds, grid, st);
    case 64: return launch_bwd_tiles_d64(a, p.c_h, mode, spec, lds, grid, st);
    case 96: return launch_bwd_tiles_d96(a, p.c_h, mode, spec, lds, grid, st);
    case 128: return launch_bwd_tiles_d128(a, p.c_h, mode, spec, lds, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool backward_fused_supported(const Problem& p) {
  if (p.fp32 || !(p.d == 32 || p.d == 64 || p.d == 96 || p.d == 128)) return false;
  if (!(p.c_h == 1 || p.c_h == 2 || p.c_h == 4)) return false;
  if ((long long)p.B * (p.M / p.c_h) * ((p.T + bwt::TB - 1) / bwt::TB) > 0x7fffffffLL) return false;
  bwt::BwArgs a{};
  return plan_tiles(p, bwt::PASS_D, a) != 0 && plan_tiles(p, bwt::PASS_K, a) != 0;
}

size_t backward_fused_workspace_bytes(const Problem& p) { return fused_layout(p).total; }

hipError_t launch_backward_fused(const Problem& p, const BwdGrads& g, const float* lse, const float* o32,
                                 void* workspace, hipStream_t st, bool* unsupported) {
  *unsupported = false;
  if (!backward_fused_supported(p)) {
    *unsupported = true;
    return hipSuccess;
  }
  char* ws = reinterpret_cast<char*>(workspace);
  const FusedLayout l = fused_layout(p);
  const size_t tens = (size_t)p.B * p.T * p.M * p.d;
  hipError_t e;

  // ---- GroupNorm / gate backward -> dO
  const __bf16* dO = reinterpret_cast<const __bf16*>(g.dout);
  if (p.gn) {
    __bf16* dOw = reinterpret_cast<__bf16*>(ws + l.dO);
    const int nch = (p.T + GN_RB - 1) / GN_RB;
    float* part_g = reinterpret_cast<float*>(ws + l.gn);
    float* part_b = part_g + (size_t)p.B * nch * p.M * p.d;
    float* part_l = part_b + (size_t)p.B * nch * p.M * p.d;
    const dim3 grid(nch, p.B * p.M);
    switch (p.d) {
      case 32: hipLaunchKernelGGL((gn_backward_kernel<__bf16, 32>), grid, dim3(MT_THREADS), 0, st, o32, dO, p.gamma, p.beta, p.lambda, dOw, part_g, part_b, part_l, p.T, p.M); break;
      case 64: hipLaunchKernelGGL((gn_backward_kernel<__bf16, 64>), grid, dim3(MT_THREADS), 0, st, o32, dO, p.gamma, p.beta, p.lambda, dOw, part_g, part_b, part_l, p.T, p.M); break;
      case 96: hipLaunchKernelGGL((gn_backward_kernel<__bf16, 96>), grid, dim3(MT_THREADS), 0, st, o32, dO, p.gamma, p.beta, p.lambda, dOw, part_g, part_b, part_l, p.T, p.M); break;
      default: hipLaunchKernelGGL((gn_backward_kernel<__bf16, 128>), grid, dim3(MT_THREADS), 0, st, o32, dO, p.gamma, p.beta, p.lambda, dOw, part_g, part_b, part_l, p.T, p.M); break;
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = sum_rows(part_g, (size_t)p.B * nch, (size_t)p.M * p.d, g.dgamma, st)) != hipSuccess) return e;
    if ((e = sum_rows(part_b, (size_t)p.B * nch, (size_t)p.M * p.d, g.dbeta, st)) != hipSuccess) return e;
    if ((e = sum_rows(part_l, (size_t)p.B * nch * p.M, 1, g.dlambda, st)) != hipSuccess) return e;
    dO = dOw;
  }

  // ---- the tile passes
  float* dq_acc = reinterpret_cast<float*>(ws + l.dq);
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((tens / 4 + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<float4*>(dq_acc), tens / 4);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwt::BwArgs a{};
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.k = reinterpret_cast<const __bf16*>(p.k);
  a.v = reinterpret_cast<const __bf16*>(p.v);
  a.dO = dO;
  a.lse = lse;
  a.dvec = reinterpret_cast<float*>(ws + l.dvec);
  a.lse_c = reinterpret_cast<float*>(ws + l.lse_c);
  a.dq_acc = dq_acc;
  a.dk = reinterpret_cast<__bf16*>(g.dk);
  a.dv = reinterpret_cast<__bf16*>(g.dv);
  a.th_pre = p.theta_pre;
  a.th_post = p.theta_post;
  a.w_pre = p.w_pre;
  a.w_post = p.w_post;
  a.part_thpre = (p.kq & KQ_PRE) ? reinterpret_cast<float*>(ws + l.thpre) : nullptr;
  a.part_thpost = (p.kq & KQ_POST) ? reinterpret_cast<float*>(ws + l.thpost) : nullptr;
  a.part_wpre = (p.mix & MIX_PRE) ? reinterpret_cast<float*>(ws + l.wpre) : nullptr;
  a.part_wpost = (p.mix & MIX_POST) ? reinterpret_cast<float*>(ws + l.wpost) : nullptr;
  a.B = p.B;
  a.T = p.T;
  a.M = p.M;
  a.G = p.M / p.c_h;
  a.scale = (float)(1.0 / __builtin_sqrt((double)p.d));
  a.n_tiles = (p.T + bwt::TB - 1) / bwt::TB;
  bwt::BwArgs ad = a, ak = a;
  const size_t lds_d = plan_tiles(p, bwt::PASS_D, ad);
  const size_t lds_k = plan_tiles(p, bwt::PASS_K, ak);
  if ((e = launch_tiles(p, ad, bwt::PASS_D, lds_d, st)) != hipSuccess) return e;
  if ((e = launch_tiles(p, ak, bwt::PASS_K, lds_k, st)) != hipSuccess) return e;
  hipLaunchKernelGGL(dq_convert_kernel, dim3((unsigned)((tens / 4 + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const float4*>(dq_acc), reinterpret_cast<uint2*>(g.dq), a.scale, tens / 4);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // ---- parameter gradients: partial sums of the key tiles, added in order
  const size_t rows = (size_t)p.B * a.n_tiles;
  const size_t th_side = (size_t)p.M * p.c_q * p.c_k, w_side = (size_t)p.M * p.c_h;
  if (p.kq & KQ_PRE)
    if ((e = sum_rows(a.part_thpre, rows, th_side, g.dtheta, st)) != hipSuccess) return e;
  if (p.kq & KQ_POST)
    if ((e = sum_rows(a.part_thpost, rows, th_side, g.dtheta + (p.kq == KQ_BOTH ? th_side : 0), st)) != hipSuccess)
      return e;
  if (p.mix & MIX_PRE)
    if ((e = sum_rows(a.part_wpre, rows, w_side, g.dw, st)) != hipSuccess) return e;
  if (p.mix & MIX_POST)
    if ((e = sum_rows(a.part_wpost, rows, w_side, g.dw + (p.mix == MIX_BOTH ? w_side : 0), st)) != hipSuccess)
      return e;
  return hipSuccess;
}

}  // namespace mta
