// Pieces shared by the two backward passes (mta_backward.hip, materialized; mta_bwd_fused.hip,
// fused): the GroupNorm / gate backward and a fixed-order sum of partial results.
#pragma once

#include <hip/hip_runtime.h>

#include "mta_map_kernels.h"

namespace mta {
namespace {

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// ---- GroupNorm + gate backward, one wave per (b, token, head) row ----------------------------
// xhat = (O - mean) / sqrt(var + eps); Y = lambda (gamma xhat + beta). With g = lambda gamma dY:
// dO = (g - mean(g) - xhat mean(g xhat)) / sqrt(var + eps). Partial sums of dgamma, dbeta
// (over the rows of the block) and dlambda go to part_*.
constexpr int GN_RB = 64;  // rows of one (b, m) per workgroup

template <typename T, int D>
__global__ __launch_bounds__(MT_THREADS) void gn_backward_kernel(const float* __restrict__ O, const T* __restrict__ dY,
                                                                const float* __restrict__ gamma,
                                                                const float* __restrict__ beta, float lambda,
                                                                T* __restrict__ dO, float* __restrict__ part_g,
                                                                float* __restrict__ part_b, float* __restrict__ part_l,
                                                                int Tn, int M) {
  constexpr int CPL = (D + 63) / 64;  // channels per lane
  __shared__ float red[4][2 * D + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bm = blockIdx.y, b = bm / M, m = bm % M;
  const int chunk = blockIdx.x, nch = gridDim.x;
  const int i0 = chunk * GN_RB;
  float gam[CPL], bet[CPL], pg[CPL], pb[CPL];
  float pl = 0.0f;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c = lane + 64 * k;
    gam[k] = c < D ? gamma[(size_t)m * D + c] : 0.0f;
    bet[k] = c < D ? beta[(size_t)m * D + c] : 0.0f;
    pg[k] = pb[k] = 0.0f;
  }
  for (int r = wave; r < GN_RB; r += 4) {
    const int i = i0 + r;
    if (i >= Tn) break;
    const size_t row = ((size_t)b * Tn + i) * M + m;
    float o[CPL], dy[CPL];
    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane + 64 * k;
      o[k] = c < D ? O[row * D + c] : 0.0f;
      dy[k] = c < D ? (float)dY[row * D + c] : 0.0f;
      s += o[k];
    }
    const float mean = wave_sum(s) * (1.0f / D);
    float sq = 0.0f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane + 64 * k;
      const float dv = c < D ? o[k] - mean : 0.0f;
      sq += dv * dv;
    }
    const float rs = 1.0f / sqrtf(wave_sum(sq) * (1.0f / D) + 1e-5f);
    float xh[CPL], g[CPL], sg = 0.0f, sgx = 0.0f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane + 64 * k;
      xh[k] = c < D ? (o[k] - mean) * rs : 0.0f;
      pl += dy[k] * (gam[k] * xh[k] + bet[k]);
      pg[k] += lambda * dy[k] * xh[k];
      pb[k] += lambda * dy[k];
      g[k] = lambda * gam[k] * dy[k];
      sg += g[k];
      sgx += g[k] * xh[k];
    }
    const float mg = wave_sum(sg) * (1.0f / D), mgx = wave_sum(sgx) * (1.0f / D);
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const int c = lane + 64 * k;
      if (c < D) dO[row * D + c] = T((g[k] - mg - xh[k] * mgx) * rs);
    }
  }
  // per-channel partials over the four waves, the gate partial over the workgroup
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c = lane + 64 * k;
    if (c < D) {
      red[wave][c] = pg[k];
      red[wave][D + c] = pb[k];
    }
  }
  pl = wave_sum(pl);
  if (lane == 0) red[wave][2 * D] = pl;
  __syncthreads();
  const size_t prow = (size_t)b * nch + chunk;
  for (int x = threadIdx.x; x < 2 * D; x += MT_THREADS) {
    const float v = (red[0][x] + red[1][x]) + (red[2][x] + red[3][x]);
    if (x < D) part_g[(prow * M + m) * D + x] = v;
    else part_b[(prow * M + m) * D + (x - D)] = v;
  }
  if (threadIdx.x == 0) part_l[prow * M + m] = (red[0][2 * D] + red[1][2 * D]) + (red[2][2 * D] + red[3][2 * D]);
}

// ---- out[k] = sum_r part[r * K + k] in a fixed order ---------------------------------------------
// A workgroup owns SR_W columns (fewer where K is smaller); its SR_THREADS / W row groups each add
// every (SR_THREADS / W)-th row in order, and a fixed pairwise tree adds the groups: the result
// does not depend on timing, so repeated calls agree bit for bit.
constexpr int SR_THREADS = 256;
constexpr int SR_W = 16;

__global__ __launch_bounds__(SR_THREADS) void sum_rows_kernel(const float* __restrict__ part, size_t R, size_t K,
                                                              int W, float* __restrict__ out) {
  __shared__ float red[SR_THREADS];
  const int t = threadIdx.x, ng = SR_THREADS / W, rg = t / W;
  const size_t k = (size_t)blockIdx.x * W + t % W;
  float s = 0.0f;
  if (k < K)
    for (size_t r = rg; r < R; r += ng) s += part[r * K + k];
  red[t] = s;
  __syncthreads();
  for (int h = ng / 2; h > 0; h >>= 1) {
    if (rg < h) red[t] += red[t + h * W];
    __syncthreads();
  }
  if (rg == 0 && k < K) out[k] = red[t];
}

hipError_t sum_rows(const float* part, size_t R, size_t K, float* out, hipStream_t st) {
  if (K == 0) return hipSuccess;
  int W = 1;
  while (W < SR_W && (size_t)W < K) W *= 2;
  hipLaunchKernelGGL(sum_rows_kernel, dim3((unsigned)((K + W - 1) / W)), dim3(SR_THREADS), 0, st, part, R, K, W, out);
  return hipGetLastError();
}

}  // namespace
}  // namespace mta
