// Backward pass of the Multi-Token Attention layer, unfused: the forward maps are recomputed
// into the workspace with the map kernels of the forward chain, then the adjoint of every
// step runs as one kernel over fp32 [B, M, T, T] maps.
//
// Forward (page "Multi-Token Attention | Summary", greeksharifa.github.io):
//   S = Q K^T / sqrt(d)              (§2)        L = mix_pre(S)                 (§3.2)
//   C = Mask_-inf(conv_pre(Mask_0 L))  (§3.1)    P = softmax(C)                 (§2)
//   E = Mask_0(conv_post(P))           (§3.1)    A = mix_post(E)                (§3.2)
//   O = A V                            (§2)      Y = lambda (gamma xhat(O) + beta)  (§3.3)
// (absent steps are identities). Adjoint chain, given dY:
//   dO, dgamma, dbeta, dlambda        GroupNorm / gate backward per (token, head)
//   dV = A^T dO,  dA = dO V^T
//   dE = mix_post^T(dA),              dw_post[u][u'] = sum dA_u . E_u'
//   dP = conv_post^T(Mask_0 dE),      dtheta_post[a][e] = sum (Mask_0 dE)[i][j] P[i-a][j-e+h0]
//   dC = P (dP - rowsum(dP P))        (softmax backward; zero above the diagonal)
//   dL = Mask_0(conv_pre^T(dC)),      dtheta_pre[a][e] = sum dC[i][j] (Mask_0 L)[i-a][j-e+h0]
//   dS = mix_pre^T(dL),               dw_pre[u][u'] = sum dL_u . S_u'
//   dQ = dS K / sqrt(d),  dK = dS^T Q / sqrt(d)
// conv^T is the adjoint convolution: (conv^T G)[r][s] = sum_{a,e} theta[a][e] G[r+a][s+e-h0].
// Parameter gradients are reduced deterministically: every workgroup writes its partial sums,
// a second kernel adds them in a fixed order.
#include <algorithm>
#include <utility>

#include "mta_backward.h"
#include "mta_bwd_common.h"
#include "mta_map_kernels.h"

namespace mta {
namespace {

// ---- out[j][c] = scale * sum_i Map[i][j] X[i][c] (Map^T X; Map is zero for i < j) --------------
// fp32 tensors (VALU): 64 output rows j of one (b, m) per workgroup; thread (j, channel quarter). Chunks of 32 map rows
// and the matching rows of X are staged in LDS.
template <typename T, int D>
__global__ __launch_bounds__(MT_THREADS) void mapT_mat_kernel(const float* __restrict__ Map, const T* __restrict__ X,
                                                             T* __restrict__ out, float scale, int Tn, int M) {
  constexpr int JT = 64, IC = 32, CPT = D / 4, LDX = D + 4;
  __shared__ __attribute__((aligned(16))) float Ms[IC * JT];
  __shared__ __attribute__((aligned(16))) float Xs[IC * LDX];
  const int bm = blockIdx.y, b = bm / M, m = bm % M;
  const int j0 = blockIdx.x * JT;
  const int tj = threadIdx.x & 63, cg = threadIdx.x >> 6;
  const int ld = map_ld(Tn);
  const T* xb = X + (size_t)b * Tn * M * D;
  float acc[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) acc[c] = 0.0f;
  for (int i0 = j0; i0 < Tn; i0 += IC) {
    __syncthreads();
    for (int x = threadIdx.x; x < IC * JT / 4; x += MT_THREADS) {
      const int r = x / (JT / 4), c4 = (x % (JT / 4)) * 4;
      const int i = i0 + r, j = j0 + c4;
      float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < Tn && j < ld) val = *reinterpret_cast<const float4*>(Map + map_index(bm, Tn, i, j));
      *reinterpret_cast<float4*>(Ms + r * JT + c4) = val;
    }
    for (int x = threadIdx.x; x < IC * D; x += MT_THREADS) {
      const int r = x / D, c = x % D;
      const int i = i0 + r;
      Xs[r * LDX + c] = i < Tn ? (float)xb[((size_t)i * M + m) * D + c] : 0.0f;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < IC; ++r) {
      const float mv = Ms[r * JT + tj];
#pragma unroll
      for (int c = 0; c < CPT; c += 4) {
        const float4 xv = *reinterpret_cast<const float4*>(Xs + r * LDX + cg * CPT + c);
        acc[c + 0] += mv * xv.x;
        acc[c + 1] += mv * xv.y;
        acc[c + 2] += mv * xv.z;
        acc[c + 3] += mv * xv.w;
      }
    }
  }
  const int j = j0 + tj;
  if (j < Tn) {
    T* dst = out + ((size_t)b * Tn + j) * M * D + (size_t)m * D + cg * CPT;
#pragma unroll
    for (int c = 0; c < CPT; ++c) dst[c] = T(acc[c] * scale);
  }
}

// ---- the same product for bf16 tensors on MFMA: out^T = X^T Map ------------------------------
// 128 output rows j per workgroup (32 per wave). Per chunk of 32 map rows i, the map chunk
// (fp32 -> bf16) and the X chunk are staged row-major in LDS, and both MFMA operands are read
// transposed (ds_read_b64_tr_b16) with the same k-slot order: chunk rows 4g..4g+3 and
// 16+4g..16+4g+3 for lane group g.
template <int D>
__global__ __launch_bounds__(MT_THREADS) void mapT_mat_bf16_kernel(const float* __restrict__ Map,
                                                                  const __bf16* __restrict__ X,
                                                                  __bf16* __restrict__ out, float scale, int Tn,
                                                                  int M) {
  constexpr int JT = 128, IC = 32, NB = D / 16;
  constexpr int LDX = D + 16, LDM = JT + 16;
  constexpr int NML = IC * JT / 4 / MT_THREADS;                        // float4 of the map chunk per thread
  constexpr int NXC = IC * D / 8;                                      // 16-byte pieces of the X chunk
  constexpr int NXL = (NXC + MT_THREADS - 1) / MT_THREADS;
  static_assert(IC * JT / 4 % MT_THREADS == 0, "map chunk split");
  __shared__ __attribute__((aligned(16))) __bf16 Xs[IC * LDX];
  __shared__ __attribute__((aligned(16))) __bf16 Ms[IC * LDM];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lq = lane & 15, lg = lane >> 4;
  const int bm = blockIdx.y, b = bm / M, m = bm % M;
  const int j0 = blockIdx.x * JT, jw = wave * 32;
  const int ld = map_ld(Tn);
  const __bf16* xb = X + (size_t)b * Tn * M * D;
  f32x4 acc[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb][0] = acc[nb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i0 = j0; i0 < Tn; i0 += IC) {
    float4 mv[NML];
    uint4 xv[NXL];
#pragma unroll
    for (int u = 0; u < NML; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      const int r = x / (JT / 4), c4 = (x % (JT / 4)) * 4;
      const int i = i0 + r, j = j0 + c4;
      mv[u] = (i < Tn && j < ld) ? *reinterpret_cast<const float4*>(Map + map_index(bm, Tn, i, j))
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < NXL; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      const int r = x / (D / 8), c = x % (D / 8);
      const bool in = (x < NXC) & (i0 + r < Tn);
      xv[u] = *reinterpret_cast<const uint4*>(xb + ((size_t)(in ? i0 + r : 0) * M + m) * D + (in ? c * 8 : 0));
      if (!in) xv[u] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();  // every wave is done with the previous chunk
#pragma unroll
    for (int u = 0; u < NML; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      const int r = x / (JT / 4), c4 = (x % (JT / 4)) * 4;
      __bf16 h[4] = {(__bf16)mv[u].x, (__bf16)mv[u].y, (__bf16)mv[u].z, (__bf16)mv[u].w};
      *reinterpret_cast<uint2*>(Ms + r * LDM + c4) = *reinterpret_cast<const uint2*>(h);
    }
#pragma unroll
    for (int u = 0; u < NXL; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      if (x < NXC) *reinterpret_cast<uint4*>(Xs + (x / (D / 8)) * LDX + (x % (D / 8)) * 8) = xv[u];
    }
    __syncthreads();
    s16x4 bm8[2][2];
#pragma unroll
    for (int jb = 0; jb < 2; ++jb) {
      bm8[jb][0] = v_transposed(Ms, 4 * lg, jw + 16 * jb, LDM, lane);
      bm8[jb][1] = v_transposed(Ms, 16 + 4 * lg, jw + 16 * jb, LDM, lane);
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s16x4 a8[2] = {v_transposed(Xs, 4 * lg, nb * 16, LDX, lane), v_transposed(Xs, 16 + 4 * lg, nb * 16, LDX, lane)};
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(a8);
#pragma unroll
      for (int jb = 0; jb < 2; ++jb) {
        const bf16x8 bf = *reinterpret_cast<const bf16x8*>(bm8[jb]);
        acc[nb][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf, acc[nb][jb], 0, 0, 0);
      }
    }
  }
  // lane (lq, lg) holds out[j0 + jw + 16 jb + lq][channels 16 nb + 4 lg .. +3]
#pragma unroll
  for (int jb = 0; jb < 2; ++jb) {
    const int j = j0 + jw + 16 * jb + lq;
    if (j < Tn) {
      __bf16* dst = out + ((size_t)b * Tn + j) * M * D + (size_t)m * D;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        __bf16 h[4] = {(__bf16)(acc[nb][jb][0] * scale), (__bf16)(acc[nb][jb][1] * scale),
                       (__bf16)(acc[nb][jb][2] * scale), (__bf16)(acc[nb][jb][3] * scale)};
        *reinterpret_cast<uint2*>(dst + nb * 16 + 4 * lg) = *reinterpret_cast<const uint2*>(h);
      }
    }
  }
}

template <typename T, int D>
hipError_t launch_mapT(const float* Map, const T* X, T* out, float scale, const Problem& p, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    hipLaunchKernelGGL(mapT_mat_bf16_kernel<D>, dim3((p.T + 127) / 128, p.B * p.M), dim3(MT_THREADS), 0, st, Map, X,
                       out, scale, p.T, p.M);
  } else {
    hipLaunchKernelGGL((mapT_mat_kernel<T, D>), dim3((p.T + 63) / 64, p.B * p.M), dim3(MT_THREADS), 0, st, Map, X,
                       out, scale, p.T, p.M);
  }
  return hipGetLastError();
}

// ---- head-mixing weights transposed: wT[g][u][u'] = w[g][u'][u] ---------------------------------
__global__ void transpose_w_kernel(const float* __restrict__ w, float* __restrict__ wT, int G, int CH) {
  const int x = blockIdx.x * blockDim.x + threadIdx.x;
  if (x >= G * CH * CH) return;
  const int g = x / (CH * CH), u = (x / CH) % CH, v = x % CH;
  wT[x] = w[((size_t)g * CH + v) * CH + u];
}

constexpr int PD_CHUNKS = 64;  // blocks per (batch, group) of the mixing backward

// ---- mixing backward in one pass over a group's maps: the mixing-weight gradient partials
// (sum over the maps of G_u * E_v per block, reduced deterministically afterwards) and
// G_u <- sum_x wT[g][u][x] G_x in place (the gradient of the mixed map's input) --------------
template <int CH>
__global__ __launch_bounds__(MT_THREADS) void mix_backward_kernel(float* __restrict__ Gm, const float* __restrict__ Em,
                                                                 const float* __restrict__ wT,
                                                                 float* __restrict__ part, int M,
                                                                 size_t n4_per_map) {
  __shared__ float red[4][CH * CH];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int bg = blockIdx.y, G = M / CH, b = bg / G, g = bg % G;
  f32x4* gb = reinterpret_cast<f32x4*>(Gm) + ((size_t)b * M + (size_t)g * CH) * n4_per_map;
  const f32x4* eb = reinterpret_cast<const f32x4*>(Em) + ((size_t)b * M + (size_t)g * CH) * n4_per_map;
  float wl[CH][CH];
#pragma unroll
  for (int u = 0; u < CH; ++u)
#pragma unroll
    for (int x = 0; x < CH; ++x) wl[u][x] = wT[((size_t)g * CH + u) * CH + x];
  float acc[CH][CH];
#pragma unroll
  for (int u = 0; u < CH; ++u)
#pragma unroll
    for (int v = 0; v < CH; ++v) acc[u][v] = 0.0f;
  for (size_t e = (size_t)blockIdx.x * MT_THREADS + threadIdx.x; e < n4_per_map; e += (size_t)gridDim.x * MT_THREADS) {
    f32x4 gv[CH], ev[CH];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      gv[u] = gb[(size_t)u * n4_per_map + e];
      ev[u] = eb[(size_t)u * n4_per_map + e];
    }
#pragma unroll
    for (int u = 0; u < CH; ++u)
#pragma unroll
      for (int v = 0; v < CH; ++v) {
        const f32x4 pr = gv[u] * ev[v];
        acc[u][v] += (pr[0] + pr[1]) + (pr[2] + pr[3]);
      }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      f32x4 o = gv[0] * wl[u][0];
#pragma unroll
      for (int x = 1; x < CH; ++x) o += gv[x] * wl[u][x];
      gb[(size_t)u * n4_per_map + e] = o;
    }
  }
#pragma unroll
  for (int u = 0; u < CH; ++u)
#pragma unroll
    for (int v = 0; v < CH; ++v) {
      const float s = wave_sum(acc[u][v]);
      if (lane == 0) red[wave][u * CH + v] = s;
    }
  __syncthreads();
  if (threadIdx.x < CH * CH) {
    const int x = threadIdx.x;
    part[(((size_t)b * gridDim.x + blockIdx.x) * G + g) * CH * CH + x] = (red[0][x] + red[1][x]) + (red[2][x] + red[3][x]);
  }
}

// ---- causal softmax backward, in place: G <- P (G - sum_j G P), zero above the diagonal ---------
template <int NV>
__global__ __launch_bounds__(MT_THREADS) void softmax_bwd_kernel(const float* __restrict__ P, float* __restrict__ G,
                                                                int Tn) {
  __shared__ float red[MT_THREADS / 64];
  const size_t row = blockIdx.x;
  const int i = (int)(row % Tn);
  const int ld = map_ld(Tn);
  const float4* p = reinterpret_cast<const float4*>(P + row * ld);
  float4* g = reinterpret_cast<float4*>(G + row * ld);
  float4 pv[NV], gv[NV];
  float dot = 0.0f;
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const int j = (c * MT_THREADS + threadIdx.x) * 4;
    pv[c] = j < ld ? p[j / 4] : make_float4(0.f, 0.f, 0.f, 0.f);
    gv[c] = j < ld ? g[j / 4] : make_float4(0.f, 0.f, 0.f, 0.f);
    if (j + 0 > i) pv[c].x = 0.0f;
    if (j + 1 > i) pv[c].y = 0.0f;
    if (j + 2 > i) pv[c].z = 0.0f;
    if (j + 3 > i) pv[c].w = 0.0f;
    dot += (pv[c].x * gv[c].x + pv[c].y * gv[c].y) + (pv[c].z * gv[c].z + pv[c].w * gv[c].w);
  }
  dot = block_reduce(dot, red, false);
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const int j = (c * MT_THREADS + threadIdx.x) * 4;
    if (j < ld)
      g[j / 4] = make_float4(pv[c].x * (gv[c].x - dot), pv[c].y * (gv[c].y - dot), pv[c].z * (gv[c].z - dot),
                             pv[c].w * (gv[c].w - dot));
  }
}

__global__ __launch_bounds__(MT_THREADS) void softmax_bwd_long_kernel(const float* __restrict__ P, float* __restrict__ G,
                                                                     int Tn) {
  __shared__ float red[MT_THREADS / 64];
  const size_t row = blockIdx.x;
  const int i = (int)(row % Tn);
  const float* p = P + row * map_ld(Tn);
  float* g = G + row * map_ld(Tn);
  float dot = 0.0f;
  for (int j = threadIdx.x; j <= i; j += MT_THREADS) dot += p[j] * g[j];
  dot = block_reduce(dot, red, false);
  for (int j = threadIdx.x; j < Tn; j += MT_THREADS) g[j] = (j <= i) ? p[j] * (g[j] - dot) : 0.0f;
}

// ---- adjoint convolution on a 64 x 64 output tile ----------------------------------------------
// Y[r][s] = sum_{a,e} theta[a][e] G0[r+a][s+e-h0] with G0 = G where 0 <= j <= i < T, else 0 (the
// masks that followed the forward convolution); Y is written zero above the diagonal. The input
// tile spans rows r0 .. r0+63+c_q-1 and columns s0-16 .. s0+79.
template <int CK>
__global__ __launch_bounds__(MT_THREADS) void conv_adjoint_kernel(const float* __restrict__ G, float* __restrict__ Y,
                                                                 const float* __restrict__ theta, int Tn, int M,
                                                                 int c_q) {
  constexpr int H0 = (CK - 1) / 2;
  constexpr int TW = 64 + 32;
  constexpr int LD = TW + 4;
  __shared__ __attribute__((aligned(16))) float tile[(64 + 7) * LD];
  __shared__ float th[8 * CK];
  const uint3 tl = xcd_tile();
  const int bm = tl.z, m = bm % M;
  const int r0 = tl.y * 64, s0 = tl.x * 64;
  const int ld = map_ld(Tn);
  const int orow = threadIdx.x >> 2, oc0 = (threadIdx.x & 3) * 16;
  if (s0 > r0 + 63) {  // above the diagonal: zero
    const int r = r0 + orow;
    if (r < Tn)
#pragma unroll
      for (int v4 = 0; v4 < 4; ++v4) {
        const int s = s0 + oc0 + 4 * v4;
        if (s < ld) *reinterpret_cast<float4*>(Y + map_index(bm, Tn, r, s)) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    return;
  }
  const int rows = 64 + c_q - 1;
  for (int x = threadIdx.x; x < c_q * CK; x += MT_THREADS) th[x] = theta[(size_t)m * c_q * CK + x];
  constexpr int NL = ((64 + 7) * (TW / 4) + MT_THREADS - 1) / MT_THREADS;
  float4 buf[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int x = threadIdx.x + u * MT_THREADS;
    const int rr = x / (TW / 4), c4 = (x % (TW / 4)) * 4;
    const int i = r0 + rr, j = s0 - 16 + c4;
    const bool in = (x < rows * (TW / 4)) & (i < Tn) & (j >= 0) & (j < ld);
    buf[u] = *reinterpret_cast<const float4*>(G + map_index(bm, Tn, in ? i : 0, in ? j : 0));
    const int lim = min(i, Tn - 1);
    buf[u].x = (in & (j + 0 <= lim)) ? buf[u].x : 0.0f;
    buf[u].y = (in & (j + 1 <= lim)) ? buf[u].y : 0.0f;
    buf[u].z = (in & (j + 2 <= lim)) ? buf[u].z : 0.0f;
    buf[u].w = (in & (j + 3 <= lim)) ? buf[u].w : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int x = threadIdx.x + u * MT_THREADS;
    if (x < rows * (TW / 4)) *reinterpret_cast<float4*>(tile + (x / (TW / 4)) * LD + (x % (TW / 4)) * 4) = buf[u];
  }
  __syncthreads();
  float acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = 0.0f;
  for (int a = 0; a < c_q; ++a) {
    // output (orow, oc0 + c) reads tile row orow + a, tile column oc0 + 16 + c + e - H0
    const float* src = tile + (orow + a) * LD + oc0 + 16 - H0;
    float seg[16 + CK - 1];
#pragma unroll
    for (int x = 0; x < 16 + CK - 1; ++x) seg[x] = src[x];
#pragma unroll
    for (int e = 0; e < CK; ++e) {
      const float t = th[a * CK + e];
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] += t * seg[c + e];
    }
  }
  const int r = r0 + orow;
  if (r < Tn) {
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int s = s0 + oc0 + 4 * v4;
      if (s < ld) {
        float4 o;
        o.x = (s + 0 > r) ? 0.0f : acc[4 * v4 + 0];
        o.y = (s + 1 > r) ? 0.0f : acc[4 * v4 + 1];
        o.z = (s + 2 > r) ? 0.0f : acc[4 * v4 + 2];
        o.w = (s + 3 > r) ? 0.0f : acc[4 * v4 + 3];
        *reinterpret_cast<float4*>(Y + map_index(bm, Tn, r, s)) = o;
      }
    }
  }
}

// ---- kernel-weight gradient partials over one 64-row strip of the output gradient ------------
// part[a][e] = sum_{(i,j) in strip} G0[i][j] In0[i-a][j-e+h0], G0 as in conv_adjoint_kernel; In0
// is the forward convolution's input: Mask_0 of the logits before softmax (PRE), the softmax
// weights after it, zero outside the map. The workgroup walks the strip's 64 x 64 tiles on and
// below the diagonal (the gradient is zero above it), staging In like conv_kernel, and keeps
// the c_q x c_k sums in registers; heavy strips (near the end of the sequence) start first.
template <int CK, bool PRE>
__global__ __launch_bounds__(MT_THREADS) void conv_dtheta_kernel(const float* __restrict__ G,
                                                                const float* __restrict__ In,
                                                                float* __restrict__ part, int Tn, int M, int c_q) {
  constexpr int H0 = (CK - 1) / 2;
  constexpr int TW = 64 + 32;
  constexpr int LD = TW + 4;
  __shared__ __attribute__((aligned(16))) float tile[(64 + 7) * LD];
  __shared__ float red[4][8 * CK];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nty = gridDim.x, ty = nty - 1 - blockIdx.x, bm = blockIdx.y, b = bm / M, m = bm % M;
  const int i0 = ty * 64;
  const int ld = map_ld(Tn);
  const int rows = 64 + c_q - 1;
  const int orow = threadIdx.x >> 2, oc0 = (threadIdx.x & 3) * 16;
  const int i = i0 + orow;
  constexpr int NL = ((64 + 7) * (TW / 4) + MT_THREADS - 1) / MT_THREADS;
  float acc[8][CK];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int e = 0; e < CK; ++e) acc[a][e] = 0.0f;
  for (int tx = 0; tx <= ty; ++tx) {
    const int j0 = tx * 64;
    float4 buf[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      const int rr = x / (TW / 4), c4 = (x % (TW / 4)) * 4;
      const int r = i0 - (c_q - 1) + rr, s = j0 - 16 + c4;
      const bool in = (x < rows * (TW / 4)) & (r >= 0) & (r < Tn) & (s >= 0) & (s < ld);
      buf[u] = *reinterpret_cast<const float4*>(In + map_index(bm, Tn, in ? r : 0, in ? s : 0));
      const int lim = PRE ? min(r, Tn - 1) : Tn - 1;
      buf[u].x = (in & (s + 0 <= lim)) ? buf[u].x : 0.0f;
      buf[u].y = (in & (s + 1 <= lim)) ? buf[u].y : 0.0f;
      buf[u].z = (in & (s + 2 <= lim)) ? buf[u].z : 0.0f;
      buf[u].w = (in & (s + 3 <= lim)) ? buf[u].w : 0.0f;
    }
    // this thread's 16 gradient values (row i, columns j0 + oc0 ..), masked
    float g[16];
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int j = j0 + oc0 + 4 * v4;
      float4 gv = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < Tn && j < ld) gv = *reinterpret_cast<const float4*>(G + map_index(bm, Tn, i, j));
      g[4 * v4 + 0] = (i < Tn && j + 0 <= i) ? gv.x : 0.0f;
      g[4 * v4 + 1] = (i < Tn && j + 1 <= i) ? gv.y : 0.0f;
      g[4 * v4 + 2] = (i < Tn && j + 2 <= i) ? gv.z : 0.0f;
      g[4 * v4 + 3] = (i < Tn && j + 3 <= i) ? gv.w : 0.0f;
    }
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      if (x < rows * (TW / 4)) *reinterpret_cast<float4*>(tile + (x / (TW / 4)) * LD + (x % (TW / 4)) * 4) = buf[u];
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      if (a < c_q) {
        // In0[i-a][j-e+h0] sits at tile row orow + c_q - 1 - a, column oc0 + c + 16 - e + H0
        const float* src = tile + (orow + c_q - 1 - a) * LD + oc0 + 16 - H0;
        float seg[16 + CK - 1];
#pragma unroll
        for (int x = 0; x < 16 + CK - 1; ++x) seg[x] = src[x];
#pragma unroll
        for (int e = 0; e < CK; ++e) {
          float s = 0.0f;
#pragma unroll
          for (int c = 0; c < 16; ++c) s += g[c] * seg[c - e + 2 * H0];
          acc[a][e] += s;
        }
      }
    }
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    if (a < c_q) {
#pragma unroll
      for (int e = 0; e < CK; ++e) {
        const float s = wave_sum(acc[a][e]);
        if (lane == 0) red[wave][a * CK + e] = s;
      }
    }
  }
  __syncthreads();
  float* dst = part + (((size_t)b * nty + ty) * M + m) * c_q * CK;
  for (int x = threadIdx.x; x < c_q * CK; x += MT_THREADS) dst[x] = (red[0][x] + red[1][x]) + (red[2][x] + red[3][x]);
}

template <int CK>
hipError_t launch_dtheta_ck(bool pre, const float* G, const float* In, float* part, const Problem& p, hipStream_t st) {
  const dim3 grid((p.T + 63) / 64, p.B * p.M);
  if (pre)
    hipLaunchKernelGGL((conv_dtheta_kernel<CK, true>), grid, dim3(MT_THREADS), 0, st, G, In, part, p.T, p.M, p.c_q);
  else
    hipLaunchKernelGGL((conv_dtheta_kernel<CK, false>), grid, dim3(MT_THREADS), 0, st, G, In, part, p.T, p.M, p.c_q);
  return hipGetLastError();
}

template <int CK>
hipError_t launch_adjoint_ck(const float* G, float* Y, const float* theta, const Problem& p, hipStream_t st) {
  const dim3 grid((p.T + 63) / 64, (p.T + 63) / 64, p.B * p.M);
  hipLaunchKernelGGL(conv_adjoint_kernel<CK>, grid, dim3(MT_THREADS), 0, st, G, Y, theta, p.T, p.M, p.c_q);
  return hipGetLastError();
}

// The gradient of one convolution: dtheta (reduced into dtheta_out) and the adjoint map.
hipError_t conv_backward(bool pre, const float* G, const float* In, float* Y, const float* theta, float* part,
                         float* dtheta_out, const Problem& p, hipStream_t st) {
  hipError_t e = hipErrorInvalidValue;
  switch (p.c_k) {
#define MTA_CK(CKV)                                                                         \
  case CKV:                                                                                 \
    if ((e = launch_dtheta_ck<CKV>(pre, G, In, part, p, st)) != hipSuccess) return e;       \
    e = launch_adjoint_ck<CKV>(G, Y, theta, p, st);                                         \
    break;
    MTA_CK(1) MTA_CK(3) MTA_CK(5) MTA_CK(7) MTA_CK(9) MTA_CK(11) MTA_CK(13) MTA_CK(15) MTA_CK(17)
#undef MTA_CK
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const size_t nstrips = (size_t)(p.T + 63) / 64;
  return sum_rows(part, (size_t)p.B * nstrips, (size_t)p.M * p.c_q * p.c_k, dtheta_out, st);
}

hipError_t launch_softmax_bwd(const float* P, float* G, const Problem& p, hipStream_t st) {
  const dim3 grid((unsigned)((size_t)p.B * p.M * p.T));
  const int nv = (map_ld(p.T) / 4 + MT_THREADS - 1) / MT_THREADS;
  if (nv <= 1) hipLaunchKernelGGL(softmax_bwd_kernel<1>, grid, dim3(MT_THREADS), 0, st, P, G, p.T);
  else if (nv <= 2) hipLaunchKernelGGL(softmax_bwd_kernel<2>, grid, dim3(MT_THREADS), 0, st, P, G, p.T);
  else if (nv <= 4) hipLaunchKernelGGL(softmax_bwd_kernel<4>, grid, dim3(MT_THREADS), 0, st, P, G, p.T);
  else if (nv <= 8) hipLaunchKernelGGL(softmax_bwd_kernel<8>, grid, dim3(MT_THREADS), 0, st, P, G, p.T);
  else if (nv <= 16) hipLaunchKernelGGL(softmax_bwd_kernel<16>, grid, dim3(MT_THREADS), 0, st, P, G, p.T);
  else hipLaunchKernelGGL(softmax_bwd_long_kernel, grid, dim3(MT_THREADS), 0, st, P, G, p.T);
  return hipGetLastError();
}

// The gradient of one head mixing in one pass over the maps: dw (reduced into dw_out) and
// G <- mix with w^T, in place.
hipError_t mix_backward(float* G, const float* In, const float* w, float* wT, float* part, float* dw_out,
                        const Problem& p, hipStream_t st) {
  const int CH = p.c_h, NG = p.M / CH;
  const size_t n4 = (size_t)p.T * map_ld(p.T) / 4;
  const dim3 grid(PD_CHUNKS, p.B * NG);
  const int n = NG * CH * CH;
  hipLaunchKernelGGL(transpose_w_kernel, dim3((n + 255) / 256), dim3(256), 0, st, w, wT, NG, CH);
  hipError_t e;
  if ((e = hipGetLastError()) != hipSuccess) return e;
  switch (CH) {
    case 1: hipLaunchKernelGGL(mix_backward_kernel<1>, grid, dim3(MT_THREADS), 0, st, G, In, wT, part, p.M, n4); break;
    case 2: hipLaunchKernelGGL(mix_backward_kernel<2>, grid, dim3(MT_THREADS), 0, st, G, In, wT, part, p.M, n4); break;
    case 4: hipLaunchKernelGGL(mix_backward_kernel<4>, grid, dim3(MT_THREADS), 0, st, G, In, wT, part, p.M, n4); break;
    default: return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return sum_rows(part, (size_t)p.B * PD_CHUNKS, (size_t)NG * CH * CH, dw_out, st);
}

// ---- workspace layout ------------------------------------------------------------------------
struct BwdLayout {
  size_t S, L, P, E, A, G, G2;  // maps (equal offsets alias)
  size_t O, dO, wT, part;       // O fp32 [B,T,M,d]; dO input dtype; wT [c_h^2 M / c_h]; partial sums
  size_t total;
};

BwdLayout bwd_layout(const Problem& p) {
  BwdLayout l{};
  const size_t map = (size_t)p.B * p.M * p.T * map_ld(p.T) * sizeof(float);
  const size_t tens = (size_t)p.B * p.T * p.M * p.d;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  l.S = take(map);
  l.L = (p.mix & MIX_PRE) ? take(map) : l.S;
  l.P = take(map);
  l.E = (p.kq & KQ_POST) ? take(map) : l.P;
  l.A = (p.mix & MIX_POST) ? take(map) : l.E;
  l.G = take(map);
  l.G2 = take(map);
  l.O = take(p.gn ? tens * sizeof(float) : 0);
  l.dO = take(p.gn ? tens * (p.fp32 ? 4 : 2) : 0);
  l.wT = take((size_t)p.M * p.c_h * sizeof(float));
  const size_t nstrips = (size_t)(p.T + 63) / 64;
  const size_t nch = (size_t)(p.T + GN_RB - 1) / GN_RB;
  size_t part = 0;
  if (p.kq) part = std::max(part, (size_t)p.B * nstrips * p.M * p.c_q * p.c_k);
  if (p.mix) part = std::max(part, (size_t)p.B * PD_CHUNKS * p.M * p.c_h);
  if (p.gn) part = std::max(part, 2 * (size_t)p.B * nch * p.M * p.d + (size_t)p.B * nch * p.M);
  l.part = take(part * sizeof(float));
  l.total = off;
  return l;
}

template <typename T, int D>
hipError_t run_backward(const Problem& p, const BwdGrads& g, char* ws, hipStream_t st) {
  const BwdLayout l = bwd_layout(p);
  auto map = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };
  float *mS = map(l.S), *mL = map(l.L), *mP = map(l.P), *mE = map(l.E), *mA = map(l.A);
  float *G = map(l.G), *G2 = map(l.G2);
  float* part = map(l.part);
  float* wT = map(l.wT);
  const T* q = reinterpret_cast<const T*>(p.q);
  const T* k = reinterpret_cast<const T*>(p.k);
  const T* v = reinterpret_cast<const T*>(p.v);
  const float scale = (float)(1.0 / __builtin_sqrt((double)p.d));
  hipError_t e;
  const dim3 lgrid((p.T + 127) / 128, (p.T + 127) / 128, p.B * p.M);

  // ---- forward maps
  hipLaunchKernelGGL((logits_kernel<T, D>), lgrid, dim3(MT_THREADS), 0, st, q, k, mS, p.T, p.M, scale);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((p.mix & MIX_PRE) && (e = launch_mix(mL, p.w_pre, p, st, mS)) != hipSuccess) return e;
  if (p.kq & KQ_PRE) {
    if ((e = launch_conv(true, mL, mP, p, st)) != hipSuccess) return e;
    if ((e = launch_softmax(mP, p, st)) != hipSuccess) return e;
  } else {
    if ((e = launch_softmax(mP, p, st, mL)) != hipSuccess) return e;
  }
  if ((p.kq & KQ_POST) && (e = launch_conv(false, mP, mE, p, st)) != hipSuccess) return e;
  if ((p.mix & MIX_POST) && (e = launch_mix(mA, p.w_post, p, st, mE)) != hipSuccess) return e;

  // ---- GroupNorm / gate backward -> dO
  const T* dO = reinterpret_cast<const T*>(g.dout);
  if (p.gn) {
    float* O = map(l.O);
    T* dOw = reinterpret_cast<T*>(ws + l.dO);
    if ((e = launch_av_to<T, D, float>(mA, v, O, nullptr, nullptr, 0.0f, 0, 1.0f, p.B, p.T, p.M, st)) != hipSuccess)
      return e;
    const int nch = (p.T + GN_RB - 1) / GN_RB;
    float* part_g = part;
    float* part_b = part + (size_t)p.B * nch * p.M * D;
    float* part_l = part_b + (size_t)p.B * nch * p.M * D;
    hipLaunchKernelGGL((gn_backward_kernel<T, D>), dim3(nch, p.B * p.M), dim3(MT_THREADS), 0, st, O, dO, p.gamma,
                       p.beta, p.lambda, dOw, part_g, part_b, part_l, p.T, p.M);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = sum_rows(part_g, (size_t)p.B * nch, (size_t)p.M * D, g.dgamma, st)) != hipSuccess) return e;
    if ((e = sum_rows(part_b, (size_t)p.B * nch, (size_t)p.M * D, g.dbeta, st)) != hipSuccess) return e;
    if ((e = sum_rows(part_l, (size_t)p.B * nch * p.M, 1, g.dlambda, st)) != hipSuccess) return e;
    dO = dOw;
  }

  // ---- dV = A^T dO, dA = dO V^T
  if ((e = launch_mapT<T, D>(mA, dO, reinterpret_cast<T*>(g.dv), 1.0f, p, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((logits_kernel<T, D>), lgrid, dim3(MT_THREADS), 0, st, dO, v, G, p.T, p.M, 1.0f);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  // ---- after softmax: mixing, then the convolution
  const size_t w_side = (size_t)p.M * p.c_h;                 // floats of one side's mixing weights
  const size_t th_side = (size_t)p.M * p.c_q * p.c_k;        // floats of one side's kernels
  float* dw_post = g.dw + ((p.mix == MIX_BOTH) ? w_side : 0);
  float* dth_post = g.dtheta + ((p.kq == KQ_BOTH) ? th_side : 0);
  if ((p.mix & MIX_POST) && (e = mix_backward(G, mE, p.w_post, wT, part, dw_post, p, st)) != hipSuccess) return e;
  if (p.kq & KQ_POST) {
    if ((e = conv_backward(false, G, mP, G2, p.theta_post, part, dth_post, p, st)) != hipSuccess) return e;
    std::swap(G, G2);
  }
  // ---- softmax, then before softmax: the convolution, then mixing
  if ((e = launch_softmax_bwd(mP, G, p, st)) != hipSuccess) return e;
  if (p.kq & KQ_PRE) {
    if ((e = conv_backward(true, G, mL, G2, p.theta_pre, part, g.dtheta, p, st)) != hipSuccess) return e;
    std::swap(G, G2);
  }
  if ((p.mix & MIX_PRE) && (e = mix_backward(G, mS, p.w_pre, wT, part, g.dw, p, st)) != hipSuccess) return e;

  // ---- dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d)
  if ((e = launch_av_to<T, D, T>(G, k, reinterpret_cast<T*>(g.dq), nullptr, nullptr, 0.0f, 0, scale, p.B, p.T, p.M,
                                 st)) != hipSuccess)
    return e;
  return launch_mapT<T, D>(G, q, reinterpret_cast<T*>(g.dk), scale, p, st);
}

}  // namespace

size_t backward_workspace_bytes(const Problem& p) { return bwd_layout(p).total; }

bool backward_supported(const Problem& p) { return materialized_supported(p); }

hipError_t launch_backward(const Problem& p, const BwdGrads& g, void* workspace, hipStream_t st, bool* unsupported) {
  *unsupported = false;
  if (!backward_supported(p)) {
    *unsupported = true;
    return hipSuccess;
  }
  char* ws = reinterpret_cast<char*>(workspace);
  if (p.fp32) {
    switch (p.d) {
      case 16: return run_backward<float, 16>(p, g, ws, st);
      case 32: return run_backward<float, 32>(p, g, ws, st);
      case 64: return run_backward<float, 64>(p, g, ws, st);
    }
  } else {
    switch (p.d) {
      case 32: return run_backward<__bf16, 32>(p, g, ws, st);
      case 64: return run_backward<__bf16, 64>(p, g, ws, st);
      case 96: return run_backward<__bf16, 96>(p, g, ws, st);
      case 128: return run_backward<__bf16, 128>(p, g, ws, st);
    }
  }
  *unsupported = true;
  return hipSuccess;
}

}  // namespace mta
