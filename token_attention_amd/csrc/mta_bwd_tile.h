// Fused backward of the Multi-Token Attention layer: the T x T maps are recomputed tile by
// tile in LDS and never stored. Forward (page "Multi-Token Attention | Summary",
// greeksharifa.github.io, §2, §3.1, §3.2):
//   S = Q K^T / sqrt(d)   L = mix_pre(S)   Z = Mask_0(L)   C = conv_pre(Z)
//   P = softmax(Mask_-inf(C))   E = Mask_0(conv_post(P))   A = mix_post(E)   O = A V
// (absent steps are identities; conv(X)[i][j] = sum_{a,e} theta[a][e] X[i-a][j-e+h0]).
// Adjoint, given dO:
//   dA = dO V^T   dw_post[u][u'] = sum dA_u E_u'   dE_u' = sum_u w_post[u][u'] dA_u
//   dP = conv_post^T(Mask_0 dE)   dtheta_post[a][e] = sum (Mask_0 dE)[i][j] P[i-a][j-e+h0]
//   dC = P (dP - D),  D_i = sum_j P[i][j] dP[i][j]
//   dL = Mask_0(conv_pre^T(dC))   dtheta_pre[a][e] = sum dC[i][j] Z[i-a][j-e+h0]
//   dw_pre[u][u'] = sum dL_u S_u'   dS_u' = sum_u w_pre[u][u'] dL_u
//   dQ = dS K / sqrt(d)   dK = dS^T Q / sqrt(d)   dV = A^T dO
// with conv^T(G)[r][s] = sum_{a,e} theta[a][e] G[r+a][s+e-h0].
//
// Two passes over 16 x 16 tiles of one (batch, head group), every head of the group in one
// workgroup (the mixing couples them position by position):
//   PASS_D  one workgroup per 16 query rows, a sweep over the key tiles: D_i.
//   PASS_K  one workgroup per 16 keys, a sweep over the query tiles: dK and dV of its keys in
//           registers, dQ added to an fp32 buffer with atomics, and partial sums of the
//           parameter gradients.
// The softmax is rebuilt from the forward's per-row log-sum-exp: P = exp(C - lse). PASS_D also
// sums each row of that P (the forward reached its lse through fp16-rounded logits, so the sum
// is 1 only to about 1e-4) and hands PASS_K lse + log(sum) and D / sum: the normalisation then
// matches this recomputation to fp32 rounding, which a row with one key (exact gradient zero)
// needs. A tile
// step recomputes each map on the region its adjoint needs (the core 16 x 16 tile grown by the
// convolutions' reach): S = QK^T and dA = dO V^T on MFMA (bf16 operands read from global
// memory), the masks, mixing, convolutions and softmax gradient in fp32 on the VALU from LDS.
#pragma once

#include <hip/hip_runtime.h>

#include "mta_device.h"
#include "mta_internal.h"

namespace mta {
namespace bwt {

constexpr int TB = 16;           // core tile: TB query rows x TB keys
constexpr int NTH = 512;         // threads per workgroup
constexpr int CKM = 17;          // largest key extent of a convolution
constexpr int NRQ = 4;           // the rows of a parameter-gradient task split in NRQ groups
constexpr int MAXR = 5;          // rounds of those tasks per thread: 5 * NTH >= 4 * 8 * 17 * NRQ
enum { PASS_D = 0, PASS_K = 1 };

typedef short s16x4 __attribute__((ext_vector_type(4)));

// A rectangle of a map, relative to the tile origin (i0, j0).
struct Reg {
  int r0, c0, nr, nc;
};
// Storage of a map in LDS: rows from r0 and columns from c0 (tile-relative), leading
// dimension ld, head stride hs, offset off (floats). Maps that alias share one storage.
struct Geo {
  int r0, c0, ld, hs, off;
};

struct BwArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dO;      // [B,T,M,D] gradient of the output before GroupNorm
  const float* lse;      // [B,T,M] natural log-sum-exp of every softmax row (forward)
  float* lse_c;          // [B,T,M] the same, renormalised to this recomputation (PASS_D writes)
  float* dvec;           // [B,T,M] D_i (PASS_D writes, PASS_K reads)
  float* dq_acc;         // [B,T,M,D] fp32, accumulated with atomics (PASS_K)
  __bf16* dk;            // [B,T,M,D]
  __bf16* dv;
  const float* th_pre;   // [M, c_q, c_k] or null
  const float* th_post;
  const float* w_pre;    // [M / CH, CH, CH] or null
  const float* w_post;
  float* part_thpre;     // [B * n_tiles][M][c_q][c_k] partial sums (PASS_K)
  float* part_thpost;
  float* part_wpre;      // [B * n_tiles][M][CH]
  float* part_wpost;
  int B, T, M, G;
  int cq, ck;
  int a1, h1, a2, h2;    // reach of the convolution before (1) / after (2) softmax, 0 if absent
  int premix, postmix;
  float scale;           // 1 / sqrt(d)
  int n_tiles;           // ceil(T / TB)
  Reg rS, rP, rdC, rdA;  // regions computed: S / Z, P, dP / dC, dA / dE
  Geo gS, gZ, gP, gE, gAc, gdA, gdC, gdL;
  int off_lse, off_d, off_th, off_w, off_red;  // small LDS arrays (floats)
  int off_bf;            // bf16 staging (PASS_K), in floats from the pool start
  int ldk;               // leading dimension of the staged Q, dO, K rows (bf16 elements)
};

#define BWT_INLINE __attribute__((always_inline))

__device__ __forceinline__ float* at(float* lds, const Geo& G, int u, int r, int c) {
  return lds + G.off + u * G.hs + (r - G.r0) * G.ld + (c - G.c0);
}

// dst[u][r][c] over region R of every head: sum_{a, e} th[u][a][e] * src[u][r + sa a][c + sa (e - h)],
// sa = -1 for the convolution, +1 for its adjoint; then fin(u, r, c, value). Each thread makes four
// consecutive columns of one row from a window of 4 + 2h source values per lag.
template <int CH, class Fin>
__device__ __forceinline__ void conv_region(float* lds, const Geo& src, const Reg& R, const float* th, int cq,
                                            int ck, int h, bool adjoint, Fin fin) {
  const int ncb = (R.nc + 3) >> 2;
  const int n = CH * R.nr * ncb;
  for (int t = threadIdx.x; t < n; t += NTH) {
    const int u = t / (R.nr * ncb);
    const int rem = t - u * R.nr * ncb;
    const int r = R.r0 + rem / ncb;
    const int c4 = R.c0 + 4 * (rem % ncb);
    const float* thu = th + u * cq * ck;
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    for (int a = 0; a < cq; ++a) {
      const int sr = adjoint ? r + a : r - a;
      const float* row = at(lds, src, u, sr, c4 - h);
      float xr[4 + CKM - 1];
#pragma unroll
      for (int x = 0; x < 4 + CKM - 1; ++x)
        if (x < 4 + 2 * h) xr[x] = row[x];
      const float* tha = thu + a * ck;
#pragma unroll
      for (int e = 0; e < CKM; ++e) {
        if (e < ck) {
          // window slot x holds column c4 - h + x: the adjoint reads c + e - h (slot q + e),
          // the convolution reads c - e' + h with e' = ck - 1 - e (slot q + e)
          const float w = tha[adjoint ? e : ck - 1 - e];
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) o[qq] = __builtin_fmaf(w, xr[qq + e], o[qq]);
        }
      }
    }
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      if (c4 + qq < R.c0 + R.nc) fin(u, r, c4 + qq, o[qq]);
  }
}

// Partial sums of dtheta[u][a][e] over the core tile: sum_{r, c} G[u][r][c] X[u][r - a][c - e + h],
// for task t = ((u * cq + a) * ck + e) * NRQ + rq covering rows rq, rq + NRQ, ...
template <int CH>
__device__ __forceinline__ void dtheta_tasks(float* lds, const Geo& gG, const Geo& gX, int cq, int ck, int h,
                                             float (&acc)[MAXR]) {
  const int n = CH * cq * ck * NRQ;
#pragma unroll
  for (int rr = 0; rr < MAXR; ++rr) {
    const int t = threadIdx.x + rr * NTH;
    if (t < n) {
      const int rq = t % NRQ;
      const int e = (t / NRQ) % ck;
      const int a = (t / (NRQ * ck)) % cq;
      const int u = t / (NRQ * ck * cq);
      float s = 0.0f;
      for (int r = rq; r < TB; r += NRQ) {
        const float* gr = at(lds, gG, u, r, 0);
        const float* xr = at(lds, gX, u, r - a, h - e);
#pragma unroll
        for (int c = 0; c < TB; ++c) s = __builtin_fmaf(gr[c], xr[c], s);
      }
      acc[rr] += s;
    }
  }
}

__device__ __forceinline__ s16x4 tr_read(const __bf16* base, int row0, int col0, int ld, int lane) {
  const int j = lane & 15;  // lane 4k + m of a 16-lane group supplies row row0 + k, columns col0 + 4m ..
  const __bf16* p = base + (size_t)(row0 + (j >> 2)) * ld + col0 + 4 * (j & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

template <int D, int CH, int MODE>
__global__ __launch_bounds__(NTH) void bwd_tile_kernel(BwArgs A) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  constexpr int NB = D / 16;
  constexpr int NKV = (2 * CH * NB + NTH / 64 - 1) / (NTH / 64);  // dK / dV blocks per wave
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 15, lg = lane >> 4;
  const int T = A.T, M = A.M;
  const int nbg = A.B * A.G;
  const int bg = (int)blockIdx.x % nbg;
  const int tile_rank = (int)blockIdx.x / nbg;  // workgroups with the longest sweeps first
  const int b = bg / A.G, g = bg % A.G;
  const int tile = MODE == PASS_D ? A.n_tiles - 1 - tile_rank : tile_rank;
  const bool pre = A.th_pre != nullptr;
  const bool post = A.th_post != nullptr;
  const size_t bT = (size_t)b * T;

  float* th_s = lds + A.off_th;  // [2][CH][cq][ck]: before softmax, then after
  float* w_s = lds + A.off_w;    // [2][CH][CH]
  float* lse_s = lds + A.off_lse;
  float* d_s = lds + A.off_d;
  const int thn = CH * A.cq * A.ck;
  for (int x = tid; x < 2 * thn; x += NTH) {
    const float* src = x < thn ? A.th_pre : A.th_post;
    const int y = x < thn ? x : x - thn;
    th_s[x] = src ? src[(size_t)g * thn + y] : 0.0f;
  }
  for (int x = tid; x < 2 * CH * CH; x += NTH) {
    const float* src = x < CH * CH ? A.w_pre : A.w_post;
    const int y = x < CH * CH ? x : x - CH * CH;
    w_s[x] = src ? src[(size_t)g * CH * CH + y] : 0.0f;
  }

  // staged bf16 rows (PASS_K): K of the workgroup's keys, Q and dO of the step's query rows,
  // and the step's dS and A tiles
  __bf16* Ks = reinterpret_cast<__bf16*>(lds + A.off_bf);
  __bf16* Qs = Ks + CH * TB * A.ldk;
  __bf16* Os = Qs + CH * TB * A.ldk;
  __bf16* dSb = Os + CH * TB * A.ldk;
  __bf16* Ab = dSb + CH * TB * 24;
  constexpr int LDT = 24;  // leading dimension of the 16 x 16 bf16 tiles

  // stage rows r0 .. r0 + 15 of head u of X (bf16) into dst[u][16][ldk]; zeros past T
  auto stage_rows = [&](__bf16* dst, const __bf16* X, int r0) BWT_INLINE {
    constexpr int PER = D / 8;  // 16-byte pieces per row
    for (int x = tid; x < CH * TB * PER; x += NTH) {
      const int u = x / (TB * PER), rr = (x / PER) % TB, c = x % PER;
      const int i = r0 + rr;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (i < T) val = *reinterpret_cast<const uint4*>(X + ((bT + i) * M + g * CH + u) * D + c * 8);
      *reinterpret_cast<uint4*>(dst + (u * TB + rr) * A.ldk + c * 8) = val;
    }
  };

  // persistent accumulators
  float acc_thpre[MAXR], acc_thpost[MAXR], acc_w[CH * CH], acc_w2[CH * CH], acc_d = 0.0f, acc_l = 0.0f;
#pragma unroll
  for (int x = 0; x < MAXR; ++x) acc_thpre[x] = acc_thpost[x] = 0.0f;
#pragma unroll
  for (int x = 0; x < CH * CH; ++x) acc_w[x] = acc_w2[x] = 0.0f;
  f32x4 acc_kv[NKV];
#pragma unroll
  for (int x = 0; x < NKV; ++x) acc_kv[x] = f32x4{0.f, 0.f, 0.f, 0.f};

  int i0, j0;
  if (MODE == PASS_K) {
    j0 = tile * TB;
    i0 = j0;
    stage_rows(Ks, A.k, j0);
  } else {
    i0 = tile * TB;
    j0 = 0;
  }

  for (;;) {
    if (MODE == PASS_K ? i0 >= T : j0 > i0) break;
    __syncthreads();  // the previous step is done with every LDS map
    auto valid = [&](int r, int c) BWT_INLINE {
      const int i = i0 + r, j = j0 + c;
      return (j >= 0) & (j <= i) & (i < T);
    };
    // ---- (1) row statistics; S = Q K^T / sqrt(d) and dA = dO V^T on MFMA
    for (int x = tid; x < CH * A.rP.nr; x += NTH) {
      const int u = x / A.rP.nr, r = A.rP.r0 + x % A.rP.nr;
      const int i = i0 + r;
      lse_s[x] = (i >= 0 && i < T) ? (MODE == PASS_D ? A.lse : A.lse_c)[(bT + i) * M + g * CH + u] : 0.0f;
    }
    if (MODE == PASS_K) {
      for (int x = tid; x < CH * A.rdC.nr; x += NTH) {
        const int u = x / A.rdC.nr, r = A.rdC.r0 + x % A.rdC.nr;
        const int i = i0 + r;
        d_s[x] = (i >= 0 && i < T) ? A.dvec[(bT + i) * M + g * CH + u] : 0.0f;
      }
    }
    {
      const int nbS = (A.rS.nr / 16) * (A.rS.nc / 16), nbA = (A.rdA.nr / 16) * (A.rdA.nc / 16);
      const int ntask = CH * (nbS + nbA);
      for (int t = wave; t < ntask; t += NTH / 64) {
        const bool isS = t < CH * nbS;
        const int tt = isS ? t : t - CH * nbS;
        const Reg& R = isS ? A.rS : A.rdA;
        const int nbc = R.nc / 16;
        const int u = tt / (isS ? nbS : nbA), blk = tt % (isS ? nbS : nbA);
        const int rb = R.r0 + 16 * (blk / nbc), cb = R.c0 + 16 * (blk % nbc);
        const int m = g * CH + u;
        const int ia = min(max(i0 + rb + lq, 0), T - 1);
        const int jb = min(max(j0 + cb + lq, 0), T - 1);
        const __bf16* pa = (isS ? A.q : A.dO) + ((bT + ia) * M + m) * D + lg * 8;
        const __bf16* pb = (isS ? A.k : A.v) + ((bT + jb) * M + m) * D + lg * 8;
        bf16x8 fa[D / 32], fb[D / 32];
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          fa[kk] = *reinterpret_cast<const bf16x8*>(pa + kk * 32);
          fb[kk] = *reinterpret_cast<const bf16x8*>(pb + kk * 32);
        }
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[kk], fb[kk], c, 0, 0, 0);
        const Geo& G = isS ? A.gS : A.gdA;
        const float sc = isS ? A.scale : 1.0f;
#pragma unroll
        for (int x = 0; x < 4; ++x) *at(lds, G, u, rb + 4 * lg + x, cb + lq) = c[x] * sc;
      }
    }
    __syncthreads();
    // ---- (2) Z = Mask_0(mix_pre(S)) over rS
    {
      const int n = A.rS.nr * A.rS.nc;
      for (int x = tid; x < n; x += NTH) {
        const int r = A.rS.r0 + x / A.rS.nc, c = A.rS.c0 + x % A.rS.nc;
        const bool ok = valid(r, c);
        float s[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) s[u] = *at(lds, A.gS, u, r, c);
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          float z = s[u];
          if (A.premix) {
            z = 0.0f;
#pragma unroll
            for (int v = 0; v < CH; ++v) z = __builtin_fmaf(w_s[u * CH + v], s[v], z);
          }
          *at(lds, A.gZ, u, r, c) = ok ? z : 0.0f;
        }
      }
    }
    __syncthreads();
    // ---- (3) P = exp(C - lse) over rP (C = conv_pre(Z), or Z); zero where masked
    {
      auto finP = [&](int u, int r, int c, float cv) BWT_INLINE {
        const float l = lse_s[u * A.rP.nr + (r - A.rP.r0)];
        *at(lds, A.gP, u, r, c) = valid(r, c) ? __builtin_amdgcn_exp2f((cv - l) * 1.4426950408889634f) : 0.0f;
      };
      if (pre) {
        conv_region<CH>(lds, A.gZ, A.rP, th_s, A.cq, A.ck, A.h1, false, finP);
      } else {
        const int n = CH * A.rP.nr * A.rP.nc;
        for (int x = tid; x < n; x += NTH) {
          const int u = x / (A.rP.nr * A.rP.nc), rem = x % (A.rP.nr * A.rP.nc);
          const int r = A.rP.r0 + rem / A.rP.nc, c = A.rP.c0 + rem % A.rP.nc;
          finP(u, r, c, *at(lds, A.gZ, u, r, c));
        }
      }
    }
    __syncthreads();
    // ---- (4) PASS_K: E = Mask_0(conv_post(P)) and A = mix_post(E) on the core tile
    if (MODE == PASS_K && (post || A.postmix)) {
      const Reg core{0, 0, TB, TB};
      if (post) {
        conv_region<CH>(lds, A.gP, core, th_s + thn, A.cq, A.ck, A.h2, false,
                        [&](int u, int r, int c, float ev) BWT_INLINE { *at(lds, A.gE, u, r, c) = valid(r, c) ? ev : 0.0f; });
        if (A.postmix) __syncthreads();
      }
      if (A.postmix) {
        for (int x = tid; x < TB * TB; x += NTH) {
          const int r = x / TB, c = x % TB;
          float e[CH];
#pragma unroll
          for (int u = 0; u < CH; ++u) e[u] = *at(lds, A.gE, u, r, c);
#pragma unroll
          for (int u = 0; u < CH; ++u) {
            float s = 0.0f;
#pragma unroll
            for (int v = 0; v < CH; ++v) s = __builtin_fmaf(w_s[CH * CH + u * CH + v], e[v], s);
            *at(lds, A.gAc, u, r, c) = s;
          }
        }
      }
      __syncthreads();
    }
    // ---- (5) dE = Mask_0(mix_post^T(dA)) over rdA, in place; PASS_K: dw_post partials
    {
      const int n = A.rdA.nr * A.rdA.nc;
      for (int x = tid; x < n; x += NTH) {
        const int r = A.rdA.r0 + x / A.rdA.nc, c = A.rdA.c0 + x % A.rdA.nc;
        const bool ok = valid(r, c);
        float da[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) da[u] = *at(lds, A.gdA, u, r, c);
        if (MODE == PASS_K && A.postmix && r >= 0 && r < TB && c >= 0 && c < TB) {
#pragma unroll
          for (int u = 0; u < CH; ++u)
#pragma unroll
            for (int v = 0; v < CH; ++v) acc_w2[u * CH + v] = __builtin_fmaf(da[u], *at(lds, A.gE, v, r, c), acc_w2[u * CH + v]);
        }
#pragma unroll
        for (int v = 0; v < CH; ++v) {
          float s = da[v];
          if (A.postmix) {
            s = 0.0f;
#pragma unroll
            for (int u = 0; u < CH; ++u) s = __builtin_fmaf(w_s[CH * CH + u * CH + v], da[u], s);
          }
          *at(lds, A.gdA, v, r, c) = ok ? s : 0.0f;
        }
      }
    }
    __syncthreads();
    // ---- (6) dP = conv_post^T(dE) over rdC; PASS_K: dtheta_post partials
    if (post) {
      conv_region<CH>(lds, A.gdA, A.rdC, th_s + thn, A.cq, A.ck, A.h2, true,
                      [&](int u, int r, int c, float pv) BWT_INLINE { *at(lds, A.gdC, u, r, c) = pv; });
      if (MODE == PASS_K) dtheta_tasks<CH>(lds, A.gdA, A.gP, A.cq, A.ck, A.h2, acc_thpost);
      __syncthreads();
    }
    if (MODE == PASS_D) {
      // ---- D_i partials: sum over the tile's keys of P dP
      if (tid < CH * TB) {
        const int u = tid / TB, r = tid % TB;
        const float* pr = at(lds, A.gP, u, r, 0);
        const float* dr = at(lds, A.gdC, u, r, 0);
        float s = 0.0f, l = 0.0f;
#pragma unroll
        for (int c = 0; c < TB; ++c) {
          s = __builtin_fmaf(pr[c], dr[c], s);
          l += pr[c];
        }
        acc_d += s;
        acc_l += l;
      }
      j0 += TB;
      continue;
    }
    // ---- (7) dC = P (dP - D) over rdC, in place
    {
      const int n = CH * A.rdC.nr * A.rdC.nc;
      for (int x = tid; x < n; x += NTH) {
        const int u = x / (A.rdC.nr * A.rdC.nc), rem = x % (A.rdC.nr * A.rdC.nc);
        const int r = A.rdC.r0 + rem / A.rdC.nc, c = A.rdC.c0 + rem % A.rdC.nc;
        float* pd = at(lds, A.gdC, u, r, c);
        *pd = *at(lds, A.gP, u, r, c) * (*pd - d_s[u * A.rdC.nr + (r - A.rdC.r0)]);
      }
    }
    __syncthreads();
    // ---- (8) dL = Mask_0(conv_pre^T(dC)) on the core tile; dtheta_pre partials
    if (pre) {
      conv_region<CH>(lds, A.gdC, Reg{0, 0, TB, TB}, th_s, A.cq, A.ck, A.h1, true,
                      [&](int u, int r, int c, float lv) BWT_INLINE { *at(lds, A.gdL, u, r, c) = valid(r, c) ? lv : 0.0f; });
      dtheta_tasks<CH>(lds, A.gdC, A.gZ, A.cq, A.ck, A.h1, acc_thpre);
      __syncthreads();
    }
    // ---- (9) dS = mix_pre^T(dL) (dw_pre partials) and A as bf16 tiles; stage Q and dO rows
    for (int x = tid; x < TB * TB; x += NTH) {
      const int r = x / TB, c = x % TB;
      float dl[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) dl[u] = *at(lds, A.gdL, u, r, c);
      if (A.premix) {
#pragma unroll
        for (int u = 0; u < CH; ++u)
#pragma unroll
          for (int v = 0; v < CH; ++v) acc_w[u * CH + v] = __builtin_fmaf(dl[u], *at(lds, A.gS, v, r, c), acc_w[u * CH + v]);
      }
#pragma unroll
      for (int v = 0; v < CH; ++v) {
        float s = dl[v];
        if (A.premix) {
          s = 0.0f;
#pragma unroll
          for (int u = 0; u < CH; ++u) s = __builtin_fmaf(w_s[u * CH + v], dl[u], s);
        }
        dSb[(v * TB + r) * LDT + c] = (__bf16)s;
        Ab[(v * TB + r) * LDT + c] = (__bf16)*at(lds, A.gAc, v, r, c);
      }
    }
    stage_rows(Qs, A.q, i0);
    stage_rows(Os, A.dO, i0);
    __syncthreads();
    // ---- (10) dK += dS^T Q, dV += A^T dO (registers); dQ += dS K (atomics)
#pragma unroll
    for (int x = 0; x < NKV; ++x) {
      const int kv = wave + x * (NTH / 64);
      if (kv < 2 * CH * NB) {
        const int kind = kv / (CH * NB), u = (kv / NB) % CH, nb = kv % NB;
        const s16x4 fa = tr_read((kind ? Ab : dSb) + u * TB * LDT, 4 * lg, 0, LDT, lane);
        const s16x4 fb = tr_read((kind ? Os : Qs) + u * TB * A.ldk, 4 * lg, nb * 16, A.ldk, lane);
        acc_kv[x] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, fb, acc_kv[x], 0, 0, 0);
      }
    }
    for (int t = wave; t < CH * NB; t += NTH / 64) {
      const int u = t / NB, nb = t % NB;
      const s16x4 fa = *reinterpret_cast<const s16x4*>(dSb + (u * TB + lq) * LDT + 4 * lg);
      const s16x4 fb = tr_read(Ks + u * TB * A.ldk, 4 * lg, nb * 16, A.ldk, lane);
      const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, fb, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const int i = i0 + 4 * lg + x;
        if (i < T) unsafeAtomicAdd(A.dq_acc + ((bT + i) * M + g * CH + u) * D + nb * 16 + lq, c[x]);
      }
    }
    i0 += TB;
  }

  if (MODE == PASS_D) {
    if (tid < CH * TB) {
      const int u = tid / TB, i = i0 + tid % TB;
      if (i < T) {
        const size_t x = (bT + i) * M + g * CH + u;
        A.dvec[x] = acc_d / acc_l;
        A.lse_c[x] = A.lse[x] + __logf(acc_l);
      }
    }
    return;
  }
  // ---- dK, dV of the workgroup's keys
#pragma unroll
  for (int x = 0; x < NKV; ++x) {
    const int kv = wave + x * (NTH / 64);
    if (kv < 2 * CH * NB) {
      const int kind = kv / (CH * NB), u = (kv / NB) % CH, nb = kv % NB;
      __bf16* dst = kind ? A.dv : A.dk;
      const float sc = kind ? 1.0f : A.scale;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int j = j0 + 4 * lg + y;
        if (j < T) dst[((bT + j) * M + g * CH + u) * D + nb * 16 + lq] = (__bf16)(acc_kv[x][y] * sc);
      }
    }
  }
  // ---- parameter-gradient partials of this workgroup: [b * n_tiles + tile][m][...]
  __syncthreads();
  float* red = lds + A.off_red;
  const size_t prow = (size_t)b * A.n_tiles + tile;
  const int ntap = CH * A.cq * A.ck;
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    float* part = side == 0 ? A.part_thpre : A.part_thpost;
    if (!part) continue;
    const float(&acc)[MAXR] = side == 0 ? acc_thpre : acc_thpost;
#pragma unroll
    for (int rr = 0; rr < MAXR; ++rr) {
      const int t = tid + rr * NTH;
      if (t < ntap * NRQ) red[t] = acc[rr];
    }
    __syncthreads();
    for (int x = tid; x < ntap; x += NTH) {
      float s = 0.0f;
      for (int rq = 0; rq < NRQ; ++rq) s += red[x * NRQ + rq];
      part[(prow * A.G + g) * ntap + x] = s;
    }
    __syncthreads();
  }
#pragma unroll
  for (int side = 0; side < 2; ++side) {
    float* part = side == 0 ? A.part_wpre : A.part_wpost;
    if (!part) continue;
    const float(&acc)[CH * CH] = side == 0 ? acc_w : acc_w2;
    // sum over the workgroup's threads in a fixed order: wave sums, then the waves in turn
#pragma unroll
    for (int x = 0; x < CH * CH; ++x) {
      float s = acc[x];
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
      if (lane == 0) red[wave * CH * CH + x] = s;
    }
    __syncthreads();
    if (tid < CH * CH) {
      float s = 0.0f;
      for (int w = 0; w < NTH / 64; ++w) s += red[w * CH * CH + tid];
      part[(prow * A.G + g) * CH * CH + tid] = s;
    }
    __syncthreads();
  }
}

// Launch of one pass for a head group of ch heads; lds = dynamic LDS bytes of the plan.
template <int D, int CH, int MODE>
hipError_t launch_one(const BwArgs& a, size_t lds, unsigned grid, hipStream_t st) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_tile_kernel<D, CH, MODE>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_tile_kernel<D, CH, MODE>), dim3(grid), dim3(NTH), lds, st, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_tiles(const BwArgs& a, int ch, int mode, size_t lds, unsigned grid, hipStream_t st) {
  if (grid == 0) return hipSuccess;
  switch (ch * 2 + mode) {
    case 2: return launch_one<D, 1, PASS_D>(a, lds, grid, st);
    case 3: return launch_one<D, 1, PASS_K>(a, lds, grid, st);
    case 4: return launch_one<D, 2, PASS_D>(a, lds, grid, st);
    case 5: return launch_one<D, 2, PASS_K>(a, lds, grid, st);
    case 8: return launch_one<D, 4, PASS_D>(a, lds, grid, st);
    case 9: return launch_one<D, 4, PASS_K>(a, lds, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace bwt
}  // namespace mta
