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

// The regions a tile step computes and their LDS storage. Maps that are not needed alias
// the storage of the map they are computed from.
struct Plan {
  int cq, ck, a1, h1, a2, h2;  // reach of the convolution before (1) / after (2) softmax, 0 if absent
  int pre, post, premix, postmix;
  Reg rS, rP, rdC, rdA;  // regions computed: S / Z, P, dP / dC, dA / dE
  Geo gS, gSc, gZ, gP, gE, gAc, gdA, gdC, gdL;  // gSc: PASS_K core copy of S (mixing before softmax)
  int off_lse, off_d, off_th, off_w, off_red;  // small LDS arrays (floats)
  int off_bf;            // bf16 staging, in floats from the pool start
  int ldk;               // leading dimension of the staged operand rows (bf16 elements)
  int nx1, nx2;          // staged rows per head: rows (PASS_K) or columns (PASS_D) of rS and rdA
  int lds_floats;        // pool size
};

__host__ __device__ constexpr int r4c(int x) { return (x + 3) & ~3; }
__host__ __device__ constexpr int r16c(int x) { return (x + 15) & ~15; }
__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr Geo own_geo(const Reg& R, int ch, int& pool) {
  Geo G{R.r0, R.c0, r4c(R.nc) + 4, 0, pool};
  G.hs = R.nr * G.ld;
  pool = r4c(pool + ch * G.hs);
  return G;
}

// kq, mix: placement bits, 1 before softmax, 2 after. The regions, from the core tile outwards:
// PASS_K: dC on the rows the adjoint of the convolution before softmax reads; P there and
// where the convolution after softmax reads for the core; S around P; dA around dC.
// PASS_D: P and dP on the core tile only.
__host__ __device__ constexpr Plan make_plan(int mode, int kq, int mix, int c_q, int c_k, int ch, int d) {
  Plan p{};
  p.pre = (kq & 1) != 0;
  p.post = (kq & 2) != 0;
  p.premix = (mix & 1) != 0;
  p.postmix = (mix & 2) != 0;
  p.cq = kq ? c_q : 1;
  p.ck = kq ? c_k : 1;
  p.a1 = p.pre ? c_q - 1 : 0;
  p.h1 = p.pre ? (c_k - 1) / 2 : 0;
  p.a2 = p.post ? c_q - 1 : 0;
  p.h2 = p.post ? (c_k - 1) / 2 : 0;
  const Reg core{0, 0, TB, TB};
  if (mode == PASS_K) {
    p.rdC = Reg{0, -p.h1, TB + p.a1, r4c(TB + 2 * p.h1)};
    const int hc = imax(p.h1, p.h2);
    const int c_end = imax(p.rdC.c0 + p.rdC.nc, TB + p.h2);
    p.rP = Reg{-p.a2, -hc, TB + p.a1 + p.a2, r4c(c_end + hc)};
  } else {
    p.rdC = core;
    p.rP = core;
  }
  p.rS = Reg{p.rP.r0 - p.a1, p.rP.c0 - p.h1, r16c(p.rP.nr + p.a1), r16c(p.rP.nc + 2 * p.h1)};
  p.rdA = Reg{0, p.rdC.c0 - p.h2, r16c(p.rdC.nr + p.a2), r16c(p.rdC.nc + 2 * p.h2)};
  int pool = 0;
  p.gS = own_geo(p.rS, ch, pool);
  p.gZ = p.gS;  // Z is formed in place
  p.gSc = (mode == PASS_K && p.premix) ? own_geo(core, ch, pool) : p.gS;
  p.gP = p.pre ? own_geo(p.rP, ch, pool) : p.gZ;
  if (mode == PASS_K) {
    p.gE = p.post ? own_geo(core, ch, pool) : p.gP;
    p.gAc = p.postmix ? own_geo(core, ch, pool) : p.gE;
  } else {
    p.gE = p.gP;
    p.gAc = p.gP;
  }
  p.gdA = own_geo(p.rdA, ch, pool);
  p.gdC = p.post ? own_geo(p.rdC, ch, pool) : p.gdA;
  p.gdL = (mode == PASS_K && p.pre) ? own_geo(core, ch, pool) : p.gdC;
  p.off_lse = pool;
  pool = r4c(pool + ch * p.rP.nr);
  p.off_d = pool;
  pool = r4c(pool + ch * p.rdC.nr);
  p.off_th = pool;
  pool = r4c(pool + 2 * ch * p.cq * p.ck);
  p.off_w = pool;
  pool = r4c(pool + 2 * ch * ch);
  p.ldk = d + 8;
  p.nx1 = mode == PASS_K ? p.rS.nr : p.rS.nc;
  p.nx2 = mode == PASS_K ? p.rdA.nr : p.rdA.nc;
  p.off_bf = pool;
  pool += (ch * (p.nx1 + p.nx2) * p.ldk) / 2;
  if (mode == PASS_K) pool += (2 * ch * TB * 24) / 2;
  p.off_red = 0;  // the end-of-sweep reductions reuse the pool from its start
  pool = imax(pool, imax(ch * p.cq * p.ck * NRQ, ch * ch * TB));
  p.lds_floats = r4c(pool);
  return p;
}

// Shapes with kernels specialised at compile time (the placements and kernel sizes of the
// benchmark workloads); spec 0 is the generic kernel that reads its plan from the arguments.
struct SpecShape {
  int kq, mix, cq, ck;
};
__host__ __device__ constexpr SpecShape spec_shape(int spec) {
  return spec == 1 ? SpecShape{2, 1, 4, 9}     // convolution after softmax, mixing before (4 x 9)
       : spec == 2 ? SpecShape{1, 2, 4, 9}     // convolution before softmax, mixing after (4 x 9)
       : spec == 3 ? SpecShape{3, 3, 4, 9}     // both on both sides (4 x 9)
       : spec == 4 ? SpecShape{1, 2, 6, 11}    // convolution before softmax, mixing after (6 x 11)
                   : SpecShape{0, 0, 1, 1};
}
constexpr int NSPEC = 5;

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
  float scale;           // 1 / sqrt(d)
  int n_tiles;           // ceil(T / TB)
  Plan P;                // the generic kernel's plan (the specialised ones carry their own)
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

template <int D, int CH, int MODE, int SPEC>
__global__ __launch_bounds__(NTH) void bwd_tile_kernel(BwArgs A) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  // the plan: compile-time constants for a specialised shape, so that loop bounds, divisors and
  // LDS offsets fold away
  Plan P;
  if constexpr (SPEC != 0) {
    constexpr SpecShape sh = spec_shape(SPEC);
    constexpr Plan KP = make_plan(MODE, sh.kq, sh.mix, sh.cq, sh.ck, CH, D);
    P = KP;
  } else {
    P = A.P;
  }
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
  const bool pre = P.pre, post = P.post;
  const size_t bT = (size_t)b * T;

  float* th_s = lds + P.off_th;  // [2][CH][cq][ck]: before softmax, then after
  float* w_s = lds + P.off_w;    // [2][CH][CH]
  float* lse_s = lds + P.off_lse;
  float* d_s = lds + P.off_d;
  const int thn = CH * P.cq * P.ck;
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
  __bf16* X1 = reinterpret_cast<__bf16*>(lds + P.off_bf);  // [CH][nx1] rows: Q (PASS_K) or K (PASS_D)
  __bf16* X2 = X1 + CH * P.nx1 * P.ldk;                        // [CH][nx2] rows: dO (PASS_K) or V (PASS_D)
  __bf16* dSb = X2 + CH * P.nx2 * P.ldk;
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
      *reinterpret_cast<uint4*>(dst + (u * TB + rr) * P.ldk + c * 8) = val;
    }
  };

  // persistent accumulators
  // acc_wpre / acc_wpost: task (u, v, r) = thread CH TB u + TB v + r < CH^2 TB of the mixing gradients,
  // row r of the core tile
  float acc_thpre[MAXR], acc_thpost[MAXR], acc_wpre = 0.0f, acc_wpost = 0.0f, acc_d = 0.0f, acc_l = 0.0f;
  const int wu = tid / (CH * TB), wv = (tid / TB) % CH, wr = tid % TB;
  const bool wtask = tid < CH * CH * TB;
#pragma unroll
  for (int x = 0; x < MAXR; ++x) acc_thpre[x] = acc_thpost[x] = 0.0f;
  f32x4 acc_kv[NKV];
#pragma unroll
  for (int x = 0; x < NKV; ++x) acc_kv[x] = f32x4{0.f, 0.f, 0.f, 0.f};

  // PASS_K: the dQ tasks of this wave (head u, 16 channels nb) and their K operand, K rows of
  // the workgroup's keys read transposed once for the whole sweep (staged through X1)
  constexpr int NQT = (CH * NB + NTH / 64 - 1) / (NTH / 64);
  s16x4 kfrag[NQT];
  int i0, j0;
  if (MODE == PASS_K) {
    j0 = tile * TB;
    i0 = j0;
    stage_rows(X1, A.k, j0);
    __syncthreads();
#pragma unroll
    for (int x = 0; x < NQT; ++x) {
      const int t = wave + x * (NTH / 64);
      if (t < CH * NB) kfrag[x] = tr_read(X1 + (t / NB) * TB * P.ldk, 4 * lg, (t % NB) * 16, P.ldk, lane);
    }
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
    // ---- (1) the operand rows that change from step to step (PASS_K: Q and dO of the query
    // rows, PASS_D: K and V of the keys) into LDS in one round of loads, with the row
    // statistics; then S = Q K^T / sqrt(d) and dA = dO V^T on MFMA, the operand that is fixed for
    // the sweep read from global memory (it stays in the caches)
    {
      constexpr int PER = D / 8;  // 16-byte pieces per row
      const int n1 = CH * P.nx1 * PER, n2 = CH * P.nx2 * PER;
      const int o1 = MODE == PASS_K ? i0 + P.rS.r0 : j0 + P.rS.c0;
      const int o2 = MODE == PASS_K ? i0 + P.rdA.r0 : j0 + P.rdA.c0;
      const __bf16* s1 = MODE == PASS_K ? A.q : A.k;
      const __bf16* s2 = MODE == PASS_K ? A.dO : A.v;
      for (int x = tid; x < n1 + n2; x += NTH) {
        const bool first = x < n1;
        const int y = first ? x : x - n1;
        const int row = y / PER, c = y % PER;  // row of [CH][n] rows
        const int n = first ? P.nx1 : P.nx2;
        const int u = row / n, rr = row - u * n;
        const int gi = (first ? o1 : o2) + rr;
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (gi >= 0 && gi < T) val = *reinterpret_cast<const uint4*>((first ? s1 : s2) + ((bT + gi) * M + g * CH + u) * D + c * 8);
        *reinterpret_cast<uint4*>((first ? X1 : X2) + (u * n + rr) * P.ldk + c * 8) = val;
      }
    }
    for (int x = tid; x < CH * P.rP.nr; x += NTH) {
      const int u = x / P.rP.nr, r = P.rP.r0 + x % P.rP.nr;
      const int i = i0 + r;
      lse_s[x] = (i >= 0 && i < T) ? (MODE == PASS_D ? A.lse : A.lse_c)[(bT + i) * M + g * CH + u] : 0.0f;
    }
    if (MODE == PASS_K) {
      for (int x = tid; x < CH * P.rdC.nr; x += NTH) {
        const int u = x / P.rdC.nr, r = P.rdC.r0 + x % P.rdC.nr;
        const int i = i0 + r;
        d_s[x] = (i >= 0 && i < T) ? A.dvec[(bT + i) * M + g * CH + u] : 0.0f;
      }
    }
    __syncthreads();
    {
      const int nbS = (P.rS.nr / 16) * (P.rS.nc / 16), nbA = (P.rdA.nr / 16) * (P.rdA.nc / 16);
      const int ntask = CH * (nbS + nbA);
      // task t: map (S or dA), head, 16 x 16 block; two tasks per wave at a time so that their
      // global loads are in flight together
      auto task = [&](int t, int& u, int& rb, int& cb, bool& isS) BWT_INLINE {
        isS = t < CH * nbS;
        const int tt = isS ? t : t - CH * nbS;
        const Reg& R = isS ? P.rS : P.rdA;
        const int nbc = R.nc / 16;
        u = tt / (isS ? nbS : nbA);
        const int blk = tt % (isS ? nbS : nbA);
        rb = R.r0 + 16 * (blk / nbc);
        cb = R.c0 + 16 * (blk % nbc);
      };
      // operand rows: the staged side from LDS, the fixed side from global memory
      auto frags = [&](int u, int rb, int cb, bool isS, bf16x8 (&fa)[D / 32], bf16x8 (&fb)[D / 32]) BWT_INLINE {
        const int m = g * CH + u;
        const __bf16* pa;
        const __bf16* pb;
        if (MODE == PASS_K) {
          pa = (isS ? X1 + (u * P.nx1 + rb - P.rS.r0 + lq) * P.ldk : X2 + (u * P.nx2 + rb - P.rdA.r0 + lq) * P.ldk) + lg * 8;
          const int jb = min(max(j0 + cb + lq, 0), T - 1);
          pb = (isS ? A.k : A.v) + ((bT + jb) * M + m) * D + lg * 8;
        } else {
          const int ia = min(max(i0 + rb + lq, 0), T - 1);
          pa = (isS ? A.q : A.dO) + ((bT + ia) * M + m) * D + lg * 8;
          pb = (isS ? X1 + (u * P.nx1 + cb - P.rS.c0 + lq) * P.ldk : X2 + (u * P.nx2 + cb - P.rdA.c0 + lq) * P.ldk) + lg * 8;
        }
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
          fa[kk] = *reinterpret_cast<const bf16x8*>(pa + kk * 32);
          fb[kk] = *reinterpret_cast<const bf16x8*>(pb + kk * 32);
        }
      };
      auto finish = [&](int u, int rb, int cb, bool isS, const bf16x8 (&fa)[D / 32], const bf16x8 (&fb)[D / 32]) BWT_INLINE {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[kk], fb[kk], c, 0, 0, 0);
        const Geo& G = isS ? P.gS : P.gdA;
        const float sc = isS ? A.scale : 1.0f;
#pragma unroll
        for (int x = 0; x < 4; ++x) *at(lds, G, u, rb + 4 * lg + x, cb + lq) = c[x] * sc;
      };
      constexpr int NW = NTH / 64;
      for (int t = wave; t < ntask; t += 2 * NW) {
        int u0, rb0, cb0, u1 = 0, rb1 = 0, cb1 = 0;
        bool s0, s1 = false;
        bf16x8 fa0[D / 32], fb0[D / 32], fa1[D / 32], fb1[D / 32];
        const bool two = t + NW < ntask;
        task(t, u0, rb0, cb0, s0);
        frags(u0, rb0, cb0, s0, fa0, fb0);
        if (two) {
          task(t + NW, u1, rb1, cb1, s1);
          frags(u1, rb1, cb1, s1, fa1, fb1);
        }
        finish(u0, rb0, cb0, s0, fa0, fb0);
        if (two) finish(u1, rb1, cb1, s1, fa1, fb1);
      }
    }
    __syncthreads();
    // ---- (2) Z = Mask_0(mix_pre(S)) over rS, in place (PASS_K keeps the core of S for dw_pre)
    {
      const int n = P.rS.nr * P.rS.nc;
      for (int x = tid; x < n; x += NTH) {
        const int r = P.rS.r0 + x / P.rS.nc, c = P.rS.c0 + x % P.rS.nc;
        const bool ok = valid(r, c);
        float s[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) s[u] = *at(lds, P.gS, u, r, c);
        if (MODE == PASS_K && P.premix && r >= 0 && r < TB && c >= 0 && c < TB) {
#pragma unroll
          for (int u = 0; u < CH; ++u) *at(lds, P.gSc, u, r, c) = s[u];
        }
#pragma unroll
        for (int u = 0; u < CH; ++u) {
          float z = s[u];
          if (P.premix) {
            z = 0.0f;
#pragma unroll
            for (int v = 0; v < CH; ++v) z = __builtin_fmaf(w_s[u * CH + v], s[v], z);
          }
          *at(lds, P.gZ, u, r, c) = ok ? z : 0.0f;
        }
      }
    }
    __syncthreads();
    // ---- (3) P = exp(C - lse) over rP (C = conv_pre(Z), or Z); zero where masked
    {
      auto finP = [&](int u, int r, int c, float cv) BWT_INLINE {
        const float l = lse_s[u * P.rP.nr + (r - P.rP.r0)];
        *at(lds, P.gP, u, r, c) = valid(r, c) ? __builtin_amdgcn_exp2f((cv - l) * 1.4426950408889634f) : 0.0f;
      };
      if (pre) {
        conv_region<CH>(lds, P.gZ, P.rP, th_s, P.cq, P.ck, P.h1, false, finP);
      } else {
        const int n = CH * P.rP.nr * P.rP.nc;
        for (int x = tid; x < n; x += NTH) {
          const int u = x / (P.rP.nr * P.rP.nc), rem = x % (P.rP.nr * P.rP.nc);
          const int r = P.rP.r0 + rem / P.rP.nc, c = P.rP.c0 + rem % P.rP.nc;
          finP(u, r, c, *at(lds, P.gZ, u, r, c));
        }
      }
    }
    __syncthreads();
    // ---- (4) PASS_K: E = Mask_0(conv_post(P)) and A = mix_post(E) on the core tile
    if (MODE == PASS_K && (post || P.postmix)) {
      const Reg core{0, 0, TB, TB};
      if (post) {
        conv_region<CH>(lds, P.gP, core, th_s + thn, P.cq, P.ck, P.h2, false,
                        [&](int u, int r, int c, float ev) BWT_INLINE { *at(lds, P.gE, u, r, c) = valid(r, c) ? ev : 0.0f; });
        if (P.postmix) __syncthreads();
      }
      if (P.postmix) {
        for (int x = tid; x < TB * TB; x += NTH) {
          const int r = x / TB, c = x % TB;
          float e[CH];
#pragma unroll
          for (int u = 0; u < CH; ++u) e[u] = *at(lds, P.gE, u, r, c);
#pragma unroll
          for (int u = 0; u < CH; ++u) {
            float s = 0.0f;
#pragma unroll
            for (int v = 0; v < CH; ++v) s = __builtin_fmaf(w_s[CH * CH + u * CH + v], e[v], s);
            *at(lds, P.gAc, u, r, c) = s;
          }
        }
      }
      __syncthreads();
      if (P.postmix) {  // dw_post partials: sum over the core row of dA_u E_v (before dA turns into dE)
        if (wtask) {
          const float* pa = at(lds, P.gdA, wu, wr, 0);
          const float* pe = at(lds, P.gE, wv, wr, 0);
          float s = 0.0f;
#pragma unroll
          for (int c = 0; c < TB; ++c) s = __builtin_fmaf(pa[c], pe[c], s);
          acc_wpost += s;
        }
        __syncthreads();
      }
    }
    // ---- (5) dE = Mask_0(mix_post^T(dA)) over rdA, in place; PASS_K: dw_post partials
    {
      const int n = P.rdA.nr * P.rdA.nc;
      for (int x = tid; x < n; x += NTH) {
        const int r = P.rdA.r0 + x / P.rdA.nc, c = P.rdA.c0 + x % P.rdA.nc;
        const bool ok = valid(r, c);
        float da[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) da[u] = *at(lds, P.gdA, u, r, c);
#pragma unroll
        for (int v = 0; v < CH; ++v) {
          float s = da[v];
          if (P.postmix) {
            s = 0.0f;
#pragma unroll
            for (int u = 0; u < CH; ++u) s = __builtin_fmaf(w_s[CH * CH + u * CH + v], da[u], s);
          }
          *at(lds, P.gdA, v, r, c) = ok ? s : 0.0f;
        }
      }
    }
    __syncthreads();
    // ---- (6) dP = conv_post^T(dE) over rdC; PASS_K: dtheta_post partials
    if (post) {
      conv_region<CH>(lds, P.gdA, P.rdC, th_s + thn, P.cq, P.ck, P.h2, true,
                      [&](int u, int r, int c, float pv) BWT_INLINE { *at(lds, P.gdC, u, r, c) = pv; });
      if (MODE == PASS_K) dtheta_tasks<CH>(lds, P.gdA, P.gP, P.cq, P.ck, P.h2, acc_thpost);
      __syncthreads();
    }
    if (MODE == PASS_D) {
      // ---- D_i partials: sum over the tile's keys of P dP
      if (tid < CH * TB) {
        const int u = tid / TB, r = tid % TB;
        const float* pr = at(lds, P.gP, u, r, 0);
        const float* dr = at(lds, P.gdC, u, r, 0);
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
      const int n = CH * P.rdC.nr * P.rdC.nc;
      for (int x = tid; x < n; x += NTH) {
        const int u = x / (P.rdC.nr * P.rdC.nc), rem = x % (P.rdC.nr * P.rdC.nc);
        const int r = P.rdC.r0 + rem / P.rdC.nc, c = P.rdC.c0 + rem % P.rdC.nc;
        float* pd = at(lds, P.gdC, u, r, c);
        *pd = *at(lds, P.gP, u, r, c) * (*pd - d_s[u * P.rdC.nr + (r - P.rdC.r0)]);
      }
    }
    __syncthreads();
    // ---- (8) dL = Mask_0(conv_pre^T(dC)) on the core tile; dtheta_pre partials
    if (pre) {
      conv_region<CH>(lds, P.gdC, Reg{0, 0, TB, TB}, th_s, P.cq, P.ck, P.h1, true,
                      [&](int u, int r, int c, float lv) BWT_INLINE { *at(lds, P.gdL, u, r, c) = valid(r, c) ? lv : 0.0f; });
      dtheta_tasks<CH>(lds, P.gdC, P.gZ, P.cq, P.ck, P.h1, acc_thpre);
      __syncthreads();
    }
    // ---- (9) dS = mix_pre^T(dL) (dw_pre partials) and A as bf16 tiles; stage Q and dO rows
    for (int x = tid; x < TB * TB; x += NTH) {
      const int r = x / TB, c = x % TB;
      float dl[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) dl[u] = *at(lds, P.gdL, u, r, c);
#pragma unroll
      for (int v = 0; v < CH; ++v) {
        float s = dl[v];
        if (P.premix) {
          s = 0.0f;
#pragma unroll
          for (int u = 0; u < CH; ++u) s = __builtin_fmaf(w_s[u * CH + v], dl[u], s);
        }
        dSb[(v * TB + r) * LDT + c] = (__bf16)s;
        Ab[(v * TB + r) * LDT + c] = (__bf16)*at(lds, P.gAc, v, r, c);
      }
    }
    if (P.premix && wtask) {  // dw_pre partials: sum over the core row of dL_u S_v
      const float* pl = at(lds, P.gdL, wu, wr, 0);
      const float* ps = at(lds, P.gSc, wv, wr, 0);
      float s = 0.0f;
#pragma unroll
      for (int c = 0; c < TB; ++c) s = __builtin_fmaf(pl[c], ps[c], s);
      acc_wpre += s;
    }
    __syncthreads();
    // ---- (10) dK += dS^T Q, dV += A^T dO (registers); dQ += dS K (atomics)
#pragma unroll
    for (int x = 0; x < NKV; ++x) {
      const int kv = wave + x * (NTH / 64);
      if (kv < 2 * CH * NB) {
        const int kind = kv / (CH * NB), u = (kv / NB) % CH, nb = kv % NB;
        const s16x4 fa = tr_read((kind ? Ab : dSb) + u * TB * LDT, 4 * lg, 0, LDT, lane);
        // the step's core query rows inside the staged Q (from row -rS.r0) and dO (from row 0)
        const __bf16* xb = kind ? X2 + u * P.nx2 * P.ldk : X1 + (u * P.nx1 - P.rS.r0) * P.ldk;
        const s16x4 fb = tr_read(xb, 4 * lg, nb * 16, P.ldk, lane);
        acc_kv[x] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, fb, acc_kv[x], 0, 0, 0);
      }
    }
#pragma unroll
    for (int y = 0; y < NQT; ++y) {
      const int t = wave + y * (NTH / 64);
      if (t >= CH * NB) break;
      const int u = t / NB, nb = t % NB;
      const s16x4 fa = *reinterpret_cast<const s16x4*>(dSb + (u * TB + lq) * LDT + 4 * lg);
      const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, kfrag[y], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
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
  float* red = lds + P.off_red;
  const size_t prow = (size_t)b * A.n_tiles + tile;
  const int ntap = CH * P.cq * P.ck;
  // dtheta: the row groups of each tap added in order
  auto emit_theta = [&](const float (&acc)[MAXR], float* part) BWT_INLINE {
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
  };
  // mixing weights: the rows of each (u, v) added in order
  auto emit_w = [&](float acc, float* part) BWT_INLINE {
    if (wtask) red[tid] = acc;
    __syncthreads();
    if (tid < CH * CH) {
      float s = 0.0f;
      for (int r = 0; r < TB; ++r) s += red[tid * TB + r];
      part[(prow * A.G + g) * CH * CH + tid] = s;
    }
    __syncthreads();
  };
  if (A.part_thpre) emit_theta(acc_thpre, A.part_thpre);
  if (A.part_thpost) emit_theta(acc_thpost, A.part_thpost);
  if (A.part_wpre) emit_w(acc_wpre, A.part_wpre);
  if (A.part_wpost) emit_w(acc_wpost, A.part_wpost);
}

// Launch of one pass for a head group of ch heads; lds = dynamic LDS bytes of the plan.
template <int D, int CH, int MODE, int SPEC>
hipError_t launch_one(const BwArgs& a, size_t lds, unsigned grid, hipStream_t st) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_tile_kernel<D, CH, MODE, SPEC>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_tile_kernel<D, CH, MODE, SPEC>), dim3(grid), dim3(NTH), lds, st, a);
  return hipGetLastError();
}

// Specialised shapes instantiated per (head size, heads per group): 1-3 for four-head groups of
// 128 channels, 4 for two- and four-head groups of 96 or 128 channels.
__host__ __device__ constexpr bool spec_built(int spec, int ch, int d) {
  return (spec >= 1 && spec <= 3 && ch == 4 && d == 128) || (spec == 4 && d >= 96 && (ch == 2 || ch == 4));
}

template <int D, int CH, int MODE>
hipError_t launch_spec(const BwArgs& a, int spec, size_t lds, unsigned grid, hipStream_t st) {
  switch (spec) {
    case 1: if constexpr (spec_built(1, CH, D)) return launch_one<D, CH, MODE, 1>(a, lds, grid, st); break;
    case 2: if constexpr (spec_built(2, CH, D)) return launch_one<D, CH, MODE, 2>(a, lds, grid, st); break;
    case 3: if constexpr (spec_built(3, CH, D)) return launch_one<D, CH, MODE, 3>(a, lds, grid, st); break;
    case 4: if constexpr (spec_built(4, CH, D)) return launch_one<D, CH, MODE, 4>(a, lds, grid, st); break;
  }
  return launch_one<D, CH, MODE, 0>(a, lds, grid, st);
}

template <int D>
hipError_t launch_tiles(const BwArgs& a, int ch, int mode, int spec, size_t lds, unsigned grid, hipStream_t st) {
  if (grid == 0) return hipSuccess;
  switch (ch * 2 + mode) {
    case 2: return launch_spec<D, 1, PASS_D>(a, spec, lds, grid, st);
    case 3: return launch_spec<D, 1, PASS_K>(a, spec, lds, grid, st);
    case 4: return launch_spec<D, 2, PASS_D>(a, spec, lds, grid, st);
    case 5: return launch_spec<D, 2, PASS_K>(a, spec, lds, grid, st);
    case 8: return launch_spec<D, 4, PASS_D>(a, spec, lds, grid, st);
    case 9: return launch_spec<D, 4, PASS_K>(a, spec, lds, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace bwt
}  // namespace mta
