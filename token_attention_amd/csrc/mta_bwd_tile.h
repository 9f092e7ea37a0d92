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
// needs.
//
// A tile step recomputes each map on the region its adjoint needs (the core 16 x 16 tile grown
// by the convolutions' reach). S = QK^T and dA = dO V^T run on MFMA, one 16 x 16 block of every
// head of the group per task, so that the mixing, the masks and (without a convolution before
// softmax) the exponential happen in registers on the MFMA result; the convolutions, the
// softmax gradient and the parameter-gradient sums run in fp32 on the VALU from LDS, the
// softmax gradient folded into the convolutions' epilogues. A step has three to five
// workgroup barriers.
#pragma once

#include <hip/hip_runtime.h>

#include "mta_device.h"
#include "mta_internal.h"

namespace mta {
namespace bwt {

constexpr int TB = 16;   // core tile: TB query rows x TB keys
constexpr int CKM = 17;  // largest key extent of a convolution
constexpr int LDT = 20;  // leading dimension of the 16 x 16 bf16 tiles
constexpr int EB = 5;     // dtheta taps per task (5 against 3: 2-3 % faster with 4 x 9 before softmax)
enum { PASS_D = 0, PASS_K = 1 };

typedef short s16x4 __attribute__((ext_vector_type(4)));

// A rectangle of a map, relative to the tile origin (i0, j0): rows [r0, r0 + nr), columns
// [c0, c0 + nc).
struct Reg {
  int r0, c0, nr, nc;
};
// Storage of a map in LDS: the rectangle it holds, leading dimension ld, head stride hs,
// offset off (floats). Maps that are not needed alias the storage they would be made from.
struct Geo {
  int r0, c0, ld, hs, off;
};

struct Plan {
  int cq, ck, a1, h1, a2, h2;  // reach of the convolution before (1) / after (2) softmax, 0 if absent
  int tq;                      // query rows of a tile step: PASS_K tq <= TB rows, PASS_D TB
  int pre, post, premix, postmix;
  Reg rZ, rP, rdC, rdE;        // regions: Z (with a convolution before softmax), P, dC, dE
  Reg mS, mA;                  // MFMA regions (16 x 16 blocks) covering Z or P, and dE
  Geo gZ, gP, gSc, gdE, gdAc, gE, gdC, gdL;
  int off_lse, off_d, off_th, off_w;  // small arrays (floats): lse and D double-buffered per step
  int ldk;               // leading dimension of the staged rows (bf16 elements)
  // operand rows resident for the whole sweep (bf16): PASS_K the keys' K (over the columns of
  // mS) and V (columns of mA), PASS_D the query rows' Q (rows of mS) and dO (rows of mA)
  int off_x, off_y, nrx, nry;
  int resident;          // 2: both; 1: the first (X) only; 0: neither (read from global memory)
  int off_bf;            // PASS_K bf16 staging: Q and dO of the core rows, dS and A tiles
  int lds_floats;        // pool size
};

__host__ __device__ constexpr int r4c(int x) { return (x + 3) & ~3; }
__host__ __device__ constexpr int r16c(int x) { return (x + 15) & ~15; }
__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }
// Leading dimension of a map of nc columns: the smallest ld >= nc that is 4 or 12 modulo 16.
// A multiple of four floats keeps every row 16-byte aligned, so the windows of the convolutions
// and of dtheta are read with wide LDS accesses; 4 or 12 modulo 16 puts rows four apart (the
// four row groups of a 16 x 16 MFMA result) on different banks. Against an odd ld (nc + 1) this
// cut the key-major pass's LDS instructions by 19 % and its bank-conflict cycles by 26 % at the
// T=4096 variant, and the fused backward's time by 7 % (880M slice) to 11 % (both sides).
__host__ __device__ constexpr int map_ld(int nc) {
  const int base = r4c(nc);
  return (base & ~15) + ((base & 15) <= 4 ? 4 : 12);
}
__host__ __device__ constexpr Geo own_geo(const Reg& R, int ch, int& pool) {
  Geo G{R.r0, R.c0, map_ld(R.nc), 0, pool};
  G.hs = R.nr * G.ld;
  pool = r4c(pool + ch * G.hs);
  return G;
}
__host__ __device__ constexpr Reg grow(const Reg& R, int up, int down, int side) {
  return Reg{R.r0 - up, R.c0 - side, R.nr + up + down, r4c(R.nc + 2 * side)};
}

// kq, mix: placement bits, 1 before softmax, 2 after.
// PASS_K: dC on the rows and columns the adjoint of the convolution before softmax reads for
// the core tile; P there and where the convolution after softmax reads for the core; Z around
// P; dE around dC. PASS_D: P and dP on the core tile, Z and dE around them.
__host__ __device__ constexpr Plan make_plan(int mode, int kq, int mix, int c_q, int c_k, int ch, int d,
                                             int resident = 2, int tq = TB) {
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
  const bool K = mode == PASS_K;
  p.tq = K ? tq : TB;
  const Reg core{0, 0, p.tq, TB};
  p.rdC = K ? Reg{0, -p.h1, p.tq + p.a1, r4c(TB + 2 * p.h1)} : core;
  if (K) {
    const int hc = imax(p.h1, p.h2);
    p.rP = Reg{-p.a2, -hc, p.tq + p.a1 + p.a2, r4c(TB + 2 * hc)};
  } else {
    p.rP = core;
  }
  p.rZ = grow(p.rP, p.a1, 0, p.h1);
  p.rdE = Reg{p.rdC.r0, p.rdC.c0 - p.h2, p.rdC.nr + p.a2, r4c(p.rdC.nc + 2 * p.h2)};
  const Reg& cover = p.pre ? p.rZ : p.rP;
  p.mS = Reg{cover.r0, cover.c0, r16c(cover.nr), r16c(cover.nc)};
  p.mA = Reg{p.rdE.r0, p.rdE.c0, r16c(p.rdE.nr), r16c(p.rdE.nc)};
  // four floats before the first map: the dtheta windows of taps beyond c_k (the last group of EB
  // taps) start up to EB - 1 columns left of the map they read and discard those values
  int pool = 4;
  p.gP = own_geo(p.rP, ch, pool);
  p.gZ = p.pre ? own_geo(p.rZ, ch, pool) : p.gP;
  p.gSc = (K && p.premix) ? own_geo(core, ch, pool) : p.gP;
  p.gdE = own_geo(p.rdE, ch, pool);
  p.gdAc = (K && p.postmix) ? own_geo(core, ch, pool) : p.gdE;
  p.gE = (K && p.post) ? own_geo(core, ch, pool) : p.gP;
  // dC: its own storage after a convolution (dP is made from dE), else in place over dE
  p.gdC = (K && p.post) ? own_geo(p.rdC, ch, pool) : p.gdE;
  p.gdL = (K && p.pre) ? own_geo(core, ch, pool) : p.gdC;
  p.off_lse = pool;
  pool = r4c(pool + 2 * ch * p.rP.nr);
  p.off_d = pool;
  pool = r4c(pool + 2 * ch * p.rdC.nr);
  p.off_th = pool;
  pool = r4c(pool + 2 * ch * p.cq * p.ck);
  p.off_w = pool;
  pool = r4c(pool + 2 * ch * ch);
  p.ldk = d + 8;
  p.nrx = K ? p.mS.nc : p.mS.nr;
  p.nry = K ? p.mA.nc : p.mA.nr;
  p.resident = resident;
  p.off_x = pool;
  if (resident >= 1) pool += (ch * p.nrx * p.ldk) / 2;
  p.off_y = pool;
  if (resident >= 2) pool += (ch * p.nry * p.ldk) / 2;
  p.off_bf = pool;
  if (K) pool += (2 * ch * TB * p.ldk + 2 * ch * TB * LDT) / 2;
  // the end-of-sweep reductions reuse the pool from its start
  pool = imax(pool, imax(EB * 512, ch * ch * TB));  // dtheta partials: at most EB per thread
  p.lds_floats = r4c(pool);
  // what does not fit the 160 KiB of a CU is read from global memory: first Y (fewer MFMA operand
  // reads: the dA map is the smaller one), then X
  if (resident > 0 && p.lds_floats * 4 > 160 * 1024)
    return make_plan(mode, kq, mix, c_q, c_k, ch, d, resident - 1, tq);
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

// Query rows per PASS_K step of a specialised shape: TB, or 13 for the convolution after softmax
// alone, where the 3 rows before the step's rows (P) and after them (dE) then make every map of
// the step exactly one 16-row MFMA block instead of two.
__host__ __device__ constexpr int spec_tq(int spec) { return spec == 1 ? TB - 3 : TB; }
// The plan of a specialised kernel (the host sizes its LDS from the same function).
__host__ __device__ constexpr Plan spec_plan(int mode, int spec, int ch, int d) {
  const SpecShape sh = spec_shape(spec);
  return make_plan(mode, sh.kq, sh.mix, sh.cq, sh.ck, ch, d, 2, mode == PASS_K ? spec_tq(spec) : TB);
}

// Threads per workgroup: 256 when two workgroups fit the LDS of a CU (their barriers then
// overlap), else 512.
__host__ __device__ constexpr int threads_for(const Plan& p) { return p.lds_floats * 4 <= 80 * 1024 ? 256 : 512; }

// Heads per stage-1 MFMA task: the whole group, or (HS = 2) half of it. Halved tasks give the
// waves that would otherwise idle a share of the products, and the mixing, which needs every
// head of a position, then runs as a pointwise pass of its own after them. Chosen per
// specialised PASS_K shape by measurement of the whole fused backward (the halved tasks must
// still give every wave at most one): used with 4 x 9 kernels (before softmax with mixing
// after, T=4096: 28.5 -> 27.2 ms; both sides, T=4096: 42.0 -> 37.1 ms; after softmax with
// 13-row steps, whose single 16-row block per map leaves two tasks: 21.3 -> 18.8 ms, against
// 19.8-20.8 ms with 16-row steps and whole-group tasks), not with 6 x 11 kernels before softmax
// and four-head groups (T=16384: 126 -> 133 ms).
__host__ __device__ constexpr int head_split(int mode, int spec, int ch, int d, int nt) {
  if (!(spec >= 1 && spec <= 3) || mode != PASS_K || ch % 2 != 0) return 1;
  const Plan p = spec_plan(mode, spec, ch, d);
  return 2 * (p.mS.nr / 16 + p.mA.nr / 16) <= nt / 64 ? 2 : 1;
}

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
__device__ __forceinline__ bool inside(const Reg& R, int r, int c) {
  return r >= R.r0 && r < R.r0 + R.nr && c >= R.c0 && c < R.c0 + R.nc;
}

// dst over region R of every head: sum_{a, e} th[u][a][e] * src[u][r + sa a][c + sa (e - h)],
// sa = -1 for the convolution, +1 for its adjoint; fin(u, r, c, value) stores it. Each thread
// makes CPT consecutive columns of one row from a window of CPT + 2h source values per lag.
template <int CH, int NT, int CPT = 4, class Fin>
__device__ __forceinline__ void conv_region(float* lds, const Geo& src, const Reg& R, const float* th, int cq,
                                            int ck, int h, bool adjoint, Fin fin, int t0 = -1, int nthreads = NT) {
  static_assert(CPT == 1 || CPT == 2 || CPT == 4, "R.nc is a multiple of 4");
  const int ncb = R.nc / CPT;
  const int n = CH * R.nr * ncb;
  for (int t = t0 < 0 ? (int)threadIdx.x : t0; t < n; t += nthreads) {
    const int u = t / (R.nr * ncb);
    const int rem = t - u * R.nr * ncb;
    const int r = R.r0 + rem / ncb;
    const int c0 = R.c0 + CPT * (rem % ncb);
    const float* thu = th + u * cq * ck;
    float o[CPT];
#pragma unroll
    for (int qq = 0; qq < CPT; ++qq) o[qq] = 0.0f;
    for (int a = 0; a < cq; ++a) {
      const int sr = adjoint ? r + a : r - a;
      const float* row = at(lds, src, u, sr, c0 - h);
      float xr[CPT + CKM - 1];
#pragma unroll
      for (int x = 0; x < CPT + CKM - 1; ++x)
        if (x < CPT + 2 * h) xr[x] = row[x];
      const float* tha = thu + a * ck;
#pragma unroll
      for (int e = 0; e < CKM; ++e) {
        if (e < ck) {
          // window slot x holds column c0 - h + x: the adjoint reads c + e - h (slot q + e),
          // the convolution reads c - e' + h with e' = ck - 1 - e (slot q + e)
          const float w = tha[adjoint ? e : ck - 1 - e];
#pragma unroll
          for (int qq = 0; qq < CPT; ++qq) o[qq] = __builtin_fmaf(w, xr[qq + e], o[qq]);
        }
      }
    }
#pragma unroll
    for (int qq = 0; qq < CPT; ++qq) fin(u, r, c0 + qq, o[qq]);
  }
}

// Partial sums of dtheta[u][a][e] over the core tile: sum_{r, c} G[u][r][c] X[u][r - a][c - e + h].
// Task t = ((u * cq + a) * neb + eb) * nrq + rq makes taps e = EB eb .. EB eb + EB - 1 from one window of
// X per row (rows rq, rq + nrq, ...; nrq row groups keep the tasks within one round).
template <int CH, int NT>
__device__ __forceinline__ void dtheta_tasks(float* lds, const Geo& gG, const Geo& gX, int cq, int ck, int h, int nrq,
                                             int rows, float (&acc)[EB]) {
  const int neb = (ck + EB - 1) / EB;
  const int t = threadIdx.x;
  if (t < CH * cq * neb * nrq) {
    const int rq = t % nrq;
    const int eb = (t / nrq) % neb;
    const int a = (t / (nrq * neb)) % cq;
    const int u = t / (nrq * neb * cq);
    const int e0 = EB * eb;
    // window slot k holds column k + h - e0 - (EB - 1); tap e0 + j reads slot c + EB - 1 - j.
    // Slots left of column -h serve only taps beyond ck and are not read.
    const int kmin = e0 + EB - 1 - 2 * h;
    for (int r = rq; r < rows; r += nrq) {
      const float* gr = at(lds, gG, u, r, 0);
      const float* xr = at(lds, gX, u, r - a, h - e0 - (EB - 1));
      float xw[TB + EB - 1];
#pragma unroll
      for (int k = 0; k < TB + EB - 1; ++k) xw[k] = k >= kmin ? xr[k] : 0.0f;
#pragma unroll
      for (int c = 0; c < TB; ++c) {
        const float gv = gr[c];
#pragma unroll
        for (int j = 0; j < EB; ++j) acc[j] = __builtin_fmaf(gv, xw[c + EB - 1 - j], acc[j]);
      }
    }
  }
}

__device__ __forceinline__ s16x4 tr_read(const __bf16* base, int row0, int col0, int ld, int lane) {
  const int j = lane & 15;  // lane 4k + m of a 16-lane group supplies row row0 + k, columns col0 + 4m ..
  const __bf16* p = base + (size_t)(row0 + (j >> 2)) * ld + col0 + 4 * (j & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

template <int D, int CH, int MODE, int SPEC, int NT>
__global__ __launch_bounds__(NT) void bwd_tile_kernel(BwArgs A) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  // the plan: compile-time constants for a specialised shape, so that loop bounds, divisors and
  // LDS offsets fold away
  Plan P;
  if constexpr (SPEC != 0) {
    constexpr Plan KP = spec_plan(MODE, SPEC, CH, D);
    P = KP;
  } else {
    P = A.P;
  }
  constexpr int NW = NT / 64;
  constexpr int NB = D / 16;
  constexpr int NKV = (2 * CH * NB + NW - 1) / NW;  // dK / dV blocks per wave
  constexpr int NQT = (CH * NB + NW - 1) / NW;      // dQ blocks per wave
  // columns per thread of the convolutions (PASS_D's D accumulation keeps four): two for 4 x 9
  // before softmax with mixing after (fused backward at T=4096: 27.4 -> 24.3 ms), four elsewhere
  // (two measured slower: +4 % after softmax, +7 % on both sides, twice the time with 6 x 11)
  constexpr int CPC = SPEC == 2 ? 2 : 4;
  constexpr int HS = head_split(MODE, SPEC, CH, D, NT);
  constexpr int CHT = CH / HS;  // heads per stage-1 task
  // query rows per step (a compile-time constant in the specialised kernels)
  constexpr int TQS = SPEC != 0 ? spec_plan(MODE, SPEC, CH, D).tq : TB;
  const int tq = SPEC != 0 ? TQS : P.tq;
  const int nrq = imax(1, min(tq, NT / (CH * P.cq * ((P.ck + EB - 1) / EB))));  // dtheta row groups
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
  const Reg core{0, 0, tq, TB};  // the step's core tile: tq query rows x TB keys

  float* th_s = lds + P.off_th;  // [2][CH][cq][ck]: before softmax, then after
  const int thn = CH * P.cq * P.ck;
  for (int x = tid; x < 2 * thn; x += NT) {
    const float* src = x < thn ? A.th_pre : A.th_post;
    const int y = x < thn ? x : x - thn;
    th_s[x] = src ? src[(size_t)g * thn + y] : 0.0f;
  }
  // the group's mixing weights, uniform across the workgroup: scalar registers
  float wm1[CH * CH], wm2[CH * CH];
#pragma unroll
  for (int x = 0; x < CH * CH; ++x) {
    wm1[x] = P.premix ? A.w_pre[(size_t)g * CH * CH + x] : 0.0f;
    wm2[x] = P.postmix ? A.w_post[(size_t)g * CH * CH + x] : 0.0f;
  }
  // resident operand rows (see Plan::off_x); PASS_K bf16 staging: Q and dO of the step's core
  // rows, the dS and A tiles
  __bf16* Xr = reinterpret_cast<__bf16*>(lds + P.off_x);
  __bf16* Yr = reinterpret_cast<__bf16*>(lds + P.off_y);
  __bf16* Qc = reinterpret_cast<__bf16*>(lds + P.off_bf);
  __bf16* Oc = Qc + CH * TB * P.ldk;
  __bf16* dSb = Oc + CH * TB * P.ldk;
  __bf16* Ab = dSb + CH * TB * LDT;

  // rows r0 .. r0 + n - 1 of every head of X (bf16) into dst[u][n][ldk]; zeros outside [0, T)
  auto stage_rows = [&](__bf16* dst, const __bf16* X, int r0, int n) BWT_INLINE {
    constexpr int PER = D / 8;  // 16-byte pieces per row
    for (int x = tid; x < CH * n * PER; x += NT) {
      const int row = x / PER, c = x % PER;
      const int u = row / n, rr = row - u * n;
      const int i = r0 + rr;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (i >= 0 && i < T) val = *reinterpret_cast<const uint4*>(X + ((bT + i) * M + g * CH + u) * D + c * 8);
      *reinterpret_cast<uint4*>(dst + (u * n + rr) * P.ldk + c * 8) = val;
    }
  };
  // the step's row statistics (lse over rP rows, D over rdC rows) into buffer slot `buf`
  auto load_stats = [&](int i_base, int buf) BWT_INLINE {
    float* ls = lds + P.off_lse + buf * CH * P.rP.nr;
    for (int x = tid; x < CH * P.rP.nr; x += NT) {
      const int u = x / P.rP.nr, i = i_base + P.rP.r0 + x % P.rP.nr;
      ls[x] = (i >= 0 && i < T) ? (MODE == PASS_D ? A.lse : A.lse_c)[(bT + i) * M + g * CH + u] : 0.0f;
    }
    if (MODE == PASS_K) {
      float* ds = lds + P.off_d + buf * CH * P.rdC.nr;
      for (int x = tid; x < CH * P.rdC.nr; x += NT) {
        const int u = x / P.rdC.nr, i = i_base + P.rdC.r0 + x % P.rdC.nr;
        ds[x] = (i >= 0 && i < T) ? A.dvec[(bT + i) * M + g * CH + u] : 0.0f;
      }
    }
  };

  // persistent accumulators. acc_wpre / acc_wpost: task (u, v, r) = thread CH TB u + TB v + r
  // < CH^2 TB of the mixing gradients, row r of the core tile. acc_d, acc_l (PASS_D): the
  // thread's share of D and of the row sum of P for its (head, row).
  float acc_thpre[EB], acc_thpost[EB], acc_wpre = 0.0f, acc_wpost = 0.0f, acc_d = 0.0f, acc_l = 0.0f;
  const int wu = tid / (CH * TB), wv = (tid / TB) % CH, wr = tid % TB;
  const bool wtask = tid < CH * CH * TB;
#pragma unroll
  for (int x = 0; x < EB; ++x) acc_thpre[x] = acc_thpost[x] = 0.0f;
  f32x4 acc_kv[NKV];
#pragma unroll
  for (int x = 0; x < NKV; ++x) acc_kv[x] = f32x4{0.f, 0.f, 0.f, 0.f};

  // PASS_K: the dQ tasks of this wave (head u, 16 channels nb) and their K operand, the K rows
  // of the workgroup's keys (inside the resident K rows) read transposed once for the sweep
  s16x4 kfrag[NQT];
  int i0, j0;
  if (MODE == PASS_K) {
    j0 = tile * TB;
    i0 = j0;
    if (P.resident >= 1) {
      stage_rows(Xr, A.k, j0 + P.mS.c0, P.nrx);
      if (P.resident >= 2) stage_rows(Yr, A.v, j0 + P.mA.c0, P.nry);
    } else {
      stage_rows(Qc, A.k, j0, TB);  // the K rows of the keys, for the transposed reads below
    }
    load_stats(i0, 0);
    __syncthreads();
    const __bf16* kc = P.resident >= 1 ? Xr - P.mS.c0 * P.ldk : Qc;  // K row j0 of head 0
    const int kstride = P.resident >= 1 ? P.nrx : TB;                  // rows per head
#pragma unroll
    for (int x = 0; x < NQT; ++x) {
      const int t = wave + x * NW;
      if (t < CH * NB) kfrag[x] = tr_read(kc + (t / NB) * kstride * P.ldk, 4 * lg, (t % NB) * 16, P.ldk, lane);
    }
    if (P.resident == 0) __syncthreads();  // Qc is rewritten by the first step
    if (tq < TB) {
      // rows of the bf16 staging past the step's tq rows: zero, so that the 16-row products of
      // stage 6 add nothing for them (the steps write only rows below tq of Qc, dSb and Ab)
      for (int x = tid; x < CH * (TB - tq) * P.ldk; x += NT) {
        const int u = x / ((TB - tq) * P.ldk), rem = x % ((TB - tq) * P.ldk);
        Qc[(u * TB + tq) * P.ldk + rem] = (__bf16)0.0f;
        Oc[(u * TB + tq) * P.ldk + rem] = (__bf16)0.0f;
      }
      for (int x = tid; x < CH * (TB - tq) * LDT; x += NT) {
        const int u = x / ((TB - tq) * LDT), rem = x % ((TB - tq) * LDT);
        dSb[(u * TB + tq) * LDT + rem] = (__bf16)0.0f;
        Ab[(u * TB + tq) * LDT + rem] = (__bf16)0.0f;
      }
    }
  } else {
    i0 = tile * TB;
    j0 = 0;
    if (P.resident >= 1) stage_rows(Xr, A.q, i0 + P.mS.r0, P.nrx);
    if (P.resident >= 2) stage_rows(Yr, A.dO, i0 + P.mA.r0, P.nry);
    load_stats(i0, 0);
    __syncthreads();
  }

  // stage-1 tasks: one row (PASS_K) or column (PASS_D) of 16 x 16 blocks of S, then of dA, for
  // CHT heads of the group: task t is block row (column) t / HS, heads CHT (t % HS) ..
  const int nS = MODE == PASS_K ? P.mS.nr / 16 : P.mS.nc / 16;
  const int nA = MODE == PASS_K ? P.mA.nr / 16 : P.mA.nc / 16;
  const int ntask = (nS + nA) * HS;
  const bool prefetch = ntask <= NW;  // a wave per task: its global operand is loaded ahead
  bf16x8 fg[CHT][D / 32];
  // task t's global operand at the tile origin (ti, tj): rows (PASS_K) or columns (PASS_D) of
  // its blocks, 16 bytes per lane and 32 channels, each of its heads
  auto load_global = [&](int t, int ti, int tj, bf16x8 (&dst)[CHT][D / 32]) BWT_INLINE {
    const int tb = t / HS, u0 = (t % HS) * CHT;
    const bool isS = tb < nS;
    const int blk = isS ? tb : tb - nS;
    const Reg& R = isS ? P.mS : P.mA;
    const int gi = MODE == PASS_K ? min(max(ti + R.r0 + 16 * blk + lq, 0), T - 1)
                                  : min(max(tj + R.c0 + 16 * blk + lq, 0), T - 1);
    const __bf16* src = MODE == PASS_K ? (isS ? A.q : A.dO) : (isS ? A.k : A.v);
    const __bf16* pg = src + ((bT + gi) * M + g * CH + u0) * D + lg * 8;
#pragma unroll
    for (int u = 0; u < CHT; ++u)
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) dst[u][kk] = *reinterpret_cast<const bf16x8*>(pg + u * D + kk * 32);
  };
  if (prefetch && wave < ntask) load_global(wave, i0, j0, fg);

  for (int step = 0;; ++step) {
    if (MODE == PASS_K ? i0 >= T : j0 > i0) break;
    const int buf = MODE == PASS_K ? (step & 1) : 0;
    const float* lse_s = lds + P.off_lse + buf * CH * P.rP.nr;
    const float* d_s = lds + P.off_d + buf * CH * P.rdC.nr;
    auto valid = [&](int r, int c) BWT_INLINE {
      const int i = i0 + r, j = j0 + c;
      return (j >= 0) & (j <= i) & (i < T);
    };
    // ---- (1) MFMA: S over mS and dA over mA for every head of the group (a task takes CHT of
    // them). A task is one row of 16 x 16 blocks (PASS_K: its Q or dO rows from global memory, once per step; K or V rows
    // from the resident LDS copy) or one column of blocks (PASS_D, the other way round).
    // S block: mixing before softmax, Mask_0, and Z into gZ (with a convolution before softmax)
    // or P = exp(Z - lse) into gP; PASS_K keeps the core of S (dw_pre). dA block: PASS_K keeps
    // the core (dw_post), then dE = Mask_0(mix_post^T(dA)) into gdE. PASS_K also copies the core
    // rows of Q and dO into Qc and Oc.
    if (MODE == PASS_K && step > 0) __syncthreads();  // the previous step's MFMAs read Qc and Oc
    {
      auto epilogue = [&](bool isS, int rb, int cb, int u0, const f32x4 (&c)[CHT]) BWT_INLINE {
        // lane holds rows rb + 4 lg + x, column cb + lq of heads u0 .. u0 + CHT - 1. With HS > 1
        // a mixed map is stored as the plain product here and mixed by the pass after the barrier.
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int r = rb + 4 * lg + x, cc = cb + lq;
          const bool ok = valid(r, cc);
          const bool in_core = r >= 0 && r < tq && cc >= 0 && cc < TB;
          float v[CHT];
#pragma unroll
          for (int u = 0; u < CHT; ++u) v[u] = isS ? c[u][x] * A.scale : c[u][x];
          if (isS) {
            if (MODE == PASS_K && P.premix && in_core) {
#pragma unroll
              for (int u = 0; u < CHT; ++u) *at(lds, P.gSc, u0 + u, r, cc) = v[u];
            }
            if (pre ? inside(P.rZ, r, cc) : inside(P.rP, r, cc)) {
#pragma unroll
              for (int u = 0; u < CHT; ++u) {
                float z = v[u];
                if constexpr (HS > 1) {
                  if (P.premix) {
                    *at(lds, pre ? P.gZ : P.gP, u0 + u, r, cc) = z;
                    continue;
                  }
                } else {
                  if (P.premix) {
                    z = 0.0f;
#pragma unroll
                    for (int w = 0; w < CH; ++w) z = __builtin_fmaf(wm1[u * CH + w], v[w], z);
                  }
                }
                if (pre) {
                  *at(lds, P.gZ, u0 + u, r, cc) = ok ? z : 0.0f;
                } else {
                  const float l = lse_s[(u0 + u) * P.rP.nr + (r - P.rP.r0)];
                  *at(lds, P.gP, u0 + u, r, cc) = ok ? __builtin_amdgcn_exp2f((z - l) * 1.4426950408889634f) : 0.0f;
                }
              }
            }
          } else {
            if (MODE == PASS_K && P.postmix && in_core) {
#pragma unroll
              for (int u = 0; u < CHT; ++u) *at(lds, P.gdAc, u0 + u, r, cc) = v[u];
            }
            if (inside(P.rdE, r, cc)) {
#pragma unroll
              for (int w = 0; w < CHT; ++w) {
                float s = v[w];
                if constexpr (HS > 1) {
                  if (P.postmix) {
                    *at(lds, P.gdE, u0 + w, r, cc) = s;
                    continue;
                  }
                } else {
                  if (P.postmix) {
                    s = 0.0f;
#pragma unroll
                    for (int u = 0; u < CH; ++u) s = __builtin_fmaf(wm2[u * CH + w], v[u], s);
                  }
                }
                *at(lds, P.gdE, u0 + w, r, cc) = ok ? s : 0.0f;
              }
            }
          }
        }
      };
      for (int t = wave; t < ntask; t += NW) {
        const int tb = t / HS, u0 = (t % HS) * CHT;
        const bool isS = tb < nS;
        const int blk = isS ? tb : tb - nS;
        const Reg& R = isS ? P.mS : P.mA;
        const __bf16* res = isS ? Xr : Yr;  // resident rows of this map
        const int nres = isS ? P.nrx : P.nry;
        // the global operand: rows (PASS_K) or columns (PASS_D) blk of the map, the task's
        // heads; prefetched by the previous step when every task has a wave of its own
        if (!prefetch) load_global(t, i0, j0, fg);
        if (MODE == PASS_K) {
          // the core rows of Q (S rows) and dO (dA rows), for the step's dK and dV products
          const int row = R.r0 + 16 * blk + lq;
          if (row >= 0 && row < tq) {
            __bf16* dst = isS ? Qc : Oc;
#pragma unroll
            for (int u = 0; u < CHT; ++u)
#pragma unroll
              for (int kk = 0; kk < D / 32; ++kk)
                *reinterpret_cast<bf16x8*>(dst + ((u0 + u) * TB + row) * P.ldk + kk * 32 + lg * 8) = fg[u][kk];
          }
        }
        const int nother = MODE == PASS_K ? R.nc / 16 : R.nr / 16;
        for (int o = 0; o < nother; ++o) {
          f32x4 c[CHT];
          // the other operand's rows: resident in LDS, or from global memory
          const __bf16* pr0;
          size_t ustride;
          if (isS ? P.resident >= 1 : P.resident >= 2) {
            pr0 = res + ((size_t)u0 * nres + 16 * o + lq) * P.ldk + lg * 8;
            ustride = (size_t)nres * P.ldk;
          } else {
            const int oi = MODE == PASS_K ? min(max(j0 + R.c0 + 16 * o + lq, 0), T - 1)
                                          : min(max(i0 + R.r0 + 16 * o + lq, 0), T - 1);
            const __bf16* src = MODE == PASS_K ? (isS ? A.k : A.v) : (isS ? A.q : A.dO);
            pr0 = src + ((bT + oi) * M + g * CH + u0) * D + lg * 8;
            ustride = D;
          }
#pragma unroll
          for (int u = 0; u < CHT; ++u) {
            const __bf16* pr = pr0 + u * ustride;
            c[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
              const bf16x8 fr = *reinterpret_cast<const bf16x8*>(pr + kk * 32);
              c[u] = MODE == PASS_K ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(fg[u][kk], fr, c[u], 0, 0, 0)
                                    : __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr, fg[u][kk], c[u], 0, 0, 0);
            }
          }
          const int rb = MODE == PASS_K ? R.r0 + 16 * blk : R.r0 + 16 * o;
          const int cb = MODE == PASS_K ? R.c0 + 16 * o : R.c0 + 16 * blk;
          epilogue(isS, rb, cb, u0, c);
        }
        if (prefetch) {  // the next step's operand, in flight through the stages that follow
          if (MODE == PASS_K ? i0 + tq < T : j0 + TB <= i0) load_global(t, MODE == PASS_K ? i0 + tq : i0,
                                                                        MODE == PASS_K ? j0 : j0 + TB, fg);
        }
      }
    }
    __syncthreads();
    if constexpr (HS > 1) {
      // ---- (1b) the mixing of the halved tasks, position by position over every head: before
      // softmax with Mask_0 into Z, or with the exponential into P; after softmax, dE
      if (P.premix || P.postmix) {
        if (P.premix) {
          const Reg& R = pre ? P.rZ : P.rP;
          const Geo& G = pre ? P.gZ : P.gP;
          for (int x = tid; x < R.nr * R.nc; x += NT) {
            const int r = R.r0 + x / R.nc, c = R.c0 + x % R.nc;
            const bool ok = valid(r, c);
            float v[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u) v[u] = *at(lds, G, u, r, c);
#pragma unroll
            for (int u = 0; u < CH; ++u) {
              float z = 0.0f;
#pragma unroll
              for (int w = 0; w < CH; ++w) z = __builtin_fmaf(wm1[u * CH + w], v[w], z);
              if (pre) {
                *at(lds, G, u, r, c) = ok ? z : 0.0f;
              } else {
                const float l = lse_s[u * P.rP.nr + (r - P.rP.r0)];
                *at(lds, G, u, r, c) = ok ? __builtin_amdgcn_exp2f((z - l) * 1.4426950408889634f) : 0.0f;
              }
            }
          }
        }
        if (P.postmix) {
          for (int x = tid; x < P.rdE.nr * P.rdE.nc; x += NT) {
            const int r = P.rdE.r0 + x / P.rdE.nc, c = P.rdE.c0 + x % P.rdE.nc;
            const bool ok = valid(r, c);
            float v[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u) v[u] = *at(lds, P.gdE, u, r, c);
#pragma unroll
            for (int w = 0; w < CH; ++w) {
              float s = 0.0f;
#pragma unroll
              for (int u = 0; u < CH; ++u) s = __builtin_fmaf(wm2[u * CH + w], v[u], s);
              *at(lds, P.gdE, w, r, c) = ok ? s : 0.0f;
            }
          }
        }
        __syncthreads();
      }
    }
    // the softmax gradient at (u, r, c) of rdC, from dP there: dC = P (dP - D_r)
    auto dC_of = [&](int u, int r, int c, float dp) BWT_INLINE {
      return *at(lds, P.gP, u, r, c) * (dp - d_s[u * P.rdC.nr + (r - P.rdC.r0)]);
    };
    // ---- (2) with a convolution before softmax: P = exp(conv_pre(Z) - lse) over rP; PASS_K
    // without one after softmax also dC there (dP = dE)
    if (pre) {
      conv_region<CH, NT, CPC>(lds, P.gZ, P.rP, th_s, P.cq, P.ck, P.h1, false, [&](int u, int r, int c, float cv) BWT_INLINE {
        const float l = lse_s[u * P.rP.nr + (r - P.rP.r0)];
        const float pv = valid(r, c) ? __builtin_amdgcn_exp2f((cv - l) * 1.4426950408889634f) : 0.0f;
        *at(lds, P.gP, u, r, c) = pv;
        if (MODE == PASS_K && !post && inside(P.rdC, r, c)) {
          float* pd = at(lds, P.gdC, u, r, c);
          *pd = pv * (*pd - d_s[u * P.rdC.nr + (r - P.rdC.r0)]);
        }
      });
      __syncthreads();
    }
    if (MODE == PASS_D) {
      // ---- D_i and the row sum of P: dP = conv_post^T(dE) (or dE) on the core tile; the four
      // threads of a row (consecutive lanes) combine their columns
      if (post) {
        conv_region<CH, NT>(lds, P.gdE, core, th_s + thn, P.cq, P.ck, P.h2, true, [&](int u, int r, int c, float dp) BWT_INLINE {
          const float pv = *at(lds, P.gP, u, r, c);
          acc_d = __builtin_fmaf(pv, dp, acc_d);
          acc_l += pv;
        });
      } else {
        for (int t = tid; t < CH * TB * 4; t += NT) {
          const int u = t / (TB * 4), r = (t / 4) % TB, c4 = 4 * (t % 4);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            const float pv = *at(lds, P.gP, u, r, c4 + qq);
            acc_d = __builtin_fmaf(pv, *at(lds, P.gdE, u, r, c4 + qq), acc_d);
            acc_l += pv;
          }
        }
      }
      j0 += TB;
      __syncthreads();  // the next step rewrites gP and gdE
      continue;
    }
    // ---- (3) PASS_K: E = Mask_0(conv_post(P)) on the core; dP = conv_post^T(dE) over rdC
    // and dC = P (dP - D) there; dtheta_post partials. Without a convolution after softmax and
    // before it either, dC = P (dE - D) in place. Q and dO of the core rows into LDS.
    if (post) {
      conv_region<CH, NT, CPC>(lds, P.gP, core, th_s + thn, P.cq, P.ck, P.h2, false,
                          [&](int u, int r, int c, float ev) BWT_INLINE { *at(lds, P.gE, u, r, c) = valid(r, c) ? ev : 0.0f; });
      conv_region<CH, NT, CPC>(lds, P.gdE, P.rdC, th_s + thn, P.cq, P.ck, P.h2, true,
                          [&](int u, int r, int c, float dp) BWT_INLINE { *at(lds, P.gdC, u, r, c) = dC_of(u, r, c, dp); });
      dtheta_tasks<CH, NT>(lds, P.gdE, P.gP, P.cq, P.ck, P.h2, nrq, tq, acc_thpost);
    } else if (!pre) {
      for (int t = tid; t < CH * P.rdC.nr * P.rdC.nc; t += NT) {
        const int u = t / (P.rdC.nr * P.rdC.nc), rem = t % (P.rdC.nr * P.rdC.nc);
        const int r = P.rdC.r0 + rem / P.rdC.nc, c = P.rdC.c0 + rem % P.rdC.nc;
        float* pd = at(lds, P.gdC, u, r, c);
        *pd = dC_of(u, r, c, *pd);
      }
    }
    __syncthreads();
    // ---- (4) with a convolution before softmax: dL = Mask_0(conv_pre^T(dC)) on the core;
    // dtheta_pre partials
    if (pre) {
      conv_region<CH, NT, CPC>(lds, P.gdC, core, th_s, P.cq, P.ck, P.h1, true,
                          [&](int u, int r, int c, float lv) BWT_INLINE { *at(lds, P.gdL, u, r, c) = valid(r, c) ? lv : 0.0f; });
      dtheta_tasks<CH, NT>(lds, P.gdC, P.gZ, P.cq, P.ck, P.h1, nrq, tq, acc_thpre);
      __syncthreads();
    }
    // ---- (5) dS = mix_pre^T(dL) and A = mix_post(E) on the core as bf16 tiles; the mixing
    // gradients' partials; the next step's row statistics
    for (int x = tid; x < tq * TB; x += NT) {
      const int r = x / TB, c = x % TB;
      float dl[CH], e[CH];
#pragma unroll
      for (int u = 0; u < CH; ++u) {
        dl[u] = *at(lds, P.gdL, u, r, c);
        e[u] = *at(lds, P.gE, u, r, c);
      }
#pragma unroll
      for (int w = 0; w < CH; ++w) {
        float s = dl[w], av = e[w];
        if (P.premix) {
          s = 0.0f;
#pragma unroll
          for (int u = 0; u < CH; ++u) s = __builtin_fmaf(wm1[u * CH + w], dl[u], s);
        }
        if (P.postmix) {
          av = 0.0f;
#pragma unroll
          for (int u = 0; u < CH; ++u) av = __builtin_fmaf(wm2[w * CH + u], e[u], av);
        }
        dSb[(w * TB + r) * LDT + c] = (__bf16)s;
        Ab[(w * TB + r) * LDT + c] = (__bf16)av;
      }
    }
    if (wtask && wr < tq) {
      if (P.premix) {  // dw_pre: the core row of dL_u S_v
        const float* pl = at(lds, P.gdL, wu, wr, 0);
        const float* ps = at(lds, P.gSc, wv, wr, 0);
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < TB; ++c) s = __builtin_fmaf(pl[c], ps[c], s);
        acc_wpre += s;
      }
      if (P.postmix) {  // dw_post: the core row of dA_u E_v
        const float* pa = at(lds, P.gdAc, wu, wr, 0);
        const float* pe = at(lds, P.gE, wv, wr, 0);
        float s = 0.0f;
#pragma unroll
        for (int c = 0; c < TB; ++c) s = __builtin_fmaf(pa[c], pe[c], s);
        acc_wpost += s;
      }
    }
    if (i0 + tq < T) load_stats(i0 + tq, buf ^ 1);
    __syncthreads();
    // ---- (6) dK += dS^T Q, dV += A^T dO (registers); dQ += dS K (atomics). The next step's
    // first stage writes none of what this one reads, so no barrier follows.
#pragma unroll
    for (int x = 0; x < NKV; ++x) {
      const int kv = wave + x * NW;
      if (kv < 2 * CH * NB) {
        const int kind = kv / (CH * NB), u = (kv / NB) % CH, nb = kv % NB;
        const s16x4 fa = tr_read((kind ? Ab : dSb) + u * TB * LDT, 4 * lg, 0, LDT, lane);
        const s16x4 fb = tr_read((kind ? Oc : Qc) + u * TB * P.ldk, 4 * lg, nb * 16, P.ldk, lane);
        acc_kv[x] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, fb, acc_kv[x], 0, 0, 0);
      }
    }
#pragma unroll
    for (int y = 0; y < NQT; ++y) {
      const int t = wave + y * NW;
      if (t < CH * NB) {
        const int u = t / NB, nb = t % NB;
        const s16x4 fa = *reinterpret_cast<const s16x4*>(dSb + (u * TB + lq) * LDT + 4 * lg);
        const f32x4 c = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(fa, kfrag[y], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int i = i0 + 4 * lg + x;
          if (4 * lg + x < tq && i < T) unsafeAtomicAdd(A.dq_acc + ((bT + i) * M + g * CH + u) * D + nb * 16 + lq, c[x]);
        }
      }
    }
    i0 += tq;
  }

  if (MODE == PASS_D) {
    // the threads of a (head, row) are four consecutive lanes; the first adds their shares
    acc_d += __shfl_xor(acc_d, 1);
    acc_l += __shfl_xor(acc_l, 1);
    acc_d += __shfl_xor(acc_d, 2);
    acc_l += __shfl_xor(acc_l, 2);
    if (tid < CH * TB * 4 && (tid & 3) == 0) {
      const int u = tid / (TB * 4), i = i0 + (tid / 4) % TB;
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
    const int kv = wave + x * NW;
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
  float* red = lds;
  const size_t prow = (size_t)b * A.n_tiles + tile;
  const int ntap = CH * P.cq * P.ck;
  // dtheta: the row groups of each tap added in order
  auto emit_theta = [&](const float (&acc)[EB], float* part) BWT_INLINE {
    const int neb = (P.ck + EB - 1) / EB;
    if (tid < CH * P.cq * neb * nrq) {
      const int rq = tid % nrq, eb = (tid / nrq) % neb, ua = tid / (nrq * neb);  // ua = u * cq + a
#pragma unroll
      for (int j = 0; j < EB; ++j)
        if (EB * eb + j < P.ck) red[(ua * P.ck + EB * eb + j) * nrq + rq] = acc[j];
    }
    __syncthreads();
    for (int x = tid; x < ntap; x += NT) {
      float s = 0.0f;
      for (int rq = 0; rq < nrq; ++rq) s += red[x * nrq + rq];
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

// Launch of one pass for a head group of CH heads; lds = dynamic LDS bytes of the plan.
template <int D, int CH, int MODE, int SPEC, int NT>
hipError_t launch_one(const BwArgs& a, size_t lds, unsigned grid, hipStream_t st) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&bwd_tile_kernel<D, CH, MODE, SPEC, NT>),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_tile_kernel<D, CH, MODE, SPEC, NT>), dim3(grid), dim3(NT), lds, st, a);
  return hipGetLastError();
}

// Specialised shapes instantiated per (head size, heads per group): 1-3 for four-head groups of
// 128 channels, 4 for two- and four-head groups of 96 or 128 channels.
__host__ __device__ constexpr bool spec_built(int spec, int ch, int d) {
  return (spec >= 1 && spec <= 3 && ch == 4 && d == 128) || (spec == 4 && d >= 96 && (ch == 2 || ch == 4));
}

template <int D, int CH, int MODE, int SPEC>
hipError_t launch_nt(const BwArgs& a, size_t lds, unsigned grid, hipStream_t st) {
  if constexpr (SPEC != 0) {
    constexpr int NT = threads_for(spec_plan(MODE, SPEC, CH, D));
    return launch_one<D, CH, MODE, SPEC, NT>(a, lds, grid, st);
  } else {
    return launch_one<D, CH, MODE, 0, 512>(a, lds, grid, st);
  }
}

template <int D, int CH, int MODE>
hipError_t launch_spec(const BwArgs& a, int spec, size_t lds, unsigned grid, hipStream_t st) {
  switch (spec) {
    case 1: if constexpr (spec_built(1, CH, D)) return launch_nt<D, CH, MODE, 1>(a, lds, grid, st); break;
    case 2: if constexpr (spec_built(2, CH, D)) return launch_nt<D, CH, MODE, 2>(a, lds, grid, st); break;
    case 3: if constexpr (spec_built(3, CH, D)) return launch_nt<D, CH, MODE, 3>(a, lds, grid, st); break;
    case 4: if constexpr (spec_built(4, CH, D)) return launch_nt<D, CH, MODE, 4>(a, lds, grid, st); break;
  }
  return launch_nt<D, CH, MODE, 0>(a, lds, grid, st);
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
