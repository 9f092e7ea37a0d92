// Map kernels shared by the unfused forward chain and the backward pass: fp32 [B, M, T, T]
// maps in HBM, one kernel per step of the layer of the page "Multi-Token Attention |
// Summary" (greeksharifa.github.io): logits (§2), head mixing (§3.2), key-query
// convolution with its masks (§3.1), causal row softmax (§2), AV with GroupNorm and gate
// (§3.3). Map indices are 64-bit (a [16, 16384, 16384] map has 2^32 entries). Map rows are
// padded to a multiple of 4 floats (LD = T rounded up) so that rows stream as float4.
#pragma once

#include "mta_device.h"
#include "mta_internal.h"

namespace mta {
namespace {

constexpr int MT_THREADS = 256;
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__host__ __device__ __forceinline__ int map_ld(int T) { return (T + 3) & ~3; }

__device__ __forceinline__ size_t map_index(int bm, int T, int i, int j) {
  return ((size_t)bm * T + i) * map_ld(T) + j;
}

// Workgroups are dispatched round-robin over the 8 XCDs (separate L2 caches). Renumber a
// 3D grid so that every XCD receives one contiguous run of tiles: neighbouring tiles, which
// share halo cache lines, then run on the same XCD at about the same time.
__device__ __forceinline__ uint3 xcd_tile() {
  const unsigned gx = gridDim.x, gy = gridDim.y, n = gx * gy * gridDim.z;
  const unsigned l = blockIdx.x + gx * (blockIdx.y + gy * blockIdx.z);
  const unsigned xcd = l % 8, k = l / 8, per = n / 8, rem = n % 8;
  const unsigned t = xcd * per + (xcd < rem ? xcd : rem) + k;
  return make_uint3(t % gx, (t / gx) % gy, t / (gx * gy));
}

// ---- logits: X[b,m,i,j] = q_i . k_j / sqrt(d) on a 128-query x 128-key tile ----------
// The K tile is staged in LDS; each wave computes S^T blocks (keys are the MFMA rows), so a
// lane holds four consecutive keys of one query and writes them as one float4.
template <typename T, int D>
__global__ __launch_bounds__(MT_THREADS) void logits_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           float* __restrict__ X, int Tn, int M, float scale) {
  typedef Mfma<T> MT;
  constexpr int KT = 128, QPW = 32;             // keys per tile, queries per wave
  constexpr int EPC = 16 / (int)sizeof(T);      // elements per 16-byte chunk
  constexpr int LDKE = D + EPC;                 // padded K row (elements)
  __shared__ __attribute__((aligned(16))) T Ks[KT * LDKE];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int bm = blockIdx.z, b = bm / M, m = bm % M;
  const int i0 = blockIdx.y * (4 * QPW) + wave * QPW, j0 = blockIdx.x * KT;
  const T* qb = q + (size_t)b * Tn * M * D;
  const T* kb = k + (size_t)b * Tn * M * D;
  {
    // all loads first (their latencies overlap), then the LDS stores; rows past T are zero
    constexpr int NL = KT * (D / EPC) / MT_THREADS;
    static_assert(KT * (D / EPC) % MT_THREADS == 0, "K staging split");
    uint4 buf[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      const int r = x / (D / EPC), c = x % (D / EPC);
      const bool in = j0 + r < Tn;
      buf[u] = *reinterpret_cast<const uint4*>(kb + ((size_t)(in ? j0 + r : 0) * M + m) * D + c * EPC);
      if (!in) buf[u] = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      *reinterpret_cast<uint4*>(Ks + (x / (D / EPC)) * LDKE + (x % (D / EPC)) * EPC) = buf[u];
    }
  }
  constexpr int KQ = D / MT::K;
  typename MT::frag qf[QPW / 16][KQ];
#pragma unroll
  for (int qb2 = 0; qb2 < QPW / 16; ++qb2) {
    const int qi = i0 + qb2 * 16 + lr;
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks)
      qf[qb2][ks] = qi < Tn ? MT::load(qb + ((size_t)qi * M + m) * D + ks * MT::K + lg * MT::KPL) : MT::zero();
  }
  __syncthreads();
  const int ld = map_ld(Tn);
#pragma unroll 2
  for (int kb2 = 0; kb2 < KT / 16; ++kb2) {
    f32x4 c[QPW / 16];
#pragma unroll
    for (int qb2 = 0; qb2 < QPW / 16; ++qb2) c[qb2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KQ; ++ks) {
      const typename MT::frag kf = MT::load(Ks + (kb2 * 16 + lr) * LDKE + ks * MT::K + lg * MT::KPL);
#pragma unroll
      for (int qb2 = 0; qb2 < QPW / 16; ++qb2) c[qb2] = MT::mma(kf, qf[qb2][ks], c[qb2]);
    }
    const int j = j0 + kb2 * 16 + 4 * lg;
#pragma unroll
    for (int qb2 = 0; qb2 < QPW / 16; ++qb2) {
      const int qi = i0 + qb2 * 16 + lr;
      if (qi < Tn && j < ld)  // columns T .. ld-1 are row padding, never read
        *reinterpret_cast<float4*>(X + map_index(bm, Tn, qi, j)) =
            make_float4(c[qb2][0] * scale, c[qb2][1] * scale, c[qb2][2] * scale, c[qb2][3] * scale);
    }
  }
}

// ---- head mixing: X_u <- sum_u' w[g][u][u'] Src_u' (Src = X: in place) -----------------
// Each thread mixes two consecutive float4 of every map of the group per step (2 x c_h
// 16-byte loads in flight).
template <int CH>
__global__ __launch_bounds__(MT_THREADS) void mix_kernel(float* X, const float* Src, const float* __restrict__ w,
                                                        int M, size_t n4_per_map) {
  const int bg = blockIdx.y;  // b * (M/CH) + g
  const int G = M / CH;
  const int b = bg / G, g = bg % G;
  float wl[CH][CH];
#pragma unroll
  for (int u = 0; u < CH; ++u)
#pragma unroll
    for (int x = 0; x < CH; ++x) wl[u][x] = w[((size_t)g * CH + u) * CH + x];
  f32x4* base = reinterpret_cast<f32x4*>(X) + ((size_t)b * M + (size_t)g * CH) * n4_per_map;
  const f32x4* src = reinterpret_cast<const f32x4*>(Src) + ((size_t)b * M + (size_t)g * CH) * n4_per_map;
  for (size_t e = ((size_t)blockIdx.x * MT_THREADS + threadIdx.x) * 2; e < n4_per_map;
       e += (size_t)gridDim.x * MT_THREADS * 2) {
    const bool two = e + 1 < n4_per_map;
    f32x4 in[CH][2];
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      in[u][0] = src[(size_t)u * n4_per_map + e];
      in[u][1] = two ? src[(size_t)u * n4_per_map + e + 1] : in[u][0];
    }
#pragma unroll
    for (int u = 0; u < CH; ++u) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        f32x4 o = in[0][h] * wl[u][0];
#pragma unroll
        for (int x = 1; x < CH; ++x) o += in[x][h] * wl[u][x];
        if (h == 0 || two) base[(size_t)u * n4_per_map + e + h] = o;
      }
    }
  }
}

// ---- key-query convolution on a 64 x 64 output tile ----------------------------------
// PRE:  input Mask_0(X) (zero for s > r and outside the map); output -inf for j > i.
// POST: input A (already zero above the diagonal); output 0 for j > i (Mask_0).
// The input tile (c_q - 1 halo rows, 16 halo columns each side) is staged with float4 loads;
// each thread computes 16 consecutive outputs of one row and stores them as four float4.
template <int CK, bool PRE>
__global__ __launch_bounds__(MT_THREADS) void conv_kernel(const float* __restrict__ X, float* __restrict__ Y,
                                                         const float* __restrict__ theta, int Tn, int M,
                                                         int c_q) {
  constexpr int H0 = (CK - 1) / 2;
  constexpr int TW = 64 + 32;     // input columns j0 - 16 .. j0 + 79
  constexpr int LD = TW + 4;
  __shared__ __attribute__((aligned(16))) float tile[(64 + 7) * LD];
  __shared__ float th[8 * CK];
  const uint3 tl = xcd_tile();
  const int bm = tl.z, m = bm % M;
  const int i0 = tl.y * 64, j0 = tl.x * 64;
  const int rows = 64 + c_q - 1;
  const int ld = map_ld(Tn);
  for (int x = threadIdx.x; x < c_q * CK; x += MT_THREADS) th[x] = theta[(size_t)m * c_q * CK + x];
  // all loads of a thread are issued before any is stored, so their latencies overlap;
  // chunks outside the map load a valid address and are zeroed afterwards
  constexpr int NL = ((64 + 7) * (TW / 4) + MT_THREADS - 1) / MT_THREADS;
  float4 buf[NL];
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int x = threadIdx.x + u * MT_THREADS;
    const int rr = x / (TW / 4), c4 = (x % (TW / 4)) * 4;
    const int r = i0 - (c_q - 1) + rr, s = j0 - 16 + c4;
    const bool in = (x < rows * (TW / 4)) & (r >= 0) & (r < Tn) & (s >= 0) & (s < ld);
    buf[u] = *reinterpret_cast<const float4*>(X + map_index(bm, Tn, in ? r : 0, in ? s : 0));
    const int lim = PRE ? min(r, Tn - 1) : Tn - 1;  // padding columns, s > r before softmax
    buf[u].x = (in & (s + 0 <= lim)) ? buf[u].x : 0.0f;
    buf[u].y = (in & (s + 1 <= lim)) ? buf[u].y : 0.0f;
    buf[u].z = (in & (s + 2 <= lim)) ? buf[u].z : 0.0f;
    buf[u].w = (in & (s + 3 <= lim)) ? buf[u].w : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < NL; ++u) {
    const int x = threadIdx.x + u * MT_THREADS;
    if (x < rows * (TW / 4)) *reinterpret_cast<float4*>(tile + (x / (TW / 4)) * LD + (x % (TW / 4)) * 4) = buf[u];
  }
  __syncthreads();
  const int orow = threadIdx.x >> 2;         // 0..63
  const int oc0 = (threadIdx.x & 3) * 16;    // 16 output columns
  float acc[16];
#pragma unroll
  for (int c = 0; c < 16; ++c) acc[c] = 0.0f;
  for (int a = 0; a < c_q; ++a) {
    // output (orow, oc0 + c) reads tile row orow + c_q - 1 - a, tile column oc0 + 16 + c - e + H0
    const float* src = tile + (orow + c_q - 1 - a) * LD + oc0 + 16 - H0;
    float seg[16 + CK - 1];
#pragma unroll
    for (int x = 0; x < 16 + CK - 1; ++x) seg[x] = src[x];
#pragma unroll
    for (int e = 0; e < CK; ++e) {
      const float t = th[a * CK + e];
#pragma unroll
      for (int c = 0; c < 16; ++c) acc[c] += t * seg[c - e + 2 * H0];
    }
  }
  const int i = i0 + orow;
  if (i < Tn) {
    const float masked = PRE ? -__builtin_inff() : 0.0f;
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int j = j0 + oc0 + 4 * v4;
      if (j < ld) {
        float4 o;
        o.x = (j + 0 > i) ? masked : acc[4 * v4 + 0];
        o.y = (j + 1 > i) ? masked : acc[4 * v4 + 1];
        o.z = (j + 2 > i) ? masked : acc[4 * v4 + 2];
        o.w = (j + 3 > i) ? masked : acc[4 * v4 + 3];
        *reinterpret_cast<float4*>(Y + map_index(bm, Tn, i, j)) = o;
      }
    }
  }
}

// ---- key-query convolution on fp16 MFMA (bf16 problems), 64 x 64 output tiles ----------
// Same masks and staging as conv_kernel, the tile held as fp16. For every query lag a the
// banded Toeplitz matrix of theta[m][a][.] (out key n x 32 window keys) is the A operand and
// 8 consecutive window keys of input row i - a the B operand, so a lane ends with four
// consecutive output keys of one query row, stored as one float4. A workgroup walks CT
// consecutive tiles of one (b, m) map: the Toeplitz operands are built once, and the next
// tile's loads are in flight while the current tile is multiplied.
constexpr int CT = 8;

template <bool PRE>
__global__ __launch_bounds__(MT_THREADS) void conv_mfma_kernel(const float* __restrict__ X, float* __restrict__ Y,
                                                              const float* __restrict__ theta, int Tn, int M,
                                                              int c_q, int c_k, int ntx, int ntiles) {
  constexpr int TW = 64 + 32;   // input columns j0 - 16 .. j0 + 79
  constexpr int LDT = TW + 8;   // fp16 row stride
  constexpr int NL = ((64 + 7) * (TW / 4) + MT_THREADS - 1) / MT_THREADS;
  __shared__ __attribute__((aligned(16))) _Float16 tile[(64 + 7) * LDT];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lq = lane & 15, lg = lane >> 4;
  const int bm = blockIdx.y, m = bm % M;
  const int h0 = (c_k - 1) / 2;
  const int rows = 64 + c_q - 1;
  const int ld = map_ld(Tn);
  const int tfirst = blockIdx.x * CT, tend = min(tfirst + CT, ntiles);
  float4 buf[NL];
  auto load_tile = [&](int t) {
    const int i0 = (t / ntx) * 64, j0 = (t % ntx) * 64;
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      const int rr = x / (TW / 4), c4 = (x % (TW / 4)) * 4;
      const int r = i0 - (c_q - 1) + rr, s = j0 - 16 + c4;
      const bool in = (x < rows * (TW / 4)) & (r >= 0) & (r < Tn) & (s >= 0) & (s < ld);
      buf[u] = *reinterpret_cast<const float4*>(X + map_index(bm, Tn, in ? r : 0, in ? s : 0));
      const int lim = PRE ? min(r, Tn - 1) : Tn - 1;
      buf[u].x = (in & (s + 0 <= lim)) ? buf[u].x : 0.0f;
      buf[u].y = (in & (s + 1 <= lim)) ? buf[u].y : 0.0f;
      buf[u].z = (in & (s + 2 <= lim)) ? buf[u].z : 0.0f;
      buf[u].w = (in & (s + 3 <= lim)) ? buf[u].w : 0.0f;
    }
  };
  load_tile(tfirst);
  // Toeplitz operands: out key n = lq, window key k = 8 lg + t, tap e = n - k + 8 + h0
  f16x8 tz[8];
  const float* th = theta + (size_t)m * c_q * c_k;
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int e = lq - (8 * lg + t) + 8 + h0;
      tz[a][t] = (_Float16)((a < c_q && e >= 0 && e < c_k) ? th[a * c_k + e] : 0.0f);
    }
  const float masked = PRE ? -__builtin_inff() : 0.0f;
  for (int t = tfirst; t < tend; ++t) {
    const int i0 = (t / ntx) * 64, j0 = (t % ntx) * 64;
    __syncthreads();  // every wave is done with the previous tile
#pragma unroll
    for (int u = 0; u < NL; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      if (x < rows * (TW / 4)) {
        const f16x4 h = {(_Float16)buf[u].x, (_Float16)buf[u].y, (_Float16)buf[u].z, (_Float16)buf[u].w};
        *reinterpret_cast<f16x4*>(tile + (x / (TW / 4)) * LDT + (x % (TW / 4)) * 4) = h;
      }
    }
    __syncthreads();
    if (t + 1 < tend) load_tile(t + 1);
    const int rl = wave * 16 + lq;  // output row within the tile
    const int i = i0 + rl;
#pragma unroll
    for (int ob = 0; ob < 4; ++ob) {
      f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int a = 0; a < 8; ++a) {
        if (a < c_q) {
          // window keys j0 + 16 ob - 8 + k: tile column 16 ob + 8 + k
          const f16x8 bz = *reinterpret_cast<const f16x8*>(tile + (rl + c_q - 1 - a) * LDT + 16 * ob + 8 + 8 * lg);
          c = __builtin_amdgcn_mfma_f32_16x16x32_f16(tz[a], bz, c, 0, 0, 0);
        }
      }
      const int j = j0 + 16 * ob + 4 * lg;
      if (i < Tn && j < ld) {
        float4 o;
        o.x = (j + 0 > i) ? masked : c[0];
        o.y = (j + 1 > i) ? masked : c[1];
        o.z = (j + 2 > i) ? masked : c[2];
        o.w = (j + 3 > i) ? masked : c[3];
        *reinterpret_cast<float4*>(Y + map_index(bm, Tn, i, j)) = o;
      }
    }
  }
}

// ---- causal row softmax, in place; one workgroup per (b, m, i) row --------------------
// The row is read once into registers (NV float4 per thread), then written once.
__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int o = 32; o > 0; o >>= 1) {
    const float t = __shfl_xor(v, o);
    v = is_max ? fmaxf(v, t) : v + t;
  }
  __syncthreads();  // red is reused between the two reductions
  if (lane == 0) red[wave] = v;
  __syncthreads();
  v = red[0];
#pragma unroll
  for (int w = 1; w < MT_THREADS / 64; ++w) v = is_max ? fmaxf(v, red[w]) : v + red[w];
  return v;
}

// reads the row from Src (= X: in place), writes it to X
template <int NV>
__global__ __launch_bounds__(MT_THREADS) void softmax_kernel(float* X, const float* Src, int Tn) {
  __shared__ float red[MT_THREADS / 64];
  const size_t row = blockIdx.x;  // (b*M + m)*T + i
  const int i = (int)(row % Tn);
  const int ld = map_ld(Tn);
  float4* x = reinterpret_cast<float4*>(X + row * ld);
  const float4* xs = reinterpret_cast<const float4*>(Src + row * ld);
  const float NEG = -__builtin_inff();
  float4 v[NV];
  float mx = NEG;
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const int j = (c * MT_THREADS + threadIdx.x) * 4;
    v[c] = j < ld ? xs[j / 4] : make_float4(NEG, NEG, NEG, NEG);
    if (j + 0 > i) v[c].x = NEG;
    if (j + 1 > i) v[c].y = NEG;
    if (j + 2 > i) v[c].z = NEG;
    if (j + 3 > i) v[c].w = NEG;
    mx = fmaxf(mx, fmaxf(fmaxf(v[c].x, v[c].y), fmaxf(v[c].z, v[c].w)));
  }
  mx = block_reduce(mx, red, true);
  float sum = 0.0f;
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    v[c] = make_float4(expf(v[c].x - mx), expf(v[c].y - mx), expf(v[c].z - mx), expf(v[c].w - mx));
    sum += (v[c].x + v[c].y) + (v[c].z + v[c].w);
  }
  const float inv = 1.0f / block_reduce(sum, red, false);
#pragma unroll
  for (int c = 0; c < NV; ++c) {
    const int j = (c * MT_THREADS + threadIdx.x) * 4;
    if (j < ld) x[j / 4] = make_float4(v[c].x * inv, v[c].y * inv, v[c].z * inv, v[c].w * inv);
  }
}

// rows longer than 16 * 4 * MT_THREADS: three passes over the row
__global__ __launch_bounds__(MT_THREADS) void softmax_long_kernel(float* X, const float* Src, int Tn) {
  __shared__ float red[MT_THREADS / 64];
  const size_t row = blockIdx.x;
  const int i = (int)(row % Tn);
  float* x = X + row * map_ld(Tn);
  const float* xs = Src + row * map_ld(Tn);
  float mx = -__builtin_inff();
  for (int j = threadIdx.x; j <= i; j += MT_THREADS) mx = fmaxf(mx, xs[j]);
  mx = block_reduce(mx, red, true);
  float sum = 0.0f;
  for (int j = threadIdx.x; j <= i; j += MT_THREADS) sum += expf(xs[j] - mx);
  const float inv = 1.0f / block_reduce(sum, red, false);
  // every thread reads its own entries before writing them (in place is safe)
  for (int j = threadIdx.x; j < Tn; j += MT_THREADS) x[j] = (j <= i) ? expf(xs[j] - mx) * inv : 0.0f;
}

// causal row softmax of Src (default: X itself) into X
hipError_t launch_softmax(float* X, const Problem& p, hipStream_t st, const float* Src = nullptr) {
  const dim3 grid((unsigned)((size_t)p.B * p.M * p.T));
  const int nv = (map_ld(p.T) / 4 + MT_THREADS - 1) / MT_THREADS;
  const float* S = Src ? Src : X;
  if (nv <= 1) hipLaunchKernelGGL(softmax_kernel<1>, grid, dim3(MT_THREADS), 0, st, X, S, p.T);
  else if (nv <= 2) hipLaunchKernelGGL(softmax_kernel<2>, grid, dim3(MT_THREADS), 0, st, X, S, p.T);
  else if (nv <= 4) hipLaunchKernelGGL(softmax_kernel<4>, grid, dim3(MT_THREADS), 0, st, X, S, p.T);
  else if (nv <= 8) hipLaunchKernelGGL(softmax_kernel<8>, grid, dim3(MT_THREADS), 0, st, X, S, p.T);
  else if (nv <= 16) hipLaunchKernelGGL(softmax_kernel<16>, grid, dim3(MT_THREADS), 0, st, X, S, p.T);
  else hipLaunchKernelGGL(softmax_long_kernel, grid, dim3(MT_THREADS), 0, st, X, S, p.T);
  return hipGetLastError();
}

// ---- AV + GroupNorm + gate: 128 query rows x d of one (b, m) per workgroup ------------
// Without GroupNorm the product is multiplied by oscale. OT: output element type.
template <typename T, int D, typename OT = T>
__global__ __launch_bounds__(MT_THREADS) void av_kernel(const float* __restrict__ A, const T* __restrict__ v,
                                                       OT* __restrict__ out, const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, float lambda, int gn,
                                                       float oscale, int Tn, int M) {
  typedef Mfma<T> MT;
  constexpr int BKA = 32;
  constexpr int PAD = 16 / (int)sizeof(T);
  constexpr int LDA = BKA + PAD;
  constexpr int LDV = BKA + PAD;
  constexpr int NB = D / 16;
  constexpr int KV = BKA / MT::K;
  __shared__ __attribute__((aligned(16))) T As[128 * LDA];
  __shared__ __attribute__((aligned(16))) T Vt[D * LDV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int bm = blockIdx.y, b = bm / M, m = bm % M;
  const int i0 = blockIdx.x * 128;
  const T* vb = v + (size_t)b * Tn * M * D;
  f32x4 acc[2][NB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < Tn; j0 += BKA) {
    __syncthreads();
    // A tile: 128 rows x 32 keys, fp32 -> T
    for (int x = threadIdx.x; x < 128 * (BKA / 4); x += MT_THREADS) {
      const int r = x / (BKA / 4), c4 = (x % (BKA / 4)) * 4;
      const int i = i0 + r;
      float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < Tn) {
        const float* src = A + map_index(bm, Tn, i, j0 + c4);
        if (j0 + c4 + 3 < Tn) {
          val = *reinterpret_cast<const float4*>(src);
        } else {
          float tmp[4] = {0.f, 0.f, 0.f, 0.f};
          for (int e = 0; e < 4; ++e)
            if (j0 + c4 + e < Tn) tmp[e] = src[e];
          val = make_float4(tmp[0], tmp[1], tmp[2], tmp[3]);
        }
      }
      T* dst = As + r * LDA + c4;
      dst[0] = T(val.x);
      dst[1] = T(val.y);
      dst[2] = T(val.z);
      dst[3] = T(val.w);
    }
    // V^T tile: Vt[c][kk] = V[j0 + kk][c], read in 16-byte chunks of one key row
    constexpr int EPC = 16 / (int)sizeof(T);
    for (int x = threadIdx.x; x < BKA * (D / EPC); x += MT_THREADS) {
      const int kk = x % BKA, c0 = (x / BKA) * EPC;
      const int j = j0 + kk;
      T vals[EPC];
      if (j < Tn) {
        *reinterpret_cast<uint4*>(vals) = *reinterpret_cast<const uint4*>(vb + ((size_t)j * M + m) * D + c0);
      } else {
#pragma unroll
        for (int e = 0; e < EPC; ++e) vals[e] = T(0.0f);
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) Vt[(c0 + e) * LDV + kk] = vals[e];
    }
    __syncthreads();
#pragma unroll
    for (int kv = 0; kv < KV; ++kv)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const typename MT::frag af = MT::load(As + (wave * 32 + rb * 16 + lr) * LDA + kv * MT::K + lg * MT::KPL);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const typename MT::frag bf = MT::load(Vt + (nb * 16 + lr) * LDV + kv * MT::K + lg * MT::KPL);
          acc[rb][nb] = MT::mma(af, bf, acc[rb][nb]);
        }
      }
  }
  OT* ob = out + (size_t)b * Tn * M * D;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = i0 + wave * 32 + rb * 16 + 4 * lg + r;
      float mean = 0.0f, inv = 1.0f;
      if (gn) {
        float s = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s += acc[rb][nb][r];
        mean = row16_sum(s) * (1.0f / D);
        float sq = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float dv = acc[rb][nb][r] - mean;
          sq += dv * dv;
        }
        inv = 1.0f / sqrtf(row16_sum(sq) * (1.0f / D) + 1e-5f);
      }
      if (i < Tn) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int c = nb * 16 + lr;
          float y = acc[rb][nb][r] * oscale;
          if (gn) y = lambda * (gamma[(size_t)m * D + c] * (acc[rb][nb][r] - mean) * inv + beta[(size_t)m * D + c]);
          ob[((size_t)i * M + m) * D + c] = OT(y);
        }
      }
    }
}

// ---- AV + GroupNorm + gate for bf16 tensors: O^T = V^T A^T on MFMA ------------------
// 128 query rows of one (b, m) per workgroup, 32 per wave. The weights stream from the fp32
// map straight into B operands: per 32 keys a lane reads two 16-byte pieces of its query row
// (keys 4g..4g+3 and 16+4g..16+4g+3 for lane group g). V tiles are staged row-major in LDS and
// read transposed (ds_read_b64_tr_b16) in the same key order.
typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ s16x4 v_transposed(const __bf16* Vs, int row0, int col0, int ld, int lane) {
  const int j = lane & 15;  // lane 4k + m of a 16-lane group supplies row row0 + k, columns col0 + 4m ..
  const __bf16* p = Vs + (size_t)(row0 + (j >> 2)) * ld + col0 + 4 * (j & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

template <int D, typename OT = __bf16>
__global__ __launch_bounds__(MT_THREADS) void av_bf16_kernel(const float* __restrict__ A, const __bf16* __restrict__ v,
                                                            OT* __restrict__ out, const float* __restrict__ gamma,
                                                            const float* __restrict__ beta, float lambda, int gn,
                                                            float oscale, int Tn, int M) {
  constexpr int BKA = 32, NB = D / 16, NQ = 2;
  constexpr int LDV = D + 16;
  __shared__ __attribute__((aligned(16))) __bf16 Vs[BKA * LDV];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int lq = lane & 15, lg = lane >> 4;
  const int bm = blockIdx.y, b = bm / M, m = bm % M;
  const int i0 = blockIdx.x * 128 + wave * 32;
  const __bf16* vb = v + (size_t)b * Tn * M * D;
  const int ld = map_ld(Tn);
  f32x4 acc[NB][NQ];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) acc[nb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto load_w = [&](int j0, float4 (&w)[NQ][2]) {
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
      const int i = i0 + qb * 16 + lq;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int j = j0 + 16 * h + 4 * lg;
        w[qb][h] = (i < Tn && j < ld) ? *reinterpret_cast<const float4*>(A + map_index(bm, Tn, i, j))
                                      : make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  };
  // V rows of a chunk: NVL 16-byte pieces per thread (the last round may be partial)
  constexpr int NVL = (BKA * (D / 8) + MT_THREADS - 1) / MT_THREADS;
  auto load_v = [&](int j0, uint4 (&vv)[NVL]) {
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      const int r = x / (D / 8), c = x % (D / 8);
      const bool in = (x < BKA * (D / 8)) & (j0 + r < Tn);
      vv[u] = *reinterpret_cast<const uint4*>(vb + ((size_t)(in ? j0 + r : 0) * M + m) * D + (in ? c * 8 : 0));
      if (!in) vv[u] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  float4 wcur[NQ][2];
  uint4 vcur[NVL];
  load_w(0, wcur);
  load_v(0, vcur);
  for (int j0 = 0; j0 < Tn; j0 += BKA) {
    __syncthreads();  // every wave is done with the previous V tile
#pragma unroll
    for (int u = 0; u < NVL; ++u) {
      const int x = threadIdx.x + u * MT_THREADS;
      if (x < BKA * (D / 8)) *reinterpret_cast<uint4*>(Vs + (x / (D / 8)) * LDV + (x % (D / 8)) * 8) = vcur[u];
    }
    float4 wnext[NQ][2];
    uint4 vnext[NVL];
    load_w(j0 + BKA, wnext);  // next chunk in flight while this one is multiplied
    load_v(j0 + BKA, vnext);
    __syncthreads();
    bf16x8 bp[NQ];
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
      const float4 lo = wcur[qb][0], hi = wcur[qb][1];
      bp[qb] = bf16x8{(__bf16)lo.x, (__bf16)lo.y, (__bf16)lo.z, (__bf16)lo.w,
                      (__bf16)hi.x, (__bf16)hi.y, (__bf16)hi.z, (__bf16)hi.w};
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      s16x4 v8[2] = {v_transposed(Vs, 4 * lg, nb * 16, LDV, lane), v_transposed(Vs, 16 + 4 * lg, nb * 16, LDV, lane)};
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(v8);
#pragma unroll
      for (int qb = 0; qb < NQ; ++qb) acc[nb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bp[qb], acc[nb][qb], 0, 0, 0);
    }
#pragma unroll
    for (int qb = 0; qb < NQ; ++qb) {
      wcur[qb][0] = wnext[qb][0];
      wcur[qb][1] = wnext[qb][1];
    }
#pragma unroll
    for (int u = 0; u < NVL; ++u) vcur[u] = vnext[u];
  }
  // lane (lq, lg) holds O[query i0 + 16 qb + lq][channels 16 nb + 4 lg .. +3]
  OT* ob = out + (size_t)b * Tn * M * D;
#pragma unroll
  for (int qb = 0; qb < NQ; ++qb) {
    const int i = i0 + qb * 16 + lq;
    float mean = 0.0f, inv = 1.0f;
    if (gn) {
      float sum = 0.0f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sum += (acc[nb][qb][0] + acc[nb][qb][1]) + (acc[nb][qb][2] + acc[nb][qb][3]);
      sum += __shfl_xor(sum, 16);
      sum += __shfl_xor(sum, 32);
      mean = sum * (1.0f / D);
      float sq = 0.0f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dv = acc[nb][qb][r] - mean;
          sq += dv * dv;
        }
      sq += __shfl_xor(sq, 16);
      sq += __shfl_xor(sq, 32);
      inv = 1.0f / sqrtf(sq * (1.0f / D) + 1e-5f);
    }
    if (i < Tn) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int c0 = nb * 16 + 4 * lg;
        float y[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          y[r] = acc[nb][qb][r] * oscale;
          if (gn) y[r] = lambda * (gamma[(size_t)m * D + c0 + r] * (acc[nb][qb][r] - mean) * inv + beta[(size_t)m * D + c0 + r]);
        }
        if constexpr (sizeof(OT) == 2) {
          __bf16 h[4] = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
          *reinterpret_cast<uint2*>(ob + ((size_t)i * M + m) * D + c0) = *reinterpret_cast<const uint2*>(h);
        } else {
          *reinterpret_cast<float4*>(ob + ((size_t)i * M + m) * D + c0) = make_float4(y[0], y[1], y[2], y[3]);
        }
      }
    }
  }
}

// out = GN(A V) (gn) or oscale * A V, for every (b, m); OT: output element type
template <typename T, int D, typename OT = T>
hipError_t launch_av_to(const float* A, const T* v, OT* out, const float* gamma, const float* beta, float lambda,
                        int gn, float oscale, int B, int Tn, int M, hipStream_t st) {
  const dim3 grid((Tn + 127) / 128, B * M);
  if constexpr (sizeof(T) == 2) {
    hipLaunchKernelGGL((av_bf16_kernel<D, OT>), grid, dim3(MT_THREADS), 0, st, A, v, out, gamma, beta, lambda, gn,
                       oscale, Tn, M);
  } else {
    hipLaunchKernelGGL((av_kernel<T, D, OT>), grid, dim3(MT_THREADS), 0, st, A, v, out, gamma, beta, lambda, gn,
                       oscale, Tn, M);
  }
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_av(const float* A, const Problem& p, hipStream_t st) {
  return launch_av_to<T, D>(A, reinterpret_cast<const T*>(p.v), reinterpret_cast<T*>(p.out), p.gamma, p.beta,
                            p.lambda, p.gn, 1.0f, p.B, p.T, p.M, st);
}

template <int CK>
hipError_t launch_conv_ck(bool pre, const float* X, float* Y, const Problem& p, hipStream_t st) {
  const dim3 grid((p.T + 63) / 64, (p.T + 63) / 64, p.B * p.M);
  if (pre)
    hipLaunchKernelGGL((conv_kernel<CK, true>), grid, dim3(MT_THREADS), 0, st, X, Y, p.theta_pre, p.T, p.M, p.c_q);
  else
    hipLaunchKernelGGL((conv_kernel<CK, false>), grid, dim3(MT_THREADS), 0, st, X, Y, p.theta_post, p.T, p.M,
                       p.c_q);
  return hipGetLastError();
}

// pre: the convolution before softmax (kernels theta_pre), else after it (theta_post)
hipError_t launch_conv(bool pre, const float* X, float* Y, const Problem& p, hipStream_t st) {
  if (!p.fp32) {  // bf16 problems: fp16 MFMA Toeplitz convolution (fp32 problems stay exact)
    const int ntx = (p.T + 63) / 64, ntiles = ntx * ntx;
    const dim3 grid((ntiles + CT - 1) / CT, p.B * p.M);
    if (pre)
      hipLaunchKernelGGL(conv_mfma_kernel<true>, grid, dim3(MT_THREADS), 0, st, X, Y, p.theta_pre, p.T, p.M, p.c_q,
                         p.c_k, ntx, ntiles);
    else
      hipLaunchKernelGGL(conv_mfma_kernel<false>, grid, dim3(MT_THREADS), 0, st, X, Y, p.theta_post, p.T, p.M,
                         p.c_q, p.c_k, ntx, ntiles);
    return hipGetLastError();
  }
  switch (p.c_k) {
    case 1: return launch_conv_ck<1>(pre, X, Y, p, st);
    case 3: return launch_conv_ck<3>(pre, X, Y, p, st);
    case 5: return launch_conv_ck<5>(pre, X, Y, p, st);
    case 7: return launch_conv_ck<7>(pre, X, Y, p, st);
    case 9: return launch_conv_ck<9>(pre, X, Y, p, st);
    case 11: return launch_conv_ck<11>(pre, X, Y, p, st);
    case 13: return launch_conv_ck<13>(pre, X, Y, p, st);
    case 15: return launch_conv_ck<15>(pre, X, Y, p, st);
    case 17: return launch_conv_ck<17>(pre, X, Y, p, st);
  }
  return hipErrorInvalidValue;
}

// w: the mixing weights of the side being applied (w_pre or w_post); mixes Src (default: X
// itself) into X
hipError_t launch_mix(float* X, const float* w, const Problem& p, hipStream_t st, const float* Src = nullptr) {
  const float* S = Src ? Src : X;
  const size_t n4 = (size_t)p.T * map_ld(p.T) / 4;  // whole padded map, padding included
  const int G = p.M / p.c_h;
  size_t want = (n4 + 2 * MT_THREADS - 1) / (2 * MT_THREADS);
  const unsigned gx = (unsigned)(want < 4096 ? want : 4096);
  const dim3 grid(gx, p.B * G);
  switch (p.c_h) {
    case 1: hipLaunchKernelGGL(mix_kernel<1>, grid, dim3(MT_THREADS), 0, st, X, S, w, p.M, n4); break;
    case 2: hipLaunchKernelGGL(mix_kernel<2>, grid, dim3(MT_THREADS), 0, st, X, S, w, p.M, n4); break;
    case 4: hipLaunchKernelGGL(mix_kernel<4>, grid, dim3(MT_THREADS), 0, st, X, S, w, p.M, n4); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace mta
