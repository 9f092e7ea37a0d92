// Fused Multi-Token Attention forward for bf16 tensors on gfx950, key-major schedule.
//
// Method: page "Multi-Token Attention | Summary" (greeksharifa.github.io), §2 (logits,
// causal softmax, AV), §3.1 (key-query convolution with Mask_0 / Mask_-inf), §3.2
// (head mixing in groups of c_h heads), §3.3 (GroupNorm + scalar gate).
//
// Orientation. Every logit tile is computed transposed, S^T = K Q^T (keys are the MFMA
// rows, queries the columns), so that in the 16x16 accumulator layout a lane owns one
// query and four consecutive keys. Consequences:
//   * softmax statistics of a query are reduced in-lane plus two cross-lane steps;
//   * the weights P^T feed the AV product O^T = V^T P^T directly as the B operand from
//     registers (no LDS round trip): the eight k-slots of lane group g are keys
//     {4g..4g+3} of one 16-key block and {16+4g..16+4g+3} of the next;
//   * V stays row-major in LDS; its transposed A operand (same k-slot permutation) is
//     read with ds_read_b64_tr_b16, which transposes a 4 x 16 block of b16 values
//     within each 16-lane group.
//
// Work split. One workgroup (4 waves) owns batch b, head group g (c_h heads) and a tile
// of R query rows; tile row t is global row i0 - (c_q - 1) + t (the first c_q - 1 rows
// are the query halo of the convolution). Wave w owns head hu = w / (4/c_h) and a slab
// of QW rows.
//
// Key tiles of BK keys stream through LDS. While a tile is being computed the next
// one is already loading into registers (global -> VGPR prefetch), written to LDS
// after the tile. With a convolution the logits of a tile cover keys
// [j0 - 8, j0 + BK + 8): 16-key blocks 0..BK/16, where block 0 equals the last block
// of the previous tile, so each tile computes only BK new key columns (sliding key
// halo); the convolution input lives in an LDS ring of BK/16 + 1 blocks per row.
//
// The c_q x c_k convolution runs on fp16 MFMA: output keys of one 16-key block read a
// 32-key window (blocks ob, ob+1); for each query lag a the banded Toeplitz matrix of
// theta[a][.] is the A operand (constant per workgroup) and the input tile shifted by a
// query rows is the B operand.
//
// Schedules:
//   one pass  (no convolution, or convolution before softmax): online softmax. With
//             mixing after softmax each wave exchanges its weights through LDS and keeps
//             c_h accumulators Acc[u'] = sum_j exp(s_u' - m_u') V_hu, rescaled with
//             head u''s running max; epilogue O = sum_u' w[hu][u'] Acc[u'] / l_u'.
//   two phase (convolution after softmax): phase 1 exact (max, sum) per row, phase 2
//             exact weights -> convolution -> Mask_0 -> AV.
// Mixing before softmax exchanges the scaled logits of the new key blocks through LDS.
#pragma once

#include "mta_device.h"
#include "mta_internal.h"

namespace mta {
namespace kmajor {

constexpr int NW = 4;
constexpr int NT = 64 * NW;
constexpr int CQ_MAX = 8;
constexpr int ZPRE = 8;  // zero rows above the tile in the convolution input ring

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct Args {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const float* theta;
  const float* w;
  const float* gamma;
  const float* beta;
  float lambda;
  __bf16* out;
  int B, T, M;
  int c_q, c_k;
  int kq, mix, gn;
  int r_out;
  int n_tiles;
  int n_groups;
  float qk_scale;  // log2(e)/sqrt(d)
  int xcd_remap;
};

template <int D_, int CH_, int QW_, int BK_, bool KQ_, bool TWO_, bool PAIRS_>
struct Cfg {
  static constexpr int D = D_, CH = CH_, QW = QW_, BK = BK_;
  static constexpr bool KQ = KQ_, TWO = TWO_, PAIRS = PAIRS_;
  static constexpr int WPH = NW / CH;        // waves per head
  static constexpr int R = QW * WPH;         // tile rows
  static constexpr int NQB = QW / 16;        // query blocks per wave
  static constexpr int NKB = BK / 16;        // new key blocks per tile
  static constexpr int LB = KQ ? NKB + 1 : NKB;  // logit blocks per tile (with the carried halo)
  static constexpr int KS = D / 32;          // k-steps of QK^T
  static constexpr int NB = D / 16;          // channel blocks
  static constexpr int NC = BK / 32;         // 32-key chunks of AV
  static constexpr int NP = PAIRS ? CH : 1;
  static constexpr int KROWS = KQ ? BK + 16 : BK;  // K rows in LDS
  static constexpr int LDK = D + 8;          // K row stride (bf16): 16-byte reads conflict-free
  static constexpr int LDV = D + 16;         // V row stride (bf16): transposed reads conflict-free
  static constexpr int ZW = LB * 16;         // ring width (keys)
  static constexpr int LDZ = ZW + 8;         // fp16 stride
  static constexpr int ZROWS = ZPRE + R;
  static constexpr int LDX = LB * 16 + 4;    // fp32 mixing exchange stride
  static constexpr size_t KS_BYTES = (size_t)CH * KROWS * LDK * 2;
  static constexpr size_t SX_BYTES = (size_t)CH * R * LDX * 4;
  static constexpr size_t U_BYTES = KS_BYTES > SX_BYTES ? KS_BYTES : SX_BYTES;
  static constexpr size_t VS_BYTES = (size_t)CH * BK * LDV * 2;
  static constexpr size_t ZB_BYTES = KQ ? (size_t)CH * ZROWS * LDZ * 2 : 0;
  static constexpr size_t PB_BYTES = PAIRS ? (size_t)CH * WPH * NQB * NC * 64 * 16 : 0;
  static constexpr size_t ST_BYTES = (size_t)CH * R * 2 * 4;
  static constexpr size_t OFF_U = 0;
  static constexpr size_t OFF_VS = OFF_U + U_BYTES;
  static constexpr size_t OFF_ZB = OFF_VS + VS_BYTES;
  static constexpr size_t OFF_PB = OFF_ZB + ZB_BYTES;
  static constexpr size_t OFF_ST = OFF_PB + PB_BYTES;
  static constexpr size_t LDS_BYTES = OFF_ST + ST_BYTES;
  // register prefetch of one regular tile (16-byte chunks per thread)
  static constexpr int KCH = CH * BK * (D / 8);
  static constexpr int VCH = CH * BK * (D / 8);
  static constexpr int KPT = (KCH + NT - 1) / NT;
  static constexpr int VPT = (VCH + NT - 1) / NT;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(QW % 16 == 0 && BK % 32 == 0 && D % 32 == 0, "tile shape");
  static_assert(KCH % NT == 0 && VCH % NT == 0, "staging split");
};

__device__ __forceinline__ bf16x8 pack_bf16(const f32x4& lo, const f32x4& hi) {
  bf16x8 r;
  r[0] = (__bf16)lo[0];
  r[1] = (__bf16)lo[1];
  r[2] = (__bf16)lo[2];
  r[3] = (__bf16)lo[3];
  r[4] = (__bf16)hi[0];
  r[5] = (__bf16)hi[1];
  r[6] = (__bf16)hi[2];
  r[7] = (__bf16)hi[3];
  return r;
}

__device__ __forceinline__ float xgroup_max(float x) {  // over the 4 lane groups (same query)
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}

__device__ __forceinline__ float xgroup_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Transposed read of V: lane i of each 16-lane group receives V[row0 + 0..3][col0 + i].
// In a group, lane 4k + m supplies the address of row row0 + k, columns col0 + 4m ..+3.
__device__ __forceinline__ s16x4 vtr(const __bf16* Vs, int row0, int col0, int ld, int lane) {
  const int j = lane & 15;
  const __bf16* p = Vs + (size_t)(row0 + (j >> 2)) * ld + col0 + 4 * (j & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

template <class C>
__global__ __launch_bounds__(NT, 1) void kmajor_kernel(Args A) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  __bf16* Ks = reinterpret_cast<__bf16*>(smem + C::OFF_U);
  float* Sx = reinterpret_cast<float*>(smem + C::OFF_U);  // aliases Ks (after QK^T)
  __bf16* Vs = reinterpret_cast<__bf16*>(smem + C::OFF_VS);
  _Float16* Zb = reinterpret_cast<_Float16*>(smem + C::OFF_ZB);
  u32x4* Pb = reinterpret_cast<u32x4*>(smem + C::OFF_PB);
  float* St_a = reinterpret_cast<float*>(smem + C::OFF_ST);
  float* St_l = St_a + C::CH * C::R;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hu = wave / C::WPH;
  const int slab = wave % C::WPH;
  const int qs0 = slab * C::QW;  // first tile row of this wave
  const int lq = lane & 15;      // query within a block (D layout column)
  const int lg = lane >> 4;      // lane group: keys 4*lg..4*lg+3 of a block

  // ---- workgroup -> (b, group, tile), heaviest tiles first ----------------------------
  const int n_bg = A.B * A.n_groups;
  int bg, rank;
  if (A.xcd_remap) {
    const int xcd = blockIdx.x & 7, kx = blockIdx.x >> 3, per = n_bg >> 3;
    rank = kx / per;
    bg = (kx % per) * 8 + xcd;
  } else {
    rank = blockIdx.x / n_bg;
    bg = blockIdx.x % n_bg;
  }
  const int qt = A.n_tiles - 1 - rank;
  const int b = bg / A.n_groups, g = bg % A.n_groups;
  const int T_ = A.T, M = A.M;
  const int cq1 = C::KQ ? A.c_q - 1 : 0;
  const int h0 = C::KQ ? (A.c_k - 1) / 2 : 0;
  const int i0 = qt * A.r_out;
  const int row0 = i0 - cq1;
  const int last_row = min(i0 + A.r_out, T_) - 1;
  const int n_kt = last_row / C::BK + 1;
  const int m_head = g * C::CH + hu;
  const bool mix_pre = A.mix == MIX_PRE;
  const int wrow_min = row0 + qs0;           // smallest global row of this wave
  const size_t bstride = (size_t)T_ * M * C::D;
  const __bf16* qb_ = A.q + b * bstride;
  const __bf16* kb_ = A.k + b * bstride;
  const __bf16* vb_ = A.v + b * bstride;

  // ---- Q^T operands (B of QK^T) in registers ------------------------------------------
  bf16x8 qf[C::NQB][C::KS];
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    const int gr = row0 + qs0 + qb * 16 + lq;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      if (gr >= 0 && gr < T_)
        qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qb_ + ((size_t)gr * M + m_head) * C::D + ks * 32 + lg * 8);
      else
        qf[qb][ks] = bf16x8{};
    }
  }

  // ---- Toeplitz A operands: out key n (row), window key k = 8*lg + s (slot) ------------
  // window key k is global key j0 - 8 + 16*ob + k; out key is j0 + 16*ob + n;
  // tap e = n - k + 8 + h0.
  f16x8 tz[C::KQ ? CQ_MAX : 1];
  if constexpr (C::KQ) {
    const float* th = A.theta + (size_t)m_head * A.c_q * A.c_k;
#pragma unroll
    for (int a = 0; a < CQ_MAX; ++a) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int e = lq - (8 * lg + s) + 8 + h0;
        float t = 0.0f;
        if (a < A.c_q && e >= 0 && e < A.c_k) t = th[a * A.c_k + e];
        tz[a][s] = (_Float16)t;
      }
    }
    for (int x = tid; x < C::CH * ZPRE * C::LDZ; x += NT) {
      const int u = x / (ZPRE * C::LDZ);
      Zb[(size_t)u * C::ZROWS * C::LDZ + (x - u * ZPRE * C::LDZ)] = (_Float16)0.0f;
    }
  }

  float wmix[C::CH];
#pragma unroll
  for (int u = 0; u < C::CH; ++u)
    wmix[u] = A.mix ? A.w[((size_t)g * C::CH + hu) * C::CH + u] : 0.0f;

  f32x4 acc[C::NP][C::NB][C::NQB];
#pragma unroll
  for (int p = 0; p < C::NP; ++p)
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) acc[p][nb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};

  float m_run[C::NQB], l_run[C::NQB];  // per query (replicated over lane groups)
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    m_run[qb] = -1e30f;
    l_run[qb] = 0.0f;  // per-lane partial sum in the one-pass schedule
  }
  const float NEG_INF = -__builtin_inff();

  // ---- staging helpers ------------------------------------------------------------------
  // K rows [kfirst, kfirst + nrows) of the group's heads -> Ks rows [lrow, lrow + nrows)
  auto stage_k_direct = [&](int kfirst, int nrows, int lrow) {
    const int total = C::CH * nrows * (C::D / 8);
    for (int c = tid; c < total; c += NT) {
      const int u = c / (nrows * (C::D / 8));
      const int rem = c - u * nrows * (C::D / 8);
      const int r = rem / (C::D / 8), cc = rem % (C::D / 8);
      const int j = kfirst + r;
      u32x4 val = u32x4{0, 0, 0, 0};
      if (j >= 0 && j < T_) val = *reinterpret_cast<const u32x4*>(kb_ + ((size_t)j * M + g * C::CH + u) * C::D + cc * 8);
      *reinterpret_cast<u32x4*>(Ks + ((size_t)u * C::KROWS + lrow + r) * C::LDK + cc * 8) = val;
    }
  };
  auto stage_v_direct = [&](int j0) {
    constexpr int total = C::CH * C::BK * (C::D / 8);
    for (int c = tid; c < total; c += NT) {
      const int u = c / (C::BK * (C::D / 8));
      const int rem = c - u * C::BK * (C::D / 8);
      const int r = rem / (C::D / 8), cc = rem % (C::D / 8);
      const int j = j0 + r;
      u32x4 val = u32x4{0, 0, 0, 0};
      if (j < T_) val = *reinterpret_cast<const u32x4*>(vb_ + ((size_t)j * M + g * C::CH + u) * C::D + cc * 8);
      *reinterpret_cast<u32x4*>(Vs + ((size_t)u * C::BK + r) * C::LDV + cc * 8) = val;
    }
  };
  u32x4 pk[C::KPT], pv[C::VPT];
  auto prefetch = [&](int kfirst, int j0, bool with_v) {
#pragma unroll
    for (int x = 0; x < C::KPT; ++x) {
      const int c = tid + x * NT;
      const int u = c / (C::BK * (C::D / 8));
      const int rem = c - u * C::BK * (C::D / 8);
      const int r = rem / (C::D / 8), cc = rem % (C::D / 8);
      const int j = kfirst + r;
      pk[x] = (j >= 0 && j < T_) ? *reinterpret_cast<const u32x4*>(kb_ + ((size_t)j * M + g * C::CH + u) * C::D + cc * 8)
                                 : u32x4{0, 0, 0, 0};
    }
    if (with_v) {
#pragma unroll
      for (int x = 0; x < C::VPT; ++x) {
        const int c = tid + x * NT;
        const int u = c / (C::BK * (C::D / 8));
        const int rem = c - u * C::BK * (C::D / 8);
        const int r = rem / (C::D / 8), cc = rem % (C::D / 8);
        const int j = j0 + r;
        pv[x] = (j < T_) ? *reinterpret_cast<const u32x4*>(vb_ + ((size_t)j * M + g * C::CH + u) * C::D + cc * 8)
                         : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto commit = [&](int lrow, bool with_v) {
#pragma unroll
    for (int x = 0; x < C::KPT; ++x) {
      const int c = tid + x * NT;
      const int u = c / (C::BK * (C::D / 8));
      const int rem = c - u * C::BK * (C::D / 8);
      const int r = rem / (C::D / 8), cc = rem % (C::D / 8);
      *reinterpret_cast<u32x4*>(Ks + ((size_t)u * C::KROWS + lrow + r) * C::LDK + cc * 8) = pk[x];
    }
    if (with_v) {
#pragma unroll
      for (int x = 0; x < C::VPT; ++x) {
        const int c = tid + x * NT;
        const int u = c / (C::BK * (C::D / 8));
        const int rem = c - u * C::BK * (C::D / 8);
        const int r = rem / (C::D / 8), cc = rem % (C::D / 8);
        *reinterpret_cast<u32x4*>(Vs + ((size_t)u * C::BK + r) * C::LDV + cc * 8) = pv[x];
      }
    }
  };

  // ---- compute helpers --------------------------------------------------------------------
  f32x4 s[C::LB][C::NQB];
  // S^T of logit blocks [lb0, lb1) from K rows at Ks row 16*lb (times the scale), then
  // the optional mixing across heads (through LDS) of the same blocks.
  auto logits = [&](int lb0, int lb1) {
#pragma unroll
    for (int lb = 0; lb < C::LB; ++lb) {
      if (lb < lb0 || lb >= lb1) continue;
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) s[lb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(
            Ks + ((size_t)hu * C::KROWS + lb * 16 + lq) * C::LDK + ks * 32 + lg * 8);
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb)
          s[lb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[qb][ks], s[lb][qb], 0, 0, 0);
      }
    }
    if (mix_pre) {
      __syncthreads();  // all waves finished reading Ks (Sx aliases it)
#pragma unroll
      for (int lb = 0; lb < C::LB; ++lb) {
        if (lb < lb0 || lb >= lb1) continue;
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb)
          *reinterpret_cast<f32x4*>(Sx + ((size_t)hu * C::R + qs0 + qb * 16 + lq) * C::LDX + (lb - lb0) * 16 + lg * 4) =
              s[lb][qb] * A.qk_scale;
      }
      __syncthreads();
#pragma unroll
      for (int lb = 0; lb < C::LB; ++lb) {
        if (lb < lb0 || lb >= lb1) continue;
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < C::CH; ++u) {
            const f32x4 o = *reinterpret_cast<const f32x4*>(
                Sx + ((size_t)u * C::R + qs0 + qb * 16 + lq) * C::LDX + (lb - lb0) * 16 + lg * 4);
            x += wmix[u] * o;
          }
          s[lb][qb] = x;
        }
      }
    } else {
#pragma unroll
      for (int lb = 0; lb < C::LB; ++lb) {
        if (lb < lb0 || lb >= lb1) continue;
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) s[lb][qb] *= A.qk_scale;
      }
    }
  };

  // convolution of the ring (logical blocks of tile kt) -> cv[ob][qb]
  f32x4 cv[C::NKB][C::NQB];
  auto ring_col = [&](int kt, int lb) { return ((kt * C::NKB + lb) % C::LB) * 16; };
  auto convolve = [&](int kt) {
#pragma unroll
    for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) cv[ob][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ob = 0; ob < C::NKB; ++ob) {
      // slots of lane group lg: window keys 8*lg .. 8*lg+7 = block ob (lg < 2) or ob+1
      const int col = ring_col(kt, ob + (lg >> 1)) + (lg & 1) * 8;
#pragma unroll
      for (int a = 0; a < CQ_MAX; ++a) {
        if (a < A.c_q) {
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            const f16x8 bz = *reinterpret_cast<const f16x8*>(
                Zb + ((size_t)hu * C::ZROWS + ZPRE + qs0 + qb * 16 + lq - a) * C::LDZ + col);
            cv[ob][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(tz[a], bz, cv[ob][qb], 0, 0, 0);
          }
        }
      }
    }
  };
  // write logit-derived values of block lb (D layout) into the ring
  auto ring_store = [&](int kt, int lb, int qb, const f32x4& val) {
    _Float16 h[4] = {(_Float16)val[0], (_Float16)val[1], (_Float16)val[2], (_Float16)val[3]};
    *reinterpret_cast<uint2*>(Zb + ((size_t)hu * C::ZROWS + ZPRE + qs0 + qb * 16 + lq) * C::LDZ + ring_col(kt, lb) +
                              lg * 4) = *reinterpret_cast<uint2*>(h);
  };

  // AV of the weight blocks pw[NKB][NQB] (out keys of this tile) against V of head hu
  auto av = [&](f32x4 (&pw)[C::NKB][C::NQB]) {
    if constexpr (C::PAIRS) {
      // publish this wave's weights in the fragment layout, then use every head's
#pragma unroll
      for (int c = 0; c < C::NC; ++c)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          const bf16x8 bp = pack_bf16(pw[2 * c][qb], pw[2 * c + 1][qb]);
          Pb[(((size_t)hu * C::WPH + slab) * C::NQB + qb) * C::NC * 64 + c * 64 + lane] =
              *reinterpret_cast<const u32x4*>(&bp);
        }
      __syncthreads();
    }
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      bf16x8 bp[C::NP][C::NQB];
#pragma unroll
      for (int p = 0; p < C::NP; ++p)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          if constexpr (C::PAIRS) {
            const u32x4 raw = Pb[(((size_t)p * C::WPH + slab) * C::NQB + qb) * C::NC * 64 + c * 64 + lane];
            bp[p][qb] = *reinterpret_cast<const bf16x8*>(&raw);
          } else {
            bp[p][qb] = pack_bf16(pw[2 * c][qb], pw[2 * c + 1][qb]);
          }
        }
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        // V^T operand: channels nb*16 + (lane & 15); k-slots = keys {4lg..4lg+3} of
        // block 2c and {16+4lg..} of block 2c+1 of this tile
        const s16x4 lo = vtr(Vs + (size_t)hu * C::BK * C::LDV, c * 32 + 4 * lg, nb * 16, C::LDV, lane);
        const s16x4 hi = vtr(Vs + (size_t)hu * C::BK * C::LDV, c * 32 + 16 + 4 * lg, nb * 16, C::LDV, lane);
        s16x4 v8[2] = {lo, hi};
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(v8);
#pragma unroll
        for (int p = 0; p < C::NP; ++p)
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb)
            acc[p][nb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bp[p][qb], acc[p][nb][qb], 0, 0, 0);
      }
    }
  };

  f32x4 pw[C::NKB][C::NQB];

  if constexpr (!C::TWO) {
    // ============================= one pass ==============================================
    if constexpr (C::KQ) stage_k_direct(-8, C::BK + 16, 0);
    else stage_k_direct(0, C::BK, 0);
    stage_v_direct(0);
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
      const int j0 = kt * C::BK;
      const bool more = kt + 1 < n_kt;
      if (more) prefetch(C::KQ ? j0 + C::BK + 8 : j0 + C::BK, j0 + C::BK, true);
      const int lb0 = (C::KQ && kt > 0) ? 1 : 0;
      logits(lb0, C::LB);
      if constexpr (C::KQ) {
        // Mask_0 on the new blocks (keys kbase + 16 lb + 4 lg + i, kbase = j0 - 8)
        const bool edge = (j0 - 8 < 0) || (j0 + C::BK + 8 - 1 > wrow_min) || (wrow_min < 0);
#pragma unroll
        for (int lb = 0; lb < C::LB; ++lb) {
          if (lb < lb0) continue;
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            f32x4 z = s[lb][qb];
            if (edge) {
              const int gr = row0 + qs0 + qb * 16 + lq;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int j = j0 - 8 + lb * 16 + 4 * lg + i;
                if (!(gr >= 0 && j >= 0 && j <= gr)) z[i] = 0.0f;
              }
            }
            ring_store(kt, lb, qb, z);
          }
        }
        __syncthreads();
        convolve(kt);
      } else {
#pragma unroll
        for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) cv[ob][qb] = s[ob][qb];
      }
      // Mask_-inf and online softmax per query
      const bool edge = (j0 + C::BK - 1 > wrow_min) || (qs0 < cq1) || (wrow_min + C::QW > T_);
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        const int t = qs0 + qb * 16 + lq;
        const int gr = row0 + t;
        const bool row_ok = t >= cq1 && gr < T_;
        float mx = NEG_INF;
#pragma unroll
        for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = cv[ob][qb][i];
            if (edge) {
              const int j = j0 + ob * 16 + 4 * lg + i;
              if (!(row_ok && j <= gr)) x = NEG_INF;
            }
            cv[ob][qb][i] = x;
            mx = fmaxf(mx, x);
          }
        mx = xgroup_max(mx);
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha = fast_exp2(m_run[qb] - m_new);
        float sum = 0.0f;
#pragma unroll
        for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = fast_exp2(cv[ob][qb][i] - m_new);
            pw[ob][qb][i] = pv;
            sum += pv;
          }
        l_run[qb] = l_run[qb] * alpha + sum;
        m_run[qb] = m_new;
        if constexpr (C::PAIRS) {
          if (lg == 0) St_a[hu * C::R + t] = alpha;
        } else {
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) acc[0][nb][qb] *= alpha;
        }
      }
      if constexpr (C::PAIRS) {
        __syncthreads();  // rescale factors of every head are visible (and Pb reuse is safe)
#pragma unroll
        for (int p = 0; p < C::NP; ++p)
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            const float al = St_a[p * C::R + qs0 + qb * 16 + lq];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) acc[p][nb][qb] *= al;
          }
      }
      av(pw);
      __syncthreads();  // every wave is done with Ks, Vs, Zb, Pb of this tile
      if (more) commit(C::KQ ? 16 : 0, true);
      __syncthreads();
    }
    // final per-query sums (partial per lane group until here)
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      l_run[qb] = xgroup_sum(l_run[qb]);
      if (lg == 0) St_l[hu * C::R + qs0 + qb * 16 + lq] = l_run[qb];
    }
    __syncthreads();
  } else {
    // ============================= two phase ============================================
    // phase 1: exact (max, sum) of every tile row of head hu (after mixing)
    stage_k_direct(0, C::BK, 0);
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
      const int j0 = kt * C::BK;
      const bool more = kt + 1 < n_kt;
      if (more) prefetch(j0 + C::BK, 0, false);
      logits(0, C::NKB);  // phase 1 needs no key halo
      const bool edge = (j0 + C::BK - 1 > wrow_min) || (wrow_min < 0) || (wrow_min + C::QW > T_);
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        const int gr = row0 + qs0 + qb * 16 + lq;
        const bool row_ok = gr >= 0 && gr < T_;
        float mx = NEG_INF;
#pragma unroll
        for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float x = s[ob][qb][i];
            if (edge) {
              const int j = j0 + ob * 16 + 4 * lg + i;
              if (!(row_ok && j <= gr)) x = NEG_INF;
            }
            s[ob][qb][i] = x;
            mx = fmaxf(mx, x);
          }
        mx = xgroup_max(mx);
        const float m_new = fmaxf(m_run[qb], mx);
        float sum = 0.0f;
#pragma unroll
        for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
          for (int i = 0; i < 4; ++i) sum += fast_exp2(s[ob][qb][i] - m_new);
        l_run[qb] = l_run[qb] * fast_exp2(m_run[qb] - m_new) + sum;
        m_run[qb] = m_new;
      }
      __syncthreads();
      if (more) commit(0, false);
      __syncthreads();
    }
    // per-query normaliser folded into the exponent: p = exp2(x - (m + log2 l))
    float shift[C::NQB];
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      const float l = xgroup_sum(l_run[qb]);
      shift[qb] = l > 0.0f ? m_run[qb] + __builtin_log2f(l) : 1e30f;
    }

    // phase 2: exact weights (sliding key halo) -> convolution -> Mask_0 -> AV
    stage_k_direct(-8, C::BK + 16, 0);
    stage_v_direct(0);
    __syncthreads();
    for (int kt = 0; kt < n_kt; ++kt) {
      const int j0 = kt * C::BK;
      const bool more = kt + 1 < n_kt;
      if (more) prefetch(j0 + C::BK + 8, j0 + C::BK, true);
      const int lb0 = kt > 0 ? 1 : 0;
      logits(lb0, C::LB);
      const bool edge = (j0 - 8 < 0) || (j0 + C::BK + 8 - 1 > wrow_min) || (wrow_min < 0) ||
                        (wrow_min + C::QW > T_);
#pragma unroll
      for (int lb = 0; lb < C::LB; ++lb) {
        if (lb < lb0) continue;
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          const int gr = row0 + qs0 + qb * 16 + lq;
          f32x4 pv;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pv[i] = fast_exp2(s[lb][qb][i] - shift[qb]);
            if (edge) {
              const int j = j0 - 8 + lb * 16 + 4 * lg + i;
              if (!(gr >= 0 && gr < T_ && j >= 0 && j <= gr)) pv[i] = 0.0f;
            }
          }
          ring_store(kt, lb, qb, pv);
        }
      }
      __syncthreads();
      convolve(kt);
      const bool edge2 = (j0 + C::BK - 1 > wrow_min) || (qs0 < cq1) || (wrow_min + C::QW > T_);
#pragma unroll
      for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          f32x4 c = cv[ob][qb];
          if (edge2) {
            const int t = qs0 + qb * 16 + lq;
            const int gr = row0 + t;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = j0 + ob * 16 + 4 * lg + i;
              if (!(t >= cq1 && gr < T_ && j <= gr)) c[i] = 0.0f;
            }
          }
          pw[ob][qb] = c;
        }
      av(pw);
      __syncthreads();
      if (more) commit(16, true);
      __syncthreads();
    }
  }

  // ============================= epilogue =================================================
  __bf16* ob_ = A.out + b * bstride;
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    const int t = qs0 + qb * 16 + lq;
    const int gr = row0 + t;
    f32x4 o[C::NB];
    if constexpr (C::PAIRS) {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < C::NP; ++p) {
        float sc = wmix[p];
        if constexpr (!C::TWO) {
          const float l = St_l[p * C::R + t];
          sc = l > 0.0f ? sc / l : 0.0f;
        }
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) o[nb] += acc[p][nb][qb] * sc;
      }
    } else {
      float sc = 1.0f;
      if constexpr (!C::TWO) sc = l_run[qb] > 0.0f ? 1.0f / l_run[qb] : 0.0f;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[nb] = acc[0][nb][qb] * sc;
    }
    float mean = 0.0f, inv = 1.0f;
    if (A.gn) {
      float sum = 0.0f;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) sum += o[nb][0] + o[nb][1] + o[nb][2] + o[nb][3];
      mean = xgroup_sum(sum) * (1.0f / C::D);
      float sq = 0.0f;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float dv = o[nb][i] - mean;
          sq += dv * dv;
        }
      inv = 1.0f / sqrtf(xgroup_sum(sq) * (1.0f / C::D) + 1e-5f);
    }
    if (t >= cq1 && gr < T_) {
      __bf16* dst = ob_ + ((size_t)gr * M + m_head) * C::D;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const int c0 = nb * 16 + 4 * lg;
        __bf16 y[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float val = o[nb][i];
          if (A.gn)
            val = A.lambda * (A.gamma[(size_t)m_head * C::D + c0 + i] * (val - mean) * inv +
                              A.beta[(size_t)m_head * C::D + c0 + i]);
          y[i] = (__bf16)val;
        }
        *reinterpret_cast<uint2*>(dst + c0) = *reinterpret_cast<const uint2*>(y);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
template <class C>
hipError_t launch(const Problem& p, hipStream_t stream) {
  Args a;
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.k = reinterpret_cast<const __bf16*>(p.k);
  a.v = reinterpret_cast<const __bf16*>(p.v);
  a.theta = p.theta;
  a.w = p.w;
  a.gamma = p.gamma;
  a.beta = p.beta;
  a.lambda = p.lambda;
  a.out = reinterpret_cast<__bf16*>(p.out);
  a.B = p.B;
  a.T = p.T;
  a.M = p.M;
  a.kq = p.kq;
  a.mix = p.mix;
  a.gn = p.gn;
  a.c_q = p.kq ? p.c_q : 1;
  a.c_k = p.kq ? p.c_k : 1;
  a.r_out = C::R - (a.c_q - 1);
  a.n_tiles = (p.T + a.r_out - 1) / a.r_out;
  a.n_groups = p.M / C::CH;
  a.qk_scale = (float)(1.4426950408889634 / __builtin_sqrt((double)p.d));
  const int n_bg = p.B * a.n_groups;
  a.xcd_remap = (n_bg % 8 == 0) ? 1 : 0;
  const long long blocks = (long long)n_bg * a.n_tiles;
  if (blocks <= 0 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kmajor_kernel<C>, dim3((unsigned)blocks), dim3(NT), 0, stream, a);
  return hipGetLastError();
}

// Tile shapes: per-pair accumulators take c_h * d * QW fp32 per wave, which limits QW.
template <int D, int CH, bool KQ, bool TWO, bool PAIRS>
hipError_t launch_shape(const Problem& p, hipStream_t stream) {
  constexpr int BK = (CH == 4) ? 32 : 64;
  constexpr int QW = (PAIRS || CH == 2) ? 32 : 64;
  return launch<Cfg<D, CH, QW, BK, KQ, TWO, PAIRS>>(p, stream);
}

template <int D, int CH>
hipError_t launch_ch(const Problem& p, hipStream_t stream) {
  const bool pairs = p.mix == MIX_POST && CH > 1;
  if (p.kq == KQ_POST) {
    if (pairs) return launch_shape<D, CH, true, true, true>(p, stream);
    return launch_shape<D, CH, true, true, false>(p, stream);
  }
  if (p.kq == KQ_PRE) {
    if (pairs) return launch_shape<D, CH, true, false, true>(p, stream);
    return launch_shape<D, CH, true, false, false>(p, stream);
  }
  if (pairs) return launch_shape<D, CH, false, false, true>(p, stream);
  return launch_shape<D, CH, false, false, false>(p, stream);
}

template <int D>
hipError_t launch_d(const Problem& p, hipStream_t stream) {
  const int ch = p.mix ? p.c_h : 1;
  switch (ch) {
    case 1: return launch_ch<D, 1>(p, stream);
    case 2: return launch_ch<D, 2>(p, stream);
    case 4: return launch_ch<D, 4>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kmajor
}  // namespace mta
