// Fused Multi-Token Attention forward for fp32 tensors on gfx950 (template implementation; one
// launch, no T x T maps in HBM). bf16 tensors run the key-major kernel of mta_kmajor_impl.h;
// this template serves the fp32 head sizes 16, 32 and 64, with every product (logits,
// Toeplitz convolution, AV) on the fp32 16x16x4 MFMA and fp32 operands in LDS.
//
// Method: page "Multi-Token Attention | Summary" (greeksharifa.github.io), §2 (logits,
// causal softmax, AV), §3.1 (key-query convolution with Mask_0 / Mask_-inf), §3.2
// (head mixing within groups of c_h heads), §3.3 (GroupNorm + scalar gate).
//
// One workgroup (4 waves) owns one batch b, one head group g (c_h heads) and one tile
// of query rows. Tile row t maps to global row i0 - (c_q-1) + t: the first c_q-1 rows
// are the query halo that the convolution reads (recomputed, never output). Each
// wave owns one head of the group and a slab of WR rows.
//
// Three schedules, chosen at compile time:
//  * one pass (no convolution, or convolution before softmax). Per key tile:
//      logits of the tile plus a 16-column key halo (fp32 MFMA)
//      -> [mix before softmax, through LDS] -> Mask_0 -> fp32 in LDS
//      -> c_q x c_k convolution as c_q banded-Toeplitz MFMAs per 16x16 block
//      -> Mask_-inf -> online softmax per (row, head)
//      -> AV. With mixing after softmax every wave keeps c_h accumulators
//         Acc[u'][v] = sum_j exp(s_u' - m_u') V_v (one per input head u' of its output
//         head v), each rescaled by its own head's running max; the mix is applied
//         once, in the epilogue: O_v = sum_u' w[v][u'] Acc[u'][v] / l_u'.
//  * two phase (convolution after softmax, which mixes rows with different
//    normalisers): phase 1 computes exact (max, sum) of every tile row (halo
//    included); phase 2 recomputes the logits with the key halo, forms the exact
//    softmax weights, convolves them (Toeplitz MFMA), applies Mask_0 and does AV.
//  * both sides (a convolution before and one after softmax, each head with its own two
//    kernels): phase 1 as the one-pass front (logits with the key halo -> Mask_0 ->
//    convolution -> Mask_-inf) for the exact (max, sum) of the softmax inputs; phase 2
//    computes the logits with twice the key halo, convolves them into softmax inputs over
//    the keys the second convolution reads, turns those into exact weights in a second
//    ring, convolves that and does AV. An output row then reads 2 (c_q - 1) query rows
//    before it, the tile's query halo.
// Epilogue: per-(row, head) GroupNorm over d, affine, gate; store in the input dtype.
//
// Exponentials use exp2 with log2(e) folded into the logit scale (the convolutions
// and the mixing are linear, so the fold commutes with them).
#pragma once
#include "mta_device.h"
#include "mta_internal.h"

namespace mta {
namespace fused {

constexpr int NWAVE = 4;
constexpr int NTHREADS = 64 * NWAVE;
constexpr int CQ_MAX = 8;     // largest supported c_q
constexpr int HALO_COLS = 16; // extra logit columns per key tile when convolving (c_k <= 17)
constexpr int ZPRE = 8;       // zero rows above the conv input tile (rows i - a < tile start)

struct FusedArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* theta;   // convolution kernels [M, c_q, c_k] (the one before softmax on both sides)
  const float* theta2;  // both sides: the kernels after softmax
  const float* w_pre;   // mixing before softmax [M/c_h, c_h, c_h]
  const float* w_post;  // mixing after softmax
  const float* gamma;
  const float* beta;
  float lambda;
  void* out;
  int B, T, M;
  int c_q, c_k;
  int kq, mix, gn;
  int row_begin;  // first output row
  int r_out;     // output rows per query tile
  int n_tiles;   // query tiles per (b, group)
  int n_groups;  // M / CH
  float qk_scale;  // log2(e) / sqrt(d)
  int xcd_remap;   // 1: keep all tiles of a (b, group) on one XCD (needs B*n_groups % 8 == 0)
};

template <typename Tin, int D_, int CH_, int WR_, int BK_, bool TWO_, bool PAIRS_, bool DUAL_ = false>
struct Cfg {
  typedef Tin T;
  typedef typename std::conditional<std::is_same<Tin, float>::value, float, _Float16>::type Tc;
  static constexpr int D = D_, CH = CH_, WR = WR_, BK = BK_;
  static constexpr bool TWO = TWO_, PAIRS = PAIRS_, DUAL = DUAL_;
  static_assert(!DUAL || TWO, "both sides use the two-phase schedule");
  static constexpr int WPH = NWAVE / CH;      // waves per head
  static constexpr int R = WR * WPH;          // computed rows per tile
  static constexpr int RB = WR / 16;          // 16-row blocks per wave
  static constexpr int KW1 = BK + HALO_COLS;  // logit columns of one convolution's key halo
  static constexpr int NB1 = KW1 / 16;
  // staged K rows and logit columns: both sides need the halo of both convolutions
  static constexpr int KWMAX = DUAL ? BK + 2 * HALO_COLS : KW1;
  static constexpr int KWB = KWMAX / 16;      // logit column blocks (with key halo)
  static constexpr int OB = BK / 16;          // output column blocks per key tile
  static constexpr int NB = D / 16;           // output channel blocks
  static constexpr int KQ = D / Mfma<Tin>::K; // k-steps of QK^T
  static constexpr int KV = BK / Mfma<Tin>::K;  // k-steps of AV
  static constexpr int KC = 32 / Mfma<Tc>::K;   // k-steps of one Toeplitz window
  static constexpr int NP = PAIRS ? CH : 1;     // accumulators per wave
  static constexpr int PAD_T = 16 / (int)sizeof(Tin);
  static constexpr int PAD_C = 16 / (int)sizeof(Tc);
  static constexpr int LDK = D + PAD_T;     // K tile row stride
  static constexpr int LDV = BK + PAD_T;    // V^T tile row stride
  static constexpr int LDP = BK + PAD_T;    // softmax-weight tile row stride
  static constexpr int LDZ = KWMAX + PAD_C; // convolution input row stride
  static constexpr int LDW = KW1 + PAD_C;   // both sides: softmax-weight ring row stride
  static constexpr int LDX = KWMAX + 4;     // fp32 exchange tile row stride (mixing)
  static constexpr int ZROWS = ZPRE + R;
  static constexpr size_t KS_BYTES = (size_t)CH * KWMAX * LDK * sizeof(Tin);
  static constexpr size_t SX_BYTES = (size_t)CH * R * LDX * sizeof(float);
  static constexpr size_t U_BYTES = KS_BYTES > SX_BYTES ? KS_BYTES : SX_BYTES;
  static constexpr size_t VT_BYTES = (size_t)CH * D * LDV * sizeof(Tin);
  static constexpr size_t ZB_BYTES = (size_t)CH * ZROWS * LDZ * sizeof(Tc);
  static constexpr size_t ZW_BYTES = DUAL ? (size_t)CH * ZROWS * LDW * sizeof(Tc) : 0;
  static constexpr size_t PB_BYTES = (size_t)CH * R * LDP * sizeof(Tin);
  static constexpr size_t ST_BYTES = (size_t)CH * R * 2 * sizeof(float);
  static constexpr size_t OFF_U = 0;
  static constexpr size_t OFF_VT = OFF_U + U_BYTES;
  static constexpr size_t OFF_ZB = OFF_VT + VT_BYTES;
  static constexpr size_t OFF_ZW = OFF_ZB + ZB_BYTES;
  static constexpr size_t OFF_PB = OFF_ZW + ZW_BYTES;
  static constexpr size_t OFF_ST = OFF_PB + PB_BYTES;
  static constexpr size_t LDS_BYTES = OFF_ST + ST_BYTES;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(D % Mfma<Tin>::K == 0 && BK % Mfma<Tin>::K == 0, "tile shape");
  static_assert(WR % 16 == 0 && NWAVE % CH == 0, "wave layout");
};

// Cooperative copy of K rows [kbase, kbase + kw) of the CH heads of group g into LDS.
template <class C>
__device__ __forceinline__ void stage_k(typename C::T* Ks, const typename C::T* kb, int g, int M,
                                        int Tn, int kbase, int kw) {
  typedef typename C::T T;
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = C::D / EPC;      // chunks per row
  const int total = C::CH * kw * CPR;
  for (int c = threadIdx.x; c < total; c += NTHREADS) {
    const int u = c / (kw * CPR);
    const int rem = c - u * kw * CPR;
    const int r = rem / CPR;
    const int cc = rem - r * CPR;
    const int j = kbase + r;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (j >= 0 && j < Tn)
      val = *reinterpret_cast<const uint4*>(kb + ((size_t)j * M + g * C::CH + u) * C::D + cc * EPC);
    *reinterpret_cast<uint4*>(Ks + ((size_t)u * C::KWMAX + r) * C::LDK + cc * EPC) = val;
  }
}

// Cooperative transposed copy V[j0 + kk][c] -> Vt[u][c][kk] for kk < BK.
template <class C>
__device__ __forceinline__ void stage_vt(typename C::T* Vt, const typename C::T* vb, int g, int M,
                                         int Tn, int j0) {
  typedef typename C::T T;
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = C::D / EPC;
  constexpr int total = C::CH * C::BK * CPR;
  for (int c = threadIdx.x; c < total; c += NTHREADS) {
    // consecutive threads take consecutive keys so that the scattered LDS writes of
    // one instruction land on consecutive addresses
    const int kk = c % C::BK;
    const int rest = c / C::BK;
    const int cc = rest % CPR;
    const int u = rest / CPR;
    const int j = j0 + kk;
    T vals[EPC];
    if (j < Tn) {
      *reinterpret_cast<uint4*>(vals) =
          *reinterpret_cast<const uint4*>(vb + ((size_t)j * M + g * C::CH + u) * C::D + cc * EPC);
    } else {
#pragma unroll
      for (int e = 0; e < EPC; ++e) vals[e] = T(0.0f);
    }
#pragma unroll
    for (int e = 0; e < EPC; ++e) Vt[((size_t)u * C::D + cc * EPC + e) * C::LDV + kk] = vals[e];
  }
}

template <class C>
__global__ __launch_bounds__(NTHREADS, 1) void mta_fused_kernel(FusedArgs A) {
  typedef typename C::T T;
  typedef typename C::Tc Tc;
  typedef Mfma<T> MT;
  typedef Mfma<Tc> MC;
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  T* Ks = reinterpret_cast<T*>(smem + C::OFF_U);
  float* Sx = reinterpret_cast<float*>(smem + C::OFF_U);  // aliases Ks (mixing before softmax)
  T* Vt = reinterpret_cast<T*>(smem + C::OFF_VT);
  Tc* Zb = reinterpret_cast<Tc*>(smem + C::OFF_ZB);
  Tc* Zw = reinterpret_cast<Tc*>(smem + C::OFF_ZW);  // both sides: the softmax weights
  T* Pb = reinterpret_cast<T*>(smem + C::OFF_PB);
  float* St_a = reinterpret_cast<float*>(smem + C::OFF_ST);  // [CH][R] rescale factors
  float* St_l = St_a + C::CH * C::R;                         // [CH][R] final row sums

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int hu = wave / C::WPH;  // head (within the group) owned by this wave
  const int ws = wave % C::WPH;  // row slab of this wave
  const int lr = lane & 15;      // D layout: column
  const int lg = lane >> 4;      // D layout: rows 4*lg .. 4*lg+3

  // ---- workgroup -> (b, group, query tile); heaviest (last) tiles first -------------
  const int n_bg = A.B * A.n_groups;
  int bg, rank;
  if (A.xcd_remap) {
    const int xcd = blockIdx.x & 7;
    const int kx = blockIdx.x >> 3;
    const int per = n_bg >> 3;
    rank = kx / per;
    bg = (kx % per) * 8 + xcd;
  } else {
    rank = blockIdx.x / n_bg;
    bg = blockIdx.x % n_bg;
  }
  const int qt = A.n_tiles - 1 - rank;
  const int b = bg / A.n_groups;
  const int g = bg % A.n_groups;
  const int T_ = A.T, M = A.M;
  const int kq = A.kq;
  const int cq1 = kq ? A.c_q - 1 : 0;
  const int halo = C::DUAL ? 2 * cq1 : cq1;  // query halo rows of the tile
  const int h0 = kq ? (A.c_k - 1) / 2 : 0;
  const int i0 = A.row_begin + qt * A.r_out;
  const int row0 = i0 - halo;  // global row of tile row 0
  const int last_row = min(i0 + A.r_out, T_) - 1;
  const int n_kt = last_row / C::BK + 1;
  const int m_head = g * C::CH + hu;
  const bool mix_pre = (A.mix & MIX_PRE) != 0;

  const size_t bstride = (size_t)T_ * M * C::D;
  const T* qb = reinterpret_cast<const T*>(A.q) + b * bstride;
  const T* kb = reinterpret_cast<const T*>(A.k) + b * bstride;
  const T* vb = reinterpret_cast<const T*>(A.v) + b * bstride;

  // ---- Q operands of this wave's rows stay in registers -----------------------------
  typename MT::frag qf[C::RB][C::KQ];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    const int gr = row0 + ws * C::WR + rb * 16 + lr;
#pragma unroll
    for (int ks = 0; ks < C::KQ; ++ks) {
      if (gr >= 0 && gr < T_)
        qf[rb][ks] = MT::load(qb + ((size_t)gr * M + m_head) * C::D + ks * MT::K + lg * MT::KPL);
      else
        qf[rb][ks] = MT::zero();
    }
  }

  // ---- banded Toeplitz operands of the c_q x c_k kernel ------------------------------
  // Output column n of a 16-column block reads input columns k of a 32-column window
  // that starts h0 keys left of the block: tap e = n - k + 2*h0.
  typedef typename MC::frag TzOps[CQ_MAX][C::KC];
  auto toeplitz = [&](TzOps& dst, const float* theta) __attribute__((always_inline)) {
    const float* th = theta + (size_t)m_head * A.c_q * A.c_k;
#pragma unroll
    for (int a = 0; a < CQ_MAX; ++a) {
#pragma unroll
      for (int kc = 0; kc < C::KC; ++kc) {
        Tc vals[MC::KPL];
#pragma unroll
        for (int e8 = 0; e8 < MC::KPL; ++e8) {
          const int kidx = kc * MC::K + lg * MC::KPL + e8;
          const int e = lr - kidx + 2 * h0;
          float t = 0.0f;
          if (a < A.c_q && e >= 0 && e < A.c_k) t = th[a * A.c_k + e];
          vals[e8] = Tc(t);
        }
        dst[a][kc] = *reinterpret_cast<typename MC::frag*>(vals);
      }
    }
  };
  TzOps tz, tz2;  // tz2: both sides, the kernel after softmax
  if (kq) {
    toeplitz(tz, A.theta);
    if constexpr (C::DUAL) toeplitz(tz2, A.theta2);
    // zero the rows above the tile that halo outputs may read
    for (int x = tid; x < C::CH * ZPRE * C::LDZ; x += NTHREADS) {
      const int u = x / (ZPRE * C::LDZ);
      const int rem = x - u * ZPRE * C::LDZ;
      Zb[(size_t)u * C::ZROWS * C::LDZ + rem] = Tc(0.0f);
    }
    if constexpr (C::DUAL) {
      for (int x = tid; x < C::CH * ZPRE * C::LDW; x += NTHREADS) {
        const int u = x / (ZPRE * C::LDW);
        const int rem = x - u * ZPRE * C::LDW;
        Zw[(size_t)u * C::ZROWS * C::LDW + rem] = Tc(0.0f);
      }
    }
  }

  float wrow[C::CH], wpost[C::CH];  // mixing weights w[g][hu][:] before / after softmax
#pragma unroll
  for (int u = 0; u < C::CH; ++u) {
    wrow[u] = (A.mix & MIX_PRE) ? A.w_pre[((size_t)g * C::CH + hu) * C::CH + u] : 0.0f;
    wpost[u] = (A.mix & MIX_POST) ? A.w_post[((size_t)g * C::CH + hu) * C::CH + u] : 0.0f;
  }

  f32x4 acc[C::NP][C::RB][C::NB];
#pragma unroll
  for (int p = 0; p < C::NP; ++p)
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) acc[p][rb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  float m_run[C::RB][4], l_run[C::RB][4];
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m_run[rb][i] = -1e30f;
      l_run[rb][i] = 0.0f;
    }

  const float NEG_INF = -__builtin_inff();
  f32x4 s[C::RB][C::KWB];

  // logits S = Q K^T * scale on nblk 16-column blocks of the staged K tile, then the
  // optional mixing of logits across the heads of the group (through LDS).
  auto logits = [&](int nblk) {
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < C::KWB; ++cb) {
        if (cb < nblk) {
          f32x4 c = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < C::KQ; ++ks) {
            const typename MT::frag bf =
                MT::load(Ks + ((size_t)hu * C::KWMAX + cb * 16 + lr) * C::LDK + ks * MT::K + lg * MT::KPL);
            c = MT::mma(qf[rb][ks], bf, c);
          }
          s[rb][cb] = c * A.qk_scale;
        }
      }
    if (mix_pre) {
      __syncthreads();  // every wave is done reading Ks, which Sx overwrites
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < C::KWB; ++cb)
          if (cb < nblk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t = ws * C::WR + rb * 16 + 4 * lg + i;
              Sx[((size_t)hu * C::R + t) * C::LDX + cb * 16 + lr] = s[rb][cb][i];
            }
      __syncthreads();
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < C::KWB; ++cb)
          if (cb < nblk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t = ws * C::WR + rb * 16 + 4 * lg + i;
              float x = 0.0f;
#pragma unroll
              for (int u = 0; u < C::CH; ++u) x += wrow[u] * Sx[((size_t)u * C::R + t) * C::LDX + cb * 16 + lr];
              s[rb][cb][i] = x;
            }
    }
  };

  // convolution of a ring of ld columns (rows shifted by the query lag a): output block ob
  // reads ring columns 16 ob .. 16 ob + 31 -> dst[rb][ob], NOB blocks
  f32x4 cv[C::RB][C::OB];
  auto convolve_ring = [&](const Tc* ring, int ld, const TzOps& tzs, auto& dst, auto nobc) __attribute__((always_inline)) {
    constexpr int NOB = decltype(nobc)::value;
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int ob = 0; ob < NOB; ++ob) dst[rb][ob] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int a = 0; a < CQ_MAX; ++a) {
      if (a < A.c_q) {
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
          const Tc* zrow = ring + ((size_t)hu * C::ZROWS + ZPRE + ws * C::WR + rb * 16 + lr - a) * ld;
#pragma unroll
          for (int ob = 0; ob < NOB; ++ob)
#pragma unroll
            for (int kc = 0; kc < C::KC; ++kc) {
              const typename MC::frag af = MC::load(zrow + ob * 16 + kc * MC::K + lg * MC::KPL);
              dst[rb][ob] = MC::mma(af, tzs[a][kc], dst[rb][ob]);
            }
        }
      }
    }
  };
  // the convolution of the logits in Zb -> cv (output keys of the tile)
  auto convolve = [&]() __attribute__((always_inline)) {
    convolve_ring(Zb, C::LDZ, tz, cv, std::integral_constant<int, C::OB>{});
  };

  // AV on the weights in Pb: acc[p] += P_{head p} V_{hu}
  auto av = [&]() {
#pragma unroll
    for (int p = 0; p < C::NP; ++p) {
      const int up = C::PAIRS ? p : hu;
#pragma unroll
      for (int kv = 0; kv < C::KV; ++kv) {
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
          const typename MT::frag af =
              MT::load(Pb + ((size_t)up * C::R + ws * C::WR + rb * 16 + lr) * C::LDP + kv * MT::K + lg * MT::KPL);
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) {
            const typename MT::frag bf =
                MT::load(Vt + ((size_t)hu * C::D + nb * 16 + lr) * C::LDV + kv * MT::K + lg * MT::KPL);
            acc[p][rb][nb] = MT::mma(af, bf, acc[p][rb][nb]);
          }
        }
      }
    }
  };

  if constexpr (!C::TWO) {
    // ===================== one pass: convolution (if any) before softmax ============
    const int nblk = kq ? C::KWB : C::OB;
    for (int kt = 0; kt < n_kt; ++kt) {
      const int j0 = kt * C::BK;
      const int kbase = j0 - h0;
      __syncthreads();  // previous tile fully consumed
      stage_k<C>(Ks, kb, g, M, T_, kq ? kbase : j0, kq ? C::KWMAX : C::BK);
      stage_vt<C>(Vt, vb, g, M, T_, j0);
      __syncthreads();
      logits(nblk);
      if (kq) {
        // Mask_0 (future keys of the source row, and positions outside the map) -> Zb
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
          for (int cb = 0; cb < C::KWB; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int t = ws * C::WR + rb * 16 + 4 * lg + i;
              const int gr = row0 + t;
              const int j = kbase + cb * 16 + lr;
              const bool keep = gr >= 0 && j >= 0 && j < T_ && j <= gr;
              Zb[((size_t)hu * C::ZROWS + ZPRE + t) * C::LDZ + cb * 16 + lr] = Tc(keep ? s[rb][cb][i] : 0.0f);
            }
        __syncthreads();
        convolve();
      } else {
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
          for (int ob = 0; ob < C::OB; ++ob) cv[rb][ob] = s[rb][ob];
      }
      // Mask_-inf and online softmax
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = ws * C::WR + rb * 16 + 4 * lg + i;
          const int gr = row0 + t;
          const bool row_ok = t >= cq1 && gr < T_;
          float mx = NEG_INF;
#pragma unroll
          for (int ob = 0; ob < C::OB; ++ob) {
            const int j = j0 + ob * 16 + lr;
            const float x = (row_ok && j <= gr) ? cv[rb][ob][i] : NEG_INF;
            cv[rb][ob][i] = x;
            mx = fmaxf(mx, x);
          }
          mx = row16_max(mx);
          const float m_new = fmaxf(m_run[rb][i], mx);
          const float alpha = fast_exp2(m_run[rb][i] - m_new);
          float sum = 0.0f;
#pragma unroll
          for (int ob = 0; ob < C::OB; ++ob) {
            const float pv = fast_exp2(cv[rb][ob][i] - m_new);
            sum += pv;
            Pb[((size_t)hu * C::R + t) * C::LDP + ob * 16 + lr] = to_elem<T>(pv);
          }
          sum = row16_sum(sum);
          l_run[rb][i] = l_run[rb][i] * alpha + sum;
          m_run[rb][i] = m_new;
          if (lr == 0) St_a[hu * C::R + t] = alpha;
        }
      }
      __syncthreads();
      // rescale the accumulators by their head's max correction, then AV
#pragma unroll
      for (int p = 0; p < C::NP; ++p) {
        const int up = C::PAIRS ? p : hu;
#pragma unroll
        for (int rb = 0; rb < C::RB; ++rb) {
          const float* al = St_a + up * C::R + ws * C::WR + rb * 16 + 4 * lg;
          const f32x4 a4 = f32x4{al[0], al[1], al[2], al[3]};
#pragma unroll
          for (int nb = 0; nb < C::NB; ++nb) acc[p][rb][nb] *= a4;
        }
      }
      av();
    }
    // final row sums of every head (the mixing epilogue needs the other heads')
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lr == 0) St_l[hu * C::R + ws * C::WR + rb * 16 + 4 * lg + i] = l_run[rb][i];
    __syncthreads();
  } else if constexpr (C::DUAL) {
    // ===================== both sides: convolutions before and after softmax ========
    // phase 1: exact (max, sum) of the softmax inputs C = conv_pre(Mask_0(L)) of tile rows
    // t >= c_q - 1 (the rows above them have no complete convolution; their weights are
    // zero in phase 2, and only non-output rows read them)
    for (int kt = 0; kt < n_kt; ++kt) {
      const int j0 = kt * C::BK;
      const int kbase = j0 - h0;
      __syncthreads();
      stage_k<C>(Ks, kb, g, M, T_, kbase, C::KW1);
      __syncthreads();
      logits(C::NB1);
      // Mask_0 -> Zb, column c holding key kbase + c
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < C::NB1; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = ws * C::WR + rb * 16 + 4 * lg + i;
            const int gr = row0 + t;
            const int j = kbase + cb * 16 + lr;
            const bool keep = gr >= 0 && j >= 0 && j < T_ && j <= gr;
            Zb[((size_t)hu * C::ZROWS + ZPRE + t) * C::LDZ + cb * 16 + lr] = Tc(keep ? s[rb][cb][i] : 0.0f);
          }
      __syncthreads();
      convolve();
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = ws * C::WR + rb * 16 + 4 * lg + i;
          const int gr = row0 + t;
          const bool row_ok = t >= cq1 && gr >= 0 && gr < T_;
          float mx = NEG_INF;
          float x[C::OB];
#pragma unroll
          for (int ob = 0; ob < C::OB; ++ob) {
            const int j = j0 + ob * 16 + lr;
            x[ob] = (row_ok && j <= gr) ? cv[rb][ob][i] : NEG_INF;
            mx = fmaxf(mx, x[ob]);
          }
          mx = row16_max(mx);
          const float m_new = fmaxf(m_run[rb][i], mx);
          float sum = 0.0f;
#pragma unroll
          for (int ob = 0; ob < C::OB; ++ob) sum += fast_exp2(x[ob] - m_new);
          sum = row16_sum(sum);
          l_run[rb][i] = l_run[rb][i] * fast_exp2(m_run[rb][i] - m_new) + sum;
          m_run[rb][i] = m_new;
        }
      }
    }
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) l_run[rb][i] = l_run[rb][i] > 0.0f ? 1.0f / l_run[rb][i] : 0.0f;

    // phase 2: logits over keys j0 - 2 h0 .. (both key halos) -> Mask_0 -> convolution into
    // the softmax inputs of keys j0 - h0 .. j0 + BK + h0 - 1 -> exact weights (Mask_-inf as
    // zero) in Zw -> convolution -> Mask_0 -> AV
    f32x4 cvp[C::RB][C::NB1];
    for (int kt = 0; kt < n_kt; ++kt) {
      const int j0 = kt * C::BK;
      const int kbase = j0 - 2 * h0;
      __syncthreads();
      stage_k<C>(Ks, kb, g, M, T_, kbase, C::KWMAX);
      stage_vt<C>(Vt, vb, g, M, T_, j0);
      __syncthreads();
      logits(C::KWB);
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < C::KWB; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = ws * C::WR + rb * 16 + 4 * lg + i;
            const int gr = row0 + t;
            const int j = kbase + cb * 16 + lr;
            const bool keep = gr >= 0 && j >= 0 && j < T_ && j <= gr;
            Zb[((size_t)hu * C::ZROWS + ZPRE + t) * C::LDZ + cb * 16 + lr] = Tc(keep ? s[rb][cb][i] : 0.0f);
          }
      __syncthreads();
      convolve_ring(Zb, C::LDZ, tz, cvp, std::integral_constant<int, C::NB1>{});
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < C::NB1; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = ws * C::WR + rb * 16 + 4 * lg + i;
            const int gr = row0 + t;
            const int j = j0 - h0 + cb * 16 + lr;
            const bool keep = t >= cq1 && gr >= 0 && gr < T_ && j >= 0 && j <= gr;
            const float pv = keep ? fast_exp2(cvp[rb][cb][i] - m_run[rb][i]) * l_run[rb][i] : 0.0f;
            Zw[((size_t)hu * C::ZROWS + ZPRE + t) * C::LDW + cb * 16 + lr] = Tc(pv);
          }
      __syncthreads();
      convolve_ring(Zw, C::LDW, tz2, cv, std::integral_constant<int, C::OB>{});
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int ob = 0; ob < C::OB; ++ob)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = ws * C::WR + rb * 16 + 4 * lg + i;
            const int gr = row0 + t;
            const int j = j0 + ob * 16 + lr;
            const bool keep = t >= halo && gr < T_ && j <= gr;
            Pb[((size_t)hu * C::R + t) * C::LDP + ob * 16 + lr] = to_elem<T>(keep ? cv[rb][ob][i] : 0.0f);
          }
      __syncthreads();
      av();
    }
  } else {
    // ===================== two phase: convolution after softmax =====================
    // phase 1: exact (max, sum) of every tile row, halo rows included
    for (int kt = 0; kt < n_kt; ++kt) {
      const int j0 = kt * C::BK;
      __syncthreads();
      stage_k<C>(Ks, kb, g, M, T_, j0, C::BK);
      __syncthreads();
      logits(C::OB);
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int gr = row0 + ws * C::WR + rb * 16 + 4 * lg + i;
          const bool row_ok = gr >= 0 && gr < T_;
          float mx = NEG_INF;
          float x[C::OB];
#pragma unroll
          for (int ob = 0; ob < C::OB; ++ob) {
            const int j = j0 + ob * 16 + lr;
            x[ob] = (row_ok && j <= gr) ? s[rb][ob][i] : NEG_INF;
            mx = fmaxf(mx, x[ob]);
          }
          mx = row16_max(mx);
          const float m_new = fmaxf(m_run[rb][i], mx);
          float sum = 0.0f;
#pragma unroll
          for (int ob = 0; ob < C::OB; ++ob) sum += fast_exp2(x[ob] - m_new);
          sum = row16_sum(sum);
          l_run[rb][i] = l_run[rb][i] * fast_exp2(m_run[rb][i] - m_new) + sum;
          m_run[rb][i] = m_new;
        }
      }
    }
    // inverse sums (0 for rows outside the map)
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
      for (int i = 0; i < 4; ++i) l_run[rb][i] = l_run[rb][i] > 0.0f ? 1.0f / l_run[rb][i] : 0.0f;

    // phase 2: exact weights with key halo -> convolution -> Mask_0 -> AV
    for (int kt = 0; kt < n_kt; ++kt) {
      const int j0 = kt * C::BK;
      const int kbase = j0 - h0;
      __syncthreads();
      stage_k<C>(Ks, kb, g, M, T_, kbase, C::KWMAX);
      stage_vt<C>(Vt, vb, g, M, T_, j0);
      __syncthreads();
      logits(C::KWB);
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int cb = 0; cb < C::KWB; ++cb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = ws * C::WR + rb * 16 + 4 * lg + i;
            const int gr = row0 + t;
            const int j = kbase + cb * 16 + lr;
            const bool keep = gr >= 0 && gr < T_ && j >= 0 && j <= gr;
            const float pv = keep ? fast_exp2(s[rb][cb][i] - m_run[rb][i]) * l_run[rb][i] : 0.0f;
            Zb[((size_t)hu * C::ZROWS + ZPRE + t) * C::LDZ + cb * 16 + lr] = Tc(pv);
          }
      __syncthreads();
      convolve();
#pragma unroll
      for (int rb = 0; rb < C::RB; ++rb)
#pragma unroll
        for (int ob = 0; ob < C::OB; ++ob)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = ws * C::WR + rb * 16 + 4 * lg + i;
            const int gr = row0 + t;
            const int j = j0 + ob * 16 + lr;
            const bool keep = t >= cq1 && gr < T_ && j <= gr;
            Pb[((size_t)hu * C::R + t) * C::LDP + ob * 16 + lr] = to_elem<T>(keep ? cv[rb][ob][i] : 0.0f);
          }
      __syncthreads();
      av();
    }
  }

  // ===================== epilogue: mixing after softmax, GroupNorm, gate ===============
  T* ob_ = reinterpret_cast<T*>(A.out) + b * bstride;
#pragma unroll
  for (int rb = 0; rb < C::RB; ++rb) {
    f32x4 o[C::NB];
    if constexpr (C::PAIRS) {
      f32x4 coef = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < C::NP; ++p) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sc = wpost[p];
          if constexpr (!C::TWO) {
            const float l = St_l[p * C::R + ws * C::WR + rb * 16 + 4 * lg + i];
            sc = l > 0.0f ? sc / l : 0.0f;
          }
          coef[i] = sc;
        }
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) o[nb] += acc[p][rb][nb] * coef;
      }
    } else {
      // a one-head group mixed after softmax scales its head by the weight w[g][0][0]
      const float wscale = (A.mix & MIX_POST) ? wpost[0] : 1.0f;
      f32x4 coef;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (!C::TWO)
          coef[i] = l_run[rb][i] > 0.0f ? wscale / l_run[rb][i] : 0.0f;
        else
          coef[i] = wscale;
      }
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[nb] = acc[0][rb][nb] * coef;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = ws * C::WR + rb * 16 + 4 * lg + i;
      const int gr = row0 + t;
      float mean = 0.0f, inv = 1.0f;
      if (A.gn) {
        float sum = 0.0f;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) sum += o[nb][i];
        mean = row16_sum(sum) * (1.0f / C::D);
        float sq = 0.0f;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const float dv = o[nb][i] - mean;
          sq += dv * dv;
        }
        const float var = row16_sum(sq) * (1.0f / C::D);
        inv = 1.0f / sqrtf(var + 1e-5f);
      }
      if (t >= halo && gr < T_) {
        T* dst = ob_ + ((size_t)gr * M + m_head) * C::D;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const int c = nb * 16 + lr;
          float y = o[nb][i];
          if (A.gn) y = A.lambda * (A.gamma[(size_t)m_head * C::D + c] * (y - mean) * inv + A.beta[(size_t)m_head * C::D + c]);
          dst[c] = to_elem<T>(y);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
template <class C>
hipError_t launch(const Problem& p, hipStream_t stream) {
  FusedArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.theta = (p.kq & KQ_PRE) ? p.theta_pre : p.theta_post;
  a.theta2 = p.theta_post;
  a.w_pre = p.w_pre;
  a.w_post = p.w_post;
  a.gamma = p.gamma;
  a.beta = p.beta;
  a.lambda = p.lambda;
  a.out = p.out;
  a.B = p.B;
  a.T = p.T;
  a.M = p.M;
  a.kq = p.kq;
  a.mix = p.mix;
  a.gn = p.gn;
  a.c_q = p.kq ? p.c_q : 1;
  a.c_k = p.kq ? p.c_k : 1;
  a.r_out = C::R - (C::DUAL ? 2 : 1) * (a.c_q - 1);
  a.row_begin = p.row_begin;
  a.n_tiles = (p.T - p.row_begin + a.r_out - 1) / a.r_out;
  a.n_groups = p.M / C::CH;
  a.qk_scale = (float)(1.4426950408889634 / __builtin_sqrt((double)p.d));
  const int n_bg = p.B * a.n_groups;
  a.xcd_remap = (n_bg % 8 == 0) ? 1 : 0;
  const long long blocks = (long long)n_bg * a.n_tiles;
  if (blocks <= 0 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mta_fused_kernel<C>, dim3((unsigned)blocks), dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

// Tile shapes per (dtype, d, c_h, schedule, pairs). Per-pair accumulators cost
// c_h * WR * d fp32 registers per wave, which caps WR at 32 when mixing after softmax. Both
// sides take 16-key tiles: their staged K rows, logits ring and weights ring of fp32 values
// then fit the LDS at d = 64 with four heads.
template <typename T, int D, int CH, bool TWO, bool PAIRS, bool DUAL = false>
hipError_t launch_shape(const Problem& p, hipStream_t stream) {
  constexpr bool F32 = std::is_same<T, float>::value;
  constexpr int BK = DUAL ? 16 : (CH == 4 || F32) ? 32 : 64;
  constexpr int WR = (CH == 4 && !PAIRS && !F32) ? 64 : 32;
  return launch<Cfg<T, D, CH, WR, BK, TWO, PAIRS, DUAL>>(p, stream);
}

template <typename T, int D, int CH>
hipError_t launch_ch(const Problem& p, hipStream_t stream) {
  const bool two = p.kq == KQ_POST;
  const bool pairs = (p.mix & MIX_POST) && CH > 1;
  if (p.kq == KQ_BOTH) {
    if (pairs) return launch_shape<T, D, CH, true, true, true>(p, stream);
    return launch_shape<T, D, CH, true, false, true>(p, stream);
  }
  if (two) {
    if (pairs) return launch_shape<T, D, CH, true, true>(p, stream);
    return launch_shape<T, D, CH, true, false>(p, stream);
  }
  if (pairs) return launch_shape<T, D, CH, false, true>(p, stream);
  return launch_shape<T, D, CH, false, false>(p, stream);
}

template <typename T, int D>
hipError_t launch_d(const Problem& p, hipStream_t stream) {
  // without mixing the head grouping does not matter: run one head per workgroup
  const int ch = p.mix ? p.c_h : 1;
  switch (ch) {
    case 1: return launch_ch<T, D, 1>(p, stream);
    case 2: return launch_ch<T, D, 2>(p, stream);
    case 4: return launch_ch<T, D, 4>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fused
}  // namespace mta
