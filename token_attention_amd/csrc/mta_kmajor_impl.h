// Fused Multi-Token Attention forward for bf16 tensors on gfx950, key-major schedule.
//
// Method: page "Multi-Token Attention | Summary" (greeksharifa.github.io), §2 (logits,
// causal softmax, AV), §3.1 (key-query convolution with Mask_0 / Mask_-inf), §3.2
// (head mixing in groups of c_h heads), §3.3 (GroupNorm + scalar gate).
//
// Orientation. Every logit tile is computed transposed, S^T = K Q^T (keys are the MFMA
// rows, queries the columns), so that in the 16x16 accumulator layout a lane owns one
// query and four consecutive keys. Consequences:
//   * softmax statistics of a query reduce in-lane plus two cross-row exchanges
//     (v_permlane16_swap / v_permlane32_swap), no LDS traffic;
//   * the weights P^T feed the AV product O^T = V^T P^T directly as the B operand from
//     registers: the eight k-slots of lane group g are keys {4g..4g+3} of one 16-key
//     block and {16+4g..16+4g+3} of the next;
//   * V stays row-major in LDS; its transposed A operand (same k-slot permutation) is
//     read with ds_read_b64_tr_b16, which transposes a 4 x 16 block of b16 values
//     within each 16-lane group.
//
// Work split. One workgroup of NW waves owns batch b, head group g (c_h heads) and a tile
// of R query rows; tile row t is global row i0 - halo + t (the first rows are the query
// halo of the convolutions). Wave w owns head hu = w / (NW/c_h) and a slab of QW rows.
// The full-size shapes have 8 waves of 32 rows (two waves per SIMD, so one wave's MFMA work
// overlaps the other's LDS and VALU work) and stage the K and V tiles of all heads of the
// group together. The key-split instantiations for a range of at most 16 rows (a decode
// step) have one wave of 16 rows per head; such a wave stages its own head's K and V and
// synchronises those with a wavefront fence only (mixing exchanges stay workgroup-wide).
//
// Key tiles of BK keys stream through LDS. The K and V rows of a later tile are loaded
// into registers (global -> VGPR prefetch) and written to LDS right after the first
// workgroup barrier that follows the last read of the buffer they replace; a later barrier
// of the same tile publishes them. With a convolution the logits of a tile cover keys
// [j0 - 8, j0 + BK + 8): 16-key blocks 0..BK/16, where block 0 equals the last block of the
// previous tile, so each tile computes only BK new key columns (sliding key halo); the
// convolution input lives in an LDS ring of BK/16 + 1 blocks per row (BK/16 more in the
// two-pass schedule, which writes the next tile's blocks while the current window is read).
//
// The c_q x c_k convolution runs on fp16 MFMA: output keys of one 16-key block read a
// 32-key window (blocks ob, ob+1); for each query lag a the banded Toeplitz matrix of
// theta[a][.] is the A operand (constant per workgroup) and the input tile shifted by a
// query rows is the B operand.
//
// Passes over the keys (every query row keeps one fixed softmax reference, the maximum of
// its first key tile, so weights exp2(x - ref) are never rescaled and the accumulators are
// touched by MFMA only; if a row sum exceeds 2^64 - a later key far above the first tile's
// maximum - the workgroup repeats with exact row maxima):
//   one pass   (no convolution after softmax, no mixing after softmax): weights against
//              the reference, AV, division by the row sum in the epilogue;
//   two passes (convolution or mixing after softmax): a statistics pass (row sums), then
//              exact normalised weights -> [convolution -> Mask_0] -> [mixing] -> AV; both
//              passes are software-pipelined one tile deep (the next tile's logits are
//              computed beside this tile's VALU work);
//   both sides (DUAL: convolutions before and after softmax): the two-pass schedule with a
//              second ring; every tile convolves the logits (first ring) into softmax inputs
//              8 keys ahead of the weights it convolves (second ring), after a lead-in tile.
// Mixing exchanges fp16 blocks of the other heads of the group through a double-buffered
// LDS buffer (one buffer with both convolutions, where ring barriers separate exchanges):
// logits before softmax (a wave's own head stays fp32), normalised weights after softmax.
//
// SPLIT instantiations cover one chunk of the key range of a row tile and write partial
// results (softmax statistics or AV sums) to a workspace for a combining kernel; they serve
// short row ranges such as a decode step, where the row tiles alone would leave the GPU idle.
//
// K and V tiles are loaded with buffer loads whose range ends at the last key row, so rows
// past the sequence read as zero (they are masked) without per-row clamping.
#pragma once

#include "mta_device.h"
#include "mta_internal.h"

namespace mta {
namespace kmajor {

// every helper lambda of the kernel is inlined: one left out of line takes its array
// arguments by reference, and those arrays then live in scratch memory
#define MTA_INLINE __attribute__((always_inline))

constexpr int ZPRE = 8;               // zero rows above the tile in the convolution input ring
// Split key ranges: partial results of row gr live at row index gr - row_begin + SPLIT_HPAD of
// the partial buffers (the rows before row_begin that a tile also computes, at most 2 (c_q - 1),
// need their softmax statistics too).
constexpr int SPLIT_HPAD = 16;
enum { SPLIT_NONE = 0, SPLIT_STATS = 1, SPLIT_PARTIAL = 2 };
constexpr float SUM_LIMIT = 0x1p64f;  // largest row sum accepted with a fixed reference

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

struct Args {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const float* theta;   // convolution kernels [M, c_q, c_k] (the one before softmax if DUAL)
  const float* theta2;  // DUAL: the kernels after softmax
  const float* w_pre;   // mixing before softmax [M/c_h, c_h, c_h]
  const float* w_post;  // mixing after softmax
  const float* gamma;
  const float* beta;
  float lambda;
  __bf16* out;
  int B, T, M;
  int c_q, c_k;
  int mix, gn;
  int row_begin;  // first output row
  int r_out;
  int n_tiles;
  int n_groups;
  float qk_scale;  // log2(e)/sqrt(d)
  int xcd_remap;
  // Split key range (SPLIT_STATS / SPLIT_PARTIAL): workgroup blockIdx.x / n_main covers key
  // tiles [split * kt_chunk, (split + 1) * kt_chunk) and writes partial results instead of out.
  int split_mode;
  int kt_zero;  // 0; the first key tile of an unsplit both-sides schedule (see kt_lo)
  int kt_chunk;
  int n_main;          // workgroups of one split (B * groups * row tiles)
  int nr;              // rows of the partial buffers: T - row_begin + SPLIT_HPAD
  float* part_stats;   // [split][B][nr][M][2]: row maximum (log2 units) and row sum against it
  float* part_o;       // [split][B][nr][M][D]: AV partial
  int n_split;         // chunks whose statistics a normalised SPLIT_PARTIAL schedule combines
  float* lse;          // unsplit, optional: [B][T][M] natural log-sum-exp of each softmax row
  float* o32;          // unsplit, optional: [B][T][M][D] output before GroupNorm, fp32
};

// KQ: a key-query convolution (TWO: after softmax); MIXPRE / MIXPOST: head mixing before /
// after softmax.
// DUAL: key-query convolutions on both sides of softmax (implies KQ and TWO). SPLIT: the
// instantiation that covers one chunk of the key range and writes partial results.
template <int D_, int CH_, int QW_, int BK_, bool KQ_, bool TWO_, bool MIXPOST_, int CQM_, bool MIXPRE_, int NW_ = 8,
          bool DUAL_ = false, bool SPLIT_ = false>
struct Cfg {
  static constexpr bool SPLIT = SPLIT_;
  static constexpr int D = D_, CH = CH_, QW = QW_, BK = BK_, CQM = CQM_;
  static constexpr int NW = NW_;               // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr bool KQ = KQ_, TWO = TWO_, MIXPOST = MIXPOST_, MIXPRE = MIXPRE_, DUAL = DUAL_;
  static_assert(!DUAL || (KQ && TWO), "both convolutions use the two-phase schedule");
  static constexpr bool MIX = MIXPRE || MIXPOST;
  // head mixing on MFMA (see mix_read): groups of four heads mixed after softmax only
  // (before softmax the VALU mixing interleaved with the next tile's logits measured faster)
  static constexpr bool XM = MIXPOST && !MIXPRE && CH == 4;
  // mixing after softmax in groups of two heads without a convolution after softmax: one pass
  // with an AV accumulator per (source head, head) pair of the group (the mixing weights and
  // each source head's row sum are applied in the epilogue)
  static constexpr bool PAIR = MIXPOST && !MIXPRE && !TWO && CH == 2 && !SPLIT;
  static constexpr int WPH = NW / CH;          // waves per head
  static constexpr bool PRIV = WPH == 1;       // a wave owns its head: private K/V staging
  static constexpr int TEAM = PRIV ? 64 : NT;  // threads staging one head set
  static constexpr int R = QW * WPH;           // tile rows
  static constexpr int NQB = QW / 16;          // query blocks per wave
  static constexpr int NKB = BK / 16;          // new key blocks per tile
  static constexpr int LB = KQ ? NKB + 1 : NKB;  // logit blocks per tile (with the carried halo)
  static constexpr int KS = D / 32;            // k-steps of QK^T
  static constexpr int NB = D / 16;            // channel blocks
  static constexpr int NC = BK / 32;           // 32-key chunks of AV
  // K rows in LDS: the one-pass convolution schedule stages a 16-key halo block in front
  static constexpr int KROWS = (KQ && !TWO) ? BK + 16 : BK;
  // convolution ring blocks per row: the window of a tile (LB blocks) and, in the pipelined
  // two-phase schedule, the NKB new blocks of the next tile, written while the window is read
  static constexpr int RB = (TWO && !DUAL) ? LB + NKB : LB;
  // K row stride (bf16) and ring row stride (fp16), chosen by measurement (LDS bank-conflict
  // counter and time): at d = 128 the two-pass schedule with LDK = D + 8 and LDZ = ZW + 8 had
  // 8.3e7 conflict cycles per launch, with D + 16 and ZW 2.8e7 and ran 5 % faster; an unpadded
  // ring made the both-sides schedule 6 % faster; a ring stride of 64 halves was 50 % slower.
  static constexpr int LDK = DUAL ? D + 8 : D + 16;
  static constexpr int LDV = D + 16;           // V row stride (bf16): transposed reads conflict-free
  static constexpr int ZW = RB * 16;           // ring width (keys)
  static constexpr int LDZ = ZW;
  static constexpr int ZROWS = ZPRE + R;
  static constexpr int XW = NKB * 4;           // exchange halves per lane and query block
  static constexpr size_t SX_HALF = (size_t)CH * R * BK;  // one exchange buffer (halves)
  static constexpr size_t KS_BYTES = (size_t)CH * KROWS * LDK * 2;
  // Exchange buffers: double buffered, unless a workgroup barrier already separates every two
  // exchanges: with both convolutions (ring writes -> convolution reads), and in the one-pass
  // convolution schedule with mixing after softmax only (the ring barrier of the next tile
  // comes between one tile's exchange reads and the next tile's writes).
  static constexpr bool ONEPASS_CONV = KQ && !TWO;
  static constexpr int XBUFS = (DUAL || (ONEPASS_CONV && !MIXPRE)) ? 1 : 2;
  static constexpr size_t SX_BYTES = (MIX && CH > 1) ? XBUFS * SX_HALF * 2 : 0;  // one head: a scalar weight
  static constexpr size_t VS_BYTES = (size_t)CH * BK * LDV * 2;
  static constexpr size_t ZRING = (size_t)CH * ZROWS * LDZ;  // halves of one ring
  // rings: the convolution input; with both convolutions the logits and the weights
  static constexpr size_t ZB_BYTES = KQ ? (DUAL ? 2 : 1) * ZRING * 2 : 0;
  static constexpr size_t OFF_KS = 0;
  static constexpr size_t OFF_SX = OFF_KS + KS_BYTES;
  static constexpr size_t OFF_VS = OFF_SX + SX_BYTES;
  static constexpr size_t OFF_ZB = OFF_VS + VS_BYTES;
  // Exact centre tap of the convolution before softmax (one-pass schedule): a second ring holds,
  // for the tile's own rows, the fp16 residual z - fp16(z) of every logit in the ring, and the
  // convolution adds the centre tap times that residual (one more MFMA per output block), so
  // the dominant term of the convolution sees the fp32 logit (error ~2^-22 |z| instead of the
  // fp16 rounding, ~2^-12 |z|, which grows with the logit's magnitude). Built where it fits the
  // LDS budget.
  static constexpr size_t ZR_RING = (size_t)CH * R * LDZ;  // halves
  static constexpr bool XC = ONEPASS_CONV && (OFF_ZB + ZB_BYTES + ZR_RING * 2 <= 160 * 1024);
  static constexpr size_t OFF_ZR = OFF_ZB + ZB_BYTES;
  static constexpr size_t ZR_BYTES = XC ? ZR_RING * 2 : 0;
  static constexpr size_t LDS_BYTES = OFF_ZR + ZR_BYTES;
  // staging: 16-byte chunks per team member for one regular tile
  static constexpr int HEADS = PRIV ? 1 : CH;
  static constexpr int CHUNKS = HEADS * BK * (D / 8);  // 16-byte chunks of one regular tile
  static constexpr int CPT = (CHUNKS + TEAM - 1) / TEAM;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget exceeded");
  static_assert(QW % 16 == 0 && BK % 32 == 0 && D % 32 == 0, "tile shape");
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

// Reductions over the four lane groups that hold the same query (lanes l, l^16, l^32,
// l^48): v_permlane16_swap(x, x) returns (x[l & ~16], x[l | 16]) in every lane, and
// v_permlane32_swap the same across halves of the wave.
__device__ __forceinline__ float xgroup_max(float x) {
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
  t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

__device__ __forceinline__ float xgroup_sum(float x) {
  auto t = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(t[0]) + __uint_as_float(t[1]);
  t = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}

// Transposed read of V: lane i of each 16-lane group receives V[row0 + 0..3][col0 + i].
// In a group, lane 4k + m supplies the address of row row0 + k, columns col0 + 4m ..+3.
__device__ __forceinline__ s16x4 vtr(const __bf16* Vs, int row0, int col0, int ld, int lane) {
  const int j = lane & 15;
  const __bf16* p = Vs + (size_t)(row0 + (j >> 2)) * ld + col0 + 4 * (j & 3);
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// Synchronises the threads that share a staged K/V tile: the workgroup, or only the
// wave itself when it owns its head (then a wavefront-scope fence keeps the LDS
// accesses of the wave in program order).
template <class C>
__device__ __forceinline__ void team_sync() {
  if constexpr (C::PRIV)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
  else
    __syncthreads();
}

template <class C>
__global__ __launch_bounds__(C::NT, 1) void kmajor_kernel(Args A) {
  __shared__ __attribute__((aligned(16))) char smem[C::LDS_BYTES];
  __bf16* Ks = reinterpret_cast<__bf16*>(smem + C::OFF_KS);
  _Float16* Sx = reinterpret_cast<_Float16*>(smem + C::OFF_SX);
  __bf16* Vs = reinterpret_cast<__bf16*>(smem + C::OFF_VS);
  _Float16* Zb = reinterpret_cast<_Float16*>(smem + C::OFF_ZB);
  _Float16* Zr = reinterpret_cast<_Float16*>(smem + C::OFF_ZR);  // residual ring (C::XC)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int hu = wave / C::WPH;
  const int slab = wave % C::WPH;
  const int qs0 = slab * C::QW;           // first tile row of this wave
  const int lq = lane & 15;               // query within a block (D layout column)
  const int lg = lane >> 4;               // lane group: keys 4*lg..4*lg+3 of a block
  const int trank = C::PRIV ? lane : tid; // rank within the staging team
  const int thead = C::PRIV ? hu : 0;     // first head staged by the team

  // ---- workgroup -> (key split, b, group, tile), heaviest tiles first --------------------
  constexpr bool split = C::SPLIT;
  const int split_id = split ? (int)blockIdx.x / A.n_main : 0;
  const int bid = split ? (int)blockIdx.x % A.n_main : (int)blockIdx.x;
  const int n_bg = A.B * A.n_groups;
  int bg, rank;
  if (A.xcd_remap) {
    const int xcd = bid & 7, kx = bid >> 3, per = n_bg >> 3;
    rank = kx / per;
    bg = (kx % per) * 8 + xcd;
  } else {
    rank = bid / n_bg;
    bg = bid % n_bg;
  }
  const int qt = A.n_tiles - 1 - rank;
  const int b = bg / A.n_groups, g = bg % A.n_groups;
  const int T_ = A.T, M = A.M;
  const int cq1 = C::KQ ? A.c_q - 1 : 0;
  // query halo: c_q - 1 rows per convolution (both: logits -> weights -> output rows)
  const int halo = C::DUAL ? 2 * cq1 : cq1;
  const int h0 = C::KQ ? (A.c_k - 1) / 2 : 0;
  const int i0 = A.row_begin + qt * A.r_out;
  const int row0 = i0 - halo;
  const int last_row = min(i0 + A.r_out, T_) - 1;
  const int n_kt = last_row / C::BK + 1;
  // key tiles of this workgroup: all of them, or one chunk when the key range is split. The
  // both-sides schedule takes its first tile from a kernel argument even when it is 0: with
  // a compile-time 0 the compiler specialises the lead-in tile (kt = -1) and the kernel runs
  // about 17 % slower.
  const int kt_lo = split ? min(split_id * A.kt_chunk, n_kt) : (C::DUAL ? A.kt_zero : 0);
  const int kt_hi = split ? min(kt_lo + A.kt_chunk, n_kt) : n_kt;
  const int j0lo = kt_lo * C::BK;
  const int m_head = g * C::CH + hu;
  constexpr bool mix_pre = C::MIXPRE;
  const int wrow_min = row0 + qs0;  // smallest global row of this wave
  const size_t bstride = (size_t)T_ * M * C::D;
  const __bf16* qb_ = A.q + b * bstride;
  const __bf16* kb_ = A.k + b * bstride;
  const __bf16* vb_ = A.v + b * bstride;
  // logits are kept unscaled; sc turns them into log2 units (mixing folds the scale in)
  const float sc = mix_pre ? 1.0f : A.qk_scale;

  // ---- Q^T operands (B of QK^T) in registers ------------------------------------------
  bf16x8 qf[C::NQB][C::KS];
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    const int gr = row0 + qs0 + qb * 16 + lq;
    const int grc = min(max(gr, 0), T_ - 1);
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      qf[qb][ks] = *reinterpret_cast<const bf16x8*>(qb_ + ((size_t)grc * M + m_head) * C::D + ks * 32 + lg * 8);
      if (gr != grc) qf[qb][ks] = bf16x8{};
    }
  }

  // ---- Toeplitz A operands: out key n (row), window key k = 8*lg + s (slot) ------------
  // window key k is global key j0 - 8 + 16*ob + k; out key is j0 + 16*ob + n;
  // tap e = n - k + 8 + h0. Before softmax the logit scale is folded in.
  f16x8 tz[C::KQ ? C::CQM : 1], tz2[C::DUAL ? C::CQM : 1];
  auto toeplitz = [&](f16x8 (&dst)[C::KQ ? C::CQM : 1], const float* theta, float tscale) MTA_INLINE {
    const float* th = theta + (size_t)m_head * A.c_q * A.c_k;
#pragma unroll
    for (int a = 0; a < C::CQM; ++a) {
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int e = lq - (8 * lg + s) + 8 + h0;
        float t = 0.0f;
        if (a < A.c_q && e >= 0 && e < A.c_k) t = th[a * A.c_k + e] * tscale;
        dst[a][s] = (_Float16)t;
      }
    }
  };
  // the centre tap alone (lag 0, key offset 0): out key n reads window key n + 8
  f16x8 tzc;
  if constexpr (C::XC) {
    const float c = A.theta[(size_t)m_head * A.c_q * A.c_k + h0] * (!mix_pre ? A.qk_scale : 1.0f);
#pragma unroll
    for (int s = 0; s < 8; ++s) tzc[s] = (_Float16)((8 * lg + s == lq + 8) ? c : 0.0f);
  }
  if constexpr (C::KQ) {
    // before softmax the logit scale is folded in (unless the mixing weights carry it)
    toeplitz(tz, A.theta, ((!C::TWO || C::DUAL) && !mix_pre) ? A.qk_scale : 1.0f);
    if constexpr (C::DUAL) toeplitz(tz2, A.theta2, 1.0f);
    // zero rows above every ring
    constexpr int NRING = C::DUAL ? 2 : 1;
    for (int x = tid; x < NRING * C::CH * ZPRE * C::LDZ; x += C::NT) {
      const int u = x / (ZPRE * C::LDZ);
      Zb[(size_t)u * C::ZROWS * C::LDZ + (x - u * ZPRE * C::LDZ)] = (_Float16)0.0f;
    }
  }

  // w[g][hu][(hu + k) % c_h] of each side; before softmax times the logit scale
  float wpre[C::CH], wpost[C::CH];
#pragma unroll
  for (int u = 0; u < C::CH; ++u) {
    const int src = (hu + u) & (C::CH - 1);
    wpre[u] = C::MIXPRE ? A.w_pre[((size_t)g * C::CH + hu) * C::CH + src] * A.qk_scale : 0.0f;
    wpost[u] = C::MIXPOST ? A.w_post[((size_t)g * C::CH + hu) * C::CH + src] : 0.0f;
  }

  f32x4 acc[C::NB][C::NQB];
  f32x4 acc2[C::PAIR ? C::NB : 1][C::PAIR ? C::NQB : 1];  // the other head's weights times V of head hu
  auto clear_acc = [&]() MTA_INLINE {
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        acc[nb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (C::PAIR) acc2[nb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
  };
  clear_acc();

  float m_run[C::NQB], l_run[C::NQB];  // reference max (logit units), per-lane partial sums
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    m_run[qb] = -1e30f;
    l_run[qb] = 0.0f;
  }
  const float NEG_INF = -__builtin_inff();
  // statistics written by SPLIT_STATS: row maximum in log2 units and the row sum against it
  float stat_m[C::NQB], stat_l[C::NQB];
  auto split_row = [&](int gr) MTA_INLINE { return ((size_t)split_id * A.B + b) * A.nr + (gr - A.row_begin + SPLIT_HPAD); };
  // normalised schedules in SPLIT_PARTIAL: the global log2 normaliser of every tile row,
  // m + log2(sum_c 2^(m_c - m) l_c) over the statistics every chunk wrote for that row
  // (loaded 8 chunks at a time, combined with a running maximum)
  auto load_shift = [&](float (&sh)[C::NQB]) MTA_INLINE {
    const size_t per_split = (size_t)A.B * A.nr * M * 2;
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      const int gr = row0 + qs0 + qb * 16 + lq;
      sh[qb] = 1e30f;
      if (gr >= 0 && gr < T_) {
        const float* st = A.part_stats + (((size_t)b * A.nr + (gr - A.row_begin + SPLIT_HPAD)) * M + m_head) * 2;
        float mx = -1e30f, l = 0.0f;
        for (int s0 = 0; s0 < A.n_split; s0 += 8) {
          float mv[8], lv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const bool in = s0 + u < A.n_split;
            mv[u] = in ? st[(size_t)(s0 + u) * per_split] : -1e30f;
            lv[u] = in ? st[(size_t)(s0 + u) * per_split + 1] : 0.0f;
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float mn = fmaxf(mx, mv[u]);
            l = l * exp2f(mx - mn) + lv[u] * exp2f(mv[u] - mn);
            mx = mn;
          }
        }
        if (l > 0.0f) sh[qb] = mx + log2f(l);
      }
    }
  };

  // ---- staging (team = the wave itself when it owns its head, else the workgroup) ------
  auto chunk_src = [&](const __bf16* base, int c, int rowfirst, int nrows_per_head) MTA_INLINE {
    const int u = thead + c / (nrows_per_head * (C::D / 8));
    const int rem = c % (nrows_per_head * (C::D / 8));
    const int r = rem / (C::D / 8), cc = rem % (C::D / 8);
    const int j = min(max(rowfirst + r, 0), T_ - 1);  // rows outside the map are masked later
    return base + ((size_t)j * M + g * C::CH + u) * C::D + cc * 8;
  };
  auto k_dst = [&](int c, int lrow, int nrows_per_head) MTA_INLINE {
    const int u = thead + c / (nrows_per_head * (C::D / 8));
    const int rem = c % (nrows_per_head * (C::D / 8));
    const int r = rem / (C::D / 8), cc = rem % (C::D / 8);
    return Ks + ((size_t)u * C::KROWS + lrow + r) * C::LDK + cc * 8;
  };
  auto v_dst = [&](int c) MTA_INLINE {
    const int u = thead + c / (C::BK * (C::D / 8));
    const int rem = c % (C::BK * (C::D / 8));
    const int r = rem / (C::D / 8), cc = rem % (C::D / 8);
    return Vs + ((size_t)u * C::BK + r) * C::LDV + cc * 8;
  };
  auto stage_k_direct = [&](int kfirst, int nrows, int lrow) MTA_INLINE {
    const int total = C::HEADS * nrows * (C::D / 8);
    for (int c = trank; c < total; c += C::TEAM)
      *reinterpret_cast<u32x4*>(k_dst(c, lrow, nrows)) = *reinterpret_cast<const u32x4*>(chunk_src(kb_, c, kfirst, nrows));
  };
  auto stage_v_direct = [&](int j0) MTA_INLINE {
    constexpr int total = C::HEADS * C::BK * (C::D / 8);
    for (int c = trank; c < total; c += C::TEAM)
      *reinterpret_cast<u32x4*>(v_dst(c)) = *reinterpret_cast<const u32x4*>(chunk_src(vb_, c, j0, C::BK));
  };
  // Regular tiles (BK rows per head, rows >= 0): chunk x of a team member is row r_x of
  // head thead + u_x, 16-byte column cc_x; its byte offset from the tile's first row and
  // its LDS element offsets do not change from tile to tile.
  // Two-phase schedules: phase 1 double-buffers K, the second buffer (BK rows per head,
  // stride LDK) in the V region, which phase 1 does not use.
  constexpr bool K2BUF = C::TWO;
  static_assert(!K2BUF || C::BK * C::LDK <= C::BK * C::LDV, "second K buffer fits the V region");
  __bf16* const Ks2 = Vs;
  // When the team's chunks advance by whole rows of one head (UNIFORM: the team covers a whole
  // number of rows, and a head's tile a whole number of team rounds), chunk x of a member is
  // its chunk 0 moved by a fixed number of rows and heads: one base offset per member plus
  // per-x constants (and a wave-uniform global row step), instead of CPT offsets per array.
  constexpr int PH = C::BK * (C::D / 8);  // chunks of one head's tile
  constexpr bool UNIFORM = C::CHUNKS % C::TEAM == 0 && PH % C::TEAM == 0 && C::TEAM % (C::D / 8) == 0;
  constexpr int NOFF = UNIFORM ? 1 : C::CPT;
  int goff[NOFF], koff[NOFF], voff[NOFF], koff2[K2BUF ? NOFF : 1];
#pragma unroll
  for (int x = 0; x < NOFF; ++x) {
    // surplus team members of the last round repeat the last chunk (identical writes)
    const int c = min(trank + x * C::TEAM, C::CHUNKS - 1);
    const int u = thead + c / PH;
    const int rem = c % PH;
    const int r = rem / (C::D / 8), cc = rem % (C::D / 8);
    goff[x] = ((r * M + g * C::CH + u) * C::D + cc * 8) * 2;
    koff[x] = (u * C::KROWS + r) * C::LDK + cc * 8;
    voff[x] = (u * C::BK + r) * C::LDV + cc * 8;
    if constexpr (K2BUF) koff2[x] = (u * C::BK + r) * C::LDK + cc * 8;
  }
  // chunk x of a UNIFORM team: du heads and dr rows after chunk 0
  auto x_du = [](int x) { return UNIFORM ? x / (PH / C::TEAM) : 0; };
  auto x_dr = [](int x) { return UNIFORM ? (x % (PH / C::TEAM)) * (C::TEAM / (C::D / 8)) : 0; };
  auto g_off = [&](int x) MTA_INLINE {
    if constexpr (UNIFORM) return goff[0];
    else return goff[x];
  };
  // the uniform part of chunk x's global byte offset (a scalar operand of the load)
  auto g_soff = [&](int x) MTA_INLINE { return UNIFORM ? (x_dr(x) * M + x_du(x)) * C::D * 2 : 0; };
  auto k_off = [&](int x) MTA_INLINE {
    if constexpr (UNIFORM) return koff[0] + (x_du(x) * C::KROWS + x_dr(x)) * C::LDK;
    else return koff[x];
  };
  auto v_off = [&](int x) MTA_INLINE {
    if constexpr (UNIFORM) return voff[0] + (x_du(x) * C::BK + x_dr(x)) * C::LDV;
    else return voff[x];
  };
  auto k2_off = [&](int x) MTA_INLINE {
    if constexpr (UNIFORM) return koff2[0] + (x_du(x) * C::BK + x_dr(x)) * C::LDK;
    else return koff2[x];
  };
  // buffer resource over rows jfirst .. T-1 of a K or V tensor of batch b
  auto tile_rsrc = [&](const __bf16* base, int jfirst) MTA_INLINE {
    const int rows = max(T_ - jfirst, 0);
    return __builtin_amdgcn_make_buffer_rsrc((void*)(base + (size_t)jfirst * M * C::D), (short)0,
                                             rows * M * C::D * 2, 0x00020000);
  };
  u32x4 pk[C::CPT], pv[C::CPT];
  auto prefetch_k = [&](int kfirst) MTA_INLINE {
    const auto rk = tile_rsrc(kb_, kfirst);
#pragma unroll
    for (int x = 0; x < C::CPT; ++x)
      pk[x] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, g_off(x), g_soff(x), 0));
  };
  auto prefetch_v = [&](int j0) MTA_INLINE {
    const auto rv = tile_rsrc(vb_, j0);
#pragma unroll
    for (int x = 0; x < C::CPT; ++x)
      pv[x] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, g_off(x), g_soff(x), 0));
  };
  auto prefetch = [&](int kfirst, int j0, bool with_v) MTA_INLINE {
    prefetch_k(kfirst);
    if (with_v) prefetch_v(j0);
  };
  auto commit_k = [&](int lrow) MTA_INLINE {
#pragma unroll
    for (int x = 0; x < C::CPT; ++x) *reinterpret_cast<u32x4*>(Ks + k_off(x) + lrow * C::LDK) = pk[x];
  };
  auto commit_k2 = [&]() MTA_INLINE {  // the second K buffer of phase 1
    if constexpr (K2BUF) {
#pragma unroll
      for (int x = 0; x < C::CPT; ++x) *reinterpret_cast<u32x4*>(Ks2 + k2_off(x)) = pk[x];
    }
  };
  auto commit_v = [&]() MTA_INLINE {
#pragma unroll
    for (int x = 0; x < C::CPT; ++x) *reinterpret_cast<u32x4*>(Vs + v_off(x)) = pv[x];
  };
  auto commit = [&](int lrow, bool with_v) MTA_INLINE {
    commit_k(lrow);
    if (with_v) commit_v();
  };

  // ---- compute helpers --------------------------------------------------------------------
  f32x4 s[C::LB][C::NQB];
  // raw S^T of logit block lb into dst[lb], from rows 16*lb - kofs .. 16*lb - kofs + 15 of
  // head hu's K rows (rph rows per head from kbuf)
  auto logit_block_from = [&](auto& dst, const __bf16* kbuf, int rph, int lb, int kofs) MTA_INLINE {
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) dst[lb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const __bf16* kr = kbuf + ((size_t)hu * rph - kofs + lq) * C::LDK + lg * 8;
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(kr + (size_t)lb * 16 * C::LDK + ks * 32);
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb)
        dst[lb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[qb][ks], dst[lb][qb], 0, 0, 0);
    }
  };
  auto logit_block = [&](int lb, int kofs = 0) MTA_INLINE {
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) s[lb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS; ++ks) {
      const bf16x8 af = *reinterpret_cast<const bf16x8*>(
          Ks + ((size_t)hu * C::KROWS + lb * 16 - kofs + lq) * C::LDK + ks * 32 + lg * 8);
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb)
        s[lb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, qf[qb][ks], s[lb][qb], 0, 0, 0);
    }
  };
  // Head mixing of blocks [LB0, LB1) of arr (logits before softmax, weights after) across
  // the heads of the group: every wave writes its blocks (fp16) to the exchange buffer,
  // lane-contiguous, and reads those of the other heads for the same rows. The buffer
  // alternates between two halves, so one barrier per exchange suffices: a half is
  // rewritten only after every wave has passed the barrier of the exchange in between.
  // mix_write / mix_read: the two halves of an exchange through buffer xb, to be separated
  // by a workgroup barrier.
  auto xslot = [&](int xb, int u, int qb) MTA_INLINE {
    return Sx + xb * C::SX_HALF + ((((size_t)u * C::WPH + slab) * C::NQB + qb) * 64 + lane) * C::XW;
  };
  // Mixing on MFMA (C::XM, weights after softmax). The exchange holds, per (head, slab, query
  // block, key block), a 16 x 16 fp16 tile stored query-major (a row of 16 keys per query; the
  // two 8-key halves of a row swap places for queries 8..15, which keeps the 16-byte reads of
  // a lane group on distinct banks). The mixed block of head hu is then one MFMA per pair of
  // heads:
  //   D[key][query] = sum over (head u, key k) of A[key][(u, k)] * B[(u, k)][query]
  // with B the stacked tiles of the pair (lane group lg reads 8 keys of head 2m + lg/2) and A
  // the constant operand w[hu][u] * delta(key, k) (zero for the wave's own head, whose fp32
  // weights enter through the accumulator's initial value instead).
  const int x_woff = lq * 16 + (((lg >> 1) ^ ((lq >> 3) & 1)) * 8) + (lg & 1) * 4;
  const int x_roff = lq * 16 + (((lg & 1) ^ ((lq >> 3) & 1)) * 8);
  auto xtile = [&](int xb, int u, int qb, int x) MTA_INLINE {
    return Sx + xb * C::SX_HALF + ((((size_t)u * C::WPH + slab) * C::NQB + qb) * C::NKB + x) * 256;
  };
  constexpr int NPAIR = C::XM ? C::CH / 2 : 1;
  f16x8 amx_pre[NPAIR], amx_post[NPAIR];
  auto build_amix = [&](f16x8 (&dst)[NPAIR], const float* w, float wscale) MTA_INLINE {
#pragma unroll
    for (int m = 0; m < NPAIR; ++m) {
      const int up = 2 * m + (lg >> 1);
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int key = 8 * (lg & 1) + s;
        float t = 0.0f;
        if (key == lq && up != hu) t = w[((size_t)g * C::CH + hu) * C::CH + up] * wscale;
        dst[m][s] = (_Float16)t;
      }
    }
  };
  if constexpr (C::XM) build_amix(amx_post, A.w_post, 1.0f);
  auto mix_write = [&](auto& arr, int xb, auto lb0c, auto lb1c) MTA_INLINE {
    constexpr int LB0 = decltype(lb0c)::value, LB1 = decltype(lb1c)::value;
    if constexpr (C::CH > 1) {
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
#pragma unroll
        for (int lb = LB0; lb < LB1; ++lb) {
          const f16x4 h = {(_Float16)arr[lb][qb][0], (_Float16)arr[lb][qb][1], (_Float16)arr[lb][qb][2],
                           (_Float16)arr[lb][qb][3]};
          if constexpr (C::XM)
            *reinterpret_cast<f16x4*>(xtile(xb, hu, qb, lb - LB0) + x_woff) = h;
          else
            *reinterpret_cast<f16x4*>(xslot(xb, hu, qb) + (lb - LB0) * 4) = h;
        }
      }
    }
  };
  // Mixed blocks of arr: arr * w[hu][hu] + bias[qb] + the other heads' contributions. bias is
  // folded into the accumulator's initial value on the MFMA path (used for the softmax offset).
  auto mix_read_b = [&](auto& arr, int xb, const float (&wrot)[C::CH], const f16x8 (&amx)[NPAIR], const float* bias,
                        auto lb0c, auto lb1c) MTA_INLINE {
    constexpr int LB0 = decltype(lb0c)::value, LB1 = decltype(lb1c)::value, XB = LB1 - LB0;
    static_assert(XB >= 1 && XB <= C::NKB, "exchange width");
    if constexpr (C::XM) {
      f16x8 bo[NPAIR][C::NQB][XB];
#pragma unroll
      for (int m = 0; m < NPAIR; ++m)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
          for (int x = 0; x < XB; ++x)
            bo[m][qb][x] = *reinterpret_cast<const f16x8*>(xtile(xb, 2 * m + (lg >> 1), qb, x) + x_roff);
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
#pragma unroll
        for (int lb = LB0; lb < LB1; ++lb) {
          f32x4 c;
#pragma unroll
          for (int i = 0; i < 4; ++i) c[i] = bias ? __builtin_fmaf(arr[lb][qb][i], wrot[0], bias[qb]) : arr[lb][qb][i] * wrot[0];
#pragma unroll
          for (int m = 0; m < NPAIR; ++m) c = __builtin_amdgcn_mfma_f32_16x16x32_f16(amx[m], bo[m][qb][lb - LB0], c, 0, 0, 0);
          arr[lb][qb] = c;
        }
      }
      return;
    }
    if constexpr (C::CH == 1) {  // a group of one head: a scalar weight
#pragma unroll
      for (int lb = LB0; lb < LB1; ++lb)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            arr[lb][qb][i] = bias ? __builtin_fmaf(arr[lb][qb][i], wrot[0], bias[qb]) : arr[lb][qb][i] * wrot[0];
    } else {
      f16x4 o[C::CH - 1][C::NQB][XB];
#pragma unroll
      for (int k = 1; k < C::CH; ++k) {
        const int u = (hu + k) & (C::CH - 1);
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
          for (int x = 0; x < XB; ++x) o[k - 1][qb][x] = *reinterpret_cast<const f16x4*>(xslot(xb, u, qb) + x * 4);
      }
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
#pragma unroll
        for (int lb = LB0; lb < LB1; ++lb) {
          f32x4 x;
#pragma unroll
          for (int i = 0; i < 4; ++i) x[i] = bias ? __builtin_fmaf(arr[lb][qb][i], wrot[0], bias[qb]) : arr[lb][qb][i] * wrot[0];
#pragma unroll
          for (int k = 1; k < C::CH; ++k)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = __builtin_fmaf(wrot[k], (float)o[k - 1][qb][lb - LB0][i], x[i]);
          arr[lb][qb] = x;
        }
      }
    }
  };
  auto mix_read = [&](auto& arr, int xb, const float (&wrot)[C::CH], const f16x8 (&amx)[NPAIR], auto lb0c,
                      auto lb1c) MTA_INLINE { mix_read_b(arr, xb, wrot, amx, nullptr, lb0c, lb1c); };
  int xbuf = 0;
  auto mix_blocks = [&](auto& arr, const float (&wrot)[C::CH], const f16x8 (&amx)[NPAIR], auto lb0c,
                        auto lb1c) MTA_INLINE {
    if constexpr (C::CH == 1) {
      mix_read(arr, 0, wrot, amx, lb0c, lb1c);
      return;
    }
    mix_write(arr, xbuf, lb0c, lb1c);
    __syncthreads();
    mix_read(arr, xbuf, wrot, amx, lb0c, lb1c);
    if constexpr (C::XBUFS == 2) xbuf ^= 1;
  };

  // Convolution of a ring (logical blocks of tile kt): output block ob covers the 16 keys
  // that start 8 keys after ring block ob, so it reads ring blocks ob and ob + 1.
  f32x4 cv[C::KQ ? C::NKB : 1][C::NQB];
  _Float16* const Zw = Zb + (C::DUAL ? C::ZRING : 0);  // ring of the weights (both convolutions)
  auto ring_col = [&](int kt, int lb) MTA_INLINE { return ((kt * C::NKB + lb) % C::RB) * 16; };
  // res_c: std::true_type adds the centre tap times the residual ring (C::XC)
  auto convolve_ring = [&](const _Float16* ring, const f16x8 (&tzs)[C::KQ ? C::CQM : 1],
                           f32x4 (&res)[C::KQ ? C::NKB : 1][C::NQB], int kt, auto res_c) MTA_INLINE {
#pragma unroll
    for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) res[ob][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ob = 0; ob < C::NKB; ++ob) {
      // slots of lane group lg: window keys 8*lg .. 8*lg+7 = block ob (lg < 2) or ob+1
      const int col = ring_col(kt, ob + (lg >> 1)) + (lg & 1) * 8;
      if constexpr (decltype(res_c)::value) {
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          const f16x8 br = *reinterpret_cast<const f16x8*>(Zr + ((size_t)hu * C::R + qs0 + qb * 16 + lq) * C::LDZ + col);
          res[ob][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(tzc, br, res[ob][qb], 0, 0, 0);
        }
      }
      // lags a >= c_q have an all-zero Toeplitz operand
#pragma unroll
      for (int a = 0; a < C::CQM; ++a) {
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          const f16x8 bz = *reinterpret_cast<const f16x8*>(
              ring + ((size_t)hu * C::ZROWS + ZPRE + qs0 + qb * 16 + lq - a) * C::LDZ + col);
          res[ob][qb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(tzs[a], bz, res[ob][qb], 0, 0, 0);
        }
      }
    }
  };
  auto convolve = [&](int kt) MTA_INLINE { convolve_ring(Zb, tz, cv, kt, std::integral_constant<bool, C::XC>{}); };
  auto ring_store_to = [&](_Float16* ring, int kt, int lb, int qb, const f32x4& val) MTA_INLINE {
    const f16x4 h = {(_Float16)val[0], (_Float16)val[1], (_Float16)val[2], (_Float16)val[3]};
    *reinterpret_cast<f16x4*>(ring + ((size_t)hu * C::ZROWS + ZPRE + qs0 + qb * 16 + lq) * C::LDZ +
                              ring_col(kt, lb) + lg * 4) = h;
  };
  auto ring_store = [&](int kt, int lb, int qb, const f32x4& val) MTA_INLINE {
    ring_store_to(Zb, kt, lb, qb, val);
    if constexpr (C::XC) {
      // residual of the fp16 rounding, for the exact centre tap
      f16x4 r;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = (_Float16)(val[i] - (float)(_Float16)val[i]);
      *reinterpret_cast<f16x4*>(Zr + ((size_t)hu * C::R + qs0 + qb * 16 + lq) * C::LDZ + ring_col(kt, lb) + lg * 4) = r;
    }
  };

  // AV of the weights of key blocks ob0 .. ob0 + NKB - 1 against V of head hu
  auto av = [&](auto& wts, auto ob0c) MTA_INLINE {
    constexpr int OB0 = decltype(ob0c)::value;
#pragma unroll
    for (int c = 0; c < C::NC; ++c) {
      bf16x8 bp[C::NQB];
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) bp[qb] = pack_bf16(wts[OB0 + 2 * c][qb], wts[OB0 + 2 * c + 1][qb]);
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        // V^T operand: channels nb*16 + (lane & 15); k-slots = keys {4lg..4lg+3} of
        // block 2c and {16+4lg..} of block 2c+1 of this tile
        const s16x4 lo = vtr(Vs + (size_t)hu * C::BK * C::LDV, c * 32 + 4 * lg, nb * 16, C::LDV, lane);
        const s16x4 hi = vtr(Vs + (size_t)hu * C::BK * C::LDV, c * 32 + 16 + 4 * lg, nb * 16, C::LDV, lane);
        s16x4 v8[2] = {lo, hi};
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(v8);
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb)
          acc[nb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bp[qb], acc[nb][qb], 0, 0, 0);
      }
    }
  };
  // Per-pair AV (C::PAIR): the wave's unnormalised bf16 weights go to the exchange buffer
  // (lane-contiguous, 16 bytes per lane and 32-key chunk), and after one barrier the other
  // head's weights for the same rows come back in the same B-operand layout; each V operand of
  // head hu then feeds both products, P_hu V_hu into acc and P_other V_hu into acc2.
  auto pair_av = [&](auto& wts) MTA_INLINE {
    if constexpr (C::PAIR) {
      bf16x8 bp[C::NC][C::NQB], bo[C::NC][C::NQB];
#pragma unroll
      for (int c = 0; c < C::NC; ++c)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          bp[c][qb] = pack_bf16(wts[2 * c][qb], wts[2 * c + 1][qb]);
          *reinterpret_cast<bf16x8*>(xslot(xbuf, hu, qb) + c * 8) = bp[c][qb];
        }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < C::NC; ++c)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) bo[c][qb] = *reinterpret_cast<const bf16x8*>(xslot(xbuf, hu ^ 1, qb) + c * 8);
      if constexpr (C::XBUFS == 2) xbuf ^= 1;
#pragma unroll
      for (int c = 0; c < C::NC; ++c) {
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
          const s16x4 lo = vtr(Vs + (size_t)hu * C::BK * C::LDV, c * 32 + 4 * lg, nb * 16, C::LDV, lane);
          const s16x4 hi = vtr(Vs + (size_t)hu * C::BK * C::LDV, c * 32 + 16 + 4 * lg, nb * 16, C::LDV, lane);
          s16x4 v8[2] = {lo, hi};
          const bf16x8 va = *reinterpret_cast<const bf16x8*>(v8);
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            acc[nb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bp[c][qb], acc[nb][qb], 0, 0, 0);
            acc2[nb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, bo[c][qb], acc2[nb][qb], 0, 0, 0);
          }
        }
      }
    }
  };
  typedef std::integral_constant<int, 0> I0;
  typedef std::integral_constant<int, 1> I1;
  typedef std::integral_constant<int, C::NKB> INKB;
  typedef std::integral_constant<int, C::LB> ILB;
  // first logit block of the tile that is new (block 0 is the carried key halo)
  typedef std::integral_constant<int, C::KQ ? 1 : 0> INEW;

  // exact weights of the last pass (mixing after softmax): no division in the epilogue
  bool normalized = false;
  if constexpr (!C::TWO) {
    // ====================== key loop without a convolution after softmax ====================
    // the softmax sees log2 units: the convolution already folded the scale in
    const float ssc = C::KQ ? 1.0f : sc;
    // Passes over the keys. Without mixing after softmax: REF (reference = the row's
    // maximum over its first key tile, weights exp2(x - ref), AV), and only if a row sum
    // exceeds 2^64: MAX (exact row maxima) then FIXED (weights against them, AV).
    // With mixing after softmax the weights of all heads must be exact before they are
    // mixed: SUM (row sums against the first-tile reference; if too large MAX then
    // SUMFIX), then NORM (exact weights, mixing, AV).
    enum { REF, MAX, FIXED, SUM, SUMFIX, NORM };
    int pass = (C::MIXPOST && !C::PAIR) ? SUM : REF;
    float shift[C::NQB];  // NORM: m * ssc + log2(l) per row
    if (C::SPLIT && C::MIXPOST && A.split_mode == SPLIT_PARTIAL) {  // statistics of the whole key range given
      load_shift(shift);
      pass = NORM;
      normalized = true;
    }
    // Synchronisation. With a workgroup barrier between the logits and the weights (the
    // convolution ring's, or the exchange of the mixing before softmax: MIDBAR), K(kt + 1)
    // is written to LDS right after it (every wave has read K(kt)) and V(kt) at the start of
    // the tile, after the tile's last barrier; that last barrier (TAIL) is the exchange of the
    // mixing after softmax when a pass mixes (V(kt) then goes to LDS after the middle barrier
    // instead), else an explicit one. Without a middle barrier a tile ends with two barriers
    // around the LDS writes of the next tile's K and V.
    constexpr bool MIDBAR = C::KQ || (mix_pre && C::CH > 1);
    for (;;) {
      const bool upd_first = pass == REF || pass == SUM;
      const bool weigh = pass != MAX;
      const bool with_av = pass == REF || pass == FIXED || pass == NORM;
      const bool tail_mix = C::MIXPOST && C::CH > 1 && with_av;  // TAIL is the mixing exchange
      // prologue: tile 0's K rows (with the left halo block) and V rows; halo block 0 of
      // the convolution input computed here so that every tile computes blocks 1..NKB
      if constexpr (C::KQ) stage_k_direct(j0lo - 8, C::BK + 16, 0);
      else stage_k_direct(j0lo, C::BK, 0);
      if constexpr (MIDBAR) {
        if (kt_lo + 1 < kt_hi) prefetch_k(C::KQ ? j0lo + C::BK + 8 : j0lo + C::BK);
        if (with_av) prefetch_v(j0lo);
      } else {
        if (with_av) stage_v_direct(j0lo);
      }
      team_sync<C>();
      if constexpr (C::KQ) {
        logit_block(0);
        if constexpr (mix_pre) mix_blocks(s, wpre, amx_pre, I0{}, I1{});
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          const int gr = row0 + qs0 + qb * 16 + lq;
          f32x4 z = s[0][qb];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int j = j0lo - 8 + 4 * lg + i;
            z[i] = ((gr >= 0) & (j >= 0) & (j <= gr)) ? z[i] : 0.0f;
          }
          ring_store(kt_lo, 0, qb, z);
        }
      }
      for (int kt = kt_lo; kt < kt_hi; ++kt) {
        const int j0 = kt * C::BK;
        const bool more = kt + 1 < kt_hi;
        auto next_v = [&]() MTA_INLINE {  // V(kt) to LDS, load V(kt + 1)
          commit_v();
          if (more) prefetch_v(j0 + C::BK);
        };
        if constexpr (MIDBAR) {
          if (with_av && !tail_mix) next_v();  // every wave finished AV(kt - 1) before TAIL
        } else {
          if (more) prefetch(j0 + C::BK, j0 + C::BK, with_av);
        }
#pragma unroll
        for (int lb = INEW::value; lb < C::LB; ++lb) logit_block(lb);
        if constexpr (mix_pre) mix_blocks(s, wpre, amx_pre, INEW{}, ILB{});
        auto next_k = [&]() MTA_INLINE {  // after the middle barrier: K(kt + 1) to LDS, load K(kt + 2)
          if (with_av && tail_mix) next_v();
          if (more) {
            commit_k(C::KQ ? 16 : 0);
            if (kt + 2 < kt_hi) prefetch_k(C::KQ ? j0 + 2 * C::BK + 8 : j0 + 2 * C::BK);
          }
        };
        if constexpr (MIDBAR && !C::KQ) next_k();
        // softmax input of this tile: cv (after the convolution) or the logits themselves
        auto& xw = [&]() MTA_INLINE -> auto& {
          if constexpr (C::KQ) return cv;
          else return s;
        }();
        if constexpr (C::KQ) {
          // Mask_0 on the new blocks (keys j0 - 8 + 16 lb + 4 lg + i)
          const bool edge = (j0 - 8 < 0) || (j0 + C::BK + 8 - 1 > wrow_min) || (wrow_min < 0);
#pragma unroll
          for (int lb = 1; lb < C::LB; ++lb) {
#pragma unroll
            for (int qb = 0; qb < C::NQB; ++qb) {
              f32x4 z = s[lb][qb];
              if (edge) {
                const int gr = row0 + qs0 + qb * 16 + lq;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int j = j0 - 8 + lb * 16 + 4 * lg + i;
                  z[i] = ((gr >= 0) & (j >= 0) & (j <= gr)) ? z[i] : 0.0f;
                }
              }
              ring_store(kt, lb, qb, z);
            }
          }
          team_sync<C>();  // rows of the neighbouring slab are read by the convolution
          next_k();
          convolve(kt);
        }
        // Mask_-inf
        const bool edge = (j0 + C::BK - 1 > wrow_min) || (qs0 < cq1) || (wrow_min + C::QW > T_);
        if (edge) {
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            const int t = qs0 + qb * 16 + lq;
            const int gr = row0 + t;
            const bool row_ok = (t >= cq1) & (gr < T_);
#pragma unroll
            for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int j = j0 + ob * 16 + 4 * lg + i;
                xw[ob][qb][i] = (row_ok & (j <= gr)) ? xw[ob][qb][i] : NEG_INF;
              }
          }
        }
        if (pass == MAX || (upd_first && kt == kt_lo)) {
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            float mx = NEG_INF;
#pragma unroll
            for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
              for (int i = 0; i < 4; ++i) mx = fmaxf(mx, xw[ob][qb][i]);
            m_run[qb] = fmaxf(m_run[qb], xgroup_max(mx));
          }
        }
        if (weigh) {
          // weights exp2(x - ref) (NORM: exact, exp2(x - shift)) in place; row sums per lane
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            const float mref = pass == NORM ? shift[qb] : m_run[qb] * ssc;
            float sum = 0.0f;
#pragma unroll
            for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float pv = fast_exp2(__builtin_fmaf(xw[ob][qb][i], ssc, -mref));
                xw[ob][qb][i] = pv;
                sum += pv;
              }
            l_run[qb] += sum;
          }
        }
        if (with_av) {
          if constexpr (C::PAIR) {
            pair_av(xw);
          } else {
            if constexpr (C::MIXPOST) mix_blocks(xw, wpost, amx_post, I0{}, INKB{});
            av(xw, I0{});
          }
        }
        if constexpr (MIDBAR) {
          if (!tail_mix) team_sync<C>();  // TAIL
        } else {
          team_sync<C>();  // the team is done with Ks and Vs of this tile
          if (more) commit(0, with_av);
          team_sync<C>();
        }
      }
      if (pass == MAX) {
        pass = (C::MIXPOST && !C::PAIR) ? SUMFIX : FIXED;
        clear_acc();
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) l_run[qb] = 0.0f;
        __syncthreads();
        continue;
      }
      if (pass == NORM) break;
      // final per-query sums (partial per lane group until here)
      bool big = false;
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        l_run[qb] = xgroup_sum(l_run[qb]);
        big |= !(l_run[qb] <= SUM_LIMIT);
      }
      if (upd_first && __syncthreads_or(big ? 1 : 0)) {
        pass = MAX;
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          m_run[qb] = -1e30f;
          l_run[qb] = 0.0f;
        }
        continue;
      }
      if (pass == SUM || pass == SUMFIX) {
        if (C::SPLIT && A.split_mode == SPLIT_STATS) {  // the chunk's statistics are the result
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            stat_m[qb] = m_run[qb] * ssc;
            stat_l[qb] = l_run[qb];
          }
          break;
        }
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb)
          shift[qb] = l_run[qb] > 0.0f ? m_run[qb] * ssc + __builtin_log2f(l_run[qb]) : 1e30f;
        pass = NORM;
        normalized = true;
        __syncthreads();
        continue;
      }
      break;
    }
    if (C::SPLIT && !C::MIXPOST) {  // unnormalised partial: its reference and row sum go with it
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        stat_m[qb] = m_run[qb] * ssc;
        stat_l[qb] = l_run[qb];
      }
    }
    if constexpr (!C::SPLIT) {  // the row statistics the epilogue reports (log-sum-exp output)
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        stat_m[qb] = normalized ? shift[qb] : m_run[qb] * ssc;
        stat_l[qb] = normalized ? 1.0f : l_run[qb];
      }
    }
  } else if constexpr (C::DUAL) {
    // ===================== convolutions before and after softmax ========================
    // Tile kt (j0 = kt * BK; kt = -1 is a lead-in tile that only fills the rings) computes
    // the logits of keys [j0 + 16, j0 + BK + 16) into logit-ring blocks 1..NKB (block b
    // holds keys j0 + 16 b ..), the convolution before softmax of keys [j0 + 8, j0 + BK + 8)
    // (it reads logit blocks ob, ob + 1), and in phase 2 the normalised weights of those
    // keys into weight-ring blocks 1..NKB (block b holds keys j0 - 8 + 16 b ..), then the
    // convolution after softmax of keys [j0, j0 + BK). The ring tile index is kt + 1. The K
    // tile of tile kt (rows j0 + 16 .. j0 + BK + 15) sits at Ks rows 0 .. BK - 1.
    //
    // Synchronisation: the barrier before the convolution before softmax (RING1) is passed
    // once every wave has read the K tile and (phase 2) finished the previous AV, so the
    // prefetched K and V rows go to LDS right after it (the hook); the barrier before the
    // convolution after softmax (phase 2) or the next tile's RING1 (phase 1) publishes them.
    // Phase 1 alternates between two K buffers (Ks and one in the V region) and needs a
    // barrier between a tile's convolution and the next tile's logit-ring writes: the
    // exchange of the mixing before softmax, else an explicit one. In phase 2 that role
    // falls to the barrier before the convolution after softmax; only with mixing on both
    // sides does a tile end with a barrier (the single exchange buffer is rewritten by the
    // next tile's mixing before softmax).
    constexpr bool XBAR = mix_pre && C::CH > 1;
    f32x4 cp[C::NKB][C::NQB];  // convolution before softmax, log2 units
    auto front = [&](int kt, const __bf16* kbuf, bool sync_before_ring, auto&& hook) MTA_INLINE {
      const int j0 = kt * C::BK, kr = kt + 1;
#pragma unroll
      for (int lb = 1; lb < C::LB; ++lb) logit_block_from(s, kbuf, C::BK, lb, 16);
      if constexpr (mix_pre) mix_blocks(s, wpre, amx_pre, I1{}, ILB{});
      if constexpr (!XBAR) {
        if (sync_before_ring) team_sync<C>();
      }
      // Mask_0 on keys j0 + 16 lb + 4 lg + i
      const bool edge0 = (j0 < 0) || (j0 + C::BK + 16 - 1 > wrow_min) || (wrow_min < 0);
#pragma unroll
      for (int lb = 1; lb < C::LB; ++lb) {
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          f32x4 z = s[lb][qb];
          if (edge0) {
            const int gr = row0 + qs0 + qb * 16 + lq;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = j0 + 16 * lb + 4 * lg + i;
              z[i] = ((gr >= 0) & (j >= 0) & (j <= gr)) ? z[i] : 0.0f;
            }
          }
          ring_store(kr, lb, qb, z);
        }
      }
      team_sync<C>();  // RING1: rows of the neighbouring slab are read by the convolution
      hook();
      convolve_ring(Zb, tz, cp, kr, std::false_type{});
      // Mask_-inf: a softmax row needs all c_q logit rows of its convolution inside the
      // tile (t >= c_q - 1) and lies in the map; keys 0 .. gr
      const bool edge1 = (j0 + 8 < 0) || (j0 + C::BK + 8 - 1 > wrow_min) || (qs0 < cq1) || (wrow_min < 0) ||
                         (wrow_min + C::QW > T_);
      if (edge1) {
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          const int t = qs0 + qb * 16 + lq;
          const int gr = row0 + t;
          const bool row_ok = (t >= cq1) & (gr >= 0) & (gr < T_);
#pragma unroll
          for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = j0 + 8 + ob * 16 + 4 * lg + i;
              cp[ob][qb][i] = (row_ok & (j >= 0) & (j <= gr)) ? cp[ob][qb][i] : NEG_INF;
            }
        }
      }
    };

    // phase 1: row sums of the softmax input against a fixed reference (the maximum of the
    // first counted tile); if a sum exceeds 2^64 the workgroup repeats the phase exactly.
    // A key chunk starting at tile kt_lo > 0 counts tiles kt_lo.. (the lead-in tile's keys
    // belong to the previous chunk); the first chunk also counts its lead-in (keys 0 .. 7).
    float lsum[C::NQB];
    float shift[C::NQB];  // p = exp2(x - (m + log2 l))
    const int kfirst = kt_lo == 0 ? -1 : kt_lo;
    if (C::SPLIT && A.split_mode == SPLIT_PARTIAL) {
      load_shift(shift);
    } else {
    for (int exact = 0;; exact = 1) {
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        m_run[qb] = -1e30f;
        l_run[qb] = 0.0f;
      }
      stage_k_direct(j0lo + 16 - C::BK, C::BK, 0);
      if (kt_lo < kt_hi) prefetch_k(kt_lo * C::BK + 16);
      team_sync<C>();
      for (int kt = kt_lo - 1; kt < kt_hi; ++kt) {
        const bool alt = ((kt - kt_lo + 1) & 1) != 0;  // this tile's K rows are in the second buffer
        if (kt + 1 < kt_hi) {
          // K(kt + 1) into the other buffer, whose last reader (the logits of tile kt - 1)
          // every wave finished before the previous RING1
          if (alt) commit_k(0);
          else commit_k2();
          if (kt + 2 < kt_hi) prefetch_k((kt + 2) * C::BK + 16);
        }
        front(kt, alt ? Ks2 : Ks, true, []() MTA_INLINE {});
        const bool counted = kt >= kfirst;
        if (counted && (exact || kt == kfirst)) {
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            float mx = NEG_INF;
#pragma unroll
            for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
              for (int i = 0; i < 4; ++i) mx = fmaxf(mx, cp[ob][qb][i]);
            const float m_new = fmaxf(m_run[qb], xgroup_max(mx));
            l_run[qb] *= fast_exp2(m_run[qb] - m_new);
            m_run[qb] = m_new;
          }
        }
        if (counted) {
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            float sum = 0.0f;
#pragma unroll
            for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
              for (int i = 0; i < 4; ++i) sum += fast_exp2(cp[ob][qb][i] - m_run[qb]);
            l_run[qb] += sum;
          }
        }
      }
      bool big = false;
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        lsum[qb] = xgroup_sum(l_run[qb]);
        big |= !(lsum[qb] <= SUM_LIMIT);
      }
      if (exact || !__syncthreads_or(big ? 1 : 0)) break;
    }
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      shift[qb] = lsum[qb] > 0.0f ? m_run[qb] + __builtin_log2f(lsum[qb]) : 1e30f;
      stat_m[qb] = m_run[qb];
      stat_l[qb] = lsum[qb];
    }
    }

    // phase 2: weights -> weight ring -> convolution after softmax -> Mask_0 -> [mixing] -> AV
    if (!C::SPLIT || A.split_mode != SPLIT_STATS) {
    team_sync<C>();  // every wave is done with both phase-1 K buffers
    stage_k_direct(j0lo + 16 - C::BK, C::BK, 0);
    if (kt_lo < kt_hi) {
      prefetch_k(kt_lo * C::BK + 16);
      prefetch_v(kt_lo * C::BK);
    }
    team_sync<C>();
    for (int kt = kt_lo - 1; kt < kt_hi; ++kt) {
      const int j0 = kt * C::BK, kr = kt + 1;
      front(kt, Ks, false, [&]() MTA_INLINE {
        // every wave has read K(kt) and finished AV(kt - 1): V(kt), K(kt + 1) to LDS
        if (kt >= kt_lo) commit_v();
        if (kt + 1 < kt_hi) {
          commit_k(0);
          if (kt + 2 < kt_hi) prefetch_k((kt + 2) * C::BK + 16);
          if (kt >= kt_lo) prefetch_v((kt + 1) * C::BK);
        }
      });
#pragma unroll
      for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          f32x4 pv;
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = fast_exp2(cp[ob][qb][i] - shift[qb]);
          ring_store_to(Zw, kr, ob + 1, qb, pv);
        }
      team_sync<C>();
      if (kt >= kt_lo) {
        convolve_ring(Zw, tz2, cv, kr, std::false_type{});
        const bool edge2 = (j0 + C::BK - 1 > wrow_min) || (qs0 < halo) || (wrow_min + C::QW > T_);
        if (edge2) {
#pragma unroll
          for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
            for (int qb = 0; qb < C::NQB; ++qb) {
              const int t = qs0 + qb * 16 + lq;
              const int gr = row0 + t;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int j = j0 + ob * 16 + 4 * lg + i;
                cv[ob][qb][i] = ((t >= halo) & (gr < T_) & (j <= gr)) ? cv[ob][qb][i] : 0.0f;
              }
            }
        }
        if constexpr (C::MIXPOST) mix_blocks(cv, wpost, amx_post, I0{}, INKB{});
        av(cv, I0{});
      }
      if constexpr (XBAR && C::MIXPOST && C::CH > 1) __syncthreads();  // the exchange buffer is reused
    }
    }
  } else {
    // ============================= two phase ============================================
    // phase 1: the row sums of head hu (after mixing) against a fixed reference, the
    // maximum of the row's first key tile; if a sum exceeds 2^64 the workgroup repeats the
    // phase as an exact online pass (running maximum, rescaled sum).
    // phase 2: exact normalised weights -> ring -> convolution -> Mask_0 -> [mixing] -> AV.
    //
    // Both phases are software-pipelined so that every stretch between two workgroup
    // barriers holds MFMA work and VALU work that do not depend on each other (the waves of
    // a SIMD run in step, so a stretch of one kind alone leaves the other unit idle):
    //   phase 1, one barrier per tile: the logits of tile kt + 1 (MFMA) beside the mixing,
    //     masking and row sums of tile kt (VALU). K tiles alternate between two buffers (Ks
    //     and one in the V region), mixing exchanges between the two exchange buffers.
    //   phase 2, two barriers per tile: stretch A computes the logits of tile kt + 1 and
    //     writes them to exchange buffer 0; stretch B convolves tile kt and multiplies it with
    //     V (MFMA) beside the mixing and the normalised weights of tile kt + 1 (VALU), which
    //     go to the ring's next NKB blocks (the ring holds LB + NKB blocks per row, so they
    //     never overwrite the window being convolved). K(kt + 2) goes to LDS in stretch B,
    //     V(kt) in stretch A; the mixing after softmax exchanges through buffer 1 inside B.
    // In phase 2 the K tile of tile kt holds rows j0 + 8 .. j0 + BK + 7 (its logit blocks
    // 1..NKB); block 0 of the first tile comes from the last block of a lead-in K tile.
    constexpr bool XBAR = mix_pre && C::CH > 1;  // mixing before softmax exchanges through LDS
    // the barriers of this schedule also order the mixing exchanges, which span the workgroup
    // even when a wave stages its own K and V
    auto tsync = [&]() MTA_INLINE {
      if constexpr (C::MIX && C::CH > 1) __syncthreads();
      else team_sync<C>();
    };
    f32x4 sn[C::LB][C::NQB];  // phase 1: the logits of the other tile of a pair
    float lsum[C::NQB];
    // per-query normaliser folded into the exponent: p = exp2(x*sc - (m*sc + log2 l))
    float shift[C::NQB];
    if (C::SPLIT && A.split_mode == SPLIT_PARTIAL) {
      load_shift(shift);
    } else {
    // tile kt: its logits are in cur and, mixing before softmax, in exchange buffer
    // (kt - kt_lo) & 1, which also names its K buffer (0: Ks, 1: the V region)
    auto p1_sums = [&](auto& cur) MTA_INLINE {
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        const float mref = m_run[qb] * sc;
        float sum = 0.0f;
#pragma unroll
        for (int lb = 1; lb < C::LB; ++lb)
#pragma unroll
          for (int i = 0; i < 4; ++i) sum += fast_exp2(__builtin_fmaf(cur[lb][qb][i], sc, -mref));
        l_run[qb] += sum;
      }
    };
    auto p1_step = [&](int kt, auto& cur, auto& nxt, bool exact) MTA_INLINE {
      const int j0 = kt * C::BK;
      const int pb = (kt - kt_lo) & 1;
      const bool more = kt + 1 < kt_hi;
      if (kt + 2 < kt_hi) {
        // K(kt + 2) into tile kt's buffer, whose logits every wave finished before the last barrier
        if (pb) commit_k2();
        else commit_k(0);
        if (kt + 3 < kt_hi) prefetch_k(j0 + 3 * C::BK);
      }
      const __bf16* kbuf = pb ? Ks : Ks2;
      const bool edge = (j0 + C::BK - 1 > wrow_min) || (wrow_min < 0) || (wrow_min + C::QW > T_);
      if (!(exact || kt == kt_lo || edge)) {
        // interior tile: one branch-free stretch, the next tile's logits (MFMA) beside this
        // tile's mixing and row sums (VALU). After the last tile of a key range the next
        // tile's logits and exchange are computed from stale rows and never used.
        constexpr int NIT = C::NKB * C::KS;      // K operands of the next tile
        constexpr int NEL = C::NKB * C::NQB * 4; // this tile's values per lane
        if constexpr (NEL % NIT == 0) {
          // Interleaved by hand (the scheduler keeps MFMAs together otherwise, and a wave
          // issues in order): this tile's exchange reads first, then per K operand (loaded
          // one step ahead) its MFMAs and an equal share of this tile's mixing and row sums;
          // scheduling barriers keep the steps apart.
          constexpr int EPI = NEL / NIT;
          f16x4 xo[C::CH > 1 ? C::CH - 1 : 1][C::NQB][C::NKB];
          if constexpr (XBAR) {
#pragma unroll
            for (int k = 1; k < C::CH; ++k)
#pragma unroll
              for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
                for (int x = 0; x < C::NKB; ++x)
                  xo[k - 1][qb][x] = *reinterpret_cast<const f16x4*>(xslot(pb, (hu + k) & (C::CH - 1), qb) + x * 4);
          }
          float mref[C::NQB], part[C::NQB];
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) {
            mref[qb] = m_run[qb] * sc;
            part[qb] = 0.0f;
          }
          const __bf16* kr = kbuf + ((size_t)hu * C::BK - 16 + lq) * C::LDK + lg * 8;
          auto kop = [&](int it) MTA_INLINE {
            return *reinterpret_cast<const bf16x8*>(kr + (size_t)(1 + it / C::KS) * 16 * C::LDK + (it % C::KS) * 32);
          };
          bf16x8 af = kop(0);
#pragma unroll
          for (int it = 0; it < NIT; ++it) {
            const int lb = 1 + it / C::KS, ks = it % C::KS;
            const bf16x8 a_it = af;
            if (it + 1 < NIT) af = kop(it + 1);
#pragma unroll
            for (int qb = 0; qb < C::NQB; ++qb) {
              if (ks == 0) nxt[lb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
              nxt[lb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_it, qf[qb][ks], nxt[lb][qb], 0, 0, 0);
            }
#pragma unroll
            for (int k = 0; k < EPI; ++k) {
              const int e = it * EPI + k;
              const int clb = 1 + e / (C::NQB * 4), cqb = (e / 4) % C::NQB, ci = e % 4;
              float x = cur[clb][cqb][ci];
              if constexpr (mix_pre) {
                x *= wpre[0];
#pragma unroll
                for (int kk = 1; kk < C::CH; ++kk) x = __builtin_fmaf(wpre[kk], (float)xo[kk - 1][cqb][clb - 1][ci], x);
              }
              part[cqb] += fast_exp2(__builtin_fmaf(x, sc, -mref[cqb]));
            }
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int qb = 0; qb < C::NQB; ++qb) l_run[qb] += part[qb];
        } else {
#pragma unroll
          for (int lb = 1; lb < C::LB; ++lb) logit_block_from(nxt, kbuf, C::BK, lb, 16);
          if constexpr (mix_pre) mix_read(cur, pb, wpre, amx_pre, I1{}, ILB{});
          p1_sums(cur);
        }
        if constexpr (mix_pre) mix_write(nxt, pb ^ 1, I1{}, ILB{});
        tsync();
        return;
      }
      if (more) {
#pragma unroll
        for (int lb = 1; lb < C::LB; ++lb) logit_block_from(nxt, kbuf, C::BK, lb, 16);
      }
      if constexpr (mix_pre) mix_read(cur, pb, wpre, amx_pre, I1{}, ILB{});
      if (edge) {
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          const int gr = row0 + qs0 + qb * 16 + lq;
          const bool row_ok = (gr >= 0) & (gr < T_);
#pragma unroll
          for (int lb = 1; lb < C::LB; ++lb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = j0 + (lb - 1) * 16 + 4 * lg + i;
              cur[lb][qb][i] = (row_ok & (j <= gr)) ? cur[lb][qb][i] : NEG_INF;
            }
        }
      }
      if (exact || kt == kt_lo) {
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          float mx = NEG_INF;
#pragma unroll
          for (int lb = 1; lb < C::LB; ++lb)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, cur[lb][qb][i]);
          const float m_new = fmaxf(m_run[qb], xgroup_max(mx));
          l_run[qb] *= fast_exp2((m_run[qb] - m_new) * sc);
          m_run[qb] = m_new;
        }
      }
      p1_sums(cur);
      if constexpr (mix_pre) {
        if (more) mix_write(nxt, pb ^ 1, I1{}, ILB{});
      }
      tsync();
    };
    for (int exact = 0;; exact = 1) {
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        m_run[qb] = -1e30f;
        l_run[qb] = 0.0f;
      }
      stage_k_direct(j0lo, C::BK, 0);  // K(kt_lo) into Ks, K(kt_lo + 1) into the second buffer
      if (kt_lo + 1 < kt_hi) {
        prefetch_k(j0lo + C::BK);
        commit_k2();
        if (kt_lo + 2 < kt_hi) prefetch_k(j0lo + 2 * C::BK);
      }
      tsync();
#pragma unroll
      for (int lb = 1; lb < C::LB; ++lb) logit_block_from(s, Ks, C::BK, lb, 16);
      if constexpr (mix_pre) mix_write(s, 0, I1{}, ILB{});
      tsync();
      for (int kt = kt_lo; kt < kt_hi; kt += 2) {
        p1_step(kt, s, sn, exact != 0);
        if (kt + 1 < kt_hi) p1_step(kt + 1, sn, s, exact != 0);
      }
      bool big = false;
#pragma unroll
      for (int qb = 0; qb < C::NQB; ++qb) {
        lsum[qb] = xgroup_sum(l_run[qb]);
        big |= !(lsum[qb] <= SUM_LIMIT);
      }
      if (exact || !__syncthreads_or(big ? 1 : 0)) break;
    }
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      const float l = lsum[qb];
      shift[qb] = l > 0.0f ? m_run[qb] * sc + __builtin_log2f(l) : 1e30f;
      stat_m[qb] = m_run[qb] * sc;
      stat_l[qb] = l;
    }
    }

    // normalised weights of blocks [L0, L1) of arr (tile kt: keys j0 - 8 + 16 lb ..) into the ring
    auto weights_edge = [&](int kt) MTA_INLINE {
      const int j0 = kt * C::BK;
      return (j0 - 8 < 0) || (j0 + C::BK + 8 - 1 > wrow_min) || (wrow_min < 0) || (wrow_min + C::QW > T_);
    };
    // With mixing before softmax the mixing step already subtracts the normaliser (its
    // accumulator starts at w[hu][hu] * x - shift), and the weights are exp2 of the result.
    float nshift[C::NQB];
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) nshift[qb] = -shift[qb];
    auto weights_exp = [&](auto& arr, auto lb0c, auto lb1c) MTA_INLINE {
      constexpr int L0 = decltype(lb0c)::value, L1 = decltype(lb1c)::value;
#pragma unroll
      for (int lb = L0; lb < L1; ++lb)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            arr[lb][qb][i] = fast_exp2(mix_pre ? arr[lb][qb][i] : __builtin_fmaf(arr[lb][qb][i], sc, -shift[qb]));
    };
    auto weights_store = [&](auto& arr, int kt, auto lb0c, auto lb1c) MTA_INLINE {
      constexpr int L0 = decltype(lb0c)::value, L1 = decltype(lb1c)::value;
#pragma unroll
      for (int lb = L0; lb < L1; ++lb)
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) ring_store(kt, lb, qb, arr[lb][qb]);
    };
    auto weights_to_ring = [&](auto& arr, int kt, auto lb0c, auto lb1c) MTA_INLINE {
      constexpr int L0 = decltype(lb0c)::value, L1 = decltype(lb1c)::value;
      const int j0 = kt * C::BK;
      weights_exp(arr, lb0c, lb1c);
      if (weights_edge(kt)) {
#pragma unroll
        for (int qb = 0; qb < C::NQB; ++qb) {
          const int gr = row0 + qs0 + qb * 16 + lq;
          const bool row_ok = (gr >= 0) & (gr < T_);
#pragma unroll
          for (int lb = L0; lb < L1; ++lb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int j = j0 - 8 + lb * 16 + 4 * lg + i;
              arr[lb][qb][i] = (row_ok & (j >= 0) & (j <= gr)) ? arr[lb][qb][i] : 0.0f;
            }
        }
      }
      weights_store(arr, kt, lb0c, lb1c);
    };

    if (!C::SPLIT || A.split_mode != SPLIT_STATS) {
    tsync();  // every wave is done with both phase-1 K buffers
    // lead-in K tile: rows j0lo - BK + 8 .. j0lo + 7, whose last block is block 0 of tile kt_lo
    stage_k_direct(j0lo - C::BK + 8, C::BK, 0);
    prefetch_k(j0lo + 8);
    prefetch_v(j0lo);
    tsync();
    logit_block_from(s, Ks, C::BK, 0, 16 - C::BK);
    if constexpr (XBAR) mix_write(s, 0, I0{}, I1{});
    tsync();  // every wave has read the lead-in rows
    if constexpr (mix_pre) mix_read_b(s, 0, wpre, amx_pre, nshift, I0{}, I1{});
    weights_to_ring(s, kt_lo, I0{}, I1{});
    commit_k(0);  // K(kt_lo)
    if (kt_lo + 1 < kt_hi) prefetch_k(j0lo + C::BK + 8);
    tsync();
    // stretches A and B of the lead-in: tile kt_lo's logits, mixing and weights
#pragma unroll
    for (int lb = 1; lb < C::LB; ++lb) logit_block_from(s, Ks, C::BK, lb, 16);
    if constexpr (XBAR) mix_write(s, 0, I1{}, ILB{});
    tsync();
    if (kt_lo + 1 < kt_hi) {
      commit_k(0);  // K(kt_lo + 1)
      if (kt_lo + 2 < kt_hi) prefetch_k(j0lo + 2 * C::BK + 8);
    }
    if constexpr (mix_pre) mix_read_b(s, 0, wpre, amx_pre, nshift, I1{}, ILB{});
    weights_to_ring(s, kt_lo, I1{}, ILB{});
    tsync();
    for (int kt = kt_lo; kt < kt_hi; ++kt) {
      const int j0 = kt * C::BK;
      const bool more = kt + 1 < kt_hi;
      // stretch A: V(kt) to LDS (every wave finished AV(kt - 1)); the logits of tile kt + 1
      commit_v();
      if (more) {
        prefetch_v(j0 + C::BK);
#pragma unroll
        for (int lb = 1; lb < C::LB; ++lb) logit_block_from(s, Ks, C::BK, lb, 16);
        if constexpr (XBAR) mix_write(s, 0, I1{}, ILB{});
      }
      tsync();
      // stretch B: K(kt + 2) to LDS (every wave read K(kt + 1)); tile kt's convolution and
      // AV beside tile kt + 1's mixing and weights
      if (kt + 2 < kt_hi) {
        commit_k(0);
        if (kt + 3 < kt_hi) prefetch_k(j0 + 3 * C::BK + 8);
      }
      const bool edge2 = (j0 + C::BK - 1 > wrow_min) || (qs0 < cq1) || (wrow_min + C::QW > T_);
      // tile kt's convolution and AV (MFMA), then tile kt + 1's mixing and weights (VALU)
      auto conv_av = [&]() MTA_INLINE {
        convolve(kt);
        if (edge2) {
#pragma unroll
          for (int ob = 0; ob < C::NKB; ++ob)
#pragma unroll
            for (int qb = 0; qb < C::NQB; ++qb) {
              const int t = qs0 + qb * 16 + lq;
              const int gr = row0 + t;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int j = j0 + ob * 16 + 4 * lg + i;
                cv[ob][qb][i] = ((t >= cq1) & (gr < T_) & (j <= gr)) ? cv[ob][qb][i] : 0.0f;
              }
            }
        }
        if constexpr (C::MIXPOST) {
          mix_write(cv, 1, I0{}, INKB{});
          if constexpr (C::CH > 1) tsync();
          mix_read(cv, 1, wpost, amx_post, I0{}, INKB{});
        }
        av(cv, I0{});
      };
      auto next_weights = [&]() MTA_INLINE {
        if (more) {
          if constexpr (mix_pre) mix_read_b(s, 0, wpre, amx_pre, nshift, I1{}, ILB{});
          weights_to_ring(s, kt + 1, I1{}, ILB{});
        }
      };
      conv_av();
      next_weights();
      tsync();
    }
    }
  }

  // ============================= split key range: partial results ==========================
  if constexpr (C::SPLIT) {
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) {
      const int t = qs0 + qb * 16 + lq;
      const int gr = row0 + t;
      if (A.split_mode == SPLIT_STATS) {
        // Each row is written by one workgroup: the tile whose output row it is, or the first
        // tile for the rows before row_begin that feed its convolutions. A tile's first c_q - 1
        // rows have no softmax of their own when a convolution precedes it (one pass, both
        // sides); after softmax alone (two phases) every tile row has its own.
        const bool own = (t >= halo) || (qt == 0 && ((C::TWO && !C::DUAL) || t >= cq1));
        if (own && lg == 0 && gr >= 0 && gr < T_) {
          float* dst = A.part_stats + (split_row(gr) * M + m_head) * 2;
          dst[0] = stat_m[qb];
          dst[1] = stat_l[qb];
        }
      } else if (t >= halo && gr < T_) {
        // output rows: the AV partial, and for unnormalised weights their reference and sum
        float* dst = A.part_o + (split_row(gr) * M + m_head) * C::D;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
          *reinterpret_cast<f32x4*>(dst + nb * 16 + 4 * lg) = acc[nb][qb];
        if (!C::TWO && !C::MIXPOST && lg == 0) {
          float* st = A.part_stats + (split_row(gr) * M + m_head) * 2;
          st[0] = stat_m[qb];
          st[1] = stat_l[qb];
        }
      }
    }
    return;
  }

  // ============================= epilogue =================================================
  // per-pair accumulators: the other head's row sums of the same rows, through the exchange
  // buffer the last tile did not use (its readers all passed that tile's barrier), or after a
  // barrier when there is one buffer
  float l_oth[C::NQB];
  if constexpr (C::PAIR) {
    if constexpr (C::XBUFS == 1) __syncthreads();
    float* xl = reinterpret_cast<float*>(Sx + xbuf * C::SX_HALF);
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb)
      if (lg == 0) xl[((hu * C::WPH + slab) * C::NQB + qb) * 16 + lq] = l_run[qb];
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < C::NQB; ++qb) l_oth[qb] = xl[(((hu ^ 1) * C::WPH + slab) * C::NQB + qb) * 16 + lq];
  }
  __bf16* ob_ = A.out + b * bstride;
#pragma unroll
  for (int qb = 0; qb < C::NQB; ++qb) {
    const int t = qs0 + qb * 16 + lq;
    const int gr = row0 + t;
    f32x4 o[C::NB];
    const float scl = (C::TWO || normalized) ? 1.0f : (l_run[qb] > 0.0f ? 1.0f / l_run[qb] : 0.0f);
    if constexpr (C::PAIR) {
      // O = w[hu][hu] (P_hu V) / l_hu + w[hu][other] (P_other V) / l_other
      const float s_own = wpost[0] * scl;
      const float s_oth = l_oth[qb] > 0.0f ? wpost[1] / l_oth[qb] : 0.0f;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[nb] = acc[nb][qb] * s_own + acc2[nb][qb] * s_oth;
    } else {
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) o[nb] = acc[nb][qb] * scl;
    }
    float mean = 0.0f, inv = 1.0f;
    if (A.gn) {
      float sum = 0.0f;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) sum += (o[nb][0] + o[nb][1]) + (o[nb][2] + o[nb][3]);
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
    if (t >= halo && gr < T_) {
      // for a backward pass: the output before GroupNorm (fp32) and the row's natural
      // log-sum-exp of the softmax input, m + log2(l) in log2 units times ln 2
      if (A.o32) {
        float* d32 = A.o32 + ((b * (size_t)T_ + gr) * M + m_head) * C::D;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) *reinterpret_cast<f32x4*>(d32 + nb * 16 + 4 * lg) = o[nb];
      }
      if (A.lse && lg == 0)
        A.lse[(b * (size_t)T_ + gr) * M + m_head] = (stat_m[qb] + __builtin_log2f(stat_l[qb])) * 0.6931471805599453f;
      __bf16* dst = ob_ + ((size_t)gr * M + m_head) * C::D;
#pragma unroll
      for (int nb = 0; nb < C::NB; ++nb) {
        const int c0 = nb * 16 + 4 * lg;
        f32x4 y = o[nb];
        if (A.gn) {
          const f32x4 ga = *reinterpret_cast<const f32x4*>(A.gamma + (size_t)m_head * C::D + c0);
          const f32x4 be = *reinterpret_cast<const f32x4*>(A.beta + (size_t)m_head * C::D + c0);
          y = A.lambda * (ga * ((y - mean) * inv) + be);
        }
        __bf16 h[4] = {(__bf16)y[0], (__bf16)y[1], (__bf16)y[2], (__bf16)y[3]};
        *reinterpret_cast<uint2*>(dst + c0) = *reinterpret_cast<const uint2*>(h);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
template <class C>
hipError_t launch(const Problem& p, hipStream_t stream) {
  if ((p.split_mode != 0) != C::SPLIT) return hipErrorInvalidValue;
  Args a;
  a.q = reinterpret_cast<const __bf16*>(p.q);
  a.k = reinterpret_cast<const __bf16*>(p.k);
  a.v = reinterpret_cast<const __bf16*>(p.v);
  a.theta = (p.kq & KQ_PRE) ? p.theta_pre : p.theta_post;
  a.theta2 = p.theta_post;
  a.w_pre = p.w_pre;
  a.w_post = p.w_post;
  a.gamma = p.gamma;
  a.beta = p.beta;
  a.lambda = p.lambda;
  a.out = reinterpret_cast<__bf16*>(p.out);
  a.B = p.B;
  a.T = p.T;
  a.M = p.M;
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
  a.split_mode = p.split_mode;
  a.kt_zero = 0;
  a.kt_chunk = p.split_mode ? p.split_keys / C::BK : 0;
  a.n_main = n_bg * a.n_tiles;
  a.nr = p.T - p.row_begin + SPLIT_HPAD;
  a.part_stats = p.part_stats;
  a.part_o = p.part_o;
  a.n_split = p.split_mode ? p.split_n : 1;
  a.lse = p.split_mode ? nullptr : p.lse;
  a.o32 = p.split_mode ? nullptr : p.o32;
  if (p.split_mode && (p.split_keys <= 0 || p.split_keys % C::BK != 0)) return hipErrorInvalidValue;
  const long long blocks = (long long)n_bg * a.n_tiles * (p.split_mode ? p.split_n : 1);
  if (blocks <= 0 || blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kmajor_kernel<C>, dim3((unsigned)blocks), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

// Query halo rows of a tile: c_q - 1 per convolution.
inline int tile_halo(const Problem& p) { return p.kq ? ((p.kq == KQ_BOTH) ? 2 : 1) * (p.c_q - 1) : 0; }
// Rows per tile of the launched shape. A split key range whose output rows fit one 16-row tile
// (a decode step) takes tiles of 16 rows with one wave per head of the group; the unsplit
// per-pair schedule of two-head groups at d = 96 takes 12 waves of 16 rows (see launch_shape);
// everything else takes 8 waves of 32 rows. The key-split plan uses the same figure.
constexpr int SMALL_R = 16;
inline bool short_rows(const Problem& p) { return p.T - p.row_begin <= SMALL_R - tile_halo(p); }
inline bool small_tiles(const Problem& p) { return p.split_mode != 0 && short_rows(p); }
inline int tile_rows(const Problem& p, bool split) {
  const int ch = p.mix ? p.c_h : 1;
  if (split && short_rows(p)) return SMALL_R;
  if (!split && !p.fp32 && p.d == 96 && ch == 2 && p.kq == KQ_PRE && p.mix == MIX_POST) return 16 * 6;
  return 32 * (8 / ch);
}

// Tile shapes: 8 waves of 32 query rows (two waves per SIMD, so one wave's MFMA work
// overlaps the other's LDS and VALU work). Key tiles of 64 keys, 32 when the LDS holds
// four heads, the fp16 exchange of a mixing group, or (convolution before softmax) when
// the ring, the convolution output and the logits are live in registers together.
// SPLIT selects the instantiations that cover one chunk of a split key range; those also come
// with 16-row tiles of one wave per head for short row ranges.
template <int D, int CH, bool KQ, bool TWO, bool MIXPOST, int CQM, bool SPLIT>
hipError_t launch_shape(const Problem& p, hipStream_t stream) {
  constexpr bool small = CH == 4 || (CH > 1 && MIXPOST) || (KQ && !TWO);
  constexpr int BK = small ? 32 : 64;
  auto go = [&](auto qwc, auto nwc) -> hipError_t {
    constexpr int QW = decltype(qwc)::value, NW = decltype(nwc)::value;
    if constexpr (!MIXPOST) {
      if (p.mix == MIX_PRE)
        return launch<Cfg<D, CH, QW, (CH > 1 ? 32 : BK), KQ, TWO, false, CQM, true, NW, false, SPLIT>>(p, stream);
    } else {
      if (p.mix == MIX_BOTH) return launch<Cfg<D, CH, QW, BK, KQ, TWO, true, CQM, true, NW, false, SPLIT>>(p, stream);
    }
    // per-pair accumulators for two-head groups at d = 96 (the 880M-model layer): 12 waves of 16
    // rows, three per SIMD (161 registers, 86 KB of LDS; 0.249 -> 0.242 ms against 8 waves of 32)
    if constexpr (!SPLIT && KQ && !TWO && MIXPOST && CH == 2 && D == 96 && QW == 32) {
      if (p.mix == MIX_POST) return launch<Cfg<D, CH, 16, BK, KQ, TWO, true, CQM, false, 12, false, SPLIT>>(p, stream);
    }
    return launch<Cfg<D, CH, QW, BK, KQ, TWO, MIXPOST, CQM, false, NW, false, SPLIT>>(p, stream);
  };
  if constexpr (SPLIT) {
    if (small_tiles(p)) return go(std::integral_constant<int, SMALL_R>{}, std::integral_constant<int, CH>{});
  }
  return go(std::integral_constant<int, 32>{}, std::integral_constant<int, 8>{});
}

template <int D, int CH, bool KQ, bool TWO, bool MIXPOST, bool SPLIT>
hipError_t launch_cq(const Problem& p, hipStream_t stream) {
  if constexpr (!KQ) {
    return launch_shape<D, CH, KQ, TWO, MIXPOST, 1, SPLIT>(p, stream);
  } else {
    // Toeplitz operands held in registers: one per query lag, rounded up
    if (p.c_q <= 4) return launch_shape<D, CH, KQ, TWO, MIXPOST, 4, SPLIT>(p, stream);
    if (p.c_q <= 6) return launch_shape<D, CH, KQ, TWO, MIXPOST, 6, SPLIT>(p, stream);
    return launch_shape<D, CH, KQ, TWO, MIXPOST, 8, SPLIT>(p, stream);
  }
}

// Convolutions on both sides: 32-key tiles (two rings, two sets of Toeplitz operands).
template <int D, int CH, bool MIXPOST, int CQM, bool SPLIT>
hipError_t launch_dual_shape(const Problem& p, hipStream_t stream) {
  auto go = [&](auto qwc, auto nwc) -> hipError_t {
    constexpr int QW = decltype(qwc)::value, NW = decltype(nwc)::value;
    if (p.mix & MIX_PRE) return launch<Cfg<D, CH, QW, 32, true, true, MIXPOST, CQM, true, NW, true, SPLIT>>(p, stream);
    return launch<Cfg<D, CH, QW, 32, true, true, MIXPOST, CQM, false, NW, true, SPLIT>>(p, stream);
  };
  if constexpr (SPLIT) {
    if (small_tiles(p)) return go(std::integral_constant<int, SMALL_R>{}, std::integral_constant<int, CH>{});
  }
  return go(std::integral_constant<int, 32>{}, std::integral_constant<int, 8>{});
}

template <int D, int CH, bool MIXPOST, bool SPLIT>
hipError_t launch_dual(const Problem& p, hipStream_t stream) {
  if (p.c_q <= 4) return launch_dual_shape<D, CH, MIXPOST, 4, SPLIT>(p, stream);
  if (p.c_q <= 6) return launch_dual_shape<D, CH, MIXPOST, 6, SPLIT>(p, stream);
  return launch_dual_shape<D, CH, MIXPOST, 8, SPLIT>(p, stream);
}

// The schedules with a convolution after softmax (POSTCONV) and the others are instantiated in
// separate translation units, which are compiled with different instruction-scheduling options.
template <int D, int CH, bool POSTCONV, bool SPLIT>
hipError_t launch_ch(const Problem& p, hipStream_t stream) {
  const bool post = (p.mix & MIX_POST) != 0;
  if constexpr (POSTCONV) {
    if (p.kq == KQ_BOTH) {
      if (post) return launch_dual<D, CH, true, SPLIT>(p, stream);
      return launch_dual<D, CH, false, SPLIT>(p, stream);
    }
    if (post) return launch_cq<D, CH, true, true, true, SPLIT>(p, stream);
    return launch_cq<D, CH, true, true, false, SPLIT>(p, stream);
  } else {
    if (p.kq == KQ_PRE) {
      if (post) return launch_cq<D, CH, true, false, true, SPLIT>(p, stream);
      return launch_cq<D, CH, true, false, false, SPLIT>(p, stream);
    }
    if (post) return launch_cq<D, CH, false, false, true, SPLIT>(p, stream);
    return launch_cq<D, CH, false, false, false, SPLIT>(p, stream);
  }
}

template <int D, bool POSTCONV, bool SPLIT>
hipError_t launch_d(const Problem& p, hipStream_t stream) {
  const int ch = p.mix ? p.c_h : 1;
  switch (ch) {
    case 1: return launch_ch<D, 1, POSTCONV, SPLIT>(p, stream);
    case 2: return launch_ch<D, 2, POSTCONV, SPLIT>(p, stream);
    case 4: return launch_ch<D, 4, POSTCONV, SPLIT>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace kmajor
}  // namespace mta
