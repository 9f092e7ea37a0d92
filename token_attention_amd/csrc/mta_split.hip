// Output rows row_begin .. T-1 of the fused layer with the key range split over workgroups.
//
// A decode step (one new row per sequence) or a short chunk has few row tiles, so the fused
// kernel would run a handful of workgroups that each walk every key. Here each row tile's keys
// are cut into chunks of split_keys keys, one workgroup per (chunk, row tile), and the partial
// results are combined afterwards, which is exact because softmax statistics and AV sums add
// up over key chunks (page "Multi-Token Attention | Summary", §2: the output is a weighted sum
// over keys; §3.1-§3.2: the convolutions and mixing act per key neighbourhood and head group):
//   * weights against a per-chunk reference (no normalisation needed before AV): one pass
//     writing (reference, row sum, AV partial) per chunk; the output is
//     sum_c 2^(m_c - m) AV_c / sum_c 2^(m_c - m) l_c;
//   * weights that must be exact first (a convolution or mixing after softmax): a statistics
//     pass per chunk, then a weighted pass per chunk that first combines every chunk's
//     statistics of its rows into one log2 normaliser per (row, head); its AV partials simply
//     add up.
// GroupNorm and the gate follow in the combining kernel.
#include <algorithm>
#include <atomic>

#include "mta_kmajor_impl.h"

namespace mta {

// Compute units of the current device (hipDeviceAttributeMultiprocessorCount), read once per
// device; 256 (MI355X) when no device can be queried, so that size queries still answer on a
// host without a GPU. The workspace-size query and the launch read the same value.
int device_compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return 256;
  }
  int cus = cached[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    return 256;
  }
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

namespace {

constexpr int HPAD = kmajor::SPLIT_HPAD;
constexpr int NSPLIT_MAX = 64;
static_assert(NSPLIT_MAX <= 64, "the output combination holds one chunk per lane");
constexpr double WG_OVERHEAD = 0.04;     // fixed cost of a workgroup, relative to a whole row tile

}  // namespace

// Number of key chunks, when the row tiles alone leave compute units idle: workgroups run in
// rounds of cus (one fused workgroup fits per compute unit), each costing the fixed overhead
// plus its share of the keys; the plan minimises
// rounds * (overhead + 1/n) (chunks are whole multiples of 64 keys). 16-row tiles of a group of
// four heads (four waves whose LDS fills a compute unit) count a round as 7/8 of the units:
// at exactly one such workgroup per unit a launch took longer than at 13/16 of that (T=4096 decode
// step: 16 chunks of 256 keys 76 us, 13 chunks of 320 keys 64 us). A decode step at T=4096
// with 16 row tiles of a four-head group gets 13 chunks of 320 keys (256 compute units), a
// 512-row chunk 5 chunks of 832 keys.
SplitPlan split_plan(const Problem& p, int cus) {
  if (p.fp32) return {1, 0};
  // row tiles of the unsplit kernel and of the split instantiations (16-row tiles for a range
  // that fits one, such as a decode step)
  const int ch = p.mix ? p.c_h : 1;
  const int halo = kmajor::tile_halo(p), rows = p.T - p.row_begin;
  const int r_out = kmajor::tile_rows(p, false) - halo, r_split = kmajor::tile_rows(p, true) - halo;
  const long long groups = (long long)p.B * (p.M / ch);
  const long long tiles = groups * ((rows + r_out - 1) / r_out);
  const long long tiles_split = groups * ((rows + r_split - 1) / r_split);
  // enough row tiles to occupy every compute unit: the unsplit kernel (heaviest tiles first)
  if (cus <= 0) cus = 1;
  if (tiles >= cus) return {1, 0};
  SplitPlan best{1, 0};
  double best_cost = (double)((tiles + cus - 1) / cus) * (WG_OVERHEAD + 1.0);
  const int nmax = std::min(NSPLIT_MAX, (p.T + 63) / 64);
  const long long per_round = (kmajor::short_rows(p) && ch >= 4) ? cus - cus / 8 : cus;
  for (int n = 2; n <= nmax; ++n) {
    const int keys = ((p.T + n - 1) / n + 63) / 64 * 64;
    const int neff = (p.T + keys - 1) / keys;
    const double rounds = (double)((tiles_split * neff + per_round - 1) / per_round);
    const double cost = rounds * (WG_OVERHEAD + 1.0 / neff);
    if (cost < best_cost * 0.999) {
      best_cost = cost;
      best = {neff, keys};
    }
  }
  return best.n <= 1 ? SplitPlan{1, 0} : best;
}

namespace {

struct SplitLayout {
  size_t nr, rows;  // rows of the partial buffers; B * nr * M
  size_t stats, o, total;
};

SplitLayout split_layout(const Problem& p, int n) {
  SplitLayout l{};
  l.nr = (size_t)(p.T - p.row_begin) + HPAD;
  l.rows = (size_t)p.B * l.nr * p.M;
  auto up = [](size_t x) { return (x + 63) & ~(size_t)63; };
  l.stats = 0;
  l.o = l.stats + up((size_t)n * l.rows * 2);
  l.total = (l.o + (size_t)n * l.rows * p.d) * sizeof(float);
  return l;
}

// statistics entries no workgroup writes stay (maximum -1e30, sum 0)
__global__ void split_fill_kernel(float* stats, size_t n) {
  const size_t x = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (x < n) {
    stats[2 * x] = -1e30f;
    stats[2 * x + 1] = 0.0f;
  }
}

// Partials of up to SBATCH chunks are loaded together so that their memory latencies overlap.
constexpr int SBATCH = 8;

// one wave per (b, output row, head): combine the AV partials, GroupNorm + gate, write out.
// Lane s holds chunk s's statistics (at most 64 chunks); the partials are loaded in batches.
template <int D>
__global__ __launch_bounds__(256) void split_out_kernel(const float* __restrict__ part_o,
                                                        const float* __restrict__ stats, int weighted,
                                                        int nsplit, int B, int nr, int M, int row_begin, int Tn,
                                                        const float* __restrict__ gamma,
                                                        const float* __restrict__ beta, float lambda, int gn,
                                                        __bf16* __restrict__ out) {
  constexpr int CPL = (D + 63) / 64;
  const int lane = threadIdx.x & 63;
  const size_t wid = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nout = Tn - row_begin;
  if (wid >= (size_t)B * nout * M) return;
  const int m = (int)(wid % M), r = (int)((wid / M) % nout), b = (int)(wid / ((size_t)M * nout));
  const size_t rows = (size_t)B * nr * M;
  const size_t idx = ((size_t)b * nr + r + HPAD) * M + m;
  float o[CPL];
#pragma unroll
  for (int k = 0; k < CPL; ++k) o[k] = 0.0f;
  // weight of chunk `lane` and the denominator (per-chunk references), else weight 1
  float wl = 1.0f, den = 0.0f;
  if (weighted) {
    const bool in = lane < nsplit;
    const float ms = in ? stats[((size_t)lane * rows + idx) * 2] : -1e30f;
    const float ls = in ? stats[((size_t)lane * rows + idx) * 2 + 1] : 0.0f;
    float mx = ms;
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    wl = in ? exp2f(ms - mx) : 0.0f;
    den = ls * wl;
    for (int off = 32; off > 0; off >>= 1) den += __shfl_xor(den, off);
  }
  for (int s0 = 0; s0 < nsplit; s0 += SBATCH) {
    float pv[SBATCH][CPL];
#pragma unroll
    for (int u = 0; u < SBATCH; ++u)
#pragma unroll
      for (int k = 0; k < CPL; ++k) {
        const int c = lane + 64 * k;
        pv[u][k] = (s0 + u < nsplit && c < D) ? part_o[((size_t)(s0 + u) * rows + idx) * D + c] : 0.0f;
      }
#pragma unroll
    for (int u = 0; u < SBATCH; ++u) {
      const float ws = __shfl(wl, (s0 + u) & 63);
#pragma unroll
      for (int k = 0; k < CPL; ++k) o[k] += ws * pv[u][k];
    }
  }
  if (weighted) {
    const float inv = den > 0.0f ? 1.0f / den : 0.0f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) o[k] *= inv;
  }
  float mean = 0.0f, rs = 1.0f;
  if (gn) {
    float sum = 0.0f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) sum += (lane + 64 * k < D) ? o[k] : 0.0f;
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off);
    mean = sum * (1.0f / D);
    float sq = 0.0f;
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
      const float dv = (lane + 64 * k < D) ? o[k] - mean : 0.0f;
      sq += dv * dv;
    }
    for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
    rs = 1.0f / sqrtf(sq * (1.0f / D) + 1e-5f);
  }
  __bf16* dst = out + (((size_t)b * Tn + row_begin + r) * M + m) * D;
#pragma unroll
  for (int k = 0; k < CPL; ++k) {
    const int c = lane + 64 * k;
    if (c < D) {
      float y = o[k];
      if (gn) y = lambda * (gamma[(size_t)m * D + c] * (y - mean) * rs + beta[(size_t)m * D + c]);
      dst[c] = (__bf16)y;
    }
  }
}

hipError_t launch_out(const Problem& p, const SplitLayout& l, float* ws, int n, bool weighted, hipStream_t st) {
  const size_t waves = (size_t)p.B * (p.T - p.row_begin) * p.M;
  const dim3 grid((unsigned)((waves + 3) / 4));
  __bf16* out = reinterpret_cast<__bf16*>(p.out);
  const int w = weighted ? 1 : 0;
  switch (p.d) {
#define MTA_D(DV)                                                                                                   \
  case DV:                                                                                                        \
    hipLaunchKernelGGL(split_out_kernel<DV>, grid, dim3(256), 0, st, ws + l.o, ws + l.stats, w, n, p.B, (int)l.nr, \
                       p.M, p.row_begin, p.T, p.gamma, p.beta, p.lambda, p.gn, out);                              \
    break;
    MTA_D(32) MTA_D(64) MTA_D(96) MTA_D(128)
#undef MTA_D
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

size_t rows_split_workspace_bytes(const Problem& p) {
  const SplitPlan plan = split_plan(p, device_compute_units());
  return plan.n <= 1 ? 0 : split_layout(p, plan.n).total;
}

hipError_t launch_rows_split(const Problem& p0, void* workspace, hipStream_t st, bool* unsupported) {
  *unsupported = false;
  const SplitPlan plan = split_plan(p0, device_compute_units());
  if (plan.n <= 1) return launch_fused(p0, st, unsupported);
  if (!fused_supported(p0)) {
    *unsupported = true;
    return hipSuccess;
  }
  const SplitLayout l = split_layout(p0, plan.n);
  float* ws = reinterpret_cast<float*>(workspace);
  Problem p = p0;
  p.split_n = plan.n;
  p.split_keys = plan.keys;
  p.part_stats = ws + l.stats;
  p.part_o = ws + l.o;
  hipError_t e;
  const size_t nstat = (size_t)plan.n * l.rows;
  hipLaunchKernelGGL(split_fill_kernel, dim3((unsigned)((nstat + 255) / 256)), dim3(256), 0, st, p.part_stats, nstat);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const bool normalised = (p.kq & KQ_POST) || (p.mix & MIX_POST);
  if (normalised) {
    p.split_mode = kmajor::SPLIT_STATS;
    if ((e = launch_fused(p, st, unsupported)) != hipSuccess || *unsupported) return e;
  }
  p.split_mode = kmajor::SPLIT_PARTIAL;
  if ((e = launch_fused(p, st, unsupported)) != hipSuccess || *unsupported) return e;
  return launch_out(p, l, ws, plan.n, !normalised, st);
}

}  // namespace mta
