// Internal interface between the C-ABI layer (mta_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace mta {

// Placements are bit sets: before softmax, after softmax, or both sides.
enum KqMode { KQ_NONE = 0, KQ_PRE = 1, KQ_POST = 2, KQ_BOTH = 3 };
enum MixMode { MIX_NONE = 0, MIX_PRE = 1, MIX_POST = 2, MIX_BOTH = 3 };

// A fully validated problem description (sizes already checked by the API layer).
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  const float* theta_pre;   // [M, c_q, c_k] kernels before softmax, or null
  const float* theta_post;  // [M, c_q, c_k] kernels after softmax, or null
  const float* w_pre;       // [M/c_h, c_h, c_h] mixing before softmax, or null
  const float* w_post;      // [M/c_h, c_h, c_h] mixing after softmax, or null
  const float* gamma;  // [M*d] or null
  const float* beta;   // [M*d] or null
  float lambda;
  void* out;
  int B, T, M, d, c_q, c_k, c_h;
  int kq;    // KqMode bits
  int mix;   // MixMode bits
  int gn;    // 0/1
  int fp32;  // 0: bf16 tensors, 1: fp32 tensors
  int row_begin = 0;  // fused path: output rows row_begin .. T-1 only
  // fused bf16 path: the key range split over split_n workgroups per row tile (0: no split)
  int split_mode = 0;            // 1: write partial softmax statistics, 2: write partial AV
  int split_keys = 0;            // keys per split, a multiple of 64
  int split_n = 1;
  float* part_stats = nullptr;   // partial buffers in the caller's workspace
  float* part_o = nullptr;
  // fused bf16 path, unsplit, optional: what a backward pass keeps from the forward
  float* lse = nullptr;          // [B, T, M] natural log-sum-exp of every softmax row
  float* o32 = nullptr;          // [B, T, M, d] output before GroupNorm, fp32
};

// Returns hipSuccess or the launch error; sets *unsupported when no kernel is
// instantiated for the shape.
hipError_t launch_fused(const Problem& p, hipStream_t stream, bool* unsupported);
bool fused_supported(const Problem& p);

// Output rows row_begin .. T-1 with the key range split over workgroups (few row tiles: a
// decode step or a short chunk); falls back to launch_fused when splitting does not pay.
size_t rows_split_workspace_bytes(const Problem& p);
// The key-split plan of a row range on a device with `cus` compute units: n chunks of `keys`
// keys each (n = 1: no split), and the current device's compute-unit count the launches use.
struct SplitPlan {
  int n, keys;
};
SplitPlan split_plan(const Problem& p, int cus);
int device_compute_units();
hipError_t launch_rows_split(const Problem& p, void* workspace, hipStream_t stream, bool* unsupported);

size_t materialized_workspace_bytes(int B, int T, int M);
hipError_t launch_materialized(const Problem& p, void* workspace, hipStream_t stream,
                               bool* unsupported);
bool materialized_supported(const Problem& p);

}  // namespace mta
