/*
 * libmta: Multi-Token Attention forward layer for AMD MI355X (gfx950).
 *
 * The layer is the one described on the page "Multi-Token Attention | Summary"
 * (greeksharifa.github.io): per-head logits QK^T/sqrt(d) (§2), a key-query
 * convolution over (query, key) with a separate c_q x c_k kernel per head, either
 * before softmax with Mask_0 before it and Mask_-inf after it, or after softmax
 * (§3.1), a head-mixing linear map inside groups of c_h heads, before or after
 * softmax (§3.2), the AV product (§2), and a per-head GroupNorm followed by a
 * scalar gate (§3.3).
 *
 * Conventions shared by every entry point
 *   Layout      q, k, v, out: [B, T, M, d] contiguous (token-major, heads
 *               concatenated, hidden size D = M*d). bf16 unless MTA_FP32 is set,
 *               then fp32. out has the input dtype.
 *   theta_kq    [M, c_q, c_k] fp32. theta[m][a][e] weighs the map entry at
 *               (query i-a, key j-e+h0), h0 = (c_k-1)/2: the query axis reaches only
 *               current and past rows (§3.1), the key axis is centred. Entries
 *               outside the T x T map count as 0. With MTA_KQ_PRE | MTA_KQ_POST it is
 *               [2, M, c_q, c_k]: the kernels before softmax, then those after.
 *   w_mix       [M/c_h, c_h, c_h] fp32, w[g][out][in] (§3.2 mixing equations);
 *               group g holds heads g*c_h .. g*c_h+c_h-1. With MTA_MIX_PRE |
 *               MTA_MIX_POST it is [2, M/c_h, c_h, c_h], the side before softmax first.
 *   GroupNorm   per (token, head) over the d channels, biased variance, eps 1e-5:
 *               out = lambda * (gamma[m*d+t] * (O_t - mean) / sqrt(var + eps) +
 *               beta[m*d+t]); gn_gamma, gn_beta are [M*d] fp32. lambda is the gate
 *               value itself (already passed through its sigmoid or depth rule).
 *   Placement   the key-query convolution acts before softmax (MTA_KQ_PRE), after
 *               it (MTA_KQ_POST), on both sides (both flags, each side with its own
 *               kernels: the default of the page's experiments, §4) or not at all;
 *               head mixing likewise (MTA_MIX_PRE, MTA_MIX_POST). On one side of
 *               softmax the two act in sequence: mixing before the convolution on
 *               the pre side, the convolution before mixing on the post side (§3.3:
 *               together they form one convolution over queries, keys and heads).
 *   Memory      every pointer is device memory owned by the caller. Nothing is
 *               retained after a call returns; buffers must stay alive until the
 *               queued work completes. q, k, v, out, workspace and (with MTA_GN)
 *               gn_gamma, gn_beta must be 16-byte aligned. The library cannot see the
 *               extent of a parameter array: theta_kq, w_mix, gn_gamma and gn_beta must
 *               hold the sizes given above for the flags passed, or the kernels read
 *               past their end.
 *   Streams     stream is a hipStream_t (NULL = the default stream). Calls are
 *               asynchronous: they validate, enqueue and return. Launch errors are
 *               reported; faults during execution surface at the caller's sync.
 *   Errors      functions return an mta_status; they never abort or throw. A
 *               thread-local message with details is kept for mta_last_error().
 *   Threads     reentrant; no global mutable state besides the per-thread message.
 */
#ifndef MTA_H
#define MTA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mta_status {
  MTA_OK = 0,
  MTA_ERR_INVALID_ARG = 1, /* sizes <= 0, M % c_h != 0, NULL/misaligned pointers,
                              unknown flag bits                                  */
  MTA_ERR_UNSUPPORTED = 2, /* valid but not built: d, dtype, c_q > 8, even c_k,
                              c_k > 17, c_h not in {1, 2, 4}, one batch of a
                              tensor (T*M*d elements) of 2 GiB or more           */
  MTA_ERR_HIP = 3,         /* the HIP runtime reported an error                   */
  MTA_ERR_WORKSPACE = 4    /* workspace missing or smaller than required          */
} mta_status;

#define MTA_KQ_PRE 0x1u   /* key-query convolution before softmax (§3.1 equation)  */
#define MTA_KQ_POST 0x2u  /* key-query convolution after softmax, then Mask_0     */
#define MTA_MIX_PRE 0x4u  /* head mixing of the logits, before softmax (§3.2)     */
#define MTA_MIX_POST 0x8u /* head mixing of the softmax weights (§3.2)            */
/* Both bits of a pair: that operation on both sides of softmax. */
#define MTA_GN 0x10u      /* per-head GroupNorm and scalar gate (§3.3)            */
#define MTA_FP32 0x20u    /* q, k, v, out are fp32 instead of bf16                */

/*
 * mta_forward: fused forward of the whole layer (§2-§3.3) in one kernel launch.
 * Flash-style: the T x T maps are never written to memory; each workgroup owns one
 * head group and one tile of query rows and recomputes the logits of the c_q-1
 * preceding rows and of the key halo it needs. Allocates nothing.
 *   q, k, v      inputs [B,T,M,d]
 *   theta_kq     required iff a KQ flag is set (ignored otherwise); [2, M, c_q, c_k]
 *                with both KQ flags
 *   w_mix        required iff a MIX flag is set (ignored otherwise); [2, M/c_h, c_h,
 *                c_h] with both MIX flags
 *   gn_gamma/beta, lambda   required iff MTA_GN (ignored otherwise)
 *   out          [B,T,M,d] output; may not alias the inputs
 *   c_q, c_k     kernel size; ignored without a KQ flag. 1 <= c_q <= 8, c_k odd <= 17
 *   c_h          head-group size; M % c_h == 0; c_h in {1,2,4}; ignored without MIX
 *   flags        MTA_* bits above
 * Supported head sizes: d in {32, 64, 96, 128} for bf16, d in {16, 32, 64} for fp32.
 * Every placement is built for both dtypes.
 */
int mta_forward(const void* q, const void* k, const void* v, const float* theta_kq,
                const float* w_mix, const float* gn_gamma, const float* gn_beta, float lambda,
                void* out, int B, int T, int M, int d, int c_q, int c_k, int c_h, unsigned flags,
                void* stream);

/*
 * mta_forward_materialized: the same layer as mta_forward computed the unfused way,
 * one kernel per step, with full fp32 [B, M, T, T] maps in the caller's workspace
 * (the memory-hungry implementation style whose cost the page's complexity table,
 * Appendix F, attributes to MTA). Same arguments as mta_forward plus:
 *   workspace        device buffer of at least mta_materialized_workspace_bytes()
 *   workspace_bytes  its size
 */
int mta_forward_materialized(const void* q, const void* k, const void* v, const float* theta_kq,
                             const float* w_mix, const float* gn_gamma, const float* gn_beta,
                             float lambda, void* out, int B, int T, int M, int d, int c_q, int c_k,
                             int c_h, unsigned flags, void* workspace, size_t workspace_bytes,
                             void* stream);

/*
 * mta_forward_rows: mta_forward for the output rows row_begin .. T-1 only, against
 * all keys 0 .. T-1. Every output row depends only on keys up to itself and on the
 * c_q-1 query rows before it, 2(c_q-1) with both KQ flags (§2 causal mask; §3.1: the
 * convolution reaches only current and past queries), so a suffix of rows can be
 * computed on its own: with a cache holding k and v (and q) of the earlier positions
 * this is the decode step (row_begin = T-1) or a prefill chunk. The rows written are
 * identical to the same rows of mta_forward.
 *   q            [B,T,M,d]; rows max(0, row_begin-(c_q-1)) .. T-1 are read with one
 *                KQ flag, max(0, row_begin-2(c_q-1)) .. T-1 with both, rows
 *                row_begin .. T-1 without; earlier rows are not read
 *   k, v         [B,T,M,d]; all rows are read
 *   out          [B,T,M,d]; rows row_begin .. T-1 are written, earlier rows are left
 *                as they were
 *   row_begin    0 <= row_begin < T, else MTA_ERR_INVALID_ARG
 * Other arguments and errors as for mta_forward. Allocates nothing.
 */
int mta_forward_rows(const void* q, const void* k, const void* v, const float* theta_kq,
                     const float* w_mix, const float* gn_gamma, const float* gn_beta, float lambda,
                     void* out, int B, int T, int M, int d, int c_q, int c_k, int c_h, int row_begin,
                     unsigned flags, void* stream);

/*
 * mta_forward_rows_split: mta_forward_rows with the key range of every row tile split over
 * several workgroups, for short row ranges (a decode step, a small prefill chunk) where the
 * row tiles alone would leave most of the GPU idle. Each workgroup covers one chunk of keys;
 * the partial softmax statistics and AV sums of the chunks are combined exactly (statistics
 * and sums over keys add up, §2), then GroupNorm and the gate are applied. With convolution
 * or mixing after softmax a statistics pass and a weighted pass run per chunk. Results equal
 * mta_forward_rows up to summation order (not bit for bit). When splitting does not pay (many
 * row tiles, or fp32 tensors) it runs mta_forward_rows and needs no workspace.
 *   workspace        device buffer of at least mta_forward_rows_split_workspace_bytes()
 *                    (may be NULL when that is 0); 16-byte aligned
 * Other arguments, reads and writes as for mta_forward_rows; errors as for
 * mta_forward_materialized. Allocates nothing.
 */
int mta_forward_rows_split(const void* q, const void* k, const void* v, const float* theta_kq,
                           const float* w_mix, const float* gn_gamma, const float* gn_beta,
                           float lambda, void* out, int B, int T, int M, int d, int c_q, int c_k,
                           int c_h, int row_begin, unsigned flags, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * mta_forward_rows_split_noalloc: mta_forward_rows_split for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). The partial results live in a scratch array inside the library instead of a
 * caller workspace: MTA_NOALLOC_SCRATCH_BYTES per device, held until the process ends. A row
 * range whose mta_forward_rows_split_workspace_bytes() exceeds that size returns
 * MTA_ERR_WORKSPACE (a decode step at B=2, T=4096, M=32, d=128 needs about 7 MiB). Every call
 * on a device shares that device's scratch, so calls that overlap on one GPU (other streams,
 * other threads) race; calls queued on one stream are ordered. The first call on a device
 * looks up the scratch address with that device current (the caller's current device must be
 * the one its stream and tensors belong to). Arguments, results and other errors as for
 * mta_forward_rows_split; allocates nothing and copies nothing.
 */
#define MTA_NOALLOC_SCRATCH_BYTES (32u << 20)
int mta_forward_rows_split_noalloc(const void* q, const void* k, const void* v,
                                   const float* theta_kq, const float* w_mix,
                                   const float* gn_gamma, const float* gn_beta, float lambda,
                                   void* out, int B, int T, int M, int d, int c_q, int c_k,
                                   int c_h, int row_begin, unsigned flags, void* stream);

/* Workspace needed by mta_forward_rows_split (0: no splitting for this shape, or invalid
 * sizes): partial statistics and AV sums of up to 64 key chunks for rows row_begin-16 .. T-1. */
size_t mta_forward_rows_split_workspace_bytes(int B, int T, int M, int d, int c_q, int c_k,
                                              int c_h, int row_begin, unsigned flags);

/* The key split mta_forward_rows_split uses on a device with compute_units compute units
 * (0: the current device, 256 when none can be queried): *n_chunks chunks of *chunk_keys keys
 * (*n_chunks = 1 and *chunk_keys = T: no split). Host-only; returns MTA_OK or
 * MTA_ERR_INVALID_ARG (invalid sizes, NULL outputs). */
int mta_forward_rows_split_plan(int B, int T, int M, int d, int c_q, int c_k, int c_h,
                                int row_begin, unsigned flags, int compute_units,
                                int* n_chunks, int* chunk_keys);

/* Workspace needed by mta_forward_materialized: two fp32 [B, M, T, LD] maps, LD = T
 * rounded up to a multiple of 4. Returns 0 for invalid sizes. */
size_t mta_materialized_workspace_bytes(int B, int T, int M, unsigned flags);

/*
 * mta_backward_materialized: gradients of the layer (the same function as mta_forward)
 * with respect to every input, for training. The loss gradient dout = dL/d(out) comes
 * in; the forward maps are recomputed into the workspace and each step's adjoint runs
 * as its own kernel over fp32 [B, M, T, T] maps (unfused, like
 * mta_forward_materialized), in the reverse order of §2-§3.3.
 *   q .. lambda      the forward arguments (same meaning and layout as mta_forward)
 *   dout             [B,T,M,d], input dtype: gradient of the output
 *   dq, dk, dv       [B,T,M,d], input dtype: written (not accumulated); distinct, and
 *                    none may alias q, k, v or dout
 *   dtheta_kq        shape of theta_kq (fp32), required iff a KQ flag is set
 *   dw_mix           shape of w_mix (fp32), required iff a MIX flag is set
 *   dgn_gamma, dgn_beta  [M*d] fp32, and dlambda (one fp32 value, the gradient of the
 *                    gate value lambda), required iff MTA_GN; all written
 *   workspace        device buffer of at least mta_backward_workspace_bytes()
 * Parameter gradients are reduced in a fixed order: repeated calls give identical
 * results. Errors as for mta_forward_materialized. Allocates nothing.
 */
int mta_backward_materialized(const void* q, const void* k, const void* v, const float* theta_kq,
                              const float* w_mix, const float* gn_gamma, const float* gn_beta,
                              float lambda, const void* dout, void* dq, void* dk, void* dv,
                              float* dtheta_kq, float* dw_mix, float* dgn_gamma, float* dgn_beta,
                              float* dlambda, int B, int T, int M, int d, int c_q, int c_k, int c_h,
                              unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace needed by mta_backward_materialized: between four and seven fp32 [B, M, T, LD]
 * maps (LD = T rounded up to a multiple of 4; one more per step that the placement
 * adds), the recomputed output before GroupNorm, and partial sums. 0 for invalid sizes. */
size_t mta_backward_workspace_bytes(int B, int T, int M, int d, int c_q, int c_k, int c_h,
                                    unsigned flags);

/*
 * mta_forward_train: mta_forward (bf16 tensors; same arguments, placements and errors) that
 * also keeps what mta_backward_fused needs, for training:
 *   lse          [B, T, M] fp32, written: the natural log-sum-exp of every softmax row,
 *                lse[b][i][m] = log sum_{j <= i} exp(C[i][j]) over the logits C that enter
 *                the softmax of head m (§2; after the convolution and mixing before softmax
 *                of §3.1-§3.2 where the placement has them). Required, 16-byte aligned.
 *   out_pre_gn   [B, T, M, d] fp32, written, or NULL: the layer output before the GroupNorm
 *                and gate of §3.3 (needed by mta_backward_fused with MTA_GN). 16-byte aligned.
 * MTA_FP32 returns MTA_ERR_UNSUPPORTED. Allocates nothing.
 */
int mta_forward_train(const void* q, const void* k, const void* v, const float* theta_kq,
                      const float* w_mix, const float* gn_gamma, const float* gn_beta, float lambda,
                      void* out, float* lse, float* out_pre_gn, int B, int T, int M, int d, int c_q,
                      int c_k, int c_h, unsigned flags, void* stream);

/*
 * mta_backward_fused: the gradients of mta_backward_materialized (same outputs, layouts and
 * parameter-gradient order) without any T x T map in memory: every map of §2-§3.2 is
 * recomputed on 16 x 16 tiles in on-chip memory, with the softmax rebuilt from the lse of
 * mta_forward_train. bf16 tensors only.
 *   lse, out_pre_gn  from mta_forward_train on the same inputs (out_pre_gn required with MTA_GN,
 *                    ignored otherwise)
 *   workspace        device buffer of at least mta_backward_fused_workspace_bytes(), 16-byte
 *                    aligned: O(B*T*M*d) bytes (an fp32 dq accumulator, dO, per-row sums and
 *                    per-tile partial sums of the parameter gradients)
 * dq is accumulated with floating-point atomics, so its last bits may differ between calls;
 * dk, dv and the parameter gradients are reduced in a fixed order. Errors as for
 * mta_backward_materialized; MTA_ERR_UNSUPPORTED for MTA_FP32 and for placements whose tiles
 * would not fit in the 160 KiB of LDS (where the resident K/V rows do not fit they are read from
 * global memory instead; with that, every shape of the supported range fits). Allocates nothing.
 */
int mta_backward_fused(const void* q, const void* k, const void* v, const float* theta_kq,
                       const float* w_mix, const float* gn_gamma, const float* gn_beta, float lambda,
                       const float* lse, const float* out_pre_gn, const void* dout, void* dq, void* dk,
                       void* dv, float* dtheta_kq, float* dw_mix, float* dgn_gamma, float* dgn_beta,
                       float* dlambda, int B, int T, int M, int d, int c_q, int c_k, int c_h,
                       unsigned flags, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace needed by mta_backward_fused; 0 for invalid sizes. */
size_t mta_backward_fused_workspace_bytes(int B, int T, int M, int d, int c_q, int c_k, int c_h,
                                          unsigned flags);

/*
 * mta_attention_plain: standard causal softmax attention softmax(QK^T/sqrt(d))V
 * (§2), computed by the same fused kernel with the convolution, mixing and
 * GroupNorm switched off. flags: 0 or MTA_FP32. Allocates nothing.
 */
int mta_attention_plain(const void* q, const void* k, const void* v, void* out, int B, int T,
                        int M, int d, unsigned flags, void* stream);

/*
 * mta_check_args: the validation mta_forward performs, without touching the GPU.
 * Pointer arguments are checked for NULL/alignment only. Returns an mta_status.
 */
int mta_check_args(const void* q, const void* k, const void* v, const float* theta_kq,
                   const float* w_mix, const float* gn_gamma, const float* gn_beta, const void* out,
                   int B, int T, int M, int d, int c_q, int c_k, int c_h, unsigned flags);

/* Static description of a status code. */
const char* mta_status_string(int status);

/* Detail message of the last failing call on this thread ("" if none). */
const char* mta_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int mta_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MTA_H */
