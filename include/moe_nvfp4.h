/*
 * moe_nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 MoE expert-FFN library.
 *
 * One quantised mixture-of-experts layer, as profiled and rebuilt in the gllm
 * pull request "perf: gather tokens per MoE expert, run large NVFP4 GEMMs on bf16
 * tensor cores #91" (sections "What changes" and "bf16 NVFP4 GEMM (CUDA)"):
 *
 *   moe_route_topk        topK routing, softmax over the picked logits
 *   moe_gather_rows       each (token, picked expert) pair -> one row of packed
 *                         n*topK-row buffers grouped by expert, plus the row copy
 *   nvfp4_expert_ffn      each expert's up -> relu^2 (or SwiGLU) -> down over its
 *                         own contiguous rows only (NVFP4 weights)
 *   moe_weighted_row_sum  dst[i] += sum_j w[i,j] * src[rows[i,j]], fixed j order
 *
 * plus two single-step entry points used on their own and by the tests:
 *   nvfp4_unpack_bf16     exact NVFP4 -> bf16 unpack that drops the global
 *   nvfp4_grouped_linear  one grouped NVFP4 projection, y = global * a . W^T
 *
 * Conventions for every entry point
 *   - Pointers named as device pointers are HIP device memory owned by the
 *     caller; the library never allocates, frees or synchronises, and never
 *     reads device memory on the host.  All work is enqueued on `stream`.
 *   - Arguments are checked on the host before anything is launched.  On
 *     MOE_INVALID_ARG, MOE_UNSUPPORTED and MOE_WORKSPACE_TOO_SMALL nothing was
 *     enqueued and no output was touched; MOE_HIP_ERROR (a failed launch) may
 *     leave earlier kernels of the same call enqueued.
 *   - Entry points are stateless and may be called from several host threads.
 *   - Results are deterministic: the same inputs give the same output bits,
 *     whatever else runs on the GPU (no floating-point atomics anywhere).
 *   - Index errors found on the device are reported, never trapped on: a
 *     kernel that meets an index outside its range skips that entry and ORs a
 *     MOE_DEVERR_* bit into a device error word (the first int32 of the
 *     workspace of moe_gather_rows and nvfp4_expert_ffn, whose first 256 bytes
 *     are reserved for it; an argument of moe_weighted_row_sum).  The word is
 *     sticky: kernels only set bits; moe_error_word_clear resets it and
 *     moe_error_word_read (a test and debugging helper) copies it to the host.
 *
 * NVFP4 tensor layout (one projection of n_experts experts):
 *   codes   uint8 [n_experts][rows][cols/2]: e2m1 codes (OCP MX E2M1: sign bit 3,
 *           magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6), element 2i of a row in the
 *           low nibble of byte i, element 2i+1 in the high nibble;
 *   scales  uint8 [n_experts][rows][cols/16]: one OCP E4M3FN scale per 16
 *           consecutive elements of a row (bias 7, max 448, 0x7F/0xFF = NaN);
 *   global  float [n_experts]: the per-tensor fp32 global of each expert;
 *   value(r, k) = global * e4m3(scale[r][k/16]) * e2m1(code(r, k)).
 *   rows = out_features, cols = in_features; cols must be a multiple of 32.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int moe_status;
#define MOE_OK 0
#define MOE_INVALID_ARG 1          /* a null pointer, a negative or inconsistent size */
#define MOE_UNSUPPORTED 2          /* a size or mode outside the limits stated below */
#define MOE_HIP_ERROR 3            /* a kernel launch failed (hipGetLastError) */
#define MOE_WORKSPACE_TOO_SMALL 4  /* ws_bytes below the size query's answer */

/* Bits of a device error word. */
#define MOE_DEVERR_EXPERT_ID 1  /* moe_gather_rows: a topk_id outside [0, n_experts) */
#define MOE_DEVERR_ROW 2        /* moe_weighted_row_sum: a rows entry outside [0, n_src_rows) */

typedef int moe_dtype;
#define MOE_F32 0   /* IEEE binary32 */
#define MOE_BF16 1  /* bfloat16, stored as uint16 bit patterns */

typedef int moe_act;
#define MOE_RELU2 0   /* h = max(u, 0)^2 */
#define MOE_SWIGLU 1  /* up rows [0, f) = gate a, rows [f, 2f) = b; h = a/(1+e^-a) * b */

/* Limits checked by every entry point. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOPK 32
#define MOE_MAX_GEMV_ROWS 32

/* One NVFP4 projection for n_experts experts; all pointers are device
 * pointers laid out as described in the file header.  codes and scales (the
 * canonical layout) may both be NULL when the repacked copies below are given
 * and rows is a multiple of 16 (32 for a SwiGLU up projection): every kernel
 * then reads the repacked copies.  So a caller keeps one copy of the
 * weights. */
typedef struct {
  const uint8_t *codes;
  const uint8_t *scales;
  const float *global;
  int rows; /* out_features */
  int cols; /* in_features, a multiple of 32 */
  /* Optional: the same scales and codes reordered by nvfp4_pack_scales and
   * nvfp4_pack_codes -- both present or both NULL, 16-byte aligned, holding
   * the same weights as `codes` / `scales`.  When both are present the decode
   * GEMV reads them, and so does the prefill GEMM when rows is a multiple of
   * 16 (SwiGLU: f too); the single-launch decode step reads only them (it
   * falls back to the per-step launches without them), and the standalone
   * unpack reads the canonical layout.  With them, one expert's repacked
   * codes (ceil(rows/16) * ceil(cols/128) KB) must stay under 2 GiB. */
  const uint8_t *scales_packed;
  const uint8_t *codes_packed;
} moe_nvfp4_weights;

/* nvfp4_packed_scales_bytes -- bytes of the reordered scales of n_experts
 * experts of rows x cols: n_experts * ceil(rows/16) * ceil(cols/128) * 128
 * (0 for non-positive sizes). */
size_t nvfp4_packed_scales_bytes(int n_experts, int rows, int cols);

/* nvfp4_pack_scales -- the optional one-time repack of a projection's e4m3
 * block scales into the order the GEMM, GEMV and single-launch decode kernels
 * read them in (the boundary's "prepack": same bytes, another order, no
 * global):
 *   dst[e][b][c][h][r][i] = scales[e][16 b + r][8 c + 4 h + i]
 * for 16-row block b, 128-column chunk c, 64-column half h < 2, row r < 16 and
 * i < 4; entries past rows or past cols/16 are zero.  In that order one 16-row
 * block's scales of one 128-wide k chunk are 128 contiguous bytes, one cache
 * line, where the canonical layout spreads them over 16 (the GEMM's scale
 * loads were a third of its requests to L2), and those of one 64-wide half
 * are 64 contiguous bytes.
 *   w       the projection (w->codes and w->global are not read)
 *   dst     device, dst_bytes >= nvfp4_packed_scales_bytes(n_experts, rows, cols)
 * Errors: MOE_INVALID_ARG for null pointers, n_experts < 1, rows < 1, cols not a
 * positive multiple of 32, or dst_bytes too small; nothing is launched then.
 * Stream-ordered on `stream`; allocates nothing. */
moe_status nvfp4_pack_scales(const moe_nvfp4_weights *w, int n_experts, uint8_t *dst, size_t dst_bytes,
                             hipStream_t stream);

/* nvfp4_packed_codes_bytes -- bytes of the reordered codes of n_experts
 * experts of rows x cols: n_experts * ceil(rows/16) * ceil(cols/128) * 1024
 * (0 for non-positive sizes). */
size_t nvfp4_packed_codes_bytes(int n_experts, int rows, int cols);

/* nvfp4_pack_codes -- the optional one-time repack of a projection's e2m1
 * codes into the order the GEMM, GEMV and single-launch decode kernels read
 * them in (same bytes, another order):
 *   dst[e][b][c][h][r][i] = codes[e][16 b + r][64 c + 32 h + i]
 * for 16-row block b, 128-column chunk c, 64-column half h < 2, row r < 16 and
 * i < 32; entries past rows or past cols/2 are zero.  One 16-row block's codes
 * of one 128-wide k chunk are then 1 KB contiguous, which one 16-byte-per-lane
 * load reads as 8 whole cache lines (16 half lines in the canonical layout),
 * and those of one 64-wide half are 512 contiguous bytes.
 *   w       the projection (w->scales and w->global are not read)
 *   dst     device, dst_bytes >= nvfp4_packed_codes_bytes(n_experts, rows, cols)
 * Errors as nvfp4_pack_scales.  Stream-ordered on `stream`; allocates nothing. */
moe_status nvfp4_pack_codes(const moe_nvfp4_weights *w, int n_experts, uint8_t *dst, size_t dst_bytes,
                            hipStream_t stream);

/* moe_route_topk -- per token, the top_k experts by router logit and their
 * weights, a softmax over the top_k picked logits only.
 *   logits        device float [n_tokens][n_experts], finite or -inf (no NaN)
 *   topk_ids      device int32 [n_tokens][top_k]: slot j holds the j-th largest
 *                 logit's expert; equal logits go to the lower expert index
 *   topk_weights  device float [n_tokens][top_k]:
 *                 w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), i = 0..top_k-1
 * Limits: 1 <= n_experts <= 1024, 1 <= top_k <= min(n_experts, 32),
 * n_tokens >= 0 (0 launches nothing).
 * Source: topK routing of the MoE layer (gllm #91 "What the profile showed":
 * 128 experts, topK 6); the weights are the per-pick weights WeightedRowSum
 * consumes ("What changes"). */
moe_status moe_route_topk(const float *logits, int n_tokens, int n_experts, int top_k,
                          int32_t *topk_ids, float *topk_weights, hipStream_t stream);

/* Workspace bytes moe_router_topk needs for n_tokens tokens and n_experts
 * experts: one counter per 16 tokens and a logits buffer [n_tokens][n_experts]
 * (used when the caller does not ask for the logits); 0 for invalid
 * arguments. */
size_t moe_router_workspace_size(int n_tokens, int n_experts);

/* moe_router_workspace_init -- prepare a router workspace once, after it is
 * allocated and before its first moe_router_topk: zeroes the counters of up
 * to n_tokens tokens (a kernel on `stream`; nothing is allocated).  Every
 * moe_router_topk call leaves them at zero again.  MOE_INVALID_ARG for a null
 * or unaligned (256-byte) workspace, MOE_WORKSPACE_TOO_SMALL if ws_bytes <
 * moe_router_workspace_size(n_tokens, 1). */
moe_status moe_router_workspace_init(void *workspace, size_t ws_bytes, int n_tokens, hipStream_t stream);

/* moe_router_topk -- the router step before routing, fused with it: the
 * logits x . W_r^T of every token on the matrix cores (bf16 operands, exact
 * products, fp32 accumulation in a fixed order), then per token the top_k
 * experts and their weights exactly as moe_route_topk computes them from
 * those logits.  (The gllm #91 page links a pull request, "perf: cut host
 * overhead from long prefills (routing, matmul scratch)", about this step.)
 *   x         device [n_tokens][d_model] of x_dtype (BF16, or F32 taken as
 *             three bf16 terms hi + mid + lo: 24 significant bits), 16-byte
 *             aligned
 *   router_w  device bf16 bits [n_experts][d_model], 16-byte aligned
 *   topk_ids, topk_weights  device [n_tokens][top_k], as moe_route_topk's
 *   logits    device float [n_tokens][n_experts] (out), or NULL: then they
 *             live in the workspace only
 *   workspace device, >= moe_router_workspace_size(n_tokens, n_experts),
 *             256-byte aligned, prepared by moe_router_workspace_init; calls
 *             that overlap on one workspace race
 * The logits of a token differ from the exact x . W_r^T by at most about
 * (d_model + 8) * 2^-24 * sum_k |x_k W_r[e][k]|, so two experts whose exact
 * logits are closer than twice that may be ranked either way; the ids and
 * weights are always those of the logits written.
 * Limits: d_model a positive multiple of 32, 1 <= n_experts <= 1024,
 * 1 <= top_k <= min(n_experts, 32); n_tokens == 0 launches nothing. */
moe_status moe_router_topk(const void *x, moe_dtype x_dtype, int n_tokens, int d_model, const uint16_t *router_w,
                           int n_experts, int top_k, int32_t *topk_ids, float *topk_weights, float *logits,
                           void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes moe_gather_rows needs for n_tokens tokens and n_experts
 * experts, the 256 reserved bytes of the error word included (0 for invalid
 * arguments). */
size_t moe_gather_workspace_size(int n_tokens, int n_experts);

/* moe_gather_rows -- the MoE gather (gllm #91 "What changes"): n x topK rows,
 * one per (token, picked expert) pair, each expert's rows contiguous, filled by
 * a single row lookup of the inputs.
 *   x               device [n_tokens][d_model] of x_dtype (F32 or BF16)
 *   topk_ids        device int32 [n_tokens][top_k], expert ids (each token
 *                   should pick an expert at most once)
 *   xg              device [n_tokens*top_k][d_model] of x_dtype (out):
 *                   xg[r] = x[row_token[r]], a bit copy; must not alias x
 *   expert_offsets  device int32 [n_experts+1] (out): exclusive scan of the
 *                   per-expert pick counts; rows of expert e are
 *                   [expert_offsets[e], expert_offsets[e+1])
 *   row_token       device int32 [n_tokens*top_k] (out): token of each row
 *   rows            device int32 [n_tokens][top_k] (out): row of pick (t, j)
 *   workspace       device scratch of ws_bytes >= moe_gather_workspace_size();
 *                   its first int32 is the error word (clear it once with
 *                   moe_error_word_clear before reading it)
 * Rows inside an expert's group are in ascending token order, so the layout is
 * unique.  A pick whose id is outside [0, n_experts) is dropped -- its
 * rows[t][j] is -1, it is not counted, and the unused tail rows (from
 * expert_offsets[n_experts] on) get row_token -1 and are not written in xg --
 * and MOE_DEVERR_EXPERT_ID is set in the workspace's error word (the
 * oracle of the tests rejects such ids: gllm #91 "Testing" checks bounds).
 * Limits: n_tokens*top_k < 2^31, d_model a multiple of 16, x and xg 16-byte
 * aligned. */
moe_status moe_gather_rows(const void *x, moe_dtype x_dtype, int n_tokens, int d_model,
                           const int32_t *topk_ids, int top_k, int n_experts, void *xg,
                           int32_t *expert_offsets, int32_t *row_token, int32_t *rows,
                           void *workspace, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes nvfp4_expert_ffn needs for n_rows packed rows of d_model
 * activations of act_dtype and an intermediate h of width d_ff (up->rows is
 * d_ff, or 2*d_ff for SwiGLU); 0 for invalid arguments.  After the 256 bytes
 * reserved for the error word it holds h as three bf16 planes (hi + mid + lo)
 * and, for fp32 activations, the activations split the same way. */
size_t nvfp4_expert_ffn_workspace_size(int n_rows, int d_model, int d_ff, moe_dtype act_dtype);

/* Workspace bytes nvfp4_grouped_linear needs (fp32 activations only; 0 for bf16). */
size_t nvfp4_grouped_linear_workspace_size(int n_rows, int k, moe_dtype a_dtype);

/* nvfp4_expert_ffn -- each expert's FFN over the rows routed to it (gllm #91
 * "What changes": up -> relu^2 -> down per expert; Glq v0.2.13 "v3b":
 * relu^2 for non-gated NemotronH; the gated experts' fused gate-up projection
 * of TensorFold issue #2265 "What ncu shows").
 *   xg              device [n_rows][up->cols] activations of act_dtype
 *   expert_offsets  device int32 [n_experts+1], non-decreasing, [0] = 0,
 *                   [n_experts] <= n_rows; rows past it are left untouched
 *   max_rows_per_expert  a host-side bound on every expert's row count (for
 *                   routed experts n_tokens, since a token picks an expert once)
 *   up, down        host structs of device pointers: up is [n_experts][f or 2f][d],
 *                   down is [n_experts][d][f]; up->cols == down->rows == d,
 *                   down->cols == f
 *   gemv_max_rows   experts with at most this many rows (1..32, normally 32)
 *                   take the decode path (fused dequant + matrix-core GEMV,
 *                   activations and h carried at fp32 accuracy); experts with
 *                   more rows take the prefill path (exact NVFP4 -> bf16 unpack
 *                   into a bf16 MFMA GEMM, global as alpha, activation rounded
 *                   to bf16 as gllm #91 "bf16 NVFP4 GEMM (CUDA)" does).  0 sends
 *                   every expert to the prefill path.  When max_rows_per_expert
 *                   <= gemv_max_rows the prefill kernels are not launched.
 *   out             device float [n_rows][down->rows]
 *   workspace       device scratch >= nvfp4_expert_ffn_workspace_size()
 * Alignment: xg, codes and the workspace 16-byte aligned, scales 2-byte.
 * Limits: when the prefill path can run (max_rows_per_expert > gemv_max_rows),
 * each activation matrix it reads as bf16 (n_rows x d, and h: n_rows x f) and
 * one expert's codes of each projection must stay under 2 GiB (it addresses
 * them with 32-bit offsets); otherwise MOE_UNSUPPORTED and nothing runs.
 * The shared expert is this call with n_experts = 1 and offsets {0, n}. */
moe_status nvfp4_expert_ffn(const void *xg, moe_dtype act_dtype, int n_rows,
                            int max_rows_per_expert, const int32_t *expert_offsets,
                            int n_experts, const moe_nvfp4_weights *up,
                            const moe_nvfp4_weights *down, moe_act act, int gemv_max_rows,
                            void *workspace, size_t ws_bytes, float *out, hipStream_t stream);

/* moe_weighted_row_sum -- WeightedRowSum (gllm #91 "What changes"):
 *   dst[i][c] += sum_{j=0..top_k-1} weights[i][j] * src[rows[i][j]][c]
 * with the j-sum taken in order from 0 by fused multiply-adds into a zero
 * accumulator and then added to dst once; one thread per output element, no
 * atomics, so the result is deterministic.
 *   dst      device float [n_tokens][d_model], read and written; no alias of src
 *   src      device float [n_src_rows][d_model]
 *   rows     device int32 [n_tokens][top_k]; an entry outside [0, n_src_rows)
 *            contributes nothing (it is skipped, never read out of bounds)
 *            and sets MOE_DEVERR_ROW in *error_word
 *   weights  device float [n_tokens][top_k]
 *   error_word  device int32, or NULL (not reported); the call has no
 *            workspace, so the caller passes the word (sticky, see above) */
moe_status moe_weighted_row_sum(float *dst, const float *src, int n_src_rows,
                                const int32_t *rows, const float *weights, int n_tokens,
                                int top_k, int d_model, int32_t *error_word, hipStream_t stream);

/* moe_weighted_row_sum_into -- the same sum written onto a zero destination,
 *   dst[i][c] = sum_{j=0..top_k-1} weights[i][j] * src[rows[i][j]][c]
 * (same order and rounding as moe_weighted_row_sum with dst = 0), for layers
 * without a shared expert. */
moe_status moe_weighted_row_sum_into(float *dst, const float *src, int n_src_rows,
                                     const int32_t *rows, const float *weights, int n_tokens,
                                     int top_k, int d_model, int32_t *error_word, hipStream_t stream);

/* moe_workspace_size -- one workspace that serves every call of a layer made
 * with the four calls in order: moe_gather_rows for n_tokens tokens and
 * n_experts experts, nvfp4_expert_ffn over the n_tokens*top_k routed rows and
 * over the n_tokens rows of a shared expert, with any d_ff up to d_ff_max and
 * either activation dtype (the largest of their sizes).  act is accepted for
 * SwiGLU's sake: h has d_ff columns for both activations, so the size does
 * not depend on it.  The calls run one after another on one stream, so they
 * may share the bytes; the first int32 (the error word) is left to the
 * gather.  0 for invalid arguments. */
size_t moe_workspace_size(int n_tokens, int top_k, int n_experts, int d_model, int d_ff_max, moe_act act);

/* moe_error_word_clear -- set a device error word to 0 (a one-thread kernel on
 * `stream`, no memset, so it may be captured in a graph). */
moe_status moe_error_word_clear(int32_t *word, hipStream_t stream);

/* moe_error_word_read -- test and debugging helper: waits for `stream`, then
 * copies the device error word to *value (host).  It is the one entry point
 * that synchronises and reads device memory on the host; the product path
 * never calls it. */
moe_status moe_error_word_read(const int32_t *word, int32_t *value, hipStream_t stream);

/* nvfp4_unpack_bf16 -- exact unpack of NVFP4 codes and scales to bf16 without
 * the per-tensor global (gllm #91 "bf16 NVFP4 GEMM (CUDA)"): a code's value
 * (2 significant bits) times its e4m3 scale (4) always fits bf16's 8.
 *   codes   device uint8 [rows][cols/2]; scales device uint8 [rows][cols/16]
 *   out     device uint16 (bf16 bits) [rows][cols] = e4m3(scale) * e2m1(code)
 * A NaN scale byte gives bf16 NaN for its 16 elements. */
moe_status nvfp4_unpack_bf16(const uint8_t *codes, const uint8_t *scales, int rows, int cols,
                             uint16_t *out, hipStream_t stream);

/* nvfp4_grouped_linear -- one NVFP4 projection per expert group:
 *   out[r][n] = global[e] * sum_k a[r][k] * e4m3 * e2m1 (W_e[n][k])  for r in expert e
 * Path choice as in nvfp4_expert_ffn (decode path: fp32-accurate; prefill path:
 * a rounded to bf16, exact bf16 weights, fp32 accumulation, global as alpha).
 * This is the single NVFP4 matmul that gllm #91 "Testing" holds to the f32
 * tolerance when fed bf16-exact activations.
 *   a    device [n_rows][w->cols] of a_dtype; out device float [n_rows][w->rows]
 *   workspace  device scratch >= nvfp4_grouped_linear_workspace_size()
 * Limits: as nvfp4_expert_ffn's for the prefill path (a as bf16 and one
 * expert's codes under 2 GiB), else MOE_UNSUPPORTED. */
moe_status nvfp4_grouped_linear(const void *a, moe_dtype a_dtype, int n_rows,
                                int max_rows_per_expert, const int32_t *expert_offsets,
                                int n_experts, const moe_nvfp4_weights *w, int gemv_max_rows,
                                void *workspace, size_t ws_bytes, float *out,
                                hipStream_t stream);

/* ------------------------------------------------------------------------- */
/* The whole layer in the fewest launches                                     */
/* ------------------------------------------------------------------------- */

/* Shapes and weights of one MoE layer.  The shared expert is optional
 * (shared_up.codes and shared_up.codes_packed both NULL: none, so the output
 * is the routed sum alone); it always uses relu^2, the routed experts use
 * `act`. */
typedef struct {
  int n_tokens;               /* n */
  int d_model;                /* d: columns of x, up.cols, down.rows */
  int n_experts;              /* routed experts E */
  int top_k;                  /* K */
  moe_dtype x_dtype;          /* activations */
  moe_act act;                /* routed experts' activation */
  int gemv_max_rows;          /* 0..32, as in nvfp4_expert_ffn */
  moe_nvfp4_weights up, down; /* routed: [E][f or 2f][d], [E][d][f] */
  moe_nvfp4_weights shared_up, shared_down; /* [1][fs][d], [1][d][fs] */
  int flags;                  /* 0, or MOE_LAYER_SINGLE_LAUNCH | MOE_LAYER_FUSED_COMBINE */
} moe_layer_desc;

/* Allows the single-launch decode step (see moe_layer_forward).  Its
 * workgroups wait on one another, so they must all be resident at once: the
 * caller promises that no other kernel -- on any stream, this library's
 * included -- runs on the device while the call's kernel does (e.g. one
 * decode loop on one stream).  Without the flag every step is made of
 * kernels that never wait on each other, which is safe under any
 * concurrency. */
#define MOE_LAYER_SINGLE_LAUNCH 1

/* Runs WeightedRowSum inside the prefill down projection instead of as its own
 * launch (gllm #91 "What changes": the combine onto the shared expert's
 * output), for prefill steps with a shared expert: every down tile stores its
 * rows device-coherently and counts them per (token, 256-column tile); the
 * tile that completes a token's count sums that token's rows in slot order,
 * with the same bits as moe_weighted_row_sum.  No workgroup waits on another,
 * so it is safe under any concurrency.  It is measured slower than the
 * separate launch on MI355X (each tile's epilogue then carries a chain of
 * device-coherent atomics and loads), so it is opt-in. */
#define MOE_LAYER_FUSED_COMBINE 2
/* A description is invalid (MOE_INVALID_ARG; workspace size 0) when, with
 * n_tokens > gemv_max_rows, an activation matrix of the prefill GEMM (x as
 * n x d; h as n*K x f; the shared h as n x fs, all bf16) or one expert's codes
 * reach 2 GiB: that GEMM addresses them with 32-bit offsets. */

/* Device pointers into a layer workspace where moe_layer_forward leaves the
 * intermediates of its last call (for inspection; computed on the host). */
typedef struct {
  int32_t *topk_ids;       /* [n][K] */
  float *topk_weights;     /* [n][K] */
  int32_t *expert_offsets; /* [E+1] */
  int32_t *row_token;      /* [n*K] */
  int32_t *rows;           /* [n][K] */
  float *yg;               /* [n*K][d]: each routed expert's output rows */
  int32_t *wait_error;     /* one word: nonzero once a bounded inter-workgroup
                              wait of the single-launch decode step (below)
                              has expired -- that call's results are invalid;
                              it stays set until moe_layer_workspace_init. */
  int32_t *decode_launch;  /* one word: calls since moe_layer_workspace_init
                              that ran the single-launch decode step. */
} moe_layer_views;
/* (moe_layer_forward does not materialise the packed activation rows: the
 * routed up projection reads x[row_token[r]] directly.) */

/* Workspace bytes moe_layer_forward needs (0 for an invalid description). */
size_t moe_layer_workspace_size(const moe_layer_desc *desc);

/* Prepare a layer workspace for moe_layer_forward: clears the launch counts
 * and the single-launch step's partial sums at its start (with a kernel on
 * `stream`; nothing is allocated).  Required once after the workspace is
 * allocated, before its first moe_layer_forward; every later call leaves them
 * ready for the next, for any token count of the same layer shape (experts,
 * top_k, d_model, d_ff, shared d_ff) whose workspace size fits ws_bytes.
 * Those partial sums are trusted by their launch-count tags, so a workspace
 * moved to a layer of another shape must be prepared again.  A workspace
 * belongs to one device.  MOE_INVALID_ARG for a bad description or an unaligned (256-byte)
 * workspace, MOE_WORKSPACE_TOO_SMALL if ws_bytes < moe_layer_workspace_size. */
moe_status moe_layer_workspace_init(const moe_layer_desc *desc, void *workspace, size_t ws_bytes,
                                    hipStream_t stream);

/* Fill `views` with the intermediates' addresses inside `workspace`. */
moe_status moe_layer_get_views(const moe_layer_desc *desc, void *workspace, moe_layer_views *views);

/* moe_layer_forward -- route -> gather -> experts -> WeightedRowSum for one
 * layer (gllm #91 "What changes"), with the same results as the four calls
 * above made in order, in fewer launches: routing and gather share one
 * workgroup for small batches, the shared and the routed experts share each
 * up and each down launch, and nothing synchronises or allocates (Glq v0.2.13
 * "Remaining gap to bf16-native": fewer launches per layer).  For a decode
 * step -- desc->flags has MOE_LAYER_SINGLE_LAUNCH, n_tokens <= min(2,
 * gemv_max_rows), d_model <= 3072 (2048 with SwiGLU), the repacked weight
 * copies given and no shared expert beside a SwiGLU FFN -- the whole layer
 * (routing, gather layout, up and down projections, combine) is ONE
 * persistent launch: each workgroup computes slices of the experts' hidden
 * width and hands its share of the down projection to the others through
 * the workspace, tagged with a launch count (waits are bounded; see
 * moe_layer_views.wait_error); its dot products run in fp32 on the vector
 * ALUs, so it agrees with the four calls to fp32 rounding rather than bit for
 * bit.  The workspace must have been prepared by
 * moe_layer_workspace_init.  Calls that overlap on one workspace race.
 *   x       device [n][d] of desc->x_dtype (16-byte aligned)
 *   logits  device float [n][E]
 *   out     device float [n][d] (written, not accumulated)
 *   workspace  device scratch >= moe_layer_workspace_size(desc), 256-byte
 *           aligned; holds every intermediate (see moe_layer_get_views) */
moe_status moe_layer_forward(const moe_layer_desc *desc, const void *x, const float *logits, float *out,
                             void *workspace, size_t ws_bytes, hipStream_t stream);

/* moe_layer_forward with timing: events[0..7] (created by the caller, timing
 * enabled) are recorded on `stream` before routing, after routing + gather,
 * after the activation split, after the decode-path up launch, after the
 * prefill up launch (the grouped GEMM; nothing runs between events 3 and 4
 * when no expert can take it), after the decode-path down launch, after the
 * prefill down launch, and after the combine, so each launch's GPU time can be
 * read with hipEventElapsedTime.  With the single-launch decode step, events
 * 1..7 are all recorded after that launch.  events == NULL records nothing. */
moe_status moe_layer_forward_profiled(const moe_layer_desc *desc, const void *x, const float *logits,
                                      float *out, void *workspace, size_t ws_bytes, hipEvent_t *events,
                                      hipStream_t stream);

/* moe_layer_forward_noalloc -- moe_layer_forward for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The layer workspace is the library's own
 * device array of MOE_NOALLOC_SCRATCH_BYTES, one per GPU, held until the
 * process ends (its address is looked up at the first call on each GPU); the
 * caller passes only x, logits and out, as for moe_layer_forward.  Nothing is
 * allocated, freed or synchronised.
 *   Limits: a description whose moe_layer_workspace_size exceeds
 *   MOE_NOALLOC_SCRATCH_BYTES (e.g. thousands of tokens at d_model 2688) is
 *   refused with MOE_UNSUPPORTED before anything runs.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (several streams or threads) race and give undefined results.  The
 *   single-launch decode step (MOE_LAYER_SINGLE_LAUNCH) clears its launch
 *   counts and partial sums with a small kernel on `stream` before each
 *   call.  The intermediates are not exposed (no views).
 * Errors as moe_layer_forward. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_layer_forward_noalloc(const moe_layer_desc *desc, const void *x, const float *logits, float *out,
                                     hipStream_t stream);

/* A short English description of a status code (a static string). */
const char *moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_NVFP4_H */
