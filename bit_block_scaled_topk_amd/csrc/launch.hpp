// launch.hpp -- internal launch functions of the HIP kernels (not part of the
// C ABI).  Each returns the launch's hipError_t; callers have already checked
// every argument against the limits of include/moe_nvfp4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_nvfp4.h"

namespace moe {

hipError_t launch_route_topk(const float *logits, int n_tokens, int n_experts, int top_k,
                             int32_t *ids, float *weights, hipStream_t stream);

// Router GEMM (x . W_r^T, bf16 weights) fused with top-K and the softmax over
// the picks.  counters: router_counter_bytes(n_tokens) bytes, zero before the
// first call (launch_router_init) and left zero by every call; logits: [n][E]
// fp32, written.
size_t router_counter_bytes(int n_tokens);
hipError_t launch_router_init(int32_t *counters, int n_tokens, hipStream_t stream);
hipError_t launch_router_topk(const void *x, bool x_f32, int n_tokens, int d_model, const uint16_t *router_w,
                              int n_experts, int top_k, float *logits, int32_t *counters, int32_t *ids,
                              float *weights, hipStream_t stream);

// Gather: bitmap layout + row copy (one workgroup for small problems).
size_t gather_workspace_bytes(int n_tokens, int n_experts);
bool gather_is_single_launch(int n_tokens, int top_k, int n_experts, int elem_bytes, int d_model);
// Routing of every token and the whole gather in one workgroup (requires
// gather_is_single_launch).
hipError_t launch_route_gather_small(const float *logits, int n_tokens, int n_experts, int top_k, int32_t *ids,
                                     float *weights, const void *x, int elem_bytes, int d_model, void *xg,
                                     int32_t *offsets, int32_t *row_token, int32_t *rows, hipStream_t stream);
// err (optional): MOE_DEVERR_EXPERT_ID is OR-ed into it for an id outside
// [0, n_experts); that pick is dropped (row -1, not counted).
hipError_t launch_gather(const void *x, int elem_bytes, int n_tokens, int d_model,
                         const int32_t *ids, int top_k, int n_experts, void *xg,
                         int32_t *offsets, int32_t *row_token, int32_t *rows, void *workspace,
                         int32_t *err, hipStream_t stream);

// error_word (optional): MOE_DEVERR_ROW is OR-ed into it for a row outside
// [0, n_src_rows); that entry contributes nothing.
hipError_t launch_weighted_row_sum(float *dst, const float *src, int n_src_rows,
                                   const int32_t *rows, const float *weights, int n_tokens,
                                   int top_k, int d_model, bool accumulate, int32_t *error_word,
                                   hipStream_t stream);

// A device error word: cleared by a one-thread kernel (no memset, so the call
// may sit in a captured graph).
hipError_t launch_error_word_clear(int32_t *word, hipStream_t stream);

hipError_t launch_unpack_bf16(const uint8_t *codes, const uint8_t *scales, long rows, int cols,
                              uint16_t *out, hipStream_t stream);

// Epilogues of the projection kernels.
enum Epilogue : int {
  EPI_F32 = 0,     // out f32 [rows][ldo] = global * acc
  EPI_RELU2 = 1,   // h = relu(global * acc)^2
  EPI_SWIGLU = 2,  // h = silu(global * acc_gate) * (global * acc_up)
};

// fp32 activations -> three bf16 planes hi, mid, lo (plane stride `plane`).
hipError_t launch_split3(const float *a, long n_elems, uint16_t *planes, long plane, hipStream_t stream);

// One grouped NVFP4 projection handled by the decode or prefill kernels.
struct ProjProblem {
  const uint16_t *a;      // bf16 activations: nt planes of [rows][lda] (plane stride `plane`)
  const int32_t *row_map; // optional: packed row r reads activation row row_map[r] (gather on load)
  long plane;
  long lda;
  long a_rows;            // rows of a (row_map values index them); loads stay inside a_rows * lda
  const int32_t *offsets; // [n_experts + 1] device (unused when known_rows >= 0)
  int n_experts;
  int n_rows;             // rows of a / out
  int known_rows;         // >= 0: one expert, rows [0, known_rows) known on the host
  int min_rows, max_rows; // experts with min_rows..max_rows rows are handled
  const uint8_t *codes;   // [n_experts][n_w][k/2]
  const uint8_t *scales;  // [n_experts][n_w][k/16]
  const uint8_t *scales_packed;  // optional: the same scales as nvfp4_pack_scales orders them
  const uint8_t *codes_packed;   // optional: the same codes as nvfp4_pack_codes orders them
  const float *global;    // [n_experts]
  int n_w, k, n_out;
  float *out_f32;         // EPI_F32 output [n_rows][ldo]
  uint16_t *out_h;        // activation epilogues: bf16 h (3 planes on the decode path)
  long ldo;
  long h_plane;
  // filled by the launchers
  int n_tiles;            // output-column tiles
  int blocks;             // workgroups of this problem
  uint32_t a_bytes;       // prefill launcher: bytes of plane 0 of a
};

// Decode path: up to two problems in one launch (e.g. the shared and the routed
// experts).  Both use the same epilogue and activation planes nt; max_active
// bounds the experts with 1..max_rows rows of each problem.
hipError_t launch_dq_gemv(ProjProblem *probs, const int *max_active, int count, int nt, int epi,
                          hipStream_t stream);

// Prefill path: up to two problems in one launch; bf16 activations (plane 0).
// The one-time scale repack: dst[e][b][c][r][i] = scales[e][16 b + r][8 c + i].
long packed_scales_bytes(long n_experts, int rows, int cols);
hipError_t launch_pack_scales(const uint8_t *scales, int n_experts, int rows, int cols, uint8_t *dst,
                              hipStream_t stream);
// The one-time code repack: dst[e][b][c][r][i] = codes[e][16 b + r][64 c + i].
long packed_codes_bytes(long n_experts, int rows, int cols);
hipError_t launch_pack_codes(const uint8_t *codes, int n_experts, int rows, int cols, uint8_t *dst,
                             hipStream_t stream);
// WeightedRowSum fused into the prefill down projection (a launch carrying the
// shared expert's problem and the routed one, EPI_F32): every tile stores its
// rows with device-coherent stores, counts each row's (token, 256-column tile)
// once the stores have completed, and the workgroup that brings a token's
// count to its number of producers -- the shared expert plus the token's picks
// whose experts take this launch (more than gmax rows) -- computes
//   out[t][c] = out[t][c] + sum_j w[t][j] * yg[rows[t][j]][c]
// for the tile's columns, j in order from a zero accumulator by fmaf: the
// bits of moe_weighted_row_sum.  counters[(t * n_ct + tile) * 16] must be zero
// when the launch starts (the up launch zeroes them: zero_counters below).
struct CombineArgs {
  int on;
  int32_t *counters;
  const int32_t *ids, *rows, *row_token, *offsets;
  const float *w;
  const float *yg;  // [n*K][d], written by this launch and earlier ones
  float *out;       // [n][d]: the shared expert's output, then the layer's
  int n, K, d, gmax, n_ct;
};
// Columns of one tile of the f32-output GEMM (the combine's column tiles).
constexpr int kGemmF32TileCols = 256;
// zero_counters: words counters[16 i], i < n_zero, are zeroed by the launch
// (grid-stride, before its tiles): the up launch prepares the down launch's
// combine counters.
hipError_t launch_dq_gemm(ProjProblem *probs, int count, int epi, hipStream_t stream,
                          const CombineArgs *combine = nullptr, int32_t *zero_counters = nullptr,
                          long n_zero = 0);

// A whole decode step (n_tokens <= 2) in one persistent launch: routing, the
// gather layout, the shared expert (up[0]/down[0], ignored unless has_shared)
// and the routed experts (up[1]/down[1]; only their weights and shapes are
// read; the repacked copies are required), and the combine.  part is
// decode_layer_part_bytes() of scratch (each work unit's share of the down
// projection, tagged with the launch's epoch), zeroed with the sync words by
// decode_layer_init; out gets (shared ? shared : 0) + sum_j w[t][j] *
// yg[rows[t][j]], and yg the routed experts' outputs.  The routing and layout
// views (ids, topk_w, offsets, row_token, rows) are written as by the separate
// routing and gather launches.  sync points to decode_layer_sync_words()
// int32 words; every launch leaves them and part ready for the next (sync[0]:
// set once a bounded wait expires; sync[1]: launches so far).  Returns hipErrorNotSupported for shapes it does not take
// (the caller then uses the per-step launches).
struct DecodeLayerProblem {
  ProjProblem up[2], down[2];
  bool has_shared;
  int max_slots;       // routed experts that can be active: min(E, n * K)
  int act;             // EPI_RELU2 or EPI_SWIGLU (routed up projection)
  const void *x;       // [n][d] activations
  bool x_f32;          // else bf16
  const float *logits; // [n][n_experts]
  void *part;
  float *out, *yg;
  int32_t *ids, *rows, *offsets, *row_token;
  float *topk_w;
  int n_tokens, n_experts, top_k, d, f, fs, n_rows;
  int32_t *sync;
};
size_t decode_layer_sync_words();
bool decode_layer_takes(int n_tokens, int top_k, int d_model);
// Bytes of DecodeLayerProblem::part (0 when the step is never taken).
size_t decode_layer_part_bytes(int n_tokens, int n_experts, int top_k, int d_model, int d_ff, int shared_d_ff);
// Zeroes the sync words and the partial sums (part may be NULL).
hipError_t decode_layer_init(int32_t *sync, void *part, size_t part_bytes, hipStream_t stream);
hipError_t launch_decode_layer(const DecodeLayerProblem &lp, hipStream_t stream);

}  // namespace moe
