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

// Gather: bitmap layout (one workgroup) + row copy.
size_t gather_workspace_bytes(int n_tokens, int n_experts);
hipError_t launch_gather(const void *x, int elem_bytes, int n_tokens, int d_model,
                         const int32_t *ids, int top_k, int n_experts, void *xg,
                         int32_t *offsets, int32_t *row_token, int32_t *rows, void *workspace,
                         hipStream_t stream);

hipError_t launch_weighted_row_sum(float *dst, const float *src, int n_src_rows,
                                   const int32_t *rows, const float *weights, int n_tokens,
                                   int top_k, int d_model, bool accumulate, hipStream_t stream);

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

// Decode path over experts with 1..max_rows rows (at most max_active of them):
// activations are nt bf16 planes; EPI_F32 writes out_f32, the activation
// epilogues write h as three bf16 planes (hi, mid, lo) with plane stride h_plane.
hipError_t launch_dq_gemv_planes(const uint16_t *a, int nt, long plane, long lda, const int32_t *offsets,
                                 int n_experts, int n_rows, int max_rows, int max_active, const uint8_t *codes,
                                 const uint8_t *scales, const float *global, int n_w, int k, int n_out,
                                 int epi, float *out_f32, uint16_t *out_h, long ldo, long h_plane,
                                 hipStream_t stream);

// Prefill path over experts with at least min_rows rows: bf16 activations;
// EPI_F32 writes out_f32, the activation epilogues write bf16 h.
hipError_t launch_dq_gemm(const uint16_t *a, long lda, const int32_t *offsets, int n_experts,
                          int min_rows, long n_rows, const uint8_t *codes, const uint8_t *scales,
                          const float *global, int n_w, int k, int n_out, int epi, float *out_f32,
                          uint16_t *out_h, long ldo, hipStream_t stream);

}  // namespace moe
