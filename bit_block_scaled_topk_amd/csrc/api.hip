// api.hip -- the C ABI (include/moe_nvfp4.h): host-side argument checks,
// workspace carving and launch planning.  Nothing here synchronises, allocates
// or reads device memory: the path choice between the decode kernels (experts
// with <= gemv_max_rows rows) and the prefill GEMM (more rows) is made on the
// device from expert_offsets, and the host only uses bounds it already knows
// (Glq v0.2.13, "v3a": host syncs inside the MoE loop dominated the host
// budget; gllm PR #91, "Results": every op synchronising was what remained).
#include <stdint.h>

#include "launch.hpp"
#include "moe_nvfp4.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_HIP_ERROR; }

bool weights_ok(const moe_nvfp4_weights *w) {
  return w && w->codes && w->scales && w->global && w->rows > 0 && w->cols > 0 &&
         aligned(w->codes, 16) && aligned(w->scales, 2) && aligned(w->global, 4);
}

// Planes of the fp32-activation split: three bf16 planes of n_rows*k.
size_t split_bytes(long n_rows, long k) { return align_up((size_t)3 * n_rows * k * sizeof(uint16_t)); }

// h as three bf16 planes of n_rows*f.
size_t h_bytes(long n_rows, long f) { return align_up((size_t)3 * n_rows * f * sizeof(uint16_t)); }

}  // namespace

extern "C" {

const char *moe_status_string(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_INVALID_ARG: return "invalid argument";
    case MOE_UNSUPPORTED: return "unsupported size or mode";
    case MOE_HIP_ERROR: return "HIP launch error";
    case MOE_WORKSPACE_TOO_SMALL: return "workspace too small";
    default: return "unknown status";
  }
}

moe_status moe_route_topk(const float *logits, int n_tokens, int n_experts, int top_k, int32_t *topk_ids,
                          float *topk_weights, hipStream_t stream) {
  if (n_tokens < 0 || n_experts < 1 || top_k < 1) return MOE_INVALID_ARG;
  if (top_k > n_experts) return MOE_INVALID_ARG;
  if (n_experts > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOPK) return MOE_UNSUPPORTED;
  if ((long)n_tokens * n_experts >= (1L << 40)) return MOE_UNSUPPORTED;
  if (n_tokens == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_INVALID_ARG;
  return hip_status(launch_route_topk(logits, n_tokens, n_experts, top_k, topk_ids, topk_weights, stream));
}

size_t moe_gather_workspace_size(int n_tokens, int n_experts) {
  if (n_tokens < 0 || n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return 0;
  return align_up(gather_workspace_bytes(n_tokens, n_experts));
}

moe_status moe_gather_rows(const void *x, moe_dtype x_dtype, int n_tokens, int d_model, const int32_t *topk_ids,
                           int top_k, int n_experts, void *xg, int32_t *expert_offsets, int32_t *row_token,
                           int32_t *rows, void *workspace, size_t ws_bytes, hipStream_t stream) {
  if (n_tokens < 0 || d_model < 0 || top_k < 1 || n_experts < 1) return MOE_INVALID_ARG;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_INVALID_ARG;
  if (n_experts > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOPK) return MOE_UNSUPPORTED;
  if (d_model % 16 != 0) return MOE_UNSUPPORTED;
  if ((long)n_tokens * top_k >= (1L << 31)) return MOE_UNSUPPORTED;
  if (!expert_offsets || !workspace) return MOE_INVALID_ARG;
  if (n_tokens > 0 && (!x || !topk_ids || !xg || !row_token || !rows)) return MOE_INVALID_ARG;
  if (n_tokens > 0 && (!aligned(x, 16) || !aligned(xg, 16))) return MOE_INVALID_ARG;
  if (x && xg && x == xg) return MOE_INVALID_ARG;
  if (ws_bytes < moe_gather_workspace_size(n_tokens, n_experts)) return MOE_WORKSPACE_TOO_SMALL;
  int elem = (x_dtype == MOE_F32) ? 4 : 2;
  return hip_status(launch_gather(x, elem, n_tokens, d_model, topk_ids, top_k, n_experts, xg, expert_offsets,
                                  row_token, rows, workspace, stream));
}

static moe_status wrs_common(float *dst, const float *src, int n_src_rows, const int32_t *rows,
                             const float *weights, int n_tokens, int top_k, int d_model, bool accumulate,
                             hipStream_t stream) {
  if (n_src_rows < 0 || n_tokens < 0 || top_k < 1 || d_model < 0) return MOE_INVALID_ARG;
  if ((long)n_tokens * d_model >= (1L << 40)) return MOE_UNSUPPORTED;
  if (n_tokens == 0 || d_model == 0) return MOE_OK;
  if (!dst || !rows || !weights || (n_src_rows > 0 && !src)) return MOE_INVALID_ARG;
  if (src && (const void *)src == (const void *)dst) return MOE_INVALID_ARG;
  return hip_status(launch_weighted_row_sum(dst, src, n_src_rows, rows, weights, n_tokens, top_k, d_model,
                                            accumulate, stream));
}

moe_status moe_weighted_row_sum(float *dst, const float *src, int n_src_rows, const int32_t *rows,
                                const float *weights, int n_tokens, int top_k, int d_model,
                                hipStream_t stream) {
  return wrs_common(dst, src, n_src_rows, rows, weights, n_tokens, top_k, d_model, true, stream);
}

moe_status moe_weighted_row_sum_into(float *dst, const float *src, int n_src_rows, const int32_t *rows,
                                     const float *weights, int n_tokens, int top_k, int d_model,
                                     hipStream_t stream) {
  return wrs_common(dst, src, n_src_rows, rows, weights, n_tokens, top_k, d_model, false, stream);
}

moe_status nvfp4_unpack_bf16(const uint8_t *codes, const uint8_t *scales, int rows, int cols, uint16_t *out,
                             hipStream_t stream) {
  if (rows < 0 || cols < 0) return MOE_INVALID_ARG;
  if (cols % 32 != 0) return MOE_UNSUPPORTED;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!codes || !scales || !out) return MOE_INVALID_ARG;
  if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(scales, 2)) return MOE_INVALID_ARG;
  return hip_status(launch_unpack_bf16(codes, scales, rows, cols, out, stream));
}

size_t nvfp4_expert_ffn_workspace_size(int n_rows, int d_model, int d_ff, moe_dtype act_dtype) {
  if (n_rows < 0 || d_model < 0 || d_ff < 0) return 0;
  if (act_dtype != MOE_F32 && act_dtype != MOE_BF16) return 0;
  size_t s = h_bytes(n_rows, d_ff);
  if (act_dtype == MOE_F32) s += split_bytes(n_rows, d_model);
  return s > 0 ? s : kAlign;
}

size_t nvfp4_grouped_linear_workspace_size(int n_rows, int k, moe_dtype a_dtype) {
  if (n_rows < 0 || k < 0) return 0;
  if (a_dtype == MOE_F32) return split_bytes(n_rows, k);
  return 0;
}

moe_status nvfp4_expert_ffn(const void *xg, moe_dtype act_dtype, int n_rows, int max_rows_per_expert,
                            const int32_t *expert_offsets, int n_experts, const moe_nvfp4_weights *up,
                            const moe_nvfp4_weights *down, moe_act act, int gemv_max_rows, void *workspace,
                            size_t ws_bytes, float *out, hipStream_t stream) {
  if (n_rows < 0 || max_rows_per_expert < 0 || n_experts < 1) return MOE_INVALID_ARG;
  if (act_dtype != MOE_F32 && act_dtype != MOE_BF16) return MOE_INVALID_ARG;
  if (act != MOE_RELU2 && act != MOE_SWIGLU) return MOE_INVALID_ARG;
  if (n_experts > MOE_MAX_EXPERTS) return MOE_UNSUPPORTED;
  if (gemv_max_rows < 0 || gemv_max_rows > MOE_MAX_GEMV_ROWS) return MOE_UNSUPPORTED;
  if (!weights_ok(up) || !weights_ok(down)) return MOE_INVALID_ARG;
  const int d = up->cols, f = down->cols, d_out = down->rows;
  if (up->rows != (act == MOE_SWIGLU ? 2 * f : f)) return MOE_INVALID_ARG;
  if (d % 32 != 0 || f % 32 != 0) return MOE_UNSUPPORTED;
  if ((long)n_rows * (d > f ? d : f) * 3 >= (1L << 40)) return MOE_UNSUPPORTED;
  if (n_rows == 0) return MOE_OK;
  if (!xg || !expert_offsets || !out || !workspace) return MOE_INVALID_ARG;
  if (!aligned(xg, 16) || !aligned(workspace, 16) || !aligned(out, 4)) return MOE_INVALID_ARG;
  if (ws_bytes < nvfp4_expert_ffn_workspace_size(n_rows, d, f, act_dtype)) return MOE_WORKSPACE_TOO_SMALL;

  const int dec_rows = gemv_max_rows < max_rows_per_expert ? gemv_max_rows : max_rows_per_expert;
  const bool use_gemm = max_rows_per_expert > gemv_max_rows;
  const int max_active = n_experts < n_rows ? n_experts : n_rows;
  const int epi = (act == MOE_SWIGLU) ? EPI_SWIGLU : EPI_RELU2;

  char *ws = (char *)workspace;
  uint16_t *h = (uint16_t *)ws;
  const long h_plane = (long)n_rows * f;
  ws += h_bytes(n_rows, f);
  const uint16_t *a = (const uint16_t *)xg;
  int nt = 1;
  long a_plane = 0;
  hipError_t err = hipSuccess;
  if (act_dtype == MOE_F32) {
    uint16_t *planes = (uint16_t *)ws;
    a_plane = (long)n_rows * d;
    err = launch_split3((const float *)xg, (long)n_rows * d, planes, a_plane, stream);
    if (err != hipSuccess) return MOE_HIP_ERROR;
    a = planes;
    nt = 3;
  }
  // up projection + activation -> h
  err = launch_dq_gemv_planes(a, nt, a_plane, d, expert_offsets, n_experts, n_rows, dec_rows, max_active, up->codes,
                              up->scales, up->global, up->rows, d, f, epi, nullptr, h, f, h_plane, stream);
  if (err != hipSuccess) return MOE_HIP_ERROR;
  if (use_gemm) {
    err = launch_dq_gemm(a, d, expert_offsets, n_experts, gemv_max_rows + 1, n_rows, up->codes, up->scales,
                         up->global, up->rows, d, f, epi, nullptr, h, f, stream);
    if (err != hipSuccess) return MOE_HIP_ERROR;
  }
  // down projection -> out
  err = launch_dq_gemv_planes(h, 3, h_plane, f, expert_offsets, n_experts, n_rows, dec_rows, max_active, down->codes,
                              down->scales, down->global, d_out, f, d_out, EPI_F32, out, nullptr, d_out, 0,
                              stream);
  if (err != hipSuccess) return MOE_HIP_ERROR;
  if (use_gemm) {
    err = launch_dq_gemm(h, f, expert_offsets, n_experts, gemv_max_rows + 1, n_rows, down->codes, down->scales,
                         down->global, d_out, f, d_out, EPI_F32, out, nullptr, d_out, stream);
    if (err != hipSuccess) return MOE_HIP_ERROR;
  }
  return MOE_OK;
}

moe_status nvfp4_grouped_linear(const void *a_in, moe_dtype a_dtype, int n_rows, int max_rows_per_expert,
                                const int32_t *expert_offsets, int n_experts, const moe_nvfp4_weights *w,
                                int gemv_max_rows, void *workspace, size_t ws_bytes, float *out,
                                hipStream_t stream) {
  if (n_rows < 0 || max_rows_per_expert < 0 || n_experts < 1) return MOE_INVALID_ARG;
  if (a_dtype != MOE_F32 && a_dtype != MOE_BF16) return MOE_INVALID_ARG;
  if (n_experts > MOE_MAX_EXPERTS) return MOE_UNSUPPORTED;
  if (gemv_max_rows < 0 || gemv_max_rows > MOE_MAX_GEMV_ROWS) return MOE_UNSUPPORTED;
  if (!weights_ok(w)) return MOE_INVALID_ARG;
  const int k = w->cols, n_out = w->rows;
  if (k % 32 != 0) return MOE_UNSUPPORTED;
  if ((long)n_rows * (k > n_out ? k : n_out) * 3 >= (1L << 40)) return MOE_UNSUPPORTED;
  if (n_rows == 0) return MOE_OK;
  if (!a_in || !expert_offsets || !out) return MOE_INVALID_ARG;
  if (!aligned(a_in, 16) || !aligned(out, 4)) return MOE_INVALID_ARG;
  const size_t need = nvfp4_grouped_linear_workspace_size(n_rows, k, a_dtype);
  if (need > 0 && (!workspace || !aligned(workspace, 16))) return MOE_INVALID_ARG;
  if (ws_bytes < need) return MOE_WORKSPACE_TOO_SMALL;

  const int dec_rows = gemv_max_rows < max_rows_per_expert ? gemv_max_rows : max_rows_per_expert;
  const bool use_gemm = max_rows_per_expert > gemv_max_rows;
  const int max_active = n_experts < n_rows ? n_experts : n_rows;
  const uint16_t *a = (const uint16_t *)a_in;
  int nt = 1;
  long a_plane = 0;
  hipError_t err;
  if (a_dtype == MOE_F32) {
    uint16_t *planes = (uint16_t *)workspace;
    a_plane = (long)n_rows * k;
    err = launch_split3((const float *)a_in, (long)n_rows * k, planes, a_plane, stream);
    if (err != hipSuccess) return MOE_HIP_ERROR;
    a = planes;
    nt = 3;
  }
  err = launch_dq_gemv_planes(a, nt, a_plane, k, expert_offsets, n_experts, n_rows, dec_rows, max_active, w->codes,
                              w->scales, w->global, n_out, k, n_out, EPI_F32, out, nullptr, n_out, 0, stream);
  if (err != hipSuccess) return MOE_HIP_ERROR;
  if (use_gemm) {
    err = launch_dq_gemm(a, k, expert_offsets, n_experts, gemv_max_rows + 1, n_rows, w->codes, w->scales,
                         w->global, n_out, k, n_out, EPI_F32, out, nullptr, n_out, stream);
    if (err != hipSuccess) return MOE_HIP_ERROR;
  }
  return MOE_OK;
}

}  // extern "C"
