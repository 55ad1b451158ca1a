// api.hip -- the C ABI (include/moe_nvfp4.h): host-side argument checks,
// workspace carving and launch planning.  Nothing here synchronises, allocates
// or reads device memory: the path choice between the decode kernels (experts
// with <= gemv_max_rows rows) and the prefill GEMM (more rows) is made on the
// device from expert_offsets, and the host only uses bounds it already knows
// (Glq v0.2.13, "v3a": host syncs inside the MoE loop dominated the host
// budget; gllm PR #91, "Results": every op synchronising was what remained).
#include <limits.h>
#include <stdint.h>

#include <mutex>

#include "launch.hpp"
#include "moe_nvfp4.h"

using namespace moe;

// The layer workspace of moe_layer_forward_noalloc: one array per GPU, held
// by the library until the process ends.  In host code `scratch` names a
// host-side stand-in, not a device address; the device address comes from
// hipGetSymbolAddress (noalloc_scratch below), once per device.
static __device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_HIP_ERROR; }

// The prefill GEMM addresses an activation matrix (bf16, a_rows x a_cols) and
// one expert's codes (w_rows x w_cols/2 bytes) with 32-bit buffer offsets that
// stay below 2^31.
bool gemm_extents_ok(long a_rows, long a_cols, long w_rows, long w_cols) {
  return a_rows * a_cols * 2 < (1L << 31) && w_rows * (w_cols / 2) < (1L << 31);
}

// The repacked copies: both or neither, 16-byte aligned, and one expert's
// repacked codes addressable with 32-bit offsets below 2^31 (the GEMM marks
// skipped loads with offset 2^31).
bool packed_ok(const moe_nvfp4_weights *w) {
  if (!w->codes_packed && !w->scales_packed) return true;
  if (!w->codes_packed || !w->scales_packed) return false;
  if (!aligned(w->codes_packed, 16) || !aligned(w->scales_packed, 16)) return false;
  return packed_codes_bytes(1, w->rows, w->cols) < (1L << 31);
}

// A projection is given by its canonical codes and scales, its repacked
// copies, or both.  Without the canonical layout every kernel that reads the
// weights must take the repacked one: whole 16-row blocks (the prefill GEMM's
// condition; SwiGLU also needs the up half block-aligned, see swiglu_ok).
bool weights_ok(const moe_nvfp4_weights *w) {
  if (!w || !w->global || w->rows <= 0 || w->cols <= 0 || !aligned(w->global, 4) || !packed_ok(w)) return false;
  if (!w->codes != !w->scales) return false;  // both canonical arrays or neither
  if (w->codes) return aligned(w->codes, 16) && aligned(w->scales, 2);
  return w->codes_packed != nullptr && w->rows % 16 == 0;
}

// SwiGLU's up projection holds 2f rows: without the canonical layout its gate
// and up halves must each be whole 16-row blocks.
bool swiglu_ok(const moe_nvfp4_weights *up) { return up->codes != nullptr || up->rows % 32 == 0; }

// Every workspace of nvfp4_expert_ffn and moe_gather_rows starts with 256
// bytes reserved for its error word (the int32 at offset 0).
constexpr size_t kErrBytes = 256;

// Planes of the fp32-activation split: three bf16 planes of n_rows*k.
size_t split_bytes(long n_rows, long k) { return align_up((size_t)3 * n_rows * k * sizeof(uint16_t)); }

// h as three bf16 planes of n_rows*f.
size_t h_bytes(long n_rows, long f) { return align_up((size_t)3 * n_rows * f * sizeof(uint16_t)); }

// A projection problem over grouped rows (offsets on the device) or over one
// expert whose rows are known on the host (known_rows >= 0).
ProjProblem make_problem(const uint16_t *a, long plane, long lda, const int32_t *offsets, int n_experts,
                         int n_rows, int known_rows, const moe_nvfp4_weights *w, int n_out, float *out_f32,
                         uint16_t *out_h, long ldo, long h_plane) {
  ProjProblem p{};
  p.a = a;
  p.row_map = nullptr;
  p.plane = plane;
  p.lda = lda;
  p.a_rows = n_rows;
  p.offsets = offsets;
  p.n_experts = n_experts;
  p.n_rows = n_rows;
  p.known_rows = known_rows;
  p.min_rows = 1;
  p.max_rows = INT_MAX;
  p.codes = w->codes;
  p.scales = w->scales;
  p.scales_packed = w->scales_packed;
  p.codes_packed = w->codes_packed;
  p.global = w->global;
  p.n_w = w->rows;
  p.k = w->cols;
  p.n_out = n_out;
  p.out_f32 = out_f32;
  p.out_h = out_h;
  p.ldo = ldo;
  p.h_plane = h_plane;
  return p;
}

// Decode-path copy of a problem: experts with 1..dec_rows rows.
ProjProblem as_decode(ProjProblem p, int dec_rows) {
  p.min_rows = 1;
  p.max_rows = dec_rows;
  return p;
}

// Prefill-path copy: experts with more than gemv_max_rows rows.  h is one bf16
// plane there (the activation rounded to bf16).
ProjProblem as_prefill(ProjProblem p, int gemv_max_rows) {
  p.min_rows = gemv_max_rows + 1;
  p.max_rows = INT_MAX;
  if (p.known_rows >= 0) p.min_rows = 1;
  return p;
}

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

size_t nvfp4_packed_scales_bytes(int n_experts, int rows, int cols) {
  if (n_experts < 1 || rows < 1 || cols < 1) return 0;
  return (size_t)packed_scales_bytes(n_experts, rows, cols);
}

moe_status nvfp4_pack_scales(const moe_nvfp4_weights *w, int n_experts, uint8_t *dst, size_t dst_bytes,
                             hipStream_t stream) {
  if (!w || !w->scales || !dst || n_experts < 1 || w->rows < 1 || w->cols < 32 || w->cols % 32 != 0)
    return MOE_INVALID_ARG;
  if (dst_bytes < (size_t)packed_scales_bytes(n_experts, w->rows, w->cols)) return MOE_INVALID_ARG;
  return hip_status(launch_pack_scales(w->scales, n_experts, w->rows, w->cols, dst, stream));
}

size_t nvfp4_packed_codes_bytes(int n_experts, int rows, int cols) {
  if (n_experts < 1 || rows < 1 || cols < 1) return 0;
  return (size_t)packed_codes_bytes(n_experts, rows, cols);
}

moe_status nvfp4_pack_codes(const moe_nvfp4_weights *w, int n_experts, uint8_t *dst, size_t dst_bytes,
                            hipStream_t stream) {
  if (!w || !w->codes || !dst || n_experts < 1 || w->rows < 1 || w->cols < 32 || w->cols % 32 != 0)
    return MOE_INVALID_ARG;
  if (dst_bytes < (size_t)packed_codes_bytes(n_experts, w->rows, w->cols)) return MOE_INVALID_ARG;
  return hip_status(launch_pack_codes(w->codes, n_experts, w->rows, w->cols, dst, stream));
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

size_t moe_router_workspace_size(int n_tokens, int n_experts) {
  if (n_tokens < 0 || n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return 0;
  return align_up(router_counter_bytes(n_tokens)) + align_up((size_t)n_tokens * n_experts * sizeof(float)) + kAlign;
}

moe_status moe_router_workspace_init(void *workspace, size_t ws_bytes, int n_tokens, hipStream_t stream) {
  if (!workspace || !aligned(workspace, kAlign) || n_tokens < 0) return MOE_INVALID_ARG;
  if (ws_bytes < moe_router_workspace_size(n_tokens, 1)) return MOE_WORKSPACE_TOO_SMALL;
  return hip_status(launch_router_init((int32_t *)workspace, n_tokens, stream));
}

moe_status moe_router_topk(const void *x, moe_dtype x_dtype, int n_tokens, int d_model, const uint16_t *router_w,
                           int n_experts, int top_k, int32_t *topk_ids, float *topk_weights, float *logits,
                           void *workspace, size_t ws_bytes, hipStream_t stream) {
  if (n_tokens < 0 || d_model < 1 || n_experts < 1 || top_k < 1 || top_k > n_experts) return MOE_INVALID_ARG;
  if (x_dtype != MOE_F32 && x_dtype != MOE_BF16) return MOE_INVALID_ARG;
  if (n_experts > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOPK) return MOE_UNSUPPORTED;
  if (d_model % 32 != 0) return MOE_UNSUPPORTED;
  if ((long)n_tokens * (n_experts > d_model ? n_experts : d_model) >= (1L << 40)) return MOE_UNSUPPORTED;
  if (n_tokens == 0) return MOE_OK;
  if (!x || !router_w || !topk_ids || !topk_weights || !workspace) return MOE_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(router_w, 16) || !aligned(workspace, kAlign)) return MOE_INVALID_ARG;
  if (logits && !aligned(logits, 4)) return MOE_INVALID_ARG;
  if (ws_bytes < moe_router_workspace_size(n_tokens, n_experts)) return MOE_WORKSPACE_TOO_SMALL;
  int32_t *counters = (int32_t *)workspace;
  float *lg = logits ? logits : (float *)((char *)workspace + align_up(router_counter_bytes(n_tokens)));
  return hip_status(launch_router_topk(x, x_dtype == MOE_F32, n_tokens, d_model, router_w, n_experts, top_k, lg,
                                       counters, topk_ids, topk_weights, stream));
}

size_t moe_gather_workspace_size(int n_tokens, int n_experts) {
  if (n_tokens < 0 || n_experts < 1 || n_experts > MOE_MAX_EXPERTS) return 0;
  return kErrBytes + align_up(gather_workspace_bytes(n_tokens, n_experts));
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
  if (n_tokens > 0 && (!aligned(x, 16) || !aligned(xg, 16) || !aligned(workspace, 16))) return MOE_INVALID_ARG;
  if (x && xg && x == xg) return MOE_INVALID_ARG;
  if (ws_bytes < moe_gather_workspace_size(n_tokens, n_experts)) return MOE_WORKSPACE_TOO_SMALL;
  int elem = (x_dtype == MOE_F32) ? 4 : 2;
  return hip_status(launch_gather(x, elem, n_tokens, d_model, topk_ids, top_k, n_experts, xg, expert_offsets,
                                  row_token, rows, (char *)workspace + kErrBytes, (int32_t *)workspace, stream));
}

static moe_status wrs_common(float *dst, const float *src, int n_src_rows, const int32_t *rows,
                             const float *weights, int n_tokens, int top_k, int d_model, bool accumulate,
                             int32_t *error_word, hipStream_t stream) {
  if (n_src_rows < 0 || n_tokens < 0 || top_k < 1 || d_model < 0) return MOE_INVALID_ARG;
  if ((long)n_tokens * d_model >= (1L << 40)) return MOE_UNSUPPORTED;
  if (n_tokens == 0 || d_model == 0) return MOE_OK;
  if (!dst || !rows || !weights || (n_src_rows > 0 && !src)) return MOE_INVALID_ARG;
  if (src && (const void *)src == (const void *)dst) return MOE_INVALID_ARG;
  if (error_word && !aligned(error_word, 4)) return MOE_INVALID_ARG;
  return hip_status(launch_weighted_row_sum(dst, src, n_src_rows, rows, weights, n_tokens, top_k, d_model,
                                            accumulate, error_word, stream));
}

moe_status moe_weighted_row_sum(float *dst, const float *src, int n_src_rows, const int32_t *rows,
                                const float *weights, int n_tokens, int top_k, int d_model, int32_t *error_word,
                                hipStream_t stream) {
  return wrs_common(dst, src, n_src_rows, rows, weights, n_tokens, top_k, d_model, true, error_word, stream);
}

moe_status moe_weighted_row_sum_into(float *dst, const float *src, int n_src_rows, const int32_t *rows,
                                     const float *weights, int n_tokens, int top_k, int d_model,
                                     int32_t *error_word, hipStream_t stream) {
  return wrs_common(dst, src, n_src_rows, rows, weights, n_tokens, top_k, d_model, false, error_word, stream);
}

moe_status moe_error_word_clear(int32_t *word, hipStream_t stream) {
  if (!word || !aligned(word, 4)) return MOE_INVALID_ARG;
  return hip_status(launch_error_word_clear(word, stream));
}

moe_status moe_error_word_read(const int32_t *word, int32_t *value, hipStream_t stream) {
  if (!word || !value || !aligned(word, 4)) return MOE_INVALID_ARG;
  if (hipMemcpyAsync(value, word, sizeof(int32_t), hipMemcpyDeviceToHost, stream) != hipSuccess)
    return MOE_HIP_ERROR;
  return hip_status(hipStreamSynchronize(stream));
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
  size_t s = kErrBytes + h_bytes(n_rows, d_ff);
  if (act_dtype == MOE_F32) s += split_bytes(n_rows, d_model);
  return s;
}

size_t moe_workspace_size(int n_tokens, int top_k, int n_experts, int d_model, int d_ff_max, moe_act act) {
  if (n_tokens < 0 || top_k < 1 || n_experts < 1 || d_model < 0 || d_ff_max < 0) return 0;
  if (act != MOE_RELU2 && act != MOE_SWIGLU) return 0;
  if (top_k > n_experts || n_experts > MOE_MAX_EXPERTS || top_k > MOE_MAX_TOPK) return 0;
  if ((long)n_tokens * top_k >= (1L << 31)) return 0;
  const int R = n_tokens * top_k;
  size_t s = moe_gather_workspace_size(n_tokens, n_experts);
  const size_t routed = nvfp4_expert_ffn_workspace_size(R, d_model, d_ff_max, MOE_F32);
  const size_t shared = nvfp4_expert_ffn_workspace_size(n_tokens, d_model, d_ff_max, MOE_F32);
  if (routed > s) s = routed;
  if (shared > s) s = shared;
  return s;
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
  if (act == MOE_SWIGLU && !swiglu_ok(up)) return MOE_INVALID_ARG;
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
  if (use_gemm && (!gemm_extents_ok(n_rows, d, up->rows, d) || !gemm_extents_ok(n_rows, f, d_out, f)))
    return MOE_UNSUPPORTED;
  const int max_active = n_experts < n_rows ? n_experts : n_rows;
  const int epi = (act == MOE_SWIGLU) ? EPI_SWIGLU : EPI_RELU2;

  char *ws = (char *)workspace + kErrBytes;
  uint16_t *h = (uint16_t *)ws;
  const long h_plane = (long)n_rows * f;
  ws += h_bytes(n_rows, f);
  const uint16_t *a = (const uint16_t *)xg;
  int nt = 1;
  long a_plane = 0;
  if (act_dtype == MOE_F32) {
    uint16_t *planes = (uint16_t *)ws;
    a_plane = (long)n_rows * d;
    if (launch_split3((const float *)xg, (long)n_rows * d, planes, a_plane, stream) != hipSuccess)
      return MOE_HIP_ERROR;
    a = planes;
    nt = 3;
  }
  ProjProblem pu = make_problem(a, a_plane, d, expert_offsets, n_experts, n_rows, -1, up, f, nullptr, h, f, h_plane);
  ProjProblem pd = make_problem(h, h_plane, f, expert_offsets, n_experts, n_rows, -1, down, d_out, out, nullptr,
                                d_out, 0);
  ProjProblem q;
  q = as_decode(pu, dec_rows);
  if (launch_dq_gemv(&q, &max_active, 1, nt, epi, stream) != hipSuccess) return MOE_HIP_ERROR;
  if (use_gemm) {
    q = as_prefill(pu, gemv_max_rows);
    if (launch_dq_gemm(&q, 1, epi, stream) != hipSuccess) return MOE_HIP_ERROR;
  }
  q = as_decode(pd, dec_rows);
  if (launch_dq_gemv(&q, &max_active, 1, 3, EPI_F32, stream) != hipSuccess) return MOE_HIP_ERROR;
  if (use_gemm) {
    q = as_prefill(pd, gemv_max_rows);
    if (launch_dq_gemm(&q, 1, EPI_F32, stream) != hipSuccess) return MOE_HIP_ERROR;
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
  if (use_gemm && !gemm_extents_ok(n_rows, k, n_out, k)) return MOE_UNSUPPORTED;
  const int max_active = n_experts < n_rows ? n_experts : n_rows;
  const uint16_t *a = (const uint16_t *)a_in;
  int nt = 1;
  long a_plane = 0;
  if (a_dtype == MOE_F32) {
    uint16_t *planes = (uint16_t *)workspace;
    a_plane = (long)n_rows * k;
    if (launch_split3((const float *)a_in, (long)n_rows * k, planes, a_plane, stream) != hipSuccess)
      return MOE_HIP_ERROR;
    a = planes;
    nt = 3;
  }
  ProjProblem p = make_problem(a, a_plane, k, expert_offsets, n_experts, n_rows, -1, w, n_out, out, nullptr, n_out, 0);
  ProjProblem q = as_decode(p, dec_rows);
  if (launch_dq_gemv(&q, &max_active, 1, nt, EPI_F32, stream) != hipSuccess) return MOE_HIP_ERROR;
  if (use_gemm) {
    q = as_prefill(p, gemv_max_rows);
    if (launch_dq_gemm(&q, 1, EPI_F32, stream) != hipSuccess) return MOE_HIP_ERROR;
  }
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// the whole layer
// ---------------------------------------------------------------------------

namespace {

struct LayerPlan {
  int n, d, E, K, f, fs, R;
  bool has_shared, f32;
  size_t off_ids, off_w, off_offsets, off_row_token, off_rows, off_yg, off_gather, off_h, off_hs, off_split,
      off_sync, off_cmb, off_part, total;
  int n_ct;  // 256-column tiles of the output (the fused combine's counters per token)
  int sync_words;
  size_t part_bytes;
};

bool plan_layer(const moe_layer_desc *dsc, LayerPlan *pl) {
  if (!dsc) return false;
  LayerPlan p{};
  p.n = dsc->n_tokens;
  p.d = dsc->d_model;
  p.E = dsc->n_experts;
  p.K = dsc->top_k;
  if (p.n < 0 || p.d <= 0 || p.E < 1 || p.K < 1 || p.K > p.E) return false;
  if (p.E > MOE_MAX_EXPERTS || p.K > MOE_MAX_TOPK) return false;
  if (dsc->x_dtype != MOE_F32 && dsc->x_dtype != MOE_BF16) return false;
  if (dsc->act != MOE_RELU2 && dsc->act != MOE_SWIGLU) return false;
  if (dsc->gemv_max_rows < 0 || dsc->gemv_max_rows > MOE_MAX_GEMV_ROWS) return false;
  if (dsc->flags & ~(MOE_LAYER_SINGLE_LAUNCH | MOE_LAYER_FUSED_COMBINE)) return false;
  if (!weights_ok(&dsc->up) || !weights_ok(&dsc->down)) return false;
  if (dsc->act == MOE_SWIGLU && !swiglu_ok(&dsc->up)) return false;
  p.f = dsc->down.cols;
  if (dsc->up.cols != p.d || dsc->down.rows != p.d) return false;
  if (dsc->up.rows != (dsc->act == MOE_SWIGLU ? 2 * p.f : p.f)) return false;
  if (p.d % 32 || p.f % 32) return false;
  p.has_shared = dsc->shared_up.codes != nullptr || dsc->shared_up.codes_packed != nullptr;
  p.fs = 0;
  if (p.has_shared) {
    if (!weights_ok(&dsc->shared_up) || !weights_ok(&dsc->shared_down)) return false;
    p.fs = dsc->shared_down.cols;
    if (dsc->shared_up.cols != p.d || dsc->shared_down.rows != p.d || dsc->shared_up.rows != p.fs) return false;
    if (p.fs % 32) return false;
  }
  if ((long)p.n * p.K >= (1L << 31)) return false;
  p.R = p.n * p.K;
  if (p.n > dsc->gemv_max_rows) {  // some expert may take the prefill GEMM
    if (!gemm_extents_ok(p.n, p.d, dsc->up.rows, p.d) || !gemm_extents_ok(p.R, p.f, p.d, p.f)) return false;
    if (p.has_shared && (!gemm_extents_ok(p.n, p.d, p.fs, p.d) || !gemm_extents_ok(p.n, p.fs, p.d, p.fs)))
      return false;
  }
  p.f32 = dsc->x_dtype == MOE_F32;
  const size_t xb = p.f32 ? 4 : 2;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align_up(bytes);
    return at;
  };
  // the decode layer's flags and counters first: the same place for every
  // description, so a workspace initialised once serves calls of any size
  p.sync_words = (int)decode_layer_sync_words();
  p.off_sync = take((size_t)p.sync_words * 4);
  // then its partial sums, tagged with launch counts: sized for a two-token
  // step whatever n is, so every token count of a layer puts them in the
  // same bytes, which nothing else writes
  p.part_bytes = p.n > 0 ? decode_layer_part_bytes(2, p.E, p.K, p.d, p.f, p.fs) : 0;
  p.off_part = take(p.part_bytes);
  p.off_ids = take((size_t)p.R * 4);
  p.off_w = take((size_t)p.R * 4);
  p.off_offsets = take((size_t)(p.E + 1) * 4);
  p.off_row_token = take((size_t)p.R * 4);
  p.off_rows = take((size_t)p.R * 4);
  p.off_yg = take((size_t)p.R * p.d * 4);
  p.off_gather = take(gather_workspace_bytes(p.n, p.E));
  p.off_h = take(h_bytes(p.R, p.f));
  p.off_hs = take(p.has_shared ? h_bytes(p.n, p.fs) : 0);
  p.off_split = take(p.f32 ? split_bytes(p.n, p.d) : 0);
  p.n_ct = (p.d + kGemmF32TileCols - 1) / kGemmF32TileCols;
  p.off_cmb = take((size_t)p.n * p.n_ct * 64);
  (void)xb;
  p.total = o;
  *pl = p;
  return true;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The current device's copy of `scratch`, its address looked up once per
// device (with that device current) and kept.
moe_status noalloc_scratch(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_HIP_ERROR;
  if (dev < 0 || dev >= kMaxDevices) return MOE_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MOE_HIP_ERROR;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

size_t moe_layer_workspace_size(const moe_layer_desc *desc) {
  LayerPlan p;
  if (!plan_layer(desc, &p)) return 0;
  return p.total;
}

moe_status moe_layer_get_views(const moe_layer_desc *desc, void *workspace, moe_layer_views *v) {
  LayerPlan p;
  if (!plan_layer(desc, &p) || !workspace || !v) return MOE_INVALID_ARG;
  char *ws = (char *)workspace;
  v->topk_ids = (int32_t *)(ws + p.off_ids);
  v->topk_weights = (float *)(ws + p.off_w);
  v->expert_offsets = (int32_t *)(ws + p.off_offsets);
  v->row_token = (int32_t *)(ws + p.off_row_token);
  v->rows = (int32_t *)(ws + p.off_rows);
  v->yg = (float *)(ws + p.off_yg);
  v->wait_error = (int32_t *)(ws + p.off_sync);
  v->decode_launch = (int32_t *)(ws + p.off_sync) + 1;
  return MOE_OK;
}

moe_status moe_layer_workspace_init(const moe_layer_desc *desc, void *workspace, size_t ws_bytes,
                                    hipStream_t stream) {
  LayerPlan p;
  if (!plan_layer(desc, &p) || !workspace || !aligned(workspace, kAlign)) return MOE_INVALID_ARG;
  if (ws_bytes < p.total) return MOE_WORKSPACE_TOO_SMALL;
  if (decode_layer_init((int32_t *)((char *)workspace + p.off_sync), (char *)workspace + p.off_part, p.part_bytes,
                        stream) != hipSuccess)
    return MOE_HIP_ERROR;
  return MOE_OK;
}

moe_status moe_layer_forward(const moe_layer_desc *dsc, const void *x, const float *logits, float *out,
                             void *workspace, size_t ws_bytes, hipStream_t stream) {
  return moe_layer_forward_profiled(dsc, x, logits, out, workspace, ws_bytes, nullptr, stream);
}

moe_status moe_layer_forward_noalloc(const moe_layer_desc *dsc, const void *x, const float *logits, float *out,
                                     hipStream_t stream) {
  LayerPlan p;
  if (!plan_layer(dsc, &p)) return MOE_INVALID_ARG;
  if (p.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_UNSUPPORTED;
  if (p.n == 0) return MOE_OK;
  if (!x || !logits || !out) return MOE_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(out, 16)) return MOE_INVALID_ARG;
  void *ws = nullptr;
  const moe_status st = noalloc_scratch(&ws);
  if (st != MOE_OK) return st;
  // the single-launch step's launch counts and partial sums start from zero
  // on every call: the array keeps whatever the last call on this GPU left
  if ((dsc->flags & MOE_LAYER_SINGLE_LAUNCH) &&
      decode_layer_init((int32_t *)((char *)ws + p.off_sync), (char *)ws + p.off_part, p.part_bytes, stream) !=
          hipSuccess)
    return MOE_HIP_ERROR;
  return moe_layer_forward_profiled(dsc, x, logits, out, ws, MOE_NOALLOC_SCRATCH_BYTES, nullptr, stream);
}

moe_status moe_layer_forward_profiled(const moe_layer_desc *dsc, const void *x, const float *logits, float *out,
                                      void *workspace, size_t ws_bytes, hipEvent_t *events, hipStream_t stream) {
  auto mark = [&](int i) { return events ? hipEventRecord(events[i], stream) : hipSuccess; };
  LayerPlan p;
  if (!plan_layer(dsc, &p)) return MOE_INVALID_ARG;
  if (p.n == 0) return MOE_OK;
  if (!x || !logits || !out || !workspace) return MOE_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(out, 16) || !aligned(workspace, kAlign)) return MOE_INVALID_ARG;
  if (ws_bytes < p.total) return MOE_WORKSPACE_TOO_SMALL;
  char *ws = (char *)workspace;
  int32_t *ids = (int32_t *)(ws + p.off_ids);
  float *w = (float *)(ws + p.off_w);
  int32_t *offsets = (int32_t *)(ws + p.off_offsets);
  int32_t *row_token = (int32_t *)(ws + p.off_row_token);
  int32_t *rows = (int32_t *)(ws + p.off_rows);
  float *yg = (float *)(ws + p.off_yg);
  uint16_t *h = (uint16_t *)(ws + p.off_h);
  uint16_t *hs = (uint16_t *)(ws + p.off_hs);
  const int elem = p.f32 ? 4 : 2;

  int32_t *sync = (int32_t *)(ws + p.off_sync);

  if (mark(0) != hipSuccess) return MOE_HIP_ERROR;
  const int gmax = dsc->gemv_max_rows;
  const int max_active = p.E < p.R ? p.E : p.R;
  const int epi = dsc->act == MOE_SWIGLU ? EPI_SWIGLU : EPI_RELU2;
  // 1-5 in one persistent launch for a decode step (at most two tokens, every
  //     expert on the decode path), when the caller has promised the device
  //     to this call alone
  if ((dsc->flags & MOE_LAYER_SINGLE_LAUNCH) && p.n <= gmax && decode_layer_takes(p.n, p.K, p.d)) {
    DecodeLayerProblem lp{};
    lp.up[1] = make_problem(nullptr, 0, p.d, nullptr, p.E, p.R, -1, &dsc->up, p.f, nullptr, nullptr, 0, 0);
    lp.down[1] = make_problem(nullptr, 0, p.f, nullptr, p.E, p.R, -1, &dsc->down, p.d, nullptr, nullptr, 0, 0);
    if (p.has_shared) {
      lp.up[0] = make_problem(nullptr, 0, p.d, nullptr, 1, p.n, p.n, &dsc->shared_up, p.fs, nullptr, nullptr, 0, 0);
      lp.down[0] =
          make_problem(nullptr, 0, p.fs, nullptr, 1, p.n, p.n, &dsc->shared_down, p.d, nullptr, nullptr, 0, 0);
    }
    lp.has_shared = p.has_shared;
    lp.max_slots = max_active;
    lp.act = epi;
    lp.x = x;
    lp.x_f32 = p.f32;
    lp.logits = logits;
    lp.part = ws + p.off_part;
    lp.out = out;
    lp.yg = yg;
    lp.ids = ids;
    lp.topk_w = w;
    lp.offsets = offsets;
    lp.row_token = row_token;
    lp.rows = rows;
    lp.n_tokens = p.n;
    lp.n_experts = p.E;
    lp.top_k = p.K;
    lp.d = p.d;
    lp.f = p.f;
    lp.fs = p.fs;
    lp.n_rows = p.R;
    lp.sync = sync;
    const hipError_t e = launch_decode_layer(lp, stream);
    if (e == hipSuccess) {
      for (int i = 1; i <= 7; ++i)
        if (mark(i) != hipSuccess) return MOE_HIP_ERROR;
      return MOE_OK;
    }
    if (e != hipErrorNotSupported) return MOE_HIP_ERROR;
  }

  // 1. routing + gather layout.  The packed activation rows are not
  //    materialised: the routed up projection reads x through row_token.
  //    The fused kernel routes every token inside one workgroup, i.e. on one
  //    CU; past kFusedRouteMaxTokens tokens, routing with a wavefront per
  //    token across CUs and then the one-workgroup layout is faster
  //    (32 tokens: 6 us less per step).
  constexpr int kFusedRouteMaxTokens = 16;
  if (p.n <= kFusedRouteMaxTokens && gather_is_single_launch(p.n, p.K, p.E, elem, p.d)) {
    if (launch_route_gather_small(logits, p.n, p.E, p.K, ids, w, x, elem, p.d, nullptr, offsets, row_token, rows,
                                  stream) != hipSuccess)
      return MOE_HIP_ERROR;
  } else {
    if (launch_route_topk(logits, p.n, p.E, p.K, ids, w, stream) != hipSuccess) return MOE_HIP_ERROR;
    if (launch_gather(x, elem, p.n, p.d, ids, p.K, p.E, nullptr, offsets, row_token, rows, ws + p.off_gather,
                      nullptr, stream) != hipSuccess)
      return MOE_HIP_ERROR;
  }
  if (mark(1) != hipSuccess) return MOE_HIP_ERROR;

  // 2. activation planes (fp32 x only: three bf16 planes of the n token rows)
  const uint16_t *a_x = (const uint16_t *)x;
  long plane_x = 0;
  int nt = 1;
  if (p.f32) {
    uint16_t *sx = (uint16_t *)(ws + p.off_split);
    plane_x = (long)p.n * p.d;
    if (launch_split3((const float *)x, plane_x, sx, plane_x, stream) != hipSuccess) return MOE_HIP_ERROR;
    a_x = sx;
    nt = 3;
  }

  const int dec_rows = gmax < p.n ? gmax : p.n;  // a routed expert has at most n rows
  const bool routed_gemm = p.n > gmax;
  const bool shared_gemv = p.has_shared && p.n <= gmax;
  const bool shared_gemm = p.has_shared && p.n > gmax;
  const long h_plane = (long)p.R * p.f, hs_plane = (long)p.n * p.fs;

  ProjProblem ru = make_problem(a_x, plane_x, p.d, offsets, p.E, p.R, -1, &dsc->up, p.f, nullptr, h, p.f, h_plane);
  ru.row_map = row_token;  // gather on load
  ru.a_rows = p.n;
  ProjProblem rd = make_problem(h, h_plane, p.f, offsets, p.E, p.R, -1, &dsc->down, p.d, yg, nullptr, p.d, 0);
  ProjProblem su{}, sd{};
  if (p.has_shared) {
    su = make_problem(a_x, plane_x, p.d, nullptr, 1, p.n, p.n, &dsc->shared_up, p.fs, nullptr, hs, p.fs, hs_plane);
    sd = make_problem(hs, hs_plane, p.fs, nullptr, 1, p.n, p.n, &dsc->shared_down, p.d, out, nullptr, p.d, 0);
  }

  // With MOE_LAYER_FUSED_COMBINE the combine joins the down GEMM when both
  // experts take it (a prefill step with a shared expert) and its coherent
  // accesses fit 32-bit offsets; the up GEMM launch zeroes its counters.
  const bool fuse_combine = (dsc->flags & MOE_LAYER_FUSED_COMBINE) && routed_gemm && shared_gemm && p.d % 4 == 0 &&
                            (long)p.R * p.d * 4 < (1L << 31) && (long)p.n * p.d * 4 < (1L << 31);
  CombineArgs cmb{};
  if (fuse_combine) {
    cmb.on = 1;
    cmb.counters = (int32_t *)(ws + p.off_cmb);
    cmb.ids = ids;
    cmb.rows = rows;
    cmb.row_token = row_token;
    cmb.offsets = offsets;
    cmb.w = w;
    cmb.yg = yg;
    cmb.out = out;
    cmb.n = p.n;
    cmb.K = p.K;
    cmb.d = p.d;
    cmb.gmax = gmax;
    cmb.n_ct = p.n_ct;
  }

  if (mark(2) != hipSuccess) return MOE_HIP_ERROR;
  // 3. up projections (+ activation); the shared expert joins the routed launch
  //    when both use the same epilogue
  {
    ProjProblem dec[2];
    int act[2];
    int c = 0;
    const bool join = shared_gemv && epi == EPI_RELU2;
    if (join) {
      dec[c] = as_decode(su, gmax);
      act[c++] = 1;
    }
    dec[c] = as_decode(ru, dec_rows);
    act[c++] = max_active;
    if (launch_dq_gemv(dec, act, c, nt, epi, stream) != hipSuccess) return MOE_HIP_ERROR;
    if (shared_gemv && !join) {
      ProjProblem s1 = as_decode(su, gmax);
      int one = 1;
      if (launch_dq_gemv(&s1, &one, 1, nt, EPI_RELU2, stream) != hipSuccess) return MOE_HIP_ERROR;
    }
    if (mark(3) != hipSuccess) return MOE_HIP_ERROR;
    ProjProblem gem[2];
    int g = 0;
    const bool gjoin = shared_gemm && epi == EPI_RELU2;
    if (gjoin) gem[g++] = as_prefill(su, gmax);
    if (routed_gemm) gem[g++] = as_prefill(ru, gmax);
    if (g > 0 && launch_dq_gemm(gem, g, epi, stream, nullptr, fuse_combine ? cmb.counters : nullptr,
                                fuse_combine ? (long)p.n * p.n_ct : 0) != hipSuccess)
      return MOE_HIP_ERROR;
    if (shared_gemm && !gjoin) {
      ProjProblem s1 = as_prefill(su, gmax);
      if (launch_dq_gemm(&s1, 1, EPI_RELU2, stream) != hipSuccess) return MOE_HIP_ERROR;
    }
  }

  if (mark(4) != hipSuccess) return MOE_HIP_ERROR;
  // 4. down projections: shared -> out, routed -> yg
  {
    ProjProblem dec[2];
    int act[2];
    int c = 0;
    if (shared_gemv) {
      dec[c] = as_decode(sd, gmax);
      act[c++] = 1;
    }
    dec[c] = as_decode(rd, dec_rows);
    act[c++] = max_active;
    if (launch_dq_gemv(dec, act, c, 3, EPI_F32, stream) != hipSuccess) return MOE_HIP_ERROR;
    if (mark(5) != hipSuccess) return MOE_HIP_ERROR;
    ProjProblem gem[2];
    int g = 0;
    if (shared_gemm) gem[g++] = as_prefill(sd, gmax);
    if (routed_gemm) gem[g++] = as_prefill(rd, gmax);
    if (g > 0 && launch_dq_gemm(gem, g, EPI_F32, stream, fuse_combine ? &cmb : nullptr) != hipSuccess)
      return MOE_HIP_ERROR;
  }

  if (mark(6) != hipSuccess) return MOE_HIP_ERROR;
  // 5. combine: out += sum_j w * yg[rows]  (onto zero without a shared
  //    expert), unless the down launch did it
  if (!fuse_combine &&
      launch_weighted_row_sum(out, yg, p.R, rows, w, p.n, p.K, p.d, p.has_shared, nullptr, stream) != hipSuccess)
    return MOE_HIP_ERROR;
  if (mark(7) != hipSuccess) return MOE_HIP_ERROR;
  return MOE_OK;
}

}  // extern "C"
