// wrs.hip -- WeightedRowSum (gllm PR #91, "What changes"):
//   dst[i][c] += sum_j w[i][j] * src[rows[i][j]][c]
// in a fixed j order: one thread per output element (four adjacent elements
// per thread when the row width allows 16-byte access), no atomics.  The j-sum
// runs in fused multiply-adds from a zero accumulator and is added to dst once.
// A row index outside [0, n_src) is skipped, so nothing is read out of bounds,
// and MOE_DEVERR_ROW is OR-ed into the caller's error word (when one is given).
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace moe {

namespace {

// KM > 0 (top_k <= KM): the K row indices and weights are loaded first, then
// all K rows, before the sums, so a thread waits for two round trips instead
// of two per row; the sums run in the same j order either way.
template <bool ACCUM, int KM>
__global__ void __launch_bounds__(256)
k_wrs_vec4(float *__restrict__ dst, const float *__restrict__ src, int n_src,
           const int32_t *__restrict__ rows, const float *__restrict__ w, int n, int K, int d4, int32_t *err) {
  long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)n * d4) return;
  int i = (int)(idx / d4);
  int c4 = (int)(idx - (long)i * d4);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if constexpr (KM > 0) {
    int r[KM];
    float wt[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < K) {
        r[j] = rows[(size_t)i * K + j];
        wt[j] = w[(size_t)i * K + j];
      }
    f32x4_t sv[KM];
#pragma unroll
    for (int j = 0; j < KM; ++j)
      if (j < K && r[j] >= 0 && r[j] < n_src) sv[j] = ((const f32x4_t *)src)[(size_t)r[j] * d4 + c4];
#pragma unroll
    for (int j = 0; j < KM; ++j) {
      if (j >= K) break;
      if (r[j] < 0 || r[j] >= n_src) {
        if (err && c4 == 0) atomicOr(err, MOE_DEVERR_ROW);
        continue;
      }
      acc.x = fmaf(wt[j], sv[j].x, acc.x);
      acc.y = fmaf(wt[j], sv[j].y, acc.y);
      acc.z = fmaf(wt[j], sv[j].z, acc.z);
      acc.w = fmaf(wt[j], sv[j].w, acc.w);
    }
  } else {
    for (int j = 0; j < K; ++j) {
      int r = rows[(size_t)i * K + j];
      float wt = w[(size_t)i * K + j];
      if (r < 0 || r >= n_src) {
        if (err && c4 == 0) atomicOr(err, MOE_DEVERR_ROW);
        continue;
      }
      f32x4_t s = ((const f32x4_t *)src)[(size_t)r * d4 + c4];
      acc.x = fmaf(wt, s.x, acc.x);
      acc.y = fmaf(wt, s.y, acc.y);
      acc.z = fmaf(wt, s.z, acc.z);
      acc.w = fmaf(wt, s.w, acc.w);
    }
  }
  if (ACCUM) {
    f32x4_t o = ((f32x4_t *)dst)[idx];
    o.x += acc.x;
    o.y += acc.y;
    o.z += acc.z;
    o.w += acc.w;
    ((f32x4_t *)dst)[idx] = o;
  } else {
    ((f32x4_t *)dst)[idx] = acc;
  }
}

template <bool ACCUM>
__global__ void __launch_bounds__(256)
k_wrs_scalar(float *__restrict__ dst, const float *__restrict__ src, int n_src,
             const int32_t *__restrict__ rows, const float *__restrict__ w, int n, int K, int d, int32_t *err) {
  long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)n * d) return;
  int i = (int)(idx / d);
  int c = (int)(idx - (long)i * d);
  float acc = 0.f;
  for (int j = 0; j < K; ++j) {
    int r = rows[(size_t)i * K + j];
    if (r < 0 || r >= n_src) {
      if (err && c == 0) atomicOr(err, MOE_DEVERR_ROW);
      continue;
    }
    acc = fmaf(w[(size_t)i * K + j], src[(size_t)r * d + c], acc);
  }
  if (ACCUM)
    dst[idx] += acc;
  else
    dst[idx] = acc;
}

}  // namespace

hipError_t launch_weighted_row_sum(float *dst, const float *src, int n_src_rows, const int32_t *rows,
                                   const float *weights, int n_tokens, int top_k, int d_model, bool accumulate,
                                   int32_t *error_word, hipStream_t stream) {
  bool vec = (d_model % 4 == 0) && ((uintptr_t)dst % 16 == 0) && ((uintptr_t)src % 16 == 0);
  long elems = (long)n_tokens * (vec ? d_model / 4 : d_model);
  long blocks = (elems + 255) / 256;
  dim3 grid((unsigned)blocks), block(256);
  const bool few = top_k <= 8;
  if (vec && accumulate && few)
    hipLaunchKernelGGL((k_wrs_vec4<true, 8>), grid, block, 0, stream, dst, src, n_src_rows, rows, weights, n_tokens,
                       top_k, d_model / 4, error_word);
  else if (vec && accumulate)
    hipLaunchKernelGGL((k_wrs_vec4<true, 0>), grid, block, 0, stream, dst, src, n_src_rows, rows, weights, n_tokens,
                       top_k, d_model / 4, error_word);
  else if (vec && few)
    hipLaunchKernelGGL((k_wrs_vec4<false, 8>), grid, block, 0, stream, dst, src, n_src_rows, rows, weights, n_tokens,
                       top_k, d_model / 4, error_word);
  else if (vec)
    hipLaunchKernelGGL((k_wrs_vec4<false, 0>), grid, block, 0, stream, dst, src, n_src_rows, rows, weights, n_tokens,
                       top_k, d_model / 4, error_word);
  else if (accumulate)
    hipLaunchKernelGGL(k_wrs_scalar<true>, grid, block, 0, stream, dst, src, n_src_rows, rows, weights,
                       n_tokens, top_k, d_model, error_word);
  else
    hipLaunchKernelGGL(k_wrs_scalar<false>, grid, block, 0, stream, dst, src, n_src_rows, rows, weights,
                       n_tokens, top_k, d_model, error_word);
  return hipGetLastError();
}

namespace {
__global__ void k_error_word_clear(int32_t *word) { *word = 0; }
}  // namespace

hipError_t launch_error_word_clear(int32_t *word, hipStream_t stream) {
  hipLaunchKernelGGL(k_error_word_clear, dim3(1), dim3(1), 0, stream, word);
  return hipGetLastError();
}

}  // namespace moe
