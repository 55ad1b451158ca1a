// gather.hip -- the MoE gather: each (token, picked expert) pair gets one row of
// packed n*topK-row buffers grouped by expert, and the activations are copied
// into those rows (gllm PR #91, "What changes": one Embedding gathers the
// inputs).  Rows inside an expert's group are in ascending token order.
//
// Layout without order-dependent atomics: a bitmap bit[e][t] marks that token t
// picked expert e (atomicOr: the result does not depend on the order), the
// per-expert prefix popcounts of the bitmap give every pick its rank among the
// expert's earlier tokens, and an exclusive scan of the counts gives the group
// offsets.  The whole layout runs in one workgroup; for small problems the
// bitmap lives in LDS and the row copy is done by the same workgroup.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace moe {

namespace {

constexpr int kLayoutThreads = 1024;
constexpr int kLdsWords = 4096;             // bitmap + prefix words kept in LDS (32 KB)
constexpr long kInlineCopyBytes = 1 << 18;  // copy inside the layout kernel below this

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ void copy_rows(const void *x, int row_bytes, const int32_t *row_token,
                                          long R, void *xg, long tid, long nthreads) {
  const int chunks = row_bytes / 16;
  const long total = R * chunks;
  for (long i = tid; i < total; i += nthreads) {
    long r = i / chunks;
    int c = (int)(i - r * chunks);
    int t = row_token[r];
    if (t < 0) continue;
    const u32x4_t *src = (const u32x4_t *)((const char *)x + (size_t)t * row_bytes) + c;
    u32x4_t *dst = (u32x4_t *)((char *)xg + (size_t)r * row_bytes) + c;
    *dst = *src;
  }
}

__global__ void __launch_bounds__(kLayoutThreads)
k_gather_layout(const int32_t *__restrict__ ids, int n, int K, int E, int32_t *__restrict__ offsets,
                int32_t *__restrict__ row_token, int32_t *__restrict__ rows, uint32_t *ws_bitmap,
                uint32_t *ws_prefix, int use_lds, const void *x, int row_bytes, void *xg,
                int inline_copy) {
  __shared__ int32_t s_count[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t s_off[MOE_MAX_EXPERTS + 1];
  __shared__ uint32_t s_words[kLdsWords];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int W = (n + 31) >> 5;
  const long picks = (long)n * K;
  uint32_t *bitmap = use_lds ? s_words : ws_bitmap;
  uint32_t *prefix = use_lds ? s_words + (size_t)E * W : ws_prefix;

  // phase 0: clear the bitmap
  for (long i = tid; i < (long)E * W; i += blockDim.x) bitmap[i] = 0u;
  __threadfence();
  __syncthreads();

  // phase 1: mark (expert, token) pairs; invalid ids are dropped
  for (long p = tid; p < picks; p += blockDim.x) {
    int e = ids[p];
    int t = (int)(p / K);
    if (e >= 0 && e < E) atomicOr(&bitmap[(size_t)e * W + (t >> 5)], 1u << (t & 31));
  }
  __threadfence();
  __syncthreads();

  // phase 2: per expert, exclusive prefix popcount over its bitmap words
  for (int e = wave; e < E; e += nwaves) {
    int running = 0;
    for (int w0 = 0; w0 < W; w0 += 64) {
      int w = w0 + lane;
      int c = (w < W) ? __popc(bitmap[(size_t)e * W + w]) : 0;
      int incl = wave_incl_scan(c, lane);
      if (w < W) prefix[(size_t)e * W + w] = running + incl - c;
      running += __shfl(incl, 63, 64);
    }
    if (lane == 0) s_count[e] = running;
  }
  __threadfence();
  __syncthreads();

  // phase 3: exclusive scan of the counts -> group offsets
  if (wave == 0) {
    int running = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      int e = e0 + lane;
      int c = (e < E) ? s_count[e] : 0;
      int incl = wave_incl_scan(c, lane);
      if (e < E) s_off[e] = running + incl - c;
      running += __shfl(incl, 63, 64);
    }
    if (lane == 0) s_off[E] = running;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += blockDim.x) offsets[e] = s_off[e];

  // phase 4: place every pick
  for (long p = tid; p < picks; p += blockDim.x) {
    int e = ids[p];
    int t = (int)(p / K);
    int32_t r = -1;
    if (e >= 0 && e < E) {
      size_t wi = (size_t)e * W + (t >> 5);
      uint32_t below = bitmap[wi] & ((1u << (t & 31)) - 1u);
      r = s_off[e] + (int32_t)prefix[wi] + __popc(below);
      row_token[r] = t;
    }
    rows[p] = r;
  }
  for (long r = s_off[E] + tid; r < picks; r += blockDim.x) row_token[r] = -1;

  if (inline_copy) {
    __threadfence();
    __syncthreads();
    copy_rows(x, row_bytes, row_token, picks, xg, tid, blockDim.x);
  }
}

__global__ void __launch_bounds__(256)
k_gather_copy(const void *__restrict__ x, int row_bytes, const int32_t *__restrict__ row_token,
              long R, void *__restrict__ xg) {
  long tid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  copy_rows(x, row_bytes, row_token, R, xg, tid, (long)gridDim.x * blockDim.x);
}

}  // namespace

size_t gather_workspace_bytes(int n_tokens, int n_experts) {
  size_t W = ((size_t)n_tokens + 31) / 32;
  size_t words = (size_t)n_experts * W;
  return 2 * words * sizeof(uint32_t) + 256;
}

hipError_t launch_gather(const void *x, int elem_bytes, int n_tokens, int d_model, const int32_t *ids,
                         int top_k, int n_experts, void *xg, int32_t *offsets, int32_t *row_token,
                         int32_t *rows, void *workspace, hipStream_t stream) {
  size_t W = ((size_t)n_tokens + 31) / 32;
  size_t words = (size_t)n_experts * W;
  int use_lds = (2 * words <= (size_t)kLdsWords) ? 1 : 0;
  uint32_t *bitmap = (uint32_t *)workspace;
  uint32_t *prefix = bitmap + words;
  int row_bytes = elem_bytes * d_model;
  long R = (long)n_tokens * top_k;
  int inline_copy = (R * row_bytes <= kInlineCopyBytes) ? 1 : 0;
  hipLaunchKernelGGL(k_gather_layout, dim3(1), dim3(kLayoutThreads), 0, stream, ids, n_tokens, top_k,
                     n_experts, offsets, row_token, rows, bitmap, prefix, use_lds, x, row_bytes, xg,
                     inline_copy);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || inline_copy) return err;
  long chunks = R * (row_bytes / 16);
  long blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_gather_copy, dim3((unsigned)blocks), dim3(256), 0, stream, x, row_bytes, row_token,
                     R, xg);
  return hipGetLastError();
}

}  // namespace moe
