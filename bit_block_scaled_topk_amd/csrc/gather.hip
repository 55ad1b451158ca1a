// gather.hip -- the MoE gather (gllm PR #91, "What changes"): a dense buffer of
// n*topK rows holds one row per (token, picked expert) pair, the rows of each
// expert contiguous, and the activations are copied into them with a single
// row lookup.  Rows inside an expert's group are in ascending token order.
//
// Layout without order-dependent atomics: a bitmap bit[e][t] marks that token t
// picked expert e (atomicOr: the result does not depend on the order), prefix
// popcounts of the bitmap give every pick its rank among the expert's earlier
// tokens, and an exclusive scan of the counts gives the group offsets.
//
// Small problems (decode) run in ONE workgroup with the bitmap in LDS, the row
// copy included, and optionally the top-K routing of every token in front of
// it (one launch for route + gather).  Large problems (prefill) use three
// launches: per-256-token chunk bitmaps and counts, then placement with the
// offsets recomputed per workgroup from the count table, then the row copy.
#include "launch.hpp"
#include "nvfp4_device.hpp"
#include "route_device.hpp"

namespace moe {

namespace {

constexpr int kSmallThreads = 1024;
constexpr int kSmallWords = 2048;  // LDS bitmap + prefix words (8 KB) for the one-workgroup path
constexpr int kSmallPicks = 2048;
constexpr long kSmallCopyBytes = 1L << 21;
constexpr int kChunkTokens = 256;  // tokens per chunk on the multi-workgroup path
constexpr int kChunkWords = kChunkTokens / 32;
constexpr int kIdBatch = 8;        // picks per thread loaded together on the multi-workgroup path

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  return v;
}

__device__ __forceinline__ void copy_rows(const void *x, int row_bytes, const int32_t *row_token, long R,
                                          void *xg, long tid, long nthreads) {
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

// Inclusive prefix sum over a wavefront: DPP row shifts inside each 16-lane
// row, then the totals of the earlier rows read with readlane.
__device__ __forceinline__ int wave_scan_incl(int v, int lane) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  return v + (lane >= 16 ? r0 : 0) + (lane >= 32 ? r1 : 0) + (lane >= 48 ? r2 : 0);
}

// Top-K of every token by ranks, with the whole workgroup: logits staged in LDS,
// each (token, expert, part) thread counts how many experts of its part beat
// the expert (larger logit, or equal logit and lower index: a strict total
// order, so ranks are unique), the parts are summed with LDS atomics, and the
// expert of rank j < K becomes slot j.  Softmax over the picks per token, the
// sum in slot order.  Requires n*E <= kRankPairs; used while every thread has
// at most 64 comparisons.
constexpr int kRankPairs = 8192;

__device__ void route_by_rank(const float *__restrict__ logits, int n, int E, int K, float *s_logit, int *s_rank,
                              int *s_sel, int32_t *ids, float *topk_w, int32_t *s_ids) {
  const int tid = threadIdx.x, nthr = blockDim.x;
  const int pairs = n * E;
  for (int i = tid; i < pairs; i += nthr) {
    s_logit[i] = logits[i];
    s_rank[i] = 0;
  }
  for (int i = tid; i < n * K; i += nthr) s_sel[i] = -1;
  __syncthreads();
  const int parts = pairs >= nthr ? 1 : nthr / pairs;
  const int span = (E + parts - 1) / parts;
  for (int i = tid; i < pairs * parts; i += nthr) {
    const int pair = i / parts, part = i - pair * parts;
    const int t = pair / E, a = pair - t * E;
    const float *row = s_logit + t * E;
    const float va = row[a];
    const int b0 = part * span, b1 = min(E, b0 + span);
    int cnt = 0;
    for (int b = b0; b < b1; ++b) {
      const float vb = row[b];
      cnt += (vb > va || (vb == va && b < a)) ? 1 : 0;
    }
    if (parts == 1)
      s_rank[pair] = cnt;
    else if (cnt)
      atomicAdd(&s_rank[pair], cnt);
  }
  __syncthreads();
  for (int i = tid; i < pairs; i += nthr) {
    const int r = s_rank[i];
    if (r < K) {
      const int t = i / E;
      s_sel[t * K + r] = i - t * E;
    }
  }
  __syncthreads();
  for (int t = tid; t < n; t += nthr) {
    const float *row = s_logit + t * E;
    const int e0 = s_sel[t * K];
    const float l0 = e0 >= 0 ? row[e0] : 0.0f;
    float sum = 0.0f;
    for (int j = 0; j < K; ++j) {
      const int e = s_sel[t * K + j];
      sum += e >= 0 ? expf(row[e] - l0) : 0.0f;
    }
    for (int j = 0; j < K; ++j) {
      const int e = s_sel[t * K + j];
      ids[(size_t)t * K + j] = e;
      topk_w[(size_t)t * K + j] = e >= 0 ? expf(row[e] - l0) / sum : 0.0f;
      s_ids[t * K + j] = e;
    }
  }
}

// One workgroup: [routing of every token ->] bitmap in LDS -> ranks -> offsets
// -> placement [-> row copy when xg is given].  Only __syncthreads between
// phases: every phase reads LDS, or global memory this workgroup wrote.
template <bool ROUTE>
__global__ void __launch_bounds__(kSmallThreads)
k_gather_small(const float *__restrict__ logits, float *__restrict__ topk_w, int32_t *ids, int n, int K, int E,
               int32_t *__restrict__ offsets, int32_t *__restrict__ row_token, int32_t *__restrict__ rows,
               const void *x, int row_bytes, void *xg, int32_t *err) {
  __shared__ uint32_t s_bits[kSmallWords];
  __shared__ int32_t s_ids[kSmallPicks];
  __shared__ int32_t s_rt[kSmallPicks];
  __shared__ int32_t s_count[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t s_off[MOE_MAX_EXPERTS + 1];
  __shared__ int32_t s_wave[kSmallThreads / 64];
  __shared__ float s_logit[ROUTE ? kRankPairs : 1];
  __shared__ int32_t s_rank[ROUTE ? kRankPairs : 1];
  __shared__ int32_t s_sel[ROUTE ? kSmallPicks : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nwaves = blockDim.x >> 6;
  const int W = (n + 31) >> 5;
  const int picks = n * K;
  uint32_t *bits = s_bits;
  uint32_t *prefix = s_bits + E * W;

  for (int i = tid; i < E * W; i += blockDim.x) bits[i] = 0u;
  if (ROUTE) {
    // ranks cost E comparisons per (token, expert): for more than a few
    // tokens a wavefront per token (K argmax rounds) is cheaper
    if (n * E <= kRankPairs && (long)n * E * E <= 64L * kSmallThreads) {
      route_by_rank(logits, n, E, K, s_logit, s_rank, s_sel, ids, topk_w, s_ids);
    } else {
      for (int t = wave; t < n; t += nwaves) {
        int my_id;
        float my_w;
        route_one_token_any(logits + (size_t)t * E, E, K, lane, my_id, my_w);
        if (lane < K) {
          ids[(size_t)t * K + lane] = my_id;
          topk_w[(size_t)t * K + lane] = my_w;
          s_ids[t * K + lane] = my_id;
        }
      }
    }
  } else {
    for (int p = tid; p < picks; p += blockDim.x) s_ids[p] = ids[p];
  }
  __syncthreads();

  for (int p = tid; p < picks; p += blockDim.x) {
    const int e = s_ids[p];
    const int t = p / K;
    if (e >= 0 && e < E)
      atomicOr(&bits[e * W + (t >> 5)], 1u << (t & 31));
    else if (err)
      atomicOr(err, MOE_DEVERR_EXPERT_ID);
  }
  __syncthreads();

  // per expert: exclusive prefix popcount over its (few) words, and its count
  for (int e = tid; e < E; e += blockDim.x) {
    int running = 0;
    for (int w = 0; w < W; ++w) {
      prefix[e * W + w] = running;
      running += __popc(bits[e * W + w]);
    }
    s_count[e] = running;
  }
  __syncthreads();

  // exclusive scan of the counts -> group offsets (E <= blockDim)
  {
    const int c = (tid < E) ? s_count[tid] : 0;
    const int incl = wave_scan_incl(c, lane);
    if (lane == 63) s_wave[wave] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_wave[w];
    if (tid < E) s_off[tid] = base + incl - c;
    if (tid == blockDim.x - 1) s_off[E] = base + incl;
  }
  __syncthreads();
  for (int e = tid; e <= E; e += blockDim.x) offsets[e] = s_off[e];

  for (int p = tid; p < picks; p += blockDim.x) {
    const int e = s_ids[p];
    const int t = p / K;
    int32_t r = -1;
    if (e >= 0 && e < E) {
      const int wi = e * W + (t >> 5);
      r = s_off[e] + (int32_t)prefix[wi] + __popc(bits[wi] & ((1u << (t & 31)) - 1u));
      row_token[r] = t;
      s_rt[r] = t;
    }
    rows[p] = r;
  }
  for (int r = s_off[E] + tid; r < picks; r += blockDim.x) {
    row_token[r] = -1;
    s_rt[r] = -1;
  }
  if (xg == nullptr) return;
  __syncthreads();
  // row copy from the LDS copy of row_token, 4 chunks in flight per thread
  const int chunks = row_bytes / 16;
  const int total = picks * chunks;
  for (int i0 = tid; i0 < total; i0 += 4 * blockDim.x) {
    u32x4_t v[4];
    int dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * blockDim.x;
      dst[u] = -1;
      if (i < total) {
        const int r = i / chunks, c = i - r * chunks;
        const int t = s_rt[r];
        if (t >= 0) {
          v[u] = *((const u32x4_t *)((const char *)x + (size_t)t * row_bytes) + c);
          dst[u] = i;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (dst[u] >= 0) {
        const int r = dst[u] / chunks, c = dst[u] - r * chunks;
        *((u32x4_t *)((char *)xg + (size_t)r * row_bytes) + c) = v[u];
      }
    }
  }
}

// Multi-workgroup path, launch 1: chunk c covers tokens [256c, 256c+256): its
// bitmap words for every expert and its per-expert pick counts.
__global__ void __launch_bounds__(256)
k_gather_bits(const int32_t *__restrict__ ids, int n, int K, int E, int W, uint32_t *__restrict__ bitmap,
              int32_t *__restrict__ chunk_count, int n_chunks, int32_t *err) {
  __shared__ uint32_t s_bits[MOE_MAX_EXPERTS * kChunkWords];
  const int c = blockIdx.x, tid = threadIdx.x;
  const int t0 = c * kChunkTokens;
  const int t1 = min(n, t0 + kChunkTokens);
  for (int i = tid; i < E * kChunkWords; i += blockDim.x) s_bits[i] = 0u;
  __syncthreads();
  // the chunk's picks, kIdBatch per thread loaded before any is used (these
  // workgroups are few, one per 256 tokens: each serial round trip shows)
  const long p_end = (long)t1 * K;
  for (long p0 = (long)t0 * K + tid; p0 < p_end; p0 += (long)kIdBatch * blockDim.x) {
    int ev[kIdBatch];
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const long p = p0 + (long)u * blockDim.x;
      ev[u] = p < p_end ? ids[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const long p = p0 + (long)u * blockDim.x;
      if (p >= p_end) break;
      const int e = ev[u], t = (int)(p / K) - t0;
      if (e >= 0 && e < E)
        atomicOr(&s_bits[e * kChunkWords + (t >> 5)], 1u << (t & 31));
      else if (err)
        atomicOr(err, MOE_DEVERR_EXPERT_ID);
    }
  }
  __syncthreads();
  const int w0 = c * kChunkWords;
  for (int i = tid; i < E * kChunkWords; i += blockDim.x) {
    int e = i / kChunkWords, wl = i - e * kChunkWords;
    if (w0 + wl < W) bitmap[(size_t)e * W + w0 + wl] = s_bits[i];
  }
  for (int e = tid; e < E; e += blockDim.x) {
    int cnt = 0;
#pragma unroll
    for (int wl = 0; wl < kChunkWords; ++wl) cnt += __popc(s_bits[e * kChunkWords + wl]);
    chunk_count[(size_t)e * n_chunks + c] = cnt;
  }
}

// Launch 2: per chunk, offsets and the chunk's base per expert from the count
// table (each workgroup recomputes them; workgroup 0 also writes offsets),
// then every pick of the chunk gets its row.
__global__ void __launch_bounds__(256)
k_gather_place(const int32_t *__restrict__ ids, int n, int K, int E, int W,
               const uint32_t *__restrict__ bitmap, const int32_t *__restrict__ chunk_count, int n_chunks,
               int32_t *__restrict__ offsets, int32_t *__restrict__ row_token, int32_t *__restrict__ rows) {
  __shared__ int32_t s_total[MOE_MAX_EXPERTS];
  __shared__ int32_t s_base[MOE_MAX_EXPERTS + 1];
  __shared__ uint32_t s_bits[MOE_MAX_EXPERTS * kChunkWords];
  __shared__ int32_t s_wave_sum[4];
  const int c = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t0 = c * kChunkTokens;
  const int t1 = min(n, t0 + kChunkTokens);
  for (int e = tid; e < E; e += blockDim.x) {
    const int32_t *row = chunk_count + (size_t)e * n_chunks;
    int pre = 0, tot = 0;
    // unrolled, so that the count loads go out in batches (these workgroups
    // are few, one per 256 tokens: each serial round trip shows)
#pragma unroll 8
    for (int cc = 0; cc < n_chunks; ++cc) {
      int v = row[cc];
      tot += v;
      if (cc < c) pre += v;
    }
    s_total[e] = tot;
    s_base[e] = pre;
  }
  const int w0 = c * kChunkWords;
  for (int i = tid; i < E * kChunkWords; i += blockDim.x) {
    int e = i / kChunkWords, wl = i - e * kChunkWords;
    s_bits[i] = (w0 + wl < W) ? bitmap[(size_t)e * W + w0 + wl] : 0u;
  }
  __syncthreads();
  // exclusive scan of s_total over experts: 4 waves x 64 lanes, E <= 1024
  int run = 0;
  if (tid == 0) s_base[E] = 0;
  for (int e0 = 0; e0 < E; e0 += 256) {
    int e = e0 + tid;
    int v = (e < E) ? s_total[e] : 0;
    int incl = wave_incl_scan(v, lane);
    if (lane == 63) s_wave_sum[wave] = incl;
    __syncthreads();
    int before = run;
    for (int w = 0; w < wave; ++w) before += s_wave_sum[w];
    int excl = before + incl - v;
    int chunk_sum = s_wave_sum[0] + s_wave_sum[1] + s_wave_sum[2] + s_wave_sum[3];
    __syncthreads();
    if (e < E) {
      if (c == 0) offsets[e] = excl;
      s_base[e] += excl;  // = offsets[e] + picks of e in earlier chunks
    }
    run += chunk_sum;
  }
  if (c == 0 && tid == 0) offsets[E] = run;
  __syncthreads();
  const long p_end = (long)t1 * K;
  for (long p0 = (long)t0 * K + tid; p0 < p_end; p0 += (long)kIdBatch * blockDim.x) {
    int ev[kIdBatch];
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const long p = p0 + (long)u * blockDim.x;
      ev[u] = p < p_end ? ids[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < kIdBatch; ++u) {
      const long p = p0 + (long)u * blockDim.x;
      if (p >= p_end) break;
      const int e = ev[u], t = (int)(p / K);
      int32_t r = -1;
      if (e >= 0 && e < E) {
        int tl = t - t0;
        int wl = tl >> 5;
        int below = 0;
        for (int ww = 0; ww < wl; ++ww) below += __popc(s_bits[e * kChunkWords + ww]);
        below += __popc(s_bits[e * kChunkWords + wl] & ((1u << (tl & 31)) - 1u));
        r = s_base[e] + below;
        row_token[r] = t;
      }
      rows[p] = r;
    }
  }
  // rows past the valid picks (only when ids were dropped)
  const long picks = (long)n * K;
  for (long r = run + (long)c * blockDim.x + tid; r < picks; r += (long)n_chunks * blockDim.x) row_token[r] = -1;
}

__global__ void __launch_bounds__(256)
k_gather_copy(const void *__restrict__ x, int row_bytes, const int32_t *__restrict__ row_token, long R,
              void *__restrict__ xg) {
  long tid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  copy_rows(x, row_bytes, row_token, R, xg, tid, (long)gridDim.x * blockDim.x);
}

bool small_path(int n, int K, int E, long row_bytes) {
  long W = ((long)n + 31) / 32;
  return 2 * (long)E * W <= kSmallWords && (long)n * K <= kSmallPicks &&
         (long)n * K * row_bytes <= kSmallCopyBytes;
}

}  // namespace

size_t gather_workspace_bytes(int n_tokens, int n_experts) {
  size_t W = ((size_t)n_tokens + 31) / 32;
  size_t n_chunks = ((size_t)n_tokens + kChunkTokens - 1) / kChunkTokens;
  return (size_t)n_experts * W * sizeof(uint32_t) + (size_t)n_experts * n_chunks * sizeof(int32_t) + 512;
}

bool gather_is_single_launch(int n_tokens, int top_k, int n_experts, int elem_bytes, int d_model) {
  return small_path(n_tokens, top_k, n_experts, (long)elem_bytes * d_model);
}

hipError_t launch_gather(const void *x, int elem_bytes, int n_tokens, int d_model, const int32_t *ids, int top_k,
                         int n_experts, void *xg, int32_t *offsets, int32_t *row_token, int32_t *rows,
                         void *workspace, int32_t *err, hipStream_t stream) {
  const int row_bytes = elem_bytes * d_model;
  if (small_path(n_tokens, top_k, n_experts, row_bytes)) {
    hipLaunchKernelGGL(k_gather_small<false>, dim3(1), dim3(kSmallThreads), 0, stream, nullptr, nullptr,
                       const_cast<int32_t *>(ids), n_tokens, top_k, n_experts, offsets, row_token, rows, x,
                       row_bytes, xg, err);
    return hipGetLastError();
  }
  const int W = (n_tokens + 31) / 32;
  const int n_chunks = (n_tokens + kChunkTokens - 1) / kChunkTokens;
  uint32_t *bitmap = (uint32_t *)workspace;
  int32_t *chunk_count = (int32_t *)(bitmap + (size_t)n_experts * W);
  hipLaunchKernelGGL(k_gather_bits, dim3(n_chunks), dim3(256), 0, stream, ids, n_tokens, top_k, n_experts, W, bitmap,
                     chunk_count, n_chunks, err);
  hipError_t he = hipGetLastError();
  if (he != hipSuccess) return he;
  hipLaunchKernelGGL(k_gather_place, dim3(n_chunks), dim3(256), 0, stream, ids, n_tokens, top_k, n_experts, W,
                     bitmap, chunk_count, n_chunks, offsets, row_token, rows);
  he = hipGetLastError();
  if (he != hipSuccess) return he;
  long R = (long)n_tokens * top_k;
  long chunks = R * (row_bytes / 16);
  long blocks = (chunks + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  if (xg == nullptr) return hipSuccess;  // the caller reads x through row_token instead
  hipLaunchKernelGGL(k_gather_copy, dim3((unsigned)blocks), dim3(256), 0, stream, x, row_bytes, row_token, R, xg);
  return hipGetLastError();
}

hipError_t launch_route_gather_small(const float *logits, int n_tokens, int n_experts, int top_k, int32_t *ids,
                                     float *weights, const void *x, int elem_bytes, int d_model, void *xg,
                                     int32_t *offsets, int32_t *row_token, int32_t *rows, hipStream_t stream) {
  hipLaunchKernelGGL(k_gather_small<true>, dim3(1), dim3(kSmallThreads), 0, stream, logits, weights, ids, n_tokens,
                     top_k, n_experts, offsets, row_token, rows, x, elem_bytes * d_model, xg, nullptr);
  return hipGetLastError();
}

}  // namespace moe
