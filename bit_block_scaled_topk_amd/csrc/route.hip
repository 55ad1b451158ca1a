// route.hip -- top-K routing with a softmax over the picked logits.
//
// The MoE layer routes each token to its topK experts (gllm PR #91, "What the
// profile showed": 128 experts, topK 6) and WeightedRowSum later weights each
// pick ("What changes").  One wavefront per token: each lane keeps its share of
// the token's logits in registers, and K rounds of a wave-wide argmax pick the
// experts in descending-logit order (equal logits: lower expert index first).
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace moe {

namespace {

constexpr int kWave = 64;
constexpr int kMaxPerLane = MOE_MAX_EXPERTS / kWave;  // 16

// (v, i) beats (bv, bi) when v is larger, or equal with a lower index.
__device__ __forceinline__ bool beats(float v, int i, float bv, int bi) {
  return (v > bv) || (v == bv && (unsigned)i < (unsigned)bi);
}

template <int PER_LANE>
__global__ void __launch_bounds__(256) k_route_topk(const float *__restrict__ logits, int n_tokens,
                                                    int n_experts, int top_k,
                                                    int32_t *__restrict__ ids,
                                                    float *__restrict__ weights) {
  const int lane = threadIdx.x & (kWave - 1);
  const int t = blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
  if (t >= n_tokens) return;
  const float *row = logits + (size_t)t * n_experts;

  float v[PER_LANE];
  bool taken[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    int e = lane + i * kWave;  // coalesced: consecutive lanes, consecutive experts
    v[i] = (e < n_experts) ? row[e] : 0.0f;
    taken[i] = !(e < n_experts);
  }

  float my_logit = 0.0f;  // lane j keeps the logit of slot j
  int my_id = 0;
  for (int j = 0; j < top_k; ++j) {
    // lane-local best among the not-yet-taken experts
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      int e = lane + i * kWave;
      if (!taken[i] && (bi < 0 || beats(v[i], e, bv, bi))) {
        bv = v[i];
        bi = e;
      }
    }
    // wave-wide argmax (butterfly; every lane ends with the same winner)
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      float ov = __shfl_xor(bv, off, kWave);
      int oi = __shfl_xor(bi, off, kWave);
      if (oi >= 0 && (bi < 0 || beats(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
      if (lane + i * kWave == bi) taken[i] = true;
    if (lane == j) {
      my_logit = bv;
      my_id = bi;
    }
  }

  // softmax over the picks: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)
  float l0 = __shfl(my_logit, 0, kWave);
  float ex = (lane < top_k) ? expf(my_logit - l0) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < top_k; ++j) sum += __shfl(ex, j, kWave);  // fixed order j = 0..K-1
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_id;
    weights[(size_t)t * top_k + lane] = ex / sum;
  }
}

}  // namespace

hipError_t launch_route_topk(const float *logits, int n_tokens, int n_experts, int top_k,
                             int32_t *ids, float *weights, hipStream_t stream) {
  const int waves_per_block = 4;
  dim3 block(kWave * waves_per_block);
  dim3 grid((n_tokens + waves_per_block - 1) / waves_per_block);
  int per_lane = (n_experts + kWave - 1) / kWave;
  if (per_lane <= 2)
    hipLaunchKernelGGL(k_route_topk<2>, grid, block, 0, stream, logits, n_tokens, n_experts, top_k, ids, weights);
  else if (per_lane <= 4)
    hipLaunchKernelGGL(k_route_topk<4>, grid, block, 0, stream, logits, n_tokens, n_experts, top_k, ids, weights);
  else
    hipLaunchKernelGGL(k_route_topk<kMaxPerLane>, grid, block, 0, stream, logits, n_tokens, n_experts, top_k, ids, weights);
  return hipGetLastError();
}

}  // namespace moe
