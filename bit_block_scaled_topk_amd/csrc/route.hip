// route.hip -- top-K routing with a softmax over the picked logits.
//
// The MoE layer routes each token to its topK experts (gllm PR #91, "What the
// profile showed": 128 experts, topK 6) and WeightedRowSum later weights each
// pick ("What changes").  One wavefront per token (route_device.hpp).
#include "launch.hpp"
#include "route_device.hpp"

namespace moe {

namespace {

template <int PER_LANE>
__global__ void __launch_bounds__(256) k_route_topk(const float *__restrict__ logits, int n_tokens, int n_experts,
                                                    int top_k, int32_t *__restrict__ ids,
                                                    float *__restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x / 64);
  if (t >= n_tokens) return;
  int my_id;
  float my_w;
  route_one_token<PER_LANE>(logits + (size_t)t * n_experts, n_experts, top_k, lane, my_id, my_w);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = my_id;
    weights[(size_t)t * top_k + lane] = my_w;
  }
}

}  // namespace

hipError_t launch_route_topk(const float *logits, int n_tokens, int n_experts, int top_k, int32_t *ids,
                             float *weights, hipStream_t stream) {
  const int waves_per_block = 4;
  dim3 block(64 * waves_per_block);
  dim3 grid((n_tokens + waves_per_block - 1) / waves_per_block);
  int per_lane = (n_experts + 63) / 64;
  if (per_lane <= 2)
    hipLaunchKernelGGL(k_route_topk<2>, grid, block, 0, stream, logits, n_tokens, n_experts, top_k, ids, weights);
  else if (per_lane <= 4)
    hipLaunchKernelGGL(k_route_topk<4>, grid, block, 0, stream, logits, n_tokens, n_experts, top_k, ids, weights);
  else
    hipLaunchKernelGGL(k_route_topk<MOE_MAX_EXPERTS / 64>, grid, block, 0, stream, logits, n_tokens, n_experts,
                       top_k, ids, weights);
  return hipGetLastError();
}

}  // namespace moe
