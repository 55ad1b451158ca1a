// route_device.hpp -- top-K selection and softmax over the picks for one token,
// computed by one wavefront (used by the routing kernel and by the fused
// route + gather kernel).
//
// Each lane keeps up to PER_LANE of the token's logits in registers (expert
// lane + 64*i).  K rounds of a wave-wide argmax pick the experts in
// descending-logit order, equal logits going to the lower expert index.  Lane j
// ends with slot j's expert and weight w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0),
// the sum taken in slot order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_nvfp4.h"

namespace moe {

__device__ __forceinline__ bool route_beats(float v, int i, float bv, int bi) {
  return (v > bv) || (v == bv && (unsigned)i < (unsigned)bi);
}

template <int PER_LANE = MOE_MAX_EXPERTS / 64>
__device__ __forceinline__ void route_one_token(const float *__restrict__ row, int n_experts, int top_k, int lane,
                                                int &my_id, float &my_w) {
  float v[PER_LANE];
  bool taken[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    int e = lane + i * 64;  // coalesced: consecutive lanes read consecutive experts
    v[i] = (e < n_experts) ? row[e] : 0.0f;
    taken[i] = !(e < n_experts);
  }
  float my_logit = 0.0f;
  my_id = 0;
  for (int j = 0; j < top_k; ++j) {
    float bv = 0.0f;
    int bi = -1;
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) {
      int e = lane + i * 64;
      if (!taken[i] && (bi < 0 || route_beats(v[i], e, bv, bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      float ov = __shfl_xor(bv, off, 64);
      int oi = __shfl_xor(bi, off, 64);
      if (oi >= 0 && (bi < 0 || route_beats(ov, oi, bv, bi))) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
      if (lane + i * 64 == bi) taken[i] = true;
    if (lane == j) {
      my_logit = bv;
      my_id = bi;
    }
  }
  float l0 = __shfl(my_logit, 0, 64);
  float ex = (lane < top_k) ? expf(my_logit - l0) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < top_k; ++j) sum += __shfl(ex, j, 64);  // fixed order j = 0..K-1
  my_w = ex / sum;
}

}  // namespace moe
