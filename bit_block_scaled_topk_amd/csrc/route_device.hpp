// route_device.hpp -- top-K selection and softmax over the picks for one token,
// computed by one wavefront (used by the routing kernel and by the fused
// route + gather kernel).
//
// Each lane keeps PER_LANE of the token's logits in registers (expert
// lane + 64*i).  K rounds of a wave-wide argmax pick the experts in
// descending-logit order, equal logits going to the lower expert index.  The
// argmax runs on DPP moves inside each 16-lane row (quad swaps, half-row and
// row mirrors) and on readlane for the four row winners, so a round costs a
// few dozen instructions and no LDS round trips.  Lane j ends with slot j's
// expert and weight w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), the sum taken
// in slot order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_nvfp4.h"

namespace moe {

__device__ __forceinline__ bool route_beats(float v, int i, float bv, int bi) {
  return (v > bv) || (v == bv && (unsigned)i < (unsigned)bi);
}

// (bv, bi) <- the better of itself and the lane DPP_CTRL names.  An index of -1
// means "nothing"; it never beats a real candidate.
template <int DPP_CTRL>
__device__ __forceinline__ void dpp_take_best(float &bv, int &bi) {
  const float ov = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(bv), DPP_CTRL, 0xF, 0xF, false));
  const int oi = __builtin_amdgcn_update_dpp(-1, bi, DPP_CTRL, 0xF, 0xF, false);
  if (oi >= 0 && (bi < 0 || route_beats(ov, oi, bv, bi))) {
    bv = ov;
    bi = oi;
  }
}

// Wave-wide argmax under route_beats; every lane returns the winner.
__device__ __forceinline__ void wave_argmax(float &bv, int &bi) {
  dpp_take_best<0xB1>(bv, bi);   // quad_perm [1,0,3,2]
  dpp_take_best<0x4E>(bv, bi);   // quad_perm [2,3,0,1]
  dpp_take_best<0x141>(bv, bi);  // row_half_mirror: quads 0 <-> 1 of each half-row
  dpp_take_best<0x140>(bv, bi);  // row_mirror: half-rows 0 <-> 1 of each row
  float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 0));
  int i = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float rv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 16 * r));
    const int ri = __builtin_amdgcn_readlane(bi, 16 * r);
    if (ri >= 0 && (i < 0 || route_beats(rv, ri, v, i))) {
      v = rv;
      i = ri;
    }
  }
  bv = v;
  bi = i;
}

template <int PER_LANE>
__device__ __forceinline__ void route_one_token(const float *__restrict__ row, int n_experts, int top_k, int lane,
                                                int &my_id, float &my_w) {
  float v[PER_LANE];
  bool taken[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + i * 64;  // coalesced: consecutive lanes read consecutive experts
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
      const int e = lane + i * 64;
      if (!taken[i] && (bi < 0 || route_beats(v[i], e, bv, bi))) {
        bv = v[i];
        bi = e;
      }
    }
    wave_argmax(bv, bi);
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i)
      if (lane + i * 64 == bi) taken[i] = true;
    if (lane == j) {
      my_logit = bv;
      my_id = bi;
    }
  }
  const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_logit), 0));
  const float ex = (lane < top_k) ? expf(my_logit - l0) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < top_k; ++j)  // fixed order j = 0..K-1
    sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  my_w = ex / sum;
}

// Dispatch on the number of logits per lane.
__device__ __forceinline__ void route_one_token_any(const float *__restrict__ row, int n_experts, int top_k,
                                                    int lane, int &my_id, float &my_w) {
  if (n_experts <= 128)
    route_one_token<2>(row, n_experts, top_k, lane, my_id, my_w);
  else if (n_experts <= 256)
    route_one_token<4>(row, n_experts, top_k, lane, my_id, my_w);
  else
    route_one_token<MOE_MAX_EXPERTS / 64>(row, n_experts, top_k, lane, my_id, my_w);
}

}  // namespace moe
