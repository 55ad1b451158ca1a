// route_device.hpp -- top-K selection and softmax over the picks for one token,
// computed by one wavefront (used by the routing kernel and by the fused
// route + gather kernel).
//
// Each lane keeps PER_LANE of the token's logits in registers (expert
// lane + 64*i), each as a 64-bit key ordered like the routing rule.  K rounds
// of a wave-wide maximum pick the experts in descending-logit order, equal
// logits going to the lower expert index.  The maximum runs branch-free on DPP
// moves inside each 16-lane row and two lane swaps across rows, so a round is
// a few dozen instructions.  Lane j ends with slot j's
// expert and weight w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), the sum taken
// in slot order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_nvfp4.h"

namespace moe {

// A candidate (logit v, expert i) as one unsigned 64-bit key whose order is
// the routing order: larger logit first, equal logits to the lower index.  The
// high word maps the float's bits monotonically to unsigned (-0 folded into +0,
// so the two zeros tie as floats do); the low word is ~i.  Key 0 is "nothing"
// (below every real key: a real key's high word is at least 0x007FFFFF, the
// image of -inf).  NaN logits are not supported.
__device__ __forceinline__ uint64_t route_key(float v, int i) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)i;
}
__device__ __forceinline__ int route_key_index(uint64_t k) { return (int)~(uint32_t)k; }
__device__ __forceinline__ float route_key_logit(uint64_t k) {
  uint32_t u = (uint32_t)(k >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

// k <- max(k, the key of the lane DPP_CTRL names), branch-free.
template <int DPP_CTRL>
__device__ __forceinline__ void dpp_max_key(uint64_t &k) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)k, DPP_CTRL, 0xF, 0xF, false);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(k >> 32), DPP_CTRL, 0xF, 0xF, false);
  const uint64_t o = ((uint64_t)hi << 32) | lo;
  k = o > k ? o : k;
}

// Wave-wide maximum key; every lane returns it.  DPP within each 16-lane row
// (quad swaps, half-row and row mirrors), then lane swaps across rows.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t k) {
  dpp_max_key<0xB1>(k);   // quad_perm [1,0,3,2]
  dpp_max_key<0x4E>(k);   // quad_perm [2,3,0,1]
  dpp_max_key<0x141>(k);  // row_half_mirror
  dpp_max_key<0x140>(k);  // row_mirror
#pragma unroll
  for (int m = 16; m <= 32; m <<= 1) {
    const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)k, m, 64);
    const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(k >> 32), m, 64);
    const uint64_t o = ((uint64_t)hi << 32) | lo;
    k = o > k ? o : k;
  }
  return k;
}

// Top-K and softmax from logits already in registers: lane keeps v[i], the
// logit of expert lane + 64 i (entries for experts >= n_experts are ignored).
// PER_LANE may exceed what n_experts needs (the extra entries are not used).
template <int PER_LANE>
__device__ __forceinline__ void route_one_token_keys(const float (&v)[PER_LANE], int n_experts, int top_k, int lane,
                                                     int &my_id, float &my_w) {
  uint64_t key[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + i * 64;
    key[i] = (e < n_experts) ? route_key(v[i], e) : 0ull;
  }
  float my_logit = 0.0f;
  my_id = 0;
  for (int j = 0; j < top_k; ++j) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < PER_LANE; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_key(best);
#pragma unroll
    for (int i = 0; i < PER_LANE; ++i) key[i] = key[i] == best ? 0ull : key[i];  // taken
    if (lane == j) {
      my_logit = route_key_logit(best);
      my_id = route_key_index(best);
    }
  }
  const float l0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_logit), 0));
  const float ex = (lane < top_k) ? expf(my_logit - l0) : 0.0f;
  float sum = 0.0f;
  for (int j = 0; j < top_k; ++j)  // fixed order j = 0..K-1
    sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
  my_w = ex / sum;
}

template <int PER_LANE>
__device__ __forceinline__ void route_one_token(const float *__restrict__ row, int n_experts, int top_k, int lane,
                                                int &my_id, float &my_w) {
  float v[PER_LANE];
#pragma unroll
  for (int i = 0; i < PER_LANE; ++i) {
    const int e = lane + i * 64;  // coalesced: consecutive lanes read consecutive experts
    v[i] = (e < n_experts) ? row[e] : 0.0f;
  }
  route_one_token_keys<PER_LANE>(v, n_experts, top_k, lane, my_id, my_w);
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
