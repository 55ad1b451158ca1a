// router.hip -- the router step before routing, fused with it: logits = x . W_r^T
// on the matrix cores, then top-K and the softmax over the picks (the linked
// PR "perf: cut host overhead from long prefills (routing, matmul scratch)" of
// the gllm #91 page is about this step; routing itself is route_device.hpp).
//
// Workgroup (mt, eg) computes the logits of tokens [16 mt, 16 mt + 16) for
// experts [16 eg, 16 eg + 16): A = 16 token rows of x, B = 16 expert rows of
// W_r (bf16), MFMA 16x16x32 with fp32 accumulation.  Its KS wavefronts split
// the 32-wide k-steps (step s goes to wavefront s % KS) and their partial
// tiles are added in LDS in wavefront order, so the logits do not depend on
// timing.  fp32 activations enter as three bf16 terms (hi + mid + lo, 24
// significant bits), each multiplied exactly.  Small batches use 16
// wavefronts per workgroup so the whole of W_r is in flight at once (one token
// reads 688 KB of router weights at d_model 2688, 128 experts); large batches
// use 4.
//
// The tile is stored with device-coherent stores and counted on the token
// tile's counter once the stores have completed.  The workgroup that brings
// the counter to the number of expert groups resets it (so every call leaves
// the counters at zero) and routes the tile's tokens from the full logits rows,
// read with device-coherent loads: one wavefront per token, exactly as the
// routing kernel does.  No workgroup waits on another.
#include "launch.hpp"
#include "nvfp4_device.hpp"
#include "route_device.hpp"

namespace moe {

namespace {

constexpr int kTileTok = 16, kTileExp = 16;
constexpr int kCntStride = 16;  // one counter per 64 bytes

template <int KS, bool XF32>
__global__ void __launch_bounds__(64 * KS)
k_router_topk(const void *__restrict__ x, int n, int d, const uint16_t *__restrict__ wr, int E, int K,
              int n_eg, float *logits, int32_t *counters, int32_t *__restrict__ ids, float *__restrict__ topk_w) {
  __shared__ f32x4_t s_part[KS][64];
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mt = blockIdx.x / n_eg, eg = blockIdx.x - mt * n_eg;
  const int t0 = mt * kTileTok, e0 = eg * kTileExp;
  const int r = lane & 15, sl = lane >> 4;  // operand row (token / expert) and k-slice of this lane
  const bool a_ok = t0 + r < n, b_ok = e0 + r < E;
  const uint16_t *brow = wr + (size_t)(b_ok ? e0 + r : 0) * d + 8 * sl;
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  const int steps = d / 32;
  if constexpr (XF32) {
    const float *arow = (const float *)x + (size_t)(a_ok ? t0 + r : 0) * d + 8 * sl;
    for (int s = wave; s < steps; s += KS) {
      const u32x4_t b = b_ok ? *(const u32x4_t *)(brow + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
      f32x4_t v0 = {0.f, 0.f, 0.f, 0.f}, v1 = {0.f, 0.f, 0.f, 0.f};
      if (a_ok) {
        v0 = *(const f32x4_t *)(arow + 32 * s);
        v1 = *(const f32x4_t *)(arow + 32 * s + 4);
      }
      u32x4_t hi, mid, lo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h0, m0, l0, h1, m1, l1;
        split3_bf16(i < 2 ? v0[2 * i] : v1[2 * i - 4], h0, m0, l0);
        split3_bf16(i < 2 ? v0[2 * i + 1] : v1[2 * i - 3], h1, m1, l1);
        hi[i] = pack_bf16x2(h0, h1);
        mid[i] = pack_bf16x2(m0, m1);
        lo[i] = pack_bf16x2(l0, l1);
      }
      acc = mfma16x16x32(hi, b, acc);
      acc = mfma16x16x32(mid, b, acc);
      acc = mfma16x16x32(lo, b, acc);
    }
  } else {
    const uint16_t *arow = (const uint16_t *)x + (size_t)(a_ok ? t0 + r : 0) * d + 8 * sl;
#pragma unroll 4
    for (int s = wave; s < steps; s += KS) {
      const u32x4_t a = a_ok ? *(const u32x4_t *)(arow + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
      const u32x4_t b = b_ok ? *(const u32x4_t *)(brow + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
      acc = mfma16x16x32(a, b, acc);
    }
  }
  s_part[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    f32x4_t v = s_part[0][lane];
#pragma unroll
    for (int w = 1; w < KS; ++w) {  // wavefront order
      const f32x4_t o = s_part[w][lane];
      v.x += o.x;
      v.y += o.y;
      v.z += o.z;
      v.w += o.w;
    }
    // lane holds D[token 4 sl + i][expert r]
    const int e = e0 + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * sl + i;
      if (t < n && e < E)
        __hip_atomic_store(logits + (size_t)t * E + e, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the stores have completed
    if (lane == 0) {
      int32_t *cnt = counters + (size_t)mt * kCntStride;
      const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == n_eg - 1;
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
      s_last = last;
    }
  }
  __syncthreads();
  if (!s_last) return;
  // the last expert group of this token tile: route its tokens
  for (int tt = wave; tt < kTileTok; tt += KS) {
    const int t = t0 + tt;
    if (t >= n) break;
    int my_id;
    float my_w;
    route_one_token_any<true>(logits + (size_t)t * E, E, K, lane, my_id, my_w);
    if (lane < K) {
      ids[(size_t)t * K + lane] = my_id;
      topk_w[(size_t)t * K + lane] = my_w;
    }
  }
}

__global__ void k_router_zero(int32_t *w, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) w[i] = 0;
}

}  // namespace

size_t router_counter_bytes(int n_tokens) {
  return (size_t)((n_tokens + kTileTok - 1) / kTileTok) * kCntStride * sizeof(int32_t);
}

hipError_t launch_router_init(int32_t *counters, int n_tokens, hipStream_t stream) {
  const long words = (long)router_counter_bytes(n_tokens) / 4;
  if (words <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_router_zero, dim3((unsigned)((words + 255) / 256)), dim3(256), 0, stream, counters, words);
  return hipGetLastError();
}

hipError_t launch_router_topk(const void *x, bool x_f32, int n_tokens, int d_model, const uint16_t *router_w,
                              int n_experts, int top_k, float *logits, int32_t *counters, int32_t *ids,
                              float *weights, hipStream_t stream) {
  const int n_tiles = (n_tokens + kTileTok - 1) / kTileTok;
  const int n_eg = (n_experts + kTileExp - 1) / kTileExp;
  const long blocks = (long)n_tiles * n_eg;
  // few workgroups: 16 wavefronts each, so the router weights stream through
  // many CUs at once; many: 4 each
  const bool wide = blocks < 512;
  dim3 grid((unsigned)blocks);
#define MOE_ROUTER_LAUNCH(KS, F)                                                                                  \
  hipLaunchKernelGGL((k_router_topk<KS, F>), grid, dim3(64 * KS), 0, stream, x, n_tokens, d_model, router_w,     \
                     n_experts, top_k, n_eg, logits, counters, ids, weights)
  if (wide && x_f32)
    MOE_ROUTER_LAUNCH(16, true);
  else if (wide)
    MOE_ROUTER_LAUNCH(16, false);
  else if (x_f32)
    MOE_ROUTER_LAUNCH(4, true);
  else
    MOE_ROUTER_LAUNCH(4, false);
#undef MOE_ROUTER_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
