// router.hip -- the router step before routing, fused with it: logits = x . W_r^T
// on the matrix cores, then top-K and the softmax over the picks (the linked
// PR "perf: cut host overhead from long prefills (routing, matmul scratch)" of
// the gllm #91 page is about this step; routing itself is route_device.hpp).
//
// Workgroup (mt, eg) computes the logits of tokens [16 mt, 16 mt + 16) for
// experts [16 eg, 16 eg + 16) (or 128 experts, see NB below): A = 16 token
// rows of x, B = 16 expert rows of W_r (bf16), MFMA 16x16x32 with fp32
// accumulation.  Its KS wavefronts split the 32-wide k-steps into contiguous
// ranges and their partial tiles are added in LDS in wavefront order, so the
// logits do not depend on timing.  fp32 activations enter as three bf16 terms (hi + mid + lo, 24
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

// PER: logits per lane when routing (ceil(E / 64), rounded up to 2, 4 or 16).
// NB: 16-expert blocks per workgroup.  NB = 1 (small batches): a token tile's
// experts are spread over many workgroups, found complete by a counter.  NB =
// 8 (large batches): one workgroup holds 128 experts of its tokens, so with up
// to 128 experts it routes them from LDS with no counter at all; the router
// weights are then read once per 16 tokens instead of once per 16 x 16 tile.
template <int KS, bool XF32, int PER, int NB>
__global__ void __launch_bounds__(64 * KS)
k_router_topk(const void *__restrict__ x, int n, int d, const uint16_t *__restrict__ wr, int E, int K,
              int n_eg, float *logits, int32_t *counters, int32_t *__restrict__ ids, float *__restrict__ topk_w) {
  __shared__ f32x4_t s_part[KS][NB][64];
  __shared__ float s_lg[NB > 1 ? kTileTok * 16 * NB : 1];  // [token][expert of the group]
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mt = blockIdx.x / n_eg, eg = blockIdx.x - mt * n_eg;
  const int t0 = mt * kTileTok, e0 = eg * kTileExp * NB;
  const int r = lane & 15, sl = lane >> 4;  // operand row (token / expert) and k-slice of this lane
  const bool a_ok = t0 + r < n;
  const uint16_t *brow[NB];
  bool b_ok[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    b_ok[j] = e0 + 16 * j + r < E;
    brow[j] = wr + (size_t)(b_ok[j] ? e0 + 16 * j + r : 0) * d + 8 * sl;
  }
  f32x4_t acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int steps = d / 32;
  // wavefront w takes the contiguous k-steps [s_lo, s_hi): consecutive steps of
  // a row share its cache lines
  const int s_lo = (int)((long)wave * steps / KS), s_hi = (int)((long)(wave + 1) * steps / KS);
  // kB k-steps per batch: every load of a batch is issued before its MFMAs,
  // so a wavefront waits out one memory round trip per batch, not per step
  constexpr int kB = NB > 1 ? 3 : (XF32 ? 4 : 8);
  if constexpr (XF32) {
    const float *arow = (const float *)x + (size_t)(a_ok ? t0 + r : 0) * d + 8 * sl;
    for (int s0 = s_lo; s0 < s_hi; s0 += kB) {
      u32x4_t b[kB][NB];
      f32x4_t v0[kB], v1[kB];
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        const int s = s0 + i;
        const bool in = s < s_hi;
#pragma unroll
        for (int j = 0; j < NB; ++j)
          b[i][j] = (in && b_ok[j]) ? *(const u32x4_t *)(brow[j] + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
        v0[i] = (in && a_ok) ? *(const f32x4_t *)(arow + 32 * s) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        v1[i] = (in && a_ok) ? *(const f32x4_t *)(arow + 32 * s + 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        if (s0 + i >= s_hi) break;  // uniform
        u32x4_t hi, mid, lo;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t h0, m0, l0, h1, m1, l1;
          split3_bf16(q < 2 ? v0[i][2 * q] : v1[i][2 * q - 4], h0, m0, l0);
          split3_bf16(q < 2 ? v0[i][2 * q + 1] : v1[i][2 * q - 3], h1, m1, l1);
          hi[q] = pack_bf16x2(h0, h1);
          mid[q] = pack_bf16x2(m0, m1);
          lo[q] = pack_bf16x2(l0, l1);
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          acc[j] = mfma16x16x32(hi, b[i][j], acc[j]);
          acc[j] = mfma16x16x32(mid, b[i][j], acc[j]);
          acc[j] = mfma16x16x32(lo, b[i][j], acc[j]);
        }
      }
    }
  } else {
    const uint16_t *arow = (const uint16_t *)x + (size_t)(a_ok ? t0 + r : 0) * d + 8 * sl;
    for (int s0 = s_lo; s0 < s_hi; s0 += kB) {
      u32x4_t a[kB], b[kB][NB];
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        const int s = s0 + i;
        const bool in = s < s_hi;
        a[i] = (in && a_ok) ? *(const u32x4_t *)(arow + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < NB; ++j)
          b[i][j] = (in && b_ok[j]) ? *(const u32x4_t *)(brow[j] + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        if (s0 + i >= s_hi) break;  // uniform
#pragma unroll
        for (int j = 0; j < NB; ++j) acc[j] = mfma16x16x32(a[i], b[i][j], acc[j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NB; ++j) s_part[wave][j][lane] = acc[j];
  __syncthreads();
  // wavefront w adds the partial tiles of expert blocks w, w + KS, ... in
  // wavefront order; lane holds D[token 4 sl + i][expert r] of each block
  const bool route_here = NB > 1 && n_eg == 1;  // every expert of these tokens is in this workgroup
  for (int j = wave; j < NB; j += KS) {
    f32x4_t v = s_part[0][j][lane];
#pragma unroll
    for (int w = 1; w < KS; ++w) {
      const f32x4_t o = s_part[w][j][lane];
      v.x += o.x;
      v.y += o.y;
      v.z += o.z;
      v.w += o.w;
    }
    const int e = e0 + 16 * j + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 4 * sl + i;
      if (route_here) {
        s_lg[(4 * sl + i) * (16 * NB) + 16 * j + r] = v[i];
        if (t < n && e < E) logits[(size_t)t * E + e] = v[i];
      } else if (t < n && e < E) {
        __hip_atomic_store(logits + (size_t)t * E + e, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  constexpr int kTokPerWave = kTileTok / KS;
  constexpr int kPer = PER;
  float lv[kTokPerWave][kPer];
  if (route_here) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kTokPerWave; ++u) {
      const int tl = wave + u * KS;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        lv[u][i] = (e < E) ? s_lg[tl * (16 * NB) + e] : 0.0f;
      }
    }
  } else {
    // the tile's logits are counted once stored; the workgroup that completes
    // its token tile's count routes the tile
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wavefront's stores have completed
    __syncthreads();
    if (tid == 0) {
      int32_t *cnt = counters + (size_t)mt * kCntStride;
      const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == n_eg - 1;
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next call
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    // a wavefront per token; each wavefront requests all of its tokens'
    // logits (device-coherent loads) first
#pragma unroll
    for (int u = 0; u < kTokPerWave; ++u) {
      const int t = t0 + wave + u * KS;
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        const int e = lane + 64 * i;
        lv[u][i] = (t < n && e < E)
                       ? __hip_atomic_load(logits + (size_t)t * E + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                       : 0.0f;
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kTokPerWave; ++u) {
    const int t = t0 + wave + u * KS;
    if (t >= n) break;  // uniform
    int my_id;
    float my_w;
    route_one_token_keys<kPer>(lv[u], E, K, lane, my_id, my_w);
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
  // few tiles: 16-expert groups and 16 wavefronts per workgroup, so the router
  // weights stream through many CUs at once; many: 128-expert groups and 4
  // wavefronts (with up to 128 experts, no counter)
  const bool wide = (long)n_tiles * ((n_experts + kTileExp - 1) / kTileExp) < 512;
  const int group = wide ? kTileExp : 8 * kTileExp;
  const int n_eg = (n_experts + group - 1) / group;
  dim3 grid((unsigned)((long)n_tiles * n_eg));
#define MOE_ROUTER_LAUNCH(KS, F, PER, NB)                                                                          \
  hipLaunchKernelGGL((k_router_topk<KS, F, PER, NB>), grid, dim3(64 * KS), 0, stream, x, n_tokens, d_model,       \
                     router_w, n_experts, top_k, n_eg, logits, counters, ids, weights)
#define MOE_ROUTER_PER(KS, F, NB)             \
  if (n_experts <= 128)                       \
    MOE_ROUTER_LAUNCH(KS, F, 2, NB);          \
  else if (n_experts <= 256)                  \
    MOE_ROUTER_LAUNCH(KS, F, 4, NB);          \
  else                                        \
    MOE_ROUTER_LAUNCH(KS, F, MOE_MAX_EXPERTS / 64, NB);
  if (wide && x_f32) {
    MOE_ROUTER_PER(16, true, 1)
  } else if (wide) {
    MOE_ROUTER_PER(16, false, 1)
  } else if (x_f32) {
    MOE_ROUTER_PER(4, true, 8)
  } else {
    MOE_ROUTER_PER(4, false, 8)
  }
#undef MOE_ROUTER_PER
#undef MOE_ROUTER_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
