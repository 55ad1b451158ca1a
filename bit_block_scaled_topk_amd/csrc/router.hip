// router.hip -- the router step before routing, fused with it: logits = x . W_r^T
// on the matrix cores, then top-K and the softmax over the picks (the linked
// PR "perf: cut host overhead from long prefills (routing, matmul scratch)" of
// the gllm #91 page is about this step; routing itself is route_device.hpp).
//
// Workgroup (mt, eg) computes the logits of tokens [16 mt, 16 mt + 16) for
// experts [16 eg, 16 eg + 16) (or 128 experts and 32 tokens, see NB and MT
// below): A = 16 token rows of x, B = 16 expert rows of W_r (bf16), MFMA
// 16x16x32 with fp32 accumulation.  Its KS wavefronts split the 32-wide
// k-steps into contiguous ranges and their partial tiles are added in LDS in
// wavefront order, so the logits do not depend on timing.  fp32 activations
// enter as three bf16 terms (hi + mid + lo, 24 significant bits), each
// multiplied exactly.  Small batches use 16 wavefronts per workgroup so the
// whole of W_r is in flight at once (one token reads 688 KB of router weights
// at d_model 2688, 128 experts); large batches use 4, or 8 with 32 tokens.
// Every workgroup of a large batch reads all of W_r from L2, so the loads are
// laid out for the vector L1: neighbouring lanes read neighbouring bytes of a
// row, and a lane rotation (ds_bpermute) puts them in the MFMA operand layout.
//
// The tile is stored with device-coherent stores and counted on the token
// tile's counter once the stores have completed.  The workgroup that brings
// the counter to the number of expert groups resets it (so every call leaves
// the counters at zero) and routes the tile's tokens from the full logits rows,
// read with device-coherent loads: one wavefront per token, exactly as the
// routing kernel does.  No workgroup waits on another.
#include <atomic>

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
// weights are then read once per token tile instead of once per 16 x 16 tile.
// MT: 16-token row blocks per workgroup (tile of 16 MT tokens).  Each router
// row a workgroup loads then serves 16 MT tokens; 2 halves the router weights'
// reads once the 16-token tiles outnumber the CUs.
template <int KS, bool XF32, int PER, int NB, int MT>
__global__ void __launch_bounds__(64 * KS)
k_router_topk(const void *__restrict__ x, int n, int d, const uint16_t *__restrict__ wr, int E, int K,
              int n_eg, float *logits, int32_t *counters, int32_t *__restrict__ ids, float *__restrict__ topk_w) {
  constexpr int kTok = kTileTok * MT;
  __shared__ f32x4_t s_part[KS][MT * NB][64];
  __shared__ float s_lg[NB > 1 ? kTok * 16 * NB : 1];  // [token][expert of the group]
  __shared__ int s_last;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mt = blockIdx.x / n_eg, eg = blockIdx.x - mt * n_eg;
  const int t0 = mt * kTok, e0 = eg * kTileExp * NB;
  const int r = lane & 15, sl = lane >> 4;  // MFMA operand row (token / expert) and k-slice of this lane
  // Loads take another lane map: four neighbouring lanes read the 64
  // contiguous bytes of one row's k-step (row cr, 16-byte piece cp), so a load
  // touches 16 64-byte segments in lane order instead of one segment per lane
  // (the vector L1 serves it in a quarter of the accesses); ds_bpermute then
  // hands lane (r, sl) the piece that lane 4 r + sl loaded.
  const int cr = lane >> 2, cp = lane & 3;
  const int src = 4 * (4 * r + sl);  // ds_bpermute takes the source lane's byte address
  auto rot = [&](u32x4_t v) {
    u32x4_t o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)v[q]);
    return o;
  };
  const uint16_t *brow[NB];
  bool b_ok[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    b_ok[j] = e0 + 16 * j + cr < E;
    brow[j] = wr + (size_t)(b_ok[j] ? e0 + 16 * j + cr : 0) * d + 8 * cp;
  }
  f32x4_t acc[MT][NB];
#pragma unroll
  for (int u = 0; u < MT; ++u)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[u][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int steps = d / 32;
  // wavefront w takes the contiguous k-steps [s_lo, s_hi): consecutive steps of
  // a row share its cache lines
  const int s_lo = (int)((long)wave * steps / KS), s_hi = (int)((long)(wave + 1) * steps / KS);
  // kB k-steps per batch: every load of a batch is issued before its MFMAs,
  // so a wavefront waits out one memory round trip per batch, not per step
  // (2 with 32 fp32 token rows, which would not fit 256 registers with 3)
  constexpr int kB = NB > 1 ? (XF32 && MT > 1 ? 2 : 3) : (XF32 ? 4 : 8);
  if constexpr (XF32) {
    // fp32 rows are loaded in the operand's own layout (32 bytes a lane): they
    // are 16 MT of the 16 (MT + NB) rows a k-step reads
    const float *arow[MT];
    bool a_ok[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      a_ok[u] = t0 + 16 * u + r < n;
      arow[u] = (const float *)x + (size_t)(a_ok[u] ? t0 + 16 * u + r : 0) * d + 8 * sl;
    }
    for (int s0 = s_lo; s0 < s_hi; s0 += kB) {
      u32x4_t b[kB][NB];
      f32x4_t v0[kB][MT], v1[kB][MT];
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        const int s = s0 + i;
        const bool in = s < s_hi;
#pragma unroll
        for (int j = 0; j < NB; ++j)
          b[i][j] = (in && b_ok[j]) ? *(const u32x4_t *)(brow[j] + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < MT; ++u) {
          v0[i][u] = (in && a_ok[u]) ? *(const f32x4_t *)(arow[u] + 32 * s) : f32x4_t{0.f, 0.f, 0.f, 0.f};
          v1[i][u] = (in && a_ok[u]) ? *(const f32x4_t *)(arow[u] + 32 * s + 4) : f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
      }
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        if (s0 + i >= s_hi) break;  // uniform
#pragma unroll
        for (int j = 0; j < NB; ++j) b[i][j] = rot(b[i][j]);
#pragma unroll
        for (int u = 0; u < MT; ++u) {
          u32x4_t hi, mid, lo;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            uint32_t h0, m0, l0, h1, m1, l1;
            split3_bf16(q < 2 ? v0[i][u][2 * q] : v1[i][u][2 * q - 4], h0, m0, l0);
            split3_bf16(q < 2 ? v0[i][u][2 * q + 1] : v1[i][u][2 * q - 3], h1, m1, l1);
            hi[q] = pack_bf16x2(h0, h1);
            mid[q] = pack_bf16x2(m0, m1);
            lo[q] = pack_bf16x2(l0, l1);
          }
#pragma unroll
          for (int j = 0; j < NB; ++j) {
            acc[u][j] = mfma16x16x32(hi, b[i][j], acc[u][j]);
            acc[u][j] = mfma16x16x32(mid, b[i][j], acc[u][j]);
            acc[u][j] = mfma16x16x32(lo, b[i][j], acc[u][j]);
          }
        }
      }
    }
  } else {
    const uint16_t *arow[MT];
    bool a_ok[MT];
#pragma unroll
    for (int u = 0; u < MT; ++u) {
      a_ok[u] = t0 + 16 * u + cr < n;
      arow[u] = (const uint16_t *)x + (size_t)(a_ok[u] ? t0 + 16 * u + cr : 0) * d + 8 * cp;
    }
    for (int s0 = s_lo; s0 < s_hi; s0 += kB) {
      u32x4_t a[kB][MT], b[kB][NB];
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        const int s = s0 + i;
        const bool in = s < s_hi;
#pragma unroll
        for (int u = 0; u < MT; ++u)
          a[i][u] = (in && a_ok[u]) ? *(const u32x4_t *)(arow[u] + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < NB; ++j)
          b[i][j] = (in && b_ok[j]) ? *(const u32x4_t *)(brow[j] + 32 * s) : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kB; ++i) {
        if (s0 + i >= s_hi) break;  // uniform
#pragma unroll
        for (int u = 0; u < MT; ++u) a[i][u] = rot(a[i][u]);
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          b[i][j] = rot(b[i][j]);
#pragma unroll
          for (int u = 0; u < MT; ++u) acc[u][j] = mfma16x16x32(a[i][u], b[i][j], acc[u][j]);
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < MT; ++u)
#pragma unroll
    for (int j = 0; j < NB; ++j) s_part[wave][u * NB + j][lane] = acc[u][j];
  __syncthreads();
  // wavefront w adds the partial tiles of blocks w, w + KS, ... (block u NB + j:
  // row block u, expert block j) in wavefront order; lane holds D[token 4 sl +
  // i][expert r] of each block
  const bool route_here = NB > 1 && n_eg == 1;  // every expert of these tokens is in this workgroup
  for (int bk = wave; bk < MT * NB; bk += KS) {
    const int u = bk / NB, j = bk - u * NB;
    f32x4_t v = s_part[0][bk][lane];
#pragma unroll
    for (int w = 1; w < KS; ++w) {
      const f32x4_t o = s_part[w][bk][lane];
      v.x += o.x;
      v.y += o.y;
      v.z += o.z;
      v.w += o.w;
    }
    const int e = e0 + 16 * j + r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tl = 16 * u + 4 * sl + i, t = t0 + tl;
      if (route_here) {
        s_lg[tl * (16 * NB) + 16 * j + r] = v[i];
        if (t < n && e < E) logits[(size_t)t * E + e] = v[i];
      } else if (t < n && e < E) {
        __hip_atomic_store(logits + (size_t)t * E + e, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  constexpr int kTokPerWave = kTok / KS;
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

// compute units of the current device, asked once per device
hipError_t device_cus(int *cus) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidValue;
  int c = dev >= 0 && dev < 64 ? cache[dev].load(std::memory_order_relaxed) : 0;
  if (c <= 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
      return hipErrorInvalidValue;
    if (dev >= 0 && dev < 64) cache[dev].store(c, std::memory_order_relaxed);
  }
  *cus = c;
  return hipSuccess;
}

constexpr int kPairWaves = 8;  // wavefronts of a 32-token workgroup

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
  // weights stream through many CUs at once; many: 128-expert groups (with up
  // to 128 experts, no counter)
  const bool wide = (long)n_tiles * ((n_experts + kTileExp - 1) / kTileExp) < 512;
  const int group = wide ? kTileExp : 8 * kTileExp;
  const int n_eg = (n_experts + group - 1) / group;
  int cus = 0;
  const hipError_t err = device_cus(&cus);
  if (err != hipSuccess) return err;
  // once the 16-token tiles outnumber the CUs, a workgroup takes 32 tokens
  // (8 wavefronts): the router weights are read half as often and no CU holds
  // two workgroups while others idle
  const bool pair = !wide && (long)n_tiles * n_eg > cus;
  const int tiles = pair ? (n_tokens + 2 * kTileTok - 1) / (2 * kTileTok) : n_tiles;
  dim3 grid((unsigned)((long)tiles * n_eg));
#define MOE_ROUTER_LAUNCH(KS, F, PER, NB, MT)                                                                       \
  hipLaunchKernelGGL((k_router_topk<KS, F, PER, NB, MT>), grid, dim3(64 * KS), 0, stream, x, n_tokens, d_model,   \
                     router_w, n_experts, top_k, n_eg, logits, counters, ids, weights)
#define MOE_ROUTER_PER(KS, F, NB, MT)         \
  if (n_experts <= 128)                       \
    MOE_ROUTER_LAUNCH(KS, F, 2, NB, MT);      \
  else if (n_experts <= 256)                  \
    MOE_ROUTER_LAUNCH(KS, F, 4, NB, MT);      \
  else                                        \
    MOE_ROUTER_LAUNCH(KS, F, MOE_MAX_EXPERTS / 64, NB, MT);
  if (wide && x_f32) {
    MOE_ROUTER_PER(16, true, 1, 1)
  } else if (wide) {
    MOE_ROUTER_PER(16, false, 1, 1)
  } else if (pair && x_f32) {
    MOE_ROUTER_PER(kPairWaves, true, 8, 2)
  } else if (pair) {
    MOE_ROUTER_PER(kPairWaves, false, 8, 2)
  } else if (x_f32) {
    MOE_ROUTER_PER(4, true, 8, 1)
  } else {
    MOE_ROUTER_PER(4, false, 8, 1)
  }
#undef MOE_ROUTER_PER
#undef MOE_ROUTER_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
