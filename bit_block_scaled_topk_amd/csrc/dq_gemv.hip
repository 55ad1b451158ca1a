// dq_gemv.hip -- decode path: fused NVFP4 dequant + matrix-core GEMV for experts
// with at most 32 rows (gllm PR #91, "Results": the NVFP4 GEMV for experts with
// <= 32 tokens; TensorFold issue #2265, "What ncu shows" / "Proposal": decode
// expert kernels must keep several k-groups of weight loads in flight).
//
// Work item = (active expert, 16 output columns).  A workgroup of WAVES
// wavefronts splits K into WAVES contiguous slices; inside a wavefront, lane
// (n = lane%16, q = lane/16) owns output column n and, per iteration, the whole
// 32-element k-group g = g0 + 4*i + q of that column's weight row: one 16-byte
// code load plus two scale bytes.  All of a chunk's weight loads are issued
// before any is used, so each wavefront keeps NI k-groups per lane in flight.
// The 32 codes become 4 bf16x8 B operands (exact: e2m1 * e4m3 has <= 6
// significant bits) and feed 4 MFMA 16x16x32 steps; the A operand holds the
// same 32 k-values of up to 16 activation rows.  Because A and B use the same
// k order, the MFMA sums the dot product over the group.
//
// Activations arrive as NT bf16 planes whose sum is the activation: NT = 1 for
// bf16 inputs (exact), NT = 3 for fp32 inputs split hi + mid + lo (24
// significant bits), so the decode path carries fp32 accuracy on bf16 MFMA.
// Partials of the WAVES slices are reduced in LDS in a fixed order, then the
// global is applied once and the epilogue stores f32, or fuses relu^2 / SwiGLU
// and writes h already split into three bf16 planes for the down projection
// (Glq v0.2.13, "v3b": the activation is applied in the final store).
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace moe {

namespace {

struct GemvArgs {
  const uint16_t *a;  // NT planes of bf16 [rows][lda]
  long plane;         // elements between planes
  long lda;
  const int32_t *offsets;
  int n_experts;
  int n_rows;          // rows of the activation / output buffers
  int max_rows;        // experts with 1..max_rows rows are handled here
  const uint8_t *codes;
  const uint8_t *scales;
  const float *global;
  int n_w;             // weight rows per expert
  int k;
  int n_out;           // output columns
  float *out_f32;      // EPI_F32: [rows][ldo]
  uint16_t *out_h;     // EPI_RELU2/SWIGLU: 3 bf16 planes [rows][ldo]
  long ldo;
  long h_plane;
};

constexpr int kNI = 8;  // k-group iterations whose weight loads are in flight per lane

// The slot-th expert (ascending id) whose row count is in [1, max_rows]; an
// expert whose row range does not lie inside [0, n_rows) is skipped, so a
// malformed offsets array can never send a load or store out of bounds.
__device__ __forceinline__ void find_expert(const int32_t *offsets, int E, int n_rows, int max_rows,
                                            int slot, int lane, int *s_info) {
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    int e = e0 + lane;
    int r0 = 0, cnt = 0;
    if (e < E) {
      r0 = offsets[e];
      cnt = offsets[e + 1] - r0;
    }
    bool flag = cnt >= 1 && cnt <= max_rows && r0 >= 0 && r0 <= n_rows - cnt;
    unsigned long long mask = __ballot(flag);
    int nflags = __popcll(mask);
    if (slot < base + nflags) {
      int pre = __popcll(mask & ((1ull << lane) - 1ull));
      if (flag && pre == slot - base) {
        s_info[0] = e;
        s_info[1] = r0;
        s_info[2] = cnt;
      }
      return;
    }
    base += nflags;
  }
  if (lane == 0) s_info[0] = -1;
}

template <int WAVES, int MT, int NT, int EPI>
__global__ void __launch_bounds__(64 * WAVES) k_dq_gemv(GemvArgs p, int n_tiles) {
  constexpr int NB = (EPI == EPI_SWIGLU) ? 2 : 1;
  __shared__ int s_info[3];
  __shared__ f32x4_t s_red[WAVES > 1 ? WAVES - 1 : 1][MT][NB][64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = blockIdx.x / n_tiles;
  const int tile = blockIdx.x - slot * n_tiles;
  if (wave == 0) find_expert(p.offsets, p.n_experts, p.n_rows, p.max_rows, slot, lane, s_info);
  __syncthreads();
  const int e = s_info[0];
  if (e < 0) return;  // uniform for the workgroup
  const int r0 = s_info[1], rows = s_info[2];

  const int nl = lane & 15, q = lane >> 4;
  const int G = p.k >> 5;
  const int gpw = (G + WAVES - 1) / WAVES;
  const int gb = wave * gpw;
  const int ge = min(G, gb + gpw);
  const int col = tile * 16 + nl;
  const bool col_ok = col < p.n_out;

  const size_t crow = (size_t)(p.k >> 1), srow = (size_t)(p.k >> 4);
  const uint8_t *wrow[NB];
  const uint8_t *sptr[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    size_t wr = (size_t)e * p.n_w + (size_t)(col_ok ? col : 0) + (size_t)b * p.n_out;
    wrow[b] = p.codes + wr * crow;
    sptr[b] = p.scales + wr * srow;
  }

  f32x4_t acc[MT][NB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[mt][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int g0 = gb; g0 < ge; g0 += 4 * kNI) {
    u32x4_t wq[NB][kNI];
    uint32_t sc[NB][kNI];
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const int g = g0 + 4 * i + q;
      const bool ok = col_ok && g < ge;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        wq[b][i] = ok ? *(const u32x4_t *)(wrow[b] + (size_t)g * 16) : u32x4_t{0u, 0u, 0u, 0u};
        sc[b][i] = ok ? (uint32_t)(*(const uint16_t *)(sptr[b] + (size_t)g * 2)) : 0u;
      }
    }
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      if (g0 + 4 * i >= ge) break;  // uniform: no group of this iteration is in range
      const int g = g0 + 4 * i + q;
      // A operands: row m = mt*16 + nl, the 32 k-values of group g, NT planes
      u32x4_t a[MT][NT][4];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int m = mt * 16 + nl;
        const bool aok = (g < ge) && (m < rows);
        const uint16_t *ap = p.a + (size_t)(r0 + (aok ? m : 0)) * p.lda + (size_t)g * 32;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int t = 0; t < 4; ++t)
            a[mt][tt][t] = aok ? *(const u32x4_t *)(ap + (size_t)tt * p.plane + 8 * t)
                               : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float s0 = e4m3_to_f32(sc[b][i] & 0xFFu);
        const float s1 = e4m3_to_f32(sc[b][i] >> 8);
        u32x4_t B[4];
        B[0] = dq8_bf16(wq[b][i][0], s0);
        B[1] = dq8_bf16(wq[b][i][1], s0);
        B[2] = dq8_bf16(wq[b][i][2], s1);
        B[3] = dq8_bf16(wq[b][i][3], s1);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          if (mt > 0 && rows <= 16 * mt) break;  // uniform
#pragma unroll
          for (int tt = 0; tt < NT; ++tt)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[mt][b] = mfma16x16x32(a[mt][tt][t], B[t], acc[mt][b]);
        }
      }
    }
  }

  // fixed-order reduction of the WAVES partial sums: slice 0 + 1 + 2 + ...
  if (WAVES > 1) {
    if (wave > 0) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int b = 0; b < NB; ++b) s_red[wave - 1][mt][b][lane] = acc[mt][b];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < WAVES - 1; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          f32x4_t v = s_red[w][mt][b][lane];
          acc[mt][b].x += v.x;
          acc[mt][b].y += v.y;
          acc[mt][b].z += v.z;
          acc[mt][b].w += v.w;
        }
  }

  // epilogue: lane holds D[m = 16*mt + 4*q + i][col], i = 0..3
  const float gl = p.global[e];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = mt * 16 + 4 * q + i;
      if (!col_ok || m >= rows) continue;
      const size_t o = (size_t)(r0 + m) * p.ldo + col;
      if (EPI == EPI_F32) {
        p.out_f32[o] = gl * acc[mt][0][i];
      } else {
        float h;
        if (EPI == EPI_RELU2) {
          float u = gl * acc[mt][0][i];
          u = u > 0.f ? u : 0.f;
          h = u * u;
        } else {
          float a = gl * acc[mt][0][i];
          float bb = gl * acc[mt][NB - 1][i];
          h = (a / (1.0f + expf(-a))) * bb;
        }
        uint32_t hi, mid, lo;
        split3_bf16(h, hi, mid, lo);
        p.out_h[o] = (uint16_t)hi;
        p.out_h[o + p.h_plane] = (uint16_t)mid;
        p.out_h[o + 2 * p.h_plane] = (uint16_t)lo;
      }
    }
  }
}

// fp32 activations -> three bf16 planes (hi, mid, lo), 4 elements per thread.
__global__ void __launch_bounds__(256)
k_split3(const float *__restrict__ a, long n_elems, uint16_t *__restrict__ planes, long plane) {
  long i = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= n_elems) return;
  f32x4_t v = *(const f32x4_t *)(a + i);
  uint32_t h[4], m[4], l[4];
  split3_bf16(v.x, h[0], m[0], l[0]);
  split3_bf16(v.y, h[1], m[1], l[1]);
  split3_bf16(v.z, h[2], m[2], l[2]);
  split3_bf16(v.w, h[3], m[3], l[3]);
  typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
  *(u32x2_t *)(planes + i) = u32x2_t{pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])};
  *(u32x2_t *)(planes + plane + i) = u32x2_t{pack_bf16x2(m[0], m[1]), pack_bf16x2(m[2], m[3])};
  *(u32x2_t *)(planes + 2 * plane + i) = u32x2_t{pack_bf16x2(l[0], l[1]), pack_bf16x2(l[2], l[3])};
}

template <int WAVES, int MT, int NT>
hipError_t dispatch_epi(const GemvArgs &g, int epi, dim3 grid, hipStream_t s, int n_tiles) {
  dim3 block(64 * WAVES);
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((k_dq_gemv<WAVES, MT, NT, EPI_F32>), grid, block, 0, s, g, n_tiles); break;
    case EPI_RELU2: hipLaunchKernelGGL((k_dq_gemv<WAVES, MT, NT, EPI_RELU2>), grid, block, 0, s, g, n_tiles); break;
    default: hipLaunchKernelGGL((k_dq_gemv<WAVES, MT, NT, EPI_SWIGLU>), grid, block, 0, s, g, n_tiles); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_split3(const float *a, long n_elems, uint16_t *planes, long plane, hipStream_t stream) {
  long threads = (n_elems + 3) / 4;
  long blocks = (threads + 255) / 256;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(k_split3, dim3((unsigned)blocks), dim3(256), 0, stream, a, n_elems, planes, plane);
  return hipGetLastError();
}

hipError_t launch_dq_gemv_planes(const uint16_t *a, int nt, long plane, long lda, const int32_t *offsets,
                                 int n_experts, int n_rows, int max_rows, int max_active, const uint8_t *codes,
                                 const uint8_t *scales, const float *global, int n_w, int k, int n_out,
                                 int epi, float *out_f32, uint16_t *out_h, long ldo, long h_plane,
                                 hipStream_t stream) {
  if (max_active <= 0 || max_rows <= 0) return hipSuccess;
  GemvArgs g;
  g.a = a; g.plane = plane; g.lda = lda; g.offsets = offsets; g.n_experts = n_experts; g.n_rows = n_rows;
  g.max_rows = max_rows; g.codes = codes; g.scales = scales; g.global = global; g.n_w = n_w;
  g.k = k; g.n_out = n_out; g.out_f32 = out_f32; g.out_h = out_h; g.ldo = ldo; g.h_plane = h_plane;
  const int n_tiles = (n_out + 15) / 16;
  dim3 grid((unsigned)((long)max_active * n_tiles));
  constexpr int W = 4;
  if (max_rows <= 16) {
    if (nt == 1) return dispatch_epi<W, 1, 1>(g, epi, grid, stream, n_tiles);
    return dispatch_epi<W, 1, 3>(g, epi, grid, stream, n_tiles);
  }
  if (nt == 1) return dispatch_epi<W, 2, 1>(g, epi, grid, stream, n_tiles);
  return dispatch_epi<W, 2, 3>(g, epi, grid, stream, n_tiles);
}

}  // namespace moe
