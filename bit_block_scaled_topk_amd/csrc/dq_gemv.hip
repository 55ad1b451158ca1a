// dq_gemv.hip -- decode path: fused NVFP4 dequant + matrix-core GEMV for experts
// with at most 32 rows (gllm PR #91, "Results": the NVFP4 GEMV for experts with
// <= 32 tokens; TensorFold issue #2265, "What ncu shows" / "Proposal": decode
// expert kernels must keep several k-groups of weight loads in flight).
//
// Work item = (expert, CT tiles of 16 output columns).  A workgroup of WAVES
// wavefronts splits K into WAVES contiguous slices; inside a wavefront, lane
// (n = lane%16, q = lane/16) owns output column n and, per iteration, the whole
// 32-element k-group g = g0 + 4*i + q of that column's weight row: one 16-byte
// code load plus two scale bytes.  A chunk's weight loads are all issued before
// any is used, so each lane keeps kNI k-groups in flight.  The 32 codes become
// 4 bf16x8 B operands (exact: a code's value times its block scale fits a bf16
// significand) and feed 4
// MFMA 16x16x32 steps; the A operand holds the same 32 k-values of up to 16
// activation rows, so the MFMA sums the dot product over the group.  The A
// operands of a k-group are loaded once and used for all CT tiles: with one
// tile per workgroup the activation rows would be read once per 16 columns,
// several times the bytes of the weights themselves.
//
// Activations arrive as NT bf16 planes whose sum is the activation: NT = 1 for
// bf16 inputs (exact), NT = 3 for fp32 inputs split hi + mid + lo (24
// significant bits), so the decode path carries fp32 accuracy on bf16 MFMA.
// The WAVES partial sums are reduced in LDS in a fixed order, the global is
// applied once, and the epilogue stores f32, or fuses relu^2 / SwiGLU and writes
// h split into three bf16 planes for the down projection (Glq v0.2.13, "v3b":
// the activation is applied in the final store).
//
// One launch may carry two problems (the shared expert and the routed experts):
// workgroups [0, blocks0) belong to the first.  Loads are unconditional: an
// out-of-range column, row or k-group reads a clamped in-range address and is
// neutralised (its scale is zeroed, or its result is not stored).
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace moe {

namespace {

#ifndef MOE_GEMV_WAVES
#define MOE_GEMV_WAVES 4
#endif
#ifndef MOE_GEMV_CT
#define MOE_GEMV_CT 4
#endif
#ifndef MOE_GEMV_NIT
#define MOE_GEMV_NIT 8
#endif
constexpr int kCT = MOE_GEMV_CT;    // 16-column tiles per workgroup
constexpr int kNIT = MOE_GEMV_NIT;  // weight loads in flight per lane (tiles x k-groups)

struct GemvBatch {
  ProjProblem p[2];
  int count;
};

// The slot-th expert (ascending id) whose row count is in [1, max_rows] and
// whose rows lie inside [0, n_rows); one round of loads: lane l reads the q+1
// offsets of experts [l*q, l*q + q).
__device__ __forceinline__ void find_expert(const int32_t *__restrict__ offsets, int E, int n_rows, int max_rows,
                                            int slot, int lane, int *s_info) {
  constexpr int kMaxQ = MOE_MAX_EXPERTS / 64;
  const int q = (E + 63) >> 6;
  const int eb = lane * q;
  int off[kMaxQ + 1];
  // unpredicated loads of clamped indices: one round trip, no branches
#pragma unroll
  for (int i = 0; i <= kMaxQ; ++i) off[i] = (i <= q) ? offsets[min(eb + i, E)] : 0;
  int local = 0;
  unsigned valid_mask = 0;
#pragma unroll
  for (int i = 0; i < kMaxQ; ++i) {
    if (i < q && eb + i < E) {
      const int r0 = off[i], cnt = off[i + 1] - off[i];
      if (cnt >= 1 && cnt <= max_rows && r0 >= 0 && r0 <= n_rows - cnt) {
        valid_mask |= 1u << i;
        ++local;
      }
    }
  }
  int incl = local;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  const int excl = incl - local;
  const int total = __shfl(incl, 63, 64);
  if (slot >= total) {
    if (lane == 0) s_info[0] = -1;
    return;
  }
  if (slot >= excl && slot < incl) {
    int want = slot - excl;
#pragma unroll
    for (int i = 0; i < kMaxQ; ++i) {
      if ((valid_mask >> i) & 1u) {
        if (want == 0) {
          s_info[0] = eb + i;
          s_info[1] = off[i];
          s_info[2] = off[i + 1] - off[i];
        }
        --want;
      }
    }
  }
}

// PK: the weights are read from their repacked copies (nvfp4_pack_codes and
// nvfp4_pack_scales: [16-row block][128-wide k chunk][64-wide half][16 rows]
// [32 or 4 bytes]),
// where the 16 rows of a round's k-groups are contiguous (one 1 KB piece of
// codes and one 128-byte line of scales per tile) instead of 16 row segments.
template <int WAVES, int MT, int NT, int EPI, int CT, bool PK>
__global__ void __launch_bounds__(64 * WAVES) k_dq_gemv(GemvBatch batch) {
  constexpr int NB = (EPI == EPI_SWIGLU) ? 2 : 1;
  constexpr int kNI = kNIT / CT > 0 ? kNIT / CT : 1;  // k-group iterations per round
  __shared__ int s_info[3];
  __shared__ f32x4_t s_red[WAVES > 1 ? WAVES - 1 : 1][CT][MT][NB][64];

  int bid = blockIdx.x;
  const bool second = batch.count > 1 && bid >= batch.p[0].blocks;
  const ProjProblem p = second ? batch.p[1] : batch.p[0];
  if (second) bid -= batch.p[0].blocks;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int slot = bid / p.n_tiles;  // n_tiles: tile blocks of CT tiles per expert
  const int tile0 = (bid - slot * p.n_tiles) * CT;
  int e, r0, rows;
  if (p.known_rows >= 0) {
    e = 0;
    r0 = 0;
    rows = p.known_rows;
  } else if (p.blocks == p.n_experts * p.n_tiles) {
    // a slot per expert: read its two offsets instead of scanning them all
    e = slot;
    r0 = p.offsets[e];
    rows = p.offsets[e + 1] - r0;
    if (rows < 1 || rows > p.max_rows || r0 < 0 || r0 > p.n_rows - rows) return;  // uniform
  } else {
    if (wave == 0) find_expert(p.offsets, p.n_experts, p.n_rows, p.max_rows, slot, lane, s_info);
    __syncthreads();
    e = s_info[0];
    if (e < 0) return;  // uniform for the workgroup
    r0 = s_info[1];
    rows = s_info[2];
  }

  const int nl = lane & 15, q = lane >> 4;
  // The wavefronts take the k-groups round-robin, an iteration (kNI chunks of
  // 4 groups) each, so that the WAVES wavefronts' loads of a round cover
  // adjacent chunks of each 16-row block: with a contiguous quarter of k per
  // wavefront, a round read 4 x CT separate runs of the weights.
  const int G = p.k >> 5;
  constexpr int kIt = 4 * kNI;  // k-groups of one iteration

  const size_t crow = (size_t)(p.k >> 1), srow = (size_t)(p.k >> 4);
  // this lane's weight row of tile ct: column (tile0 + ct) * 16 + nl (clamped)
  auto wrow_of = [&](int ct, int b, const uint8_t *base, size_t pitch) {
    const int col = min((tile0 + ct) * 16 + nl, p.n_out - 1);
    return base + ((size_t)e * p.n_w + (size_t)col + (size_t)b * p.n_out) * pitch;
  };
  // repacked: slot (block-chunk index x 16 + row in the block) of k-group g of
  // a weight row; the k-group's 16 code bytes and 2 scale bytes sit in half
  // (g >> 1) & 1 of the block-chunk, at byte 16 (g & 1) / 2 (g & 1) of the row
  const int nch = (p.k + 127) >> 7;
  const size_t pk_rows = (size_t)((p.n_w + 15) >> 4) * (size_t)nch * 16;  // 16-row slots of one expert
  auto pk_slot = [&](int ct, int b, int g) -> size_t {
    const int row = min((tile0 + ct) * 16 + nl, p.n_out - 1) + b * p.n_out;
    return (size_t)e * pk_rows + ((size_t)(row >> 4) * nch + (g >> 2)) * 16 + (row & 15);
  };
  const uint16_t *arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = min(mt * 16 + nl, rows - 1);
    const int ar = p.row_map ? max(p.row_map[r0 + m], 0) : r0 + m;
    arow[mt] = p.a + (size_t)ar * p.lda;
  }

  f32x4_t acc[CT][MT][NB];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[ct][mt][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int g0 = wave * kIt; g0 < G; g0 += WAVES * kIt) {
    u32x4_t wq[CT][NB][kNI];
    uint32_t sc[CT][NB][kNI];
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      const int g = g0 + 4 * i + q;
      const int gc = min(g, G - 1);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          if constexpr (PK) {
            const size_t slot = pk_slot(ct, b, gc);
            const size_t bc = slot >> 4, rr = slot & 15, hf = (gc >> 1) & 1, qt = gc & 1;
            wq[ct][b][i] = *(const u32x4_t *)(p.codes_packed + bc * 1024 + hf * 512 + rr * 32 + qt * 16);
            const uint32_t s2 = *(const uint16_t *)(p.scales_packed + bc * 128 + hf * 64 + rr * 4 + qt * 2);
            sc[ct][b][i] = (g < G) ? s2 : 0u;  // a zero scale neutralises a clamped group
            continue;
          }
          wq[ct][b][i] = *(const u32x4_t *)(wrow_of(ct, b, p.codes, crow) + (size_t)gc * 16);
          const uint32_t s2 = *(const uint16_t *)(wrow_of(ct, b, p.scales, srow) + (size_t)gc * 2);
          sc[ct][b][i] = (g < G) ? s2 : 0u;  // a zero scale neutralises a clamped group
        }
    }
#pragma unroll
    for (int i = 0; i < kNI; ++i) {
      if (g0 + 4 * i >= G) break;  // uniform: no group of this iteration is in range
      const int gc = min(g0 + 4 * i + q, G - 1);
      u32x4_t a[MT][NT][4];  // loaded once, used for every tile
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const uint16_t *ap = arow[mt] + (size_t)gc * 32;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int t = 0; t < 4; ++t) a[mt][tt][t] = *(const u32x4_t *)(ap + (size_t)tt * p.plane + 8 * t);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          float s0, s1;
          e4m3x2_to_f32(sc[ct][b][i], s0, s1);
          u32x4_t B[4];
          B[0] = dq8_bf16(wq[ct][b][i][0], s0);
          B[1] = dq8_bf16(wq[ct][b][i][1], s0);
          B[2] = dq8_bf16(wq[ct][b][i][2], s1);
          B[3] = dq8_bf16(wq[ct][b][i][3], s1);
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            if (mt > 0 && rows <= 16 * mt) break;  // uniform
#pragma unroll
            for (int tt = 0; tt < NT; ++tt)
#pragma unroll
              for (int t = 0; t < 4; ++t) acc[ct][mt][b] = mfma16x16x32(a[mt][tt][t], B[t], acc[ct][mt][b]);
          }
        }
    }
  }

  // fixed-order reduction of the WAVES partial sums: slice 0 + 1 + 2 + ...
  if (WAVES > 1) {
    if (wave > 0) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int b = 0; b < NB; ++b) s_red[wave - 1][ct][mt][b][lane] = acc[ct][mt][b];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < WAVES - 1; ++w)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const f32x4_t v = s_red[w][ct][mt][b][lane];
            acc[ct][mt][b].x += v.x;
            acc[ct][mt][b].y += v.y;
            acc[ct][mt][b].z += v.z;
            acc[ct][mt][b].w += v.w;
          }
  }

  // epilogue: lane holds D[m = 16*mt + 4*q + i][col], i = 0..3
  const float gl = p.global[e];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int col = (tile0 + ct) * 16 + nl;
    if (col >= p.n_out) continue;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = mt * 16 + 4 * q + i;
        if (m >= rows) continue;
        const size_t o = (size_t)(r0 + m) * p.ldo + col;
        if (EPI == EPI_F32) {
          p.out_f32[o] = gl * acc[ct][mt][0][i];
        } else {
          float h;
          if (EPI == EPI_RELU2) {
            float u = gl * acc[ct][mt][0][i];
            u = u > 0.f ? u : 0.f;
            h = u * u;
          } else {
            const float a = gl * acc[ct][mt][0][i];
            const float bb = gl * acc[ct][mt][NB - 1][i];
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
hipError_t dispatch_epi(const GemvBatch &b, int epi, dim3 grid, hipStream_t s) {
  dim3 block(64 * WAVES);
  bool pk = true;  // every problem carries both repacked copies
  for (int i = 0; i < b.count; ++i) pk = pk && b.p[i].codes_packed && b.p[i].scales_packed;
  for (int i = 0; i < b.count; ++i)  // the canonical layout is read otherwise
    if (!pk && (!b.p[i].codes || !b.p[i].scales)) return hipErrorInvalidValue;
  switch (epi * 2 + (pk ? 1 : 0)) {
    case EPI_F32 * 2: hipLaunchKernelGGL((k_dq_gemv<WAVES, MT, NT, EPI_F32, kCT, false>), grid, block, 0, s, b); break;
    case EPI_F32 * 2 + 1: hipLaunchKernelGGL((k_dq_gemv<WAVES, MT, NT, EPI_F32, kCT, true>), grid, block, 0, s, b); break;
    case EPI_RELU2 * 2:
      hipLaunchKernelGGL((k_dq_gemv<WAVES, MT, NT, EPI_RELU2, kCT, false>), grid, block, 0, s, b);
      break;
    case EPI_RELU2 * 2 + 1:
      hipLaunchKernelGGL((k_dq_gemv<WAVES, MT, NT, EPI_RELU2, kCT, true>), grid, block, 0, s, b);
      break;
    case EPI_SWIGLU * 2:
      hipLaunchKernelGGL((k_dq_gemv<WAVES, MT, NT, EPI_SWIGLU, kCT, false>), grid, block, 0, s, b);
      break;
    default: hipLaunchKernelGGL((k_dq_gemv<WAVES, MT, NT, EPI_SWIGLU, kCT, true>), grid, block, 0, s, b); break;
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

hipError_t launch_dq_gemv(ProjProblem *probs, const int *max_active, int count, int nt, int epi,
                          hipStream_t stream) {
  GemvBatch b;
  b.count = 0;
  int rows_bound = 0;
  long total = 0;
  for (int i = 0; i < count; ++i) {
    ProjProblem p = probs[i];
    if (p.known_rows >= 0) {
      if (p.known_rows < 1 || p.known_rows > p.max_rows) continue;
    } else if (max_active[i] <= 0 || p.max_rows <= 0) {
      continue;
    }
    p.n_tiles = ((p.n_out + 15) / 16 + kCT - 1) / kCT;  // blocks of kCT tiles
    const int slots = p.known_rows >= 0 ? 1 : max_active[i];
    p.blocks = slots * p.n_tiles;
    const int rb = p.known_rows >= 0 ? p.known_rows : p.max_rows;
    if (rb > rows_bound) rows_bound = rb;
    total += p.blocks;
    b.p[b.count++] = p;
  }
  if (b.count == 0) return hipSuccess;
  if (b.count == 1) b.p[1] = b.p[0];
  dim3 grid((unsigned)total);
  constexpr int W = MOE_GEMV_WAVES;
  if (rows_bound <= 16) {
    if (nt == 1) return dispatch_epi<W, 1, 1>(b, epi, grid, stream);
    return dispatch_epi<W, 1, 3>(b, epi, grid, stream);
  }
  if (nt == 1) return dispatch_epi<W, 2, 1>(b, epi, grid, stream);
  return dispatch_epi<W, 2, 3>(b, epi, grid, stream);
}

}  // namespace moe
