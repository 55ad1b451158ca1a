// dq_gemm.hip -- prefill path: grouped bf16 MFMA GEMM over experts with more
// than gemv_max_rows rows, with the exact NVFP4 -> bf16 unpack fused into the
// weight loader and the fp32 global applied as alpha (gllm PR #91, "bf16 NVFP4
// GEMM (CUDA)": unpack dropping the global, exact in bf16; global in alpha;
// activation rounded to bf16).
//
// One workgroup (4 wavefronts, 2 x 2) computes a 128-row x 128-column tile of
// one expert; the tile list is derived on the device from expert_offsets, so
// the host never reads routing results.  Per 64-wide k step, the activation
// tile (bf16) and the unpacked weight tile (bf16, decoded from 16-byte code
// loads in registers) are staged through LDS; the next step's global loads are
// issued before the current step's MFMAs.  Each wavefront owns a 64 x 64
// sub-tile as 4 x 4 MFMA 16x16x32 accumulators.
#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128, BK = 64, LDK = BK + 8;  // +8 bf16 pad per LDS row

struct GemmBatch {
  ProjProblem p[2];
  int count;
};

// Which expert and which of its 128-row tiles the m-tile index `mt` names.
// Experts whose row range is not inside [0, n_rows) are skipped.
__device__ __forceinline__ void find_tile(const int32_t *offsets, int E, int n_rows, int min_rows, int max_rows,
                                          int mt, int lane, int *s_info) {
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    int e = e0 + lane;
    int r0 = 0, cnt = 0;
    if (e < E) {
      r0 = offsets[e];
      cnt = offsets[e + 1] - r0;
    }
    bool inside = r0 >= 0 && cnt > 0 && r0 <= n_rows - cnt;
    int tiles = (cnt >= min_rows && cnt <= max_rows && inside) ? (cnt + BM - 1) / BM : 0;
    int incl = tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    int total = __shfl(incl, 63, 64);
    if (mt < base + total) {
      int excl = incl - tiles;
      if (tiles > 0 && mt >= base + excl && mt < base + incl) {
        int j = mt - base - excl;
        s_info[0] = e;
        s_info[1] = r0 + j * BM;
        s_info[2] = min(BM, cnt - j * BM);
      }
      return;
    }
    base += total;
  }
  if (lane == 0) s_info[0] = -1;
}

template <int EPI>
__global__ void __launch_bounds__(256) k_dq_gemm(GemmBatch batch) {
  __shared__ int s_info[3];
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * LDK];
  __shared__ __attribute__((aligned(16))) uint16_t sB[BN * LDK];

  int bid = blockIdx.x;
  const bool second = batch.count > 1 && bid >= batch.p[0].blocks;
  const ProjProblem p = second ? batch.p[1] : batch.p[0];
  if (second) bid -= batch.p[0].blocks;
  const int n_ntiles = p.n_tiles;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int mt = bid / n_ntiles;
  const int nt = bid - mt * n_ntiles;
  int e, r0, mrows;
  if (p.known_rows >= 0) {
    e = 0;
    r0 = mt * BM;
    mrows = min(BM, p.known_rows - r0);
    if (mrows <= 0) return;
  } else {
    if (wave == 0) find_tile(p.offsets, p.n_experts, p.n_rows, p.min_rows, p.max_rows, mt, lane, s_info);
    __syncthreads();
    e = s_info[0];
    if (e < 0) return;
    r0 = s_info[1];
    mrows = s_info[2];
  }

  // loader roles: thread -> (tile row, 32-wide half of the k step)
  const int lrow = tid >> 1, lhalf = tid & 1;
  const bool a_ok = lrow < mrows;
  const int a_row = p.row_map ? max(p.row_map[r0 + (a_ok ? lrow : 0)], 0) : r0 + (a_ok ? lrow : 0);
  const uint16_t *a_ptr = p.a + (size_t)a_row * p.lda + lhalf * 32;

  int hcol, wrow_idx;
  if (EPI == EPI_SWIGLU) {
    // LDS row j: wavefront-column wn = j/64, sub-tile s = (j%64)/16: s = 0,1 gate, 2,3 up
    const int wn = lrow >> 6, s = (lrow & 63) >> 4, jj = lrow & 15;
    hcol = nt * 64 + wn * 32 + (s & 1) * 16 + jj;
    wrow_idx = hcol + (s >> 1) * p.n_out;
  } else {
    hcol = nt * BN + lrow;
    wrow_idx = hcol;
  }
  const bool b_ok = hcol < p.n_out;
  const size_t wr = (size_t)e * p.n_w + (size_t)(b_ok ? wrow_idx : 0);
  const uint8_t *c_ptr = p.codes + wr * (size_t)(p.k >> 1) + lhalf * 16;
  const uint8_t *s_ptr = p.scales + wr * (size_t)(p.k >> 4) + lhalf * 2;

  const int nl = lane & 15, q = lane >> 4;
  const int wm = wave >> 1, wn = wave & 1;

  f32x4_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t ra[4];
  u32x4_t rc;
  uint32_t rs;
  auto load = [&](int k0) {
    const bool kin = (k0 + lhalf * 32) < p.k;
#pragma unroll
    for (int t = 0; t < 4; ++t)
      ra[t] = (a_ok && kin) ? *(const u32x4_t *)(a_ptr + k0 + 8 * t) : u32x4_t{0u, 0u, 0u, 0u};
    rc = (b_ok && kin) ? *(const u32x4_t *)(c_ptr + (k0 >> 1)) : u32x4_t{0u, 0u, 0u, 0u};
    rs = (b_ok && kin) ? (uint32_t)(*(const uint16_t *)(s_ptr + (k0 >> 4))) : 0u;
  };

  load(0);
  for (int k0 = 0; k0 < p.k; k0 += BK) {
    // registers -> LDS (weights unpacked exactly to bf16 on the way)
    u32x4_t *da = (u32x4_t *)(sA + lrow * LDK + lhalf * 32);
#pragma unroll
    for (int t = 0; t < 4; ++t) da[t] = ra[t];
    float s0, s1;
    e4m3x2_to_f32(rs, s0, s1);
    u32x4_t *db = (u32x4_t *)(sB + lrow * LDK + lhalf * 32);
    db[0] = dq8_bf16(rc[0], s0);
    db[1] = dq8_bf16(rc[1], s0);
    db[2] = dq8_bf16(rc[2], s1);
    db[3] = dq8_bf16(rc[3], s1);
    __syncthreads();
    if (k0 + BK < p.k) load(k0 + BK);
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      u32x4_t af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *(const u32x4_t *)(sA + (wm * 64 + i * 16 + nl) * LDK + kk * 32 + q * 8);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = *(const u32x4_t *)(sB + (wn * 64 + j * 16 + nl) * LDK + kk * 32 + q * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma16x16x32(af[i], bf[j], acc[i][j]);
    }
    __syncthreads();
  }

  // epilogue: lane holds D[m = wm*64 + i*16 + 4q + r][n = wn*64 + j*16 + nl]
  const float gl = p.global[e];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = wm * 64 + i * 16 + 4 * q + r;
      if (m >= mrows) continue;
      const size_t orow = (size_t)(r0 + m) * p.ldo;
      if (EPI == EPI_SWIGLU) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = nt * 64 + wn * 32 + j * 16 + nl;
          if (col >= p.n_out) continue;
          const float a = gl * acc[i][j][r];
          const float b = gl * acc[i][j + 2][r];
          const float h = (a / (1.0f + expf(-a))) * b;
          p.out_h[orow + col] = (uint16_t)f32_to_bf16_rne(h);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = nt * BN + wn * 64 + j * 16 + nl;
          if (col >= p.n_out) continue;
          float u = gl * acc[i][j][r];
          if (EPI == EPI_F32) {
            p.out_f32[orow + col] = u;
          } else {
            u = u > 0.f ? u : 0.f;
            p.out_h[orow + col] = (uint16_t)f32_to_bf16_rne(u * u);
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_dq_gemm(ProjProblem *probs, int count, int epi, hipStream_t stream) {
  GemmBatch b;
  b.count = 0;
  long total = 0;
  for (int i = 0; i < count; ++i) {
    ProjProblem p = probs[i];
    if (p.n_rows <= 0) continue;
    long m_tiles;
    if (p.known_rows >= 0) {
      if (p.known_rows < p.min_rows || p.known_rows < 1) continue;
      m_tiles = (p.known_rows + BM - 1) / BM;
    } else {
      // sum over big experts of ceil(rows/BM) <= n_rows/BM + (number of big experts)
      const int min_rows = p.min_rows < 1 ? 1 : p.min_rows;
      long big = p.n_rows / min_rows;
      if (big > p.n_experts) big = p.n_experts;
      m_tiles = (p.n_rows + BM - 1) / BM + big;
    }
    p.n_tiles = (epi == EPI_SWIGLU) ? (p.n_out + 63) / 64 : (p.n_out + BN - 1) / BN;
    p.blocks = (int)(m_tiles * p.n_tiles);
    total += p.blocks;
    b.p[b.count++] = p;
  }
  if (b.count == 0) return hipSuccess;
  if (b.count == 1) b.p[1] = b.p[0];
  dim3 grid((unsigned)total), block(256);
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL(k_dq_gemm<EPI_F32>, grid, block, 0, stream, b); break;
    case EPI_RELU2: hipLaunchKernelGGL(k_dq_gemm<EPI_RELU2>, grid, block, 0, stream, b); break;
    default: hipLaunchKernelGGL(k_dq_gemm<EPI_SWIGLU>, grid, block, 0, stream, b); break;
  }
  return hipGetLastError();
}

}  // namespace moe
