// dq_gemm.hip -- prefill path: grouped bf16 MFMA GEMM over experts with more
// than gemv_max_rows rows, with the exact NVFP4 -> bf16 unpack fused into the
// weight loader and the fp32 global applied as alpha (gllm PR #91, "bf16 NVFP4
// GEMM (CUDA)": unpack dropping the global, exact in bf16; global in alpha;
// activation rounded to bf16).
//
// Workgroups take 128-row x 256-column tiles of one expert (4 wavefronts, each
// all 128 rows x 64 columns); the tile list is derived on the device from
// expert_offsets, so the host never reads routing results.  The weights are
// decoded in registers straight into MFMA operands (no bf16 copy in LDS or
// HBM); only the activation tile is staged through LDS.
#include <type_traits>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace moe {

namespace {

constexpr int BM = 128, BN = 256, BK = 128;
constexpr int A_BYTES = BM * BK * 2;  // one LDS activation buffer: 128 rows x 256 B, XOR-swizzled
constexpr uint32_t OOB = 0x80000000u; // a buffer offset past every extent: the load returns 0

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kSc1 = 16;  // cache-policy bit of a buffer access: device-coherent (past the per-XCD L2)
static_assert(BN == kGemmF32TileCols, "the combine's column tiles are the f32 GEMM's");

struct GemmBatch {
  ProjProblem p[2];
  int count;
  CombineArgs cmb;
  int32_t *zero;  // words zero[16 i], i < n_zero, set to 0 before the tiles
  long n_zero;
};

// Half of dq8_bf16: code bytes 2h and 2h + 1 of `w` (elements 4h .. 4h + 3)
// into r[2h], r[2h + 1], exactly as dq8_bf16 decodes them.
__device__ __forceinline__ void dq4_bf16(uint32_t w, float scale, int h, u32x4_t &r) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    f32x2_t v;
    switch (2 * h + jj) {  // the byte selector must be an immediate
      case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0); break;
      case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1); break;
      case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2); break;
      default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3); break;
    }
    const uint32_t lo = __float_as_uint(v.x * scale);
    const uint32_t hi = __float_as_uint(v.y * scale);
    r[2 * h + jj] = __builtin_amdgcn_perm(hi, lo, 0x07060302u);  // {hi[31:16], lo[31:16]}
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Wait until this wavefront's loads have landed (register and LDS
// destinations), then a workgroup barrier that orders LDS only.
__device__ __forceinline__ void loads_done_barrier() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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

// One workgroup: a 128-row x 256-column tile of one expert (SwiGLU: 128 h
// columns, i.e. 128 gate + 128 up weight rows).  Wavefront w owns weight
// columns [64w, 64w + 64) of the tile and all 128 rows: 8 x 4 MFMA 16x16x32
// accumulators.
//
// The weights never pass through LDS.  Per 128-wide k chunk, lane (n, q) of a
// wavefront loads 16 bytes of codes -- 32 consecutive k of column n, at
// k = 32q .. 32q + 31 -- and the two e4m3 scales of those 32 k, for each of its
// four 16-column blocks, and decodes them in registers, exactly, into the
// B operands of four MFMA steps s = 0..3 (step s takes k = 32q + 8s .. +7).
// The k order inside a chunk is thereby permuted relative to the MFMA's own
// (slice q = k 8q .. 8q + 7); the activation fragments are read from LDS in
// the same permuted order, so every product still pairs equal k.  Each weight
// element is loaded and decoded once per workgroup.
//
// The activation tile (bf16, 128 rows x 128 k) is double-buffered in LDS and
// filled one chunk ahead by buffer-to-LDS loads: 16-byte cell c of row r sits
// in slot c ^ (r & 15) of the row, so the 16 rows an MFMA fragment reads fall
// in distinct banks, while each load instruction still fills 1 KB of LDS
// contiguously.  Rows past the expert's and k past K load as zero (offsets
// beyond the buffer's extent), so partial tiles need no branches.  One barrier
// per chunk.
//
// SM, how the weights are loaded: 0, one 2-byte scale load per chunk and
// block from the canonical layout; 2, the same from the repacked scales (a
// block's 16 rows of one chunk in one 128-byte line instead of 16 lines); 3,
// as 2 with the codes repacked too (a block's chunk, 2 halves x 16 rows x 32 bytes, is
// 1 KB contiguous: one load reads 8 whole lines instead of 16 half lines); 1 (K a
// multiple of 64, scales 4-byte aligned, no repacked copy): loaded
// for a pair of chunks at a time -- lane (n, q) loads bytes 4q .. 4q + 3 of
// the pair's 16 bytes of its weight row (chunk q >> 1, k-slices 2 (q & 1) and
// 2 (q & 1) + 1) -- and handed to the lanes that use them with ds_bpermute.
// The 2-byte loads, one per chunk and block, were a third of the kernel's
// requests to L2 (each row's 8 bytes on its own cache line); a timing probe
// without any scale loads ran 10-17 % faster.
template <int EPI, int SM>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) k_dq_gemm(GemmBatch batch) {
  constexpr bool SP = SM == 1;
  __shared__ int s_info[3];
  __shared__ __attribute__((aligned(1024))) uint8_t sA[2 * A_BYTES];
  __shared__ int s_last[BM + 1];  // the combine: tokens this tile completes, and their count

  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < batch.n_zero; i += (long)gridDim.x * blockDim.x)
    batch.zero[16 * i] = 0;

  // Tile order.  Workgroups are dealt round-robin over the 8 XCDs.  f32
  // outputs (the down projection): launch order, column tile fastest.  Other
  // outputs (the up projection): m-tile pairs dealt round-robin to the XCDs,
  // all column tiles of a pair on one XCD with the pair's two m-tiles
  // adjacent in time (grid padded to whole rounds of 8 pairs; padding tiles
  // find no rows and return), which measured about 1.5 % faster for the up
  // launch and 2 % slower for the down launch than launch order.  (Grouping
  // each XCD's tiles by m-tile was measured 20-40 % slower.)
  int t = (int)blockIdx.x;
  const bool second = batch.count > 1 && t >= batch.p[0].blocks;
  const ProjProblem p = second ? batch.p[1] : batch.p[0];
  if (second) t -= batch.p[0].blocks;
  const int n_ntiles = p.n_tiles;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int mt, nt;
  if constexpr (EPI != EPI_F32) {
    const int per = 2 * n_ntiles, xcd = t & 7, sl = t >> 3;  // the XCD's sl-th tile
    const int pair = xcd + 8 * (sl / per), ii = sl - (sl / per) * per;
    mt = 2 * pair + (ii & 1);
    nt = ii >> 1;
  } else {
    mt = t / n_ntiles;
    nt = t - mt * n_ntiles;
  }
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
  const int K = p.k;

  // Activation loads: instruction i of wavefront w fills rows 4g .. 4g + 3,
  // g = 8w + i; lane l takes row 4g + l/16, slot l%16, i.e. cell
  // (l%16) ^ (row & 15) of the row.
  uint32_t a_off[8];
  int a_k[8];  // first k of the lane's cell
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * (8 * wave + i) + (lane >> 4);
    const int c = (lane & 15) ^ (r & 15);
    const bool ok = r < mrows;
    const int src = p.row_map ? p.row_map[r0 + (ok ? r : 0)] : r0 + (ok ? r : 0);
    a_off[i] = (ok && src >= 0) ? (uint32_t)src * (uint32_t)(p.lda * 2) + 16u * c : OOB;
    a_k[i] = 8 * c;
  }

  // Weight loads: lane (nl, q), four 16-column blocks j of this wavefront.
  const int nl = lane & 15, q = lane >> 4;
  const size_t e_rows = (size_t)e * p.n_w;
  const uint32_t nch_c = (uint32_t)(K + 127) >> 7, pkc_bytes = (uint32_t)((p.n_w + 15) >> 4) * nch_c * 1024u;
  const __amdgpu_buffer_rsrc_t c_rsrc =
      SM == 3 ? make_rsrc(p.codes_packed + (size_t)e * pkc_bytes, pkc_bytes)
              : make_rsrc(p.codes + e_rows * (size_t)(K >> 1), (uint32_t)p.n_w * (uint32_t)(K >> 1));
  // repacked scales (SM 2): [16-row block][128-wide chunk][64-wide half][16 rows][4 bytes] per expert
  const uint32_t nch = (uint32_t)(K + 127) >> 7, pk_bytes = (uint32_t)((p.n_w + 15) >> 4) * nch * 128u;
  const __amdgpu_buffer_rsrc_t s_rsrc =
      SM >= 2 ? make_rsrc(p.scales_packed + (size_t)e * pk_bytes, pk_bytes)
              : make_rsrc(p.scales + e_rows * (size_t)(K >> 4), (uint32_t)p.n_w * (uint32_t)(K >> 4));
  int wrow0, dj[4];
  if (EPI == EPI_SWIGLU) {  // blocks 0, 1: gate rows; 2, 3: the matching up rows
    wrow0 = nt * 128 + wave * 32 + nl;
#pragma unroll
    for (int j = 0; j < 4; ++j) dj[j] = (j & 1) * 16 + (j >> 1) * p.n_out;
  } else {
    wrow0 = nt * BN + wave * 64 + nl;
#pragma unroll
    for (int j = 0; j < 4; ++j) dj[j] = 16 * j;
  }
  // a column past n_out reads past the expert's rows (zero), or -- for the
  // gate half of a partial SwiGLU tile -- rows whose results are not stored
  const uint32_t c_off0 = (uint32_t)wrow0 * (uint32_t)(K >> 1) + 16u * q;
  const uint32_t s_off0 = SM >= 2 ? 64u * (uint32_t)(q >> 1) + 4u * (uint32_t)nl + 2u * (uint32_t)(q & 1) : (uint32_t)wrow0 * (uint32_t)(K >> 4) + (SP ? 4u : 2u) * q;
  // A wavefront whose output columns all lie past n_out (the last column tile
  // of a ragged width, e.g. 1856 = 7 x 256 + 64) skips its MFMAs and decode:
  // it still fills its share of the activation tile and meets every barrier,
  // and its zero accumulators are never stored.
  const int first_col = (EPI == EPI_SWIGLU) ? nt * 128 + wave * 32 : nt * BN + wave * 64;
  const bool idle = __builtin_amdgcn_readfirstlane(first_col) >= p.n_out;

  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  u32x4_t rc[4];
  // Scales as loaded (SP: a chunk pair) and those of the chunk (pair) in use.
  // The 2-byte loads stay 16-bit until they are used after the next barrier:
  // widened where they are loaded, the compiler waits for the loads just
  // issued (s_waitcnt vmcnt) to zero-extend them.
  uint32_t rs32[4], cs[4];
  uint16_t rs16[4];
  auto load = [&](int k0, uint8_t *abuf, __amdgpu_buffer_rsrc_t a_rsrc, bool with_scales) {
    uint8_t *dst = abuf + wave * 8192;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t off = (k0 + a_k[i] < K) ? a_off[i] + 2u * (uint32_t)k0 : OOB;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void *)(dst + i * 1024), 16, off, 0, 0, 0);
    }
    const bool b_in = k0 + 32 * q < K;
    // SP: this lane's two k-slices of the pair (64 k, so whole or absent)
    const bool s_in = SP ? k0 + 128 * (q >> 1) + 64 * (q & 1) < K : b_in;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t co;
      if constexpr (SM == 3) {  // the block's chunk: 2 halves x 16 rows x 32 bytes, zero past K (no test)
        const uint32_t blk = (uint32_t)((wrow0 - nl + dj[j]) >> 4) * nch_c + (uint32_t)(k0 >> 7);
        co = blk * 1024u + (uint32_t)(q >> 1) * 512u + (uint32_t)nl * 32u + 16u * (uint32_t)(q & 1);
      } else
        co = b_in ? c_off0 + (uint32_t)(dj[j] * (K >> 1)) + (uint32_t)(k0 >> 1) : OOB;
      rc[j] = __builtin_amdgcn_raw_buffer_load_b128(c_rsrc, co, 0, 0);
      uint32_t so;
      if constexpr (SM >= 2)  // this lane's row's 16-row block, chunk k0 / 128 (zero past K: no test)
        so = s_off0 + ((uint32_t)((wrow0 - nl + dj[j]) >> 4) * nch + (uint32_t)(k0 >> 7)) * 128u;
      else
        so = s_in ? s_off0 + (uint32_t)(dj[j] * (K >> 4)) + (uint32_t)(k0 >> 4) : OOB;
      if constexpr (SP) {
        if (with_scales) rs32[j] = __builtin_amdgcn_raw_buffer_load_b32(s_rsrc, so, 0, 0);
      } else {
        rs16[j] = __builtin_amdgcn_raw_buffer_load_b16(s_rsrc, so, 0, 0);
      }
    }
  };

  // LDS byte offset of fragment (i, s) for this lane: row 16 i + nl, cell 4q + s
  uint32_t fa[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) fa[s] = nl * 256 + (((4 * q + s) ^ nl) << 4);

  // One chunk: wait for its operands, request the next chunk's into the other
  // buffer, compute.  `cur` and `nxt` are declared non-aliasing so that the
  // compiler does not make the LDS reads of `cur` wait for the buffer-to-LDS
  // loads into `nxt` (it cannot tell them apart otherwise, and inserts a
  // vmcnt wait that serialises every chunk's loads with its compute).  Across
  // chunks the roles swap; the explicit vmcnt(0) and barrier at the top of
  // each chunk order those accesses.  The activation resource is built here
  // from a restrict pointer so that the loads carry their own alias scope.
  // The expert's global, requested before the first chunk's operands (its
  // wait then comes with theirs).
  const float gl_v = p.global[e];
  // f32 outputs whose 16-byte row pieces are aligned, with no combine, are
  // stored during the last chunk: each fragment's 16 rows as soon as its last
  // MFMAs are issued, so the stores drain under the chunk's remaining MFMAs
  // instead of after them (a wavefront ends only once its stores complete).
  // The resource ends at the tile's last row (rows past it are dropped);
  // columns past n_out take an offset past every extent.
  const bool early = EPI == EPI_F32 && !batch.cmb.on && ((uintptr_t)p.out_f32 & 15) == 0 && p.ldo % 4 == 0 &&
                     p.n_out % 4 == 0 && (size_t)BM * p.ldo * 4 < (1u << 31);
  const __amdgpu_buffer_rsrc_t st_rsrc =
      make_rsrc(early ? p.out_f32 + (size_t)r0 * p.ldo : nullptr, early ? (uint32_t)(mrows * p.ldo * 4) : 0u);
  auto store_frag = [&](int i, float g) {
    if constexpr (EPI == EPI_F32) {
      if (!early) return;
      const int c0 = nt * BN + wave * 64;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = c0 + 16 * j + 4 * q;
        const uint32_t voff = (uint32_t)(16 * i + nl) * (uint32_t)(p.ldo * 4) + (col < p.n_out ? 4u * col : OOB);
        const f32x4_t v = {g * acc[i][j][0], g * acc[i][j][1], g * acc[i][j][2], g * acc[i][j][3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), st_rsrc, voff, 0, 0);
      }
    }
  };

  auto chunk = [&](auto last, const uint8_t *__restrict__ cur, uint8_t *__restrict__ nxt,
                   const void *__restrict__ a_src, int k0) {
    constexpr bool LAST = decltype(last)::value;
    // SP: the chunk's place in its pair; the pair's scales (loaded with the
    // pair's first chunk's codes) stay in rs32 through both of its chunks, and
    // the next pair's are requested only after this copy
    const int par = (k0 / BK) & 1;
    loads_done_barrier();
    const float gs = LAST ? __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, gl_v))) : 0.f;
    u32x4_t cc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cc[j] = rc[j];
      if constexpr (SP)
        cs[j] = rs32[j];
      else
        cs[j] = rs16[j];
    }
    if (k0 + BK < K) load(k0 + BK, nxt, make_rsrc(a_src, p.a_bytes), !SP || par == 1);
    if (idle) return;
    float s0[4], s1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t two = cs[j];
      if constexpr (SP) {  // slice q of chunk PAR: lane 2 PAR + (q >> 1) of this row, half q & 1
        two = (uint32_t)__builtin_amdgcn_ds_bpermute(4 * (nl + 16 * (2 * par + (q >> 1))), (int)two);
        two >>= 16 * (q & 1);
      }
      e4m3x2_to_f32(two, s0[j], s1[j]);
    }
    // Software pipeline over the chunk's 32 groups g = 8 s + i (step s,
    // fragment i): group g issues the LDS read of fragment g + 2, its four
    // MFMAs, and an eighth of the next step's weight decode (half of one
    // block's word); sched_barriers keep that order, so LDS latency and the
    // decode hide under the MFMAs.
    u32x4_t bw[4], bn[4], af[3];
    // A wavefront computing a chunk issues ahead of the CU's others (at the
    // barrier, issuing requests).  It keeps that priority through its tile's
    // end: the f32 outputs are stored inside the last chunk's loop; the bf16
    // outputs after it, which at the default priority lost to the other
    // workgroup's MFMAs (measured: down 3.5-5.5 %, up 2.5 % faster)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int j = 0; j < 4; ++j) bw[j] = dq8_bf16(cc[j][0], s0[j]);
    af[0] = *(const u32x4_t *)(cur + fa[0]);
    af[1] = *(const u32x4_t *)(cur + fa[0] + 4096);
#pragma unroll
    for (int g = 0; g < 32; ++g) {
      const int st = g >> 3, i = g & 7;
      if (g + 2 < 32) {
        const int g2 = g + 2;
        af[g2 % 3] = *(const u32x4_t *)(cur + fa[g2 >> 3] + (g2 & 7) * 4096);
      }
      // f32 outputs: weights as the MFMA's A operand and activations as its
      // B, so the product comes out transposed and each lane holds four
      // consecutive columns of one row (16-byte output stores)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = EPI == EPI_F32 ? mfma16x16x32(bw[j], af[g % 3], acc[i][j]) : mfma16x16x32(af[g % 3], bw[j], acc[i][j]);
      if (st < 3) dq4_bf16(cc[i >> 1][st + 1], st + 1 < 2 ? s0[i >> 1] : s1[i >> 1], i & 1, bn[i >> 1]);
      if (st < 3 && i == 7) {
#pragma unroll
        for (int j = 0; j < 4; ++j) bw[j] = bn[j];
      }
      if constexpr (LAST)
        if (st == 3 && i > 0) store_frag(i - 1, gs);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (EPI == EPI_F32 || !LAST) __builtin_amdgcn_s_setprio(0);
    if constexpr (LAST) store_frag(7, gs);
  };

  load(0, sA, make_rsrc(p.a, p.a_bytes), true);
  int k0 = 0, buf = 0;
  for (; k0 + BK < K; k0 += BK, buf ^= 1)
    chunk(std::false_type{}, sA + buf * A_BYTES, sA + (buf ^ 1) * A_BYTES, p.a, k0);
  chunk(std::true_type{}, sA + buf * A_BYTES, sA + (buf ^ 1) * A_BYTES, p.a, k0);
  if (early) return;

  // Epilogue.  f32 outputs (transposed product): lane holds D[m = 16 i + nl]
  // [column 16 j + 4 q + r of the wavefront], r = 0..3, written with one
  // 16-byte store per (i, j); four 4-byte element stores per lane, as the
  // other order gives, cost the down projection about 9 % of its time.  The
  // aligned case without the combine has stored them during the last chunk.
  // Other outputs: lane holds D[m = 16 i + 4 q + r][column 16 j + nl of the
  // wavefront].  A bf16 h tile is staged in LDS (the activation buffers are
  // free now) and written back as whole rows with 16-byte stores: 2-byte
  // element stores of 16-column row pieces cost the up projection about a
  // quarter of its time.  Both take 16-byte aligned rows whose width n_out is
  // a whole number of 16-byte chunks; other outputs get element stores.
  const float gl = gl_v;
  auto value = [&](int i, int j, int r) -> float {  // the output of accumulator (i, j, r)
    if (EPI == EPI_F32) return gl * acc[i][j][r];
    if (EPI == EPI_SWIGLU) {
      const float a = gl * acc[i][j][r];
      const float b = gl * acc[i][j + 2][r];
      return (a / (1.0f + expf(-a))) * b;
    }
    float u = gl * acc[i][j][r];
    u = u > 0.f ? u : 0.f;
    return u * u;
  };
  constexpr int JN = (EPI == EPI_SWIGLU) ? 2 : 4;      // output column blocks per wavefront
  constexpr int HC = (EPI == EPI_SWIGLU) ? 128 : BN;   // output columns of the tile
  constexpr int EB = (EPI == EPI_F32) ? 4 : 2;         // output element bytes
  constexpr int PER = 16 / EB;                         // elements per 16-byte chunk
  const uintptr_t obase = EPI == EPI_F32 ? (uintptr_t)p.out_f32 : (uintptr_t)p.out_h;
  if constexpr (EPI == EPI_F32) {
    const bool aligned = (((uintptr_t)p.out_f32 | (uintptr_t)(p.ldo * 4)) & 15) == 0 && p.n_out % 4 == 0;
    const int c0 = nt * BN + wave * 64;  // first output column of this wavefront
    const CombineArgs &cmb = batch.cmb;
    // the combine stores the tile device-coherently (the host only fuses it
    // with aligned outputs under 2 GiB)
    const __amdgpu_buffer_rsrc_t o_rsrc =
        make_rsrc(p.out_f32, cmb.on ? (uint32_t)((size_t)p.n_rows * p.ldo * 4) : 0u);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int m = 16 * i + nl;
      if (m >= mrows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = c0 + 16 * j + 4 * q;  // a multiple of 4
        if (col >= p.n_out) continue;
        const size_t o = (size_t)(r0 + m) * p.ldo + col;
        if (aligned) {  // n_out % 4 == 0: all four columns are in range
          f32x4_t v;
          v.x = value(i, j, 0);
          v.y = value(i, j, 1);
          v.z = value(i, j, 2);
          v.w = value(i, j, 3);
          if (cmb.on)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), o_rsrc, (uint32_t)(o * 4), 0,
                                                   kSc1);
          else
            *(f32x4_t *)(p.out_f32 + o) = v;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (col + r < p.n_out) p.out_f32[o + r] = value(i, j, r);
        }
      }
    }
    if (!cmb.on) return;
    // Count this tile's rows for their tokens once every store of the
    // workgroup has completed; collect the tokens whose count is complete.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    if (tid == 0) s_last[BM] = 0;
    __syncthreads();
    if (tid < mrows) {
      const int t = p.known_rows >= 0 ? r0 + tid : cmb.row_token[r0 + tid];
      int target = 1;  // the shared expert's row
      for (int j = 0; j < cmb.K; ++j) {
        const int ej = cmb.ids[(size_t)t * cmb.K + j];
        target += (cmb.offsets[ej + 1] - cmb.offsets[ej]) > cmb.gmax ? 1 : 0;
      }
      int32_t *ctr = cmb.counters + ((size_t)t * cmb.n_ct + nt) * 16;
      const int old = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (old + 1 == target) s_last[atomicAdd(&s_last[BM], 1)] = t;
    }
    __syncthreads();
    // out[t][c..c+3] = out + sum_j w_j * yg[rows[t][j]] for the tile's 256
    // columns: four tokens at a time, 64 threads x 4 columns each
    const int n_last = s_last[BM];
    const __amdgpu_buffer_rsrc_t y_rsrc = make_rsrc(cmb.yg, (uint32_t)((size_t)cmb.n * cmb.K * cmb.d * 4));
    const __amdgpu_buffer_rsrc_t s_rsrc = make_rsrc(cmb.out, (uint32_t)((size_t)cmb.n * cmb.d * 4));
    const int c = nt * BN + 4 * lane;
    for (int li = wave; li < n_last; li += 4) {
      const int t = s_last[li];
      if (c >= cmb.d) continue;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < cmb.K; ++j) {
        const int r = cmb.rows[(size_t)t * cmb.K + j];
        const float wt = cmb.w[(size_t)t * cmb.K + j];
        const f32x4_t y = __builtin_bit_cast(
            f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(y_rsrc, (uint32_t)(((size_t)r * cmb.d + c) * 4), 0, kSc1));
        acc.x = fmaf(wt, y.x, acc.x);
        acc.y = fmaf(wt, y.y, acc.y);
        acc.z = fmaf(wt, y.z, acc.z);
        acc.w = fmaf(wt, y.w, acc.w);
      }
      f32x4_t o = __builtin_bit_cast(
          f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(s_rsrc, (uint32_t)(((size_t)t * cmb.d + c) * 4), 0, kSc1));
      o.x += acc.x;
      o.y += acc.y;
      o.z += acc.z;
      o.w += acc.w;
      *(f32x4_t *)(cmb.out + (size_t)t * cmb.d + c) = o;
    }
  } else {
    const bool vec = ((obase | (uintptr_t)(p.ldo * EB)) & 15) == 0 && p.n_out % PER == 0;
    const int c0 = nt * HC + wave * (16 * JN);  // first output column of this wavefront
    if (!vec) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = 16 * i + 4 * q + r;
          if (m >= mrows) continue;
#pragma unroll
          for (int j = 0; j < JN; ++j) {
            const int col = c0 + 16 * j + nl;
            if (col >= p.n_out) continue;
            p.out_h[(size_t)(r0 + m) * p.ldo + col] = (uint16_t)f32_to_bf16_rne(value(i, j, r));
          }
        }
      return;
    }
    // the 64 KB activation buffers hold the whole bf16 tile
    static_assert(BM * HC * EB <= 2 * A_BYTES, "the staged tile fits the activation buffers");
    __syncthreads();  // every wavefront is done reading the activation buffers
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ml = 16 * i + 4 * q + r;
#pragma unroll
        for (int j = 0; j < JN; ++j) {
          const int cl = wave * (16 * JN) + 16 * j + nl;
          ((uint16_t *)sA)[ml * HC + cl] = (uint16_t)f32_to_bf16_rne(value(i, j, r));
        }
      }
    __syncthreads();
    constexpr int CPR = HC / PER;  // 16-byte chunks per row
    for (int c = tid; c < BM * CPR; c += 256) {
      const int ml = c / CPR, ch = c - ml * CPR;
      const int col = nt * HC + PER * ch;
      if (ml < mrows && col < p.n_out)
        *(u32x4_t *)(obase + ((size_t)(r0 + ml) * p.ldo + col) * EB) = *(const u32x4_t *)(sA + (ml * CPR + ch) * 16);
    }
  }
}

}  // namespace

hipError_t launch_dq_gemm(ProjProblem *probs, int count, int epi, hipStream_t stream, const CombineArgs *combine,
                          int32_t *zero_counters, long n_zero) {
  GemmBatch b;
  b.count = 0;
  b.cmb = CombineArgs{};
  if (combine && combine->on) {
    if (epi != EPI_F32) return hipErrorInvalidValue;
    b.cmb = *combine;
  }
  b.zero = zero_counters;
  b.n_zero = zero_counters ? n_zero : 0;
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
    // the kernel addresses a (plane 0) and one expert's codes and scales with
    // 32-bit buffer offsets, and marks skipped loads with offsets >= 2^31
    const long a_bytes = p.a_rows * p.lda * 2;
    if (a_bytes >= (1L << 31) || (long)p.n_w * (p.k >> 1) >= (1L << 31)) return hipErrorInvalidValue;
    p.a_bytes = (uint32_t)a_bytes;
    p.n_tiles = (epi == EPI_SWIGLU) ? (p.n_out + 127) / 128 : (p.n_out + BN - 1) / BN;
    // up projections: whole rounds of 8 m-tile pairs (see the kernel's tile order)
    p.blocks = epi != EPI_F32 ? (int)(16 * ((m_tiles + 15) / 16) * p.n_tiles) : (int)(m_tiles * p.n_tiles);
    total += p.blocks;
    b.p[b.count++] = p;
  }
  if (b.count == 0) return hipSuccess;
  if (b.count == 1) b.p[1] = b.p[0];
  // the repacked scales when every problem has them and whole 16-row blocks
  // (SwiGLU: its gate and up halves too); else a chunk pair of scales at a
  // time when every problem's k is a multiple of 64 and its scales are 4-byte
  // aligned; else one chunk's at a time
  bool pk = true, sp = true;
  for (int i = 0; i < b.count; ++i) {
    const ProjProblem &q = b.p[i];
    pk = pk && q.scales_packed != nullptr && q.n_w % 16 == 0 && (epi != EPI_SWIGLU || q.n_out % 16 == 0);
    sp = sp && q.k % 64 == 0 && ((uintptr_t)q.scales & 3) == 0;
  }
  bool pc = pk;
  for (int i = 0; i < b.count; ++i) pc = pc && b.p[i].codes_packed != nullptr;
  const int sm = pc ? 3 : pk ? 2 : sp ? 1 : 0;
  for (int i = 0; i < b.count; ++i)  // modes 0-2 read the canonical codes (and 0-1 the canonical scales)
    if (sm != 3 && (!b.p[i].codes || (sm < 2 && !b.p[i].scales))) return hipErrorInvalidValue;
  dim3 grid((unsigned)total), block(256);
  switch (epi * 4 + sm) {
#define MOE_GEMM_CASE(E, M) \
  case E * 4 + M: hipLaunchKernelGGL((k_dq_gemm<E, M>), grid, block, 0, stream, b); break;
    MOE_GEMM_CASE(EPI_F32, 0) MOE_GEMM_CASE(EPI_F32, 1) MOE_GEMM_CASE(EPI_F32, 2) MOE_GEMM_CASE(EPI_F32, 3)
    MOE_GEMM_CASE(EPI_RELU2, 0) MOE_GEMM_CASE(EPI_RELU2, 1) MOE_GEMM_CASE(EPI_RELU2, 2) MOE_GEMM_CASE(EPI_RELU2, 3)
    MOE_GEMM_CASE(EPI_SWIGLU, 0) MOE_GEMM_CASE(EPI_SWIGLU, 1) MOE_GEMM_CASE(EPI_SWIGLU, 2) MOE_GEMM_CASE(EPI_SWIGLU, 3)
#undef MOE_GEMM_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// One 4-byte unit u = (((e nrb + b) nch + c) 2 + h) 16 + r of the repacked
// scales per thread: row 16 b + r of expert e, bytes 8 c + 4 h .. + 3 of its kb
// scale bytes (the scales of k 128 c + 64 h .. + 63; zero past the row count or
// past kb).
__global__ void __launch_bounds__(256) k_pack_scales(const uint8_t *__restrict__ s, int rows, int kb, int nrb, int nch,
                                                     long units, uint8_t *__restrict__ dst) {
  const long u = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  const int r = (int)(u & 15);
  const int h = (int)((u >> 4) & 1);
  long t = u >> 5;
  const int c = (int)(t % nch);
  t /= nch;
  const int blk = (int)(t % nrb);
  const long e = t / nrb;
  const int row = 16 * blk + r, col = 8 * c + 4 * h;
  uint32_t w = 0u;
  if (row < rows) {
    const uint8_t *src = s + (e * rows + row) * (long)kb + col;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (col + i < kb) w |= (uint32_t)src[i] << (8 * i);
  }
  ((uint32_t *)dst)[u] = w;
}

long packed_scales_bytes(long n_experts, int rows, int cols) {
  return n_experts * (long)((rows + 15) / 16) * (long)((cols + 127) / 128) * 128L;
}

hipError_t launch_pack_scales(const uint8_t *scales, int n_experts, int rows, int cols, uint8_t *dst,
                              hipStream_t stream) {
  const int nrb = (rows + 15) / 16, nch = (cols + 127) / 128;
  const long units = (long)n_experts * nrb * nch * 32;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_scales, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream, scales, rows,
                     cols / 16, nrb, nch, units, dst);
  return hipGetLastError();
}

// One 16-byte piece u = ((((e nrb + b) nch + c) 2 + h) 16 + r) 2 + i of the
// repacked codes per thread: row 16 b + r of expert e, bytes 64 c + 32 h + 16 i
// .. + 15 of its kc code bytes (the codes of k 128 c + 64 h + 32 i .. + 31;
// zero past the row count or past kc).
__global__ void __launch_bounds__(256) k_pack_codes(const uint8_t *__restrict__ s, int rows, int kc, int nrb, int nch,
                                                    long units, uint8_t *__restrict__ dst) {
  const long u = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (u >= units) return;
  const int piece = (int)(u & 1);
  const int r = (int)((u >> 1) & 15);
  const int h = (int)((u >> 5) & 1);
  long t = u >> 6;
  const int c = (int)(t % nch);
  t /= nch;
  const int blk = (int)(t % nrb);
  const long e = t / nrb;
  const int row = 16 * blk + r, col = 64 * c + 32 * h + 16 * piece;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row < rows && col < kc) {
    const uint8_t *src = s + (e * rows + row) * (long)kc + col;
    if (col + 16 <= kc && ((uintptr_t)src & 15) == 0) {
      v = *(const u32x4_t *)src;
    } else {
      uint32_t w[4] = {0u, 0u, 0u, 0u};
      for (int i = 0; i < 16 && col + i < kc; ++i) w[i >> 2] |= (uint32_t)src[i] << (8 * (i & 3));
      v = u32x4_t{w[0], w[1], w[2], w[3]};
    }
  }
  ((u32x4_t *)dst)[u] = v;
}

long packed_codes_bytes(long n_experts, int rows, int cols) {
  return n_experts * (long)((rows + 15) / 16) * (long)((cols + 127) / 128) * 1024L;
}

hipError_t launch_pack_codes(const uint8_t *codes, int n_experts, int rows, int cols, uint8_t *dst,
                             hipStream_t stream) {
  const int nrb = (rows + 15) / 16, nch = (cols + 127) / 128;
  const long units = (long)n_experts * nrb * nch * 64;
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_pack_codes, dim3((unsigned)((units + 255) / 256)), dim3(256), 0, stream, codes, rows,
                     cols / 2, nrb, nch, units, dst);
  return hipGetLastError();
}

}  // namespace moe
