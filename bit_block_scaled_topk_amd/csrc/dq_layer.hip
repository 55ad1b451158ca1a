// dq_layer.hip -- a whole decode step (one or two tokens) of the MoE layer in
// ONE persistent launch: routing, the gather layout, the shared and routed
// experts' up projections (+ activation) and down projections, and the
// WeightedRowSum combine (gllm PR #91, "What changes"; Glq v0.2.13, "Remaining
// gap to bf16-native": a single-launch parallel-experts kernel is the way past
// per-expert launches).
//
// Work units.  An expert's FFN is split over its hidden width: unit (expert,
// s) owns the 64 hidden columns [64 s, 64 s + 64).  It computes those columns
// of h from all of x (64 rows of W_up; with SwiGLU also the 64 matching rows
// of the other half), and from them the down projection's share of every
// output column (the k-slice [64 s, 64 s + 64) of W_down):
//     part[unit][row][c] = sum_{k in slice} W_down[c][k] * h[row][k].
// So no unit waits for another while it computes: its weights stream into
// registers from the repacked layout, a window of kWin loads in flight per
// wavefront (issuing all of them at once was measured 2.3x slower: the
// memory pipeline stalls the issuing wavefront), each piece is used as soon as
// it has landed, and h never leaves the workgroup.  One workgroup per CU, all
// resident; workgroup w takes units w, w + grid, ...: the shared expert's
// units first (their workgroups compute them before they route), then each
// active routed expert's, in slot order.
//
// Then one hand-off.  Each partial sum is stored with the launch's epoch in
// its upper half (one 64-bit device-coherent store, no wait).  Workgroup b
// owns output columns [16 b, 16 b + 16): it loads the partials of those
// columns until every one carries this launch's epoch, sums each expert's in
// slice order (y = global * sum) and computes out = shared + sum_j w_j * y_j
// with fmaf in j order.
//
// Lane maps.  The repacked weights hold, per expert, 16-row block and
// 128-wide k chunk, two 64-wide halves of 16 rows x 32 bytes of codes (1 KB in
// all) and of 16 rows x 4 scales (128 B in all).  Up rows: one load of a
// wavefront reads a whole chunk of one block -- lane (n, q) = (l % 16, l / 16)
// gets row n's codes for k = 128 c + 32 q .. + 31; the unit's (chunk, tile)
// pieces, tile fastest, are dealt round-robin to the wavefronts, so each
// wavefront keeps one tile.  Down: one load covers the unit's k-slice of two
// blocks, which is one half of a chunk, 512 contiguous bytes per block --
// lane l takes block 2 p + l / 32, row (l % 32) / 2 and quarter l % 2 of the
// slice; block pair p goes to wavefront p % 8.  Each piece's two scales come
// with it (a 2-byte load).  The dot products run on the vector ALUs in fp32
// (bf16 x through the bf16 dot instruction: exact products, fp32 sums), each
// 16-element block's sum scaled by its e4m3 scale.  (A matrix-core tile would
// be 1/16 used here, and gfx950's FP4 converters apply only the exponent of a
// scale, so an exact bf16 decode would cost more ALU work than these dot
// products.)  The up sums of a tile's wavefronts and 4 k-quarters meet in LDS
// and are added in a fixed order; the two halves of a down row by one DPP
// move.
//
// sync[0] is the error word, sync[1] the launch count, sync[2 + w] workgroup
// w's launch count, read at start (e) and stored as e + 1 at the end: e + 1
// is this launch's epoch (every workgroup holds the same count between
// launches).  decode_layer_init zeroes the words and the partial sums once;
// every launch leaves them ready for the next.  Every wait is bounded
// (kSpinLimit sleeps); on expiry the error word is set and the kernel still
// finishes.  No workgroup waits before it has stored its partial sums, so
// every wait ends once the whole grid is resident (the host checks that with
// the occupancy query).
#include <algorithm>

#include "launch.hpp"
#include "nvfp4_device.hpp"
#include "route_device.hpp"

namespace moe {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSlice = 64;             // hidden columns of one work unit
constexpr int kSpinLimit = 1 << 22;
constexpr int kSc1 = 16;               // cache-policy bit of a buffer load: device-coherent access
constexpr int kLdsLimit = 160 * 1024;  // LDS of one CU
constexpr int kMaxRows = 2;            // tokens of a step
constexpr int kMaxPicks = kMaxRows * MOE_MAX_TOPK;  // <= 64: one wavefront
constexpr int kMaxGrid = 1024;
constexpr int kSyncWords = 2 + kMaxGrid;
constexpr int kMaxD = 3072;            // d_model the register tiles cover
constexpr int kLogitsPerThread = kMaxRows * MOE_MAX_EXPERTS / kThreads;
constexpr int kXLoads = kMaxRows * kMaxD * 4 / 16 / kThreads;  // 16-byte pieces of x per thread (fp32 x)
// Floats of a unit's up partial sums in LDS: per row, wavefront and lane
// (one tile per wavefront), or, when the up pieces go chunk-fastest, per tile,
// wavefront, row and column (4 NB tiles).
constexpr int up_part_floats(int NB) {
  return kMaxRows * kThreads > 4 * NB * kWaves * kMaxRows * 16 ? kMaxRows * kThreads : 4 * NB * kWaves * kMaxRows * 16;
}
constexpr int kSumGroup = 8;           // slices one reducer thread adds
constexpr int kRedCols = 16;           // output columns one reducer block combines
constexpr int kWin = 6;                // weight loads in flight per wavefront
constexpr int kKeyRow = 2 * MOE_MAX_EXPERTS;  // routing keys of one token, padded
// LDS of a wavefront's scale copies, in whole 1 KB buffer-to-LDS loads (every
// lane writes its 16 bytes, zeros past the data): the up scales of one block,
// every chunk (kMaxD / 128 chunks x 128 B), then the down scales of up to 12
// block pairs (2 blocks x 64 B each, 1.5 KB in two loads).
constexpr int kScUp = (kMaxD / 128 * 128 + 1023) / 1024 * 1024;
constexpr int kScW = kScUp + (12 * 2 * 64 + 1023) / 1024 * 1024;
constexpr int kOob = 0x40000000;               // a buffer offset past every extent: the load reads nothing
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer straight into LDS: lane l writes dst + 16 l
// (dst the same for the whole wavefront).
__device__ __forceinline__ void load16_to_lds(__amdgpu_buffer_rsrc_t rsrc, uint8_t *dst, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)dst, 16, voffset, 0, 0, 0);
}

struct StepArgs {
  DecodeLayerProblem lp;
  int grid;
  int ns, nr;    // units of the shared expert (0 without one) and of a routed expert
  int dch;       // 128-wide chunks of an up row: ceil(d / 128)
  int dblk;      // 16-row blocks of a down projection: d / 16
  int rk_two;    // routing: two ranking passes (else one over all of a token's keys)
  int rk_gs;     // ... the first pass ranks in groups of 2^rk_gs experts (two passes)
  int rk_kc;     // ... candidates kept per group: min(K, 2^rk_gs)
  int rk_c, rk_cp;   // ... candidates per token, and their padded row
  int rk_ep;     // ... padded key row
  int rk_p1, rk_p2;  // ... log2 of the threads per item in the first and second pass
  int rk_s1, rk_s2;  // ... keys each thread compares (multiples of 16)
  int sgroups;   // reducer: groups of kSumGroup slices (of the wider expert)
  int x_stride;  // elements of one token's x in LDS (dch * 128, zero-padded)
  int x_lds;     // LDS bytes of x
  int sc_off;    // LDS byte offset of the wavefronts' scale regions (kScW each)
};

// Workgroup barrier for LDS only: unlike __syncthreads it does not wait for
// this wavefront's outstanding global loads and stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void *base, size_t bytes) {
  const int nb = bytes > 0x7FFFFFF0u ? (int)0x7FFFFFF0u : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, nb, 0x00020000);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Sum over a group of `parts` consecutive lanes (a power of two <= 16) by DPP
// moves inside 16-lane rows; every lane of the group ends with it.
__device__ __forceinline__ int group_sum(int v, int parts) {
  if (parts >= 2) v += __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false);   // quad [1,0,3,2]
  if (parts >= 4) v += __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false);   // quad [2,3,0,1]
  if (parts >= 8) v += __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false);  // half-row mirror
  if (parts >= 16) v += __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); // row mirror
  return v;
}

// 16 e2m1 codes (two words, element 0 in the low nibble of byte 0) times 16
// fp32 activations: four chains of four elements in order, then
// (c0 + c1) + (c2 + c3).
__device__ __forceinline__ float dot16v(uint32_t w0, uint32_t w1, const f32x4_t &x0, const f32x4_t &x1,
                                        const f32x4_t &x2, const f32x4_t &x3) {
  const f32x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 0);
  const f32x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 1);
  const f32x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 2);
  const f32x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w0, 1.0f, 3);
  const f32x2_t v4 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w1, 1.0f, 0);
  const f32x2_t v5 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w1, 1.0f, 1);
  const f32x2_t v6 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w1, 1.0f, 2);
  const f32x2_t v7 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w1, 1.0f, 3);
  float c0 = v0.x * x0.x, c1 = v2.x * x1.x, c2 = v4.x * x2.x, c3 = v6.x * x3.x;
  c0 = fmaf(v0.y, x0.y, c0);
  c1 = fmaf(v2.y, x1.y, c1);
  c2 = fmaf(v4.y, x2.y, c2);
  c3 = fmaf(v6.y, x3.y, c3);
  c0 = fmaf(v1.x, x0.z, c0);
  c1 = fmaf(v3.x, x1.z, c1);
  c2 = fmaf(v5.x, x2.z, c2);
  c3 = fmaf(v7.x, x3.z, c3);
  c0 = fmaf(v1.y, x0.w, c0);
  c1 = fmaf(v3.y, x1.w, c1);
  c2 = fmaf(v5.y, x2.w, c2);
  c3 = fmaf(v7.y, x3.w, c3);
  return (c0 + c1) + (c2 + c3);
}

// 16 e2m1 codes (two words) times 16 bf16 activations (8 packed pairs) with
// the bf16 dot-product instruction (exact products, fp32 sums): two chains of
// four pairs in order, then added.
__device__ __forceinline__ float dot16_bf16(uint32_t w0, uint32_t w1, const u32x4_t &xa, const u32x4_t &xb) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
  auto pair = [](uint32_t v) { return __builtin_bit_cast(bf16x2_t, v); };
  auto cvt = [](uint32_t w, int sel) {
    switch (sel) {  // the byte selector must be an immediate
      case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
      case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
      case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
      default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
    }
  };
  float c0 = __builtin_amdgcn_fdot2_f32_bf16(cvt(w0, 0), pair(xa.x), 0.f, false);
  float c1 = __builtin_amdgcn_fdot2_f32_bf16(cvt(w1, 0), pair(xb.x), 0.f, false);
  c0 = __builtin_amdgcn_fdot2_f32_bf16(cvt(w0, 1), pair(xa.y), c0, false);
  c1 = __builtin_amdgcn_fdot2_f32_bf16(cvt(w1, 1), pair(xb.y), c1, false);
  c0 = __builtin_amdgcn_fdot2_f32_bf16(cvt(w0, 2), pair(xa.z), c0, false);
  c1 = __builtin_amdgcn_fdot2_f32_bf16(cvt(w1, 2), pair(xb.z), c1, false);
  c0 = __builtin_amdgcn_fdot2_f32_bf16(cvt(w0, 3), pair(xa.w), c0, false);
  c1 = __builtin_amdgcn_fdot2_f32_bf16(cvt(w1, 3), pair(xb.w), c1, false);
  return c0 + c1;
}

// The hidden value from the up sums: relu(gl * a)^2, or silu(gl * a) * (gl * b)
// (SwiGLU, a the gate row).
template <int EPI>
__device__ __forceinline__ float epilogue(float gl, float a, float b) {
  if (EPI == EPI_RELU2) {
    float u = gl * a;
    u = u > 0.f ? u : 0.f;
    return u * u;
  }
  const float av = gl * a, bv = gl * b;
  return (av / (1.0f + expf(-av))) * bv;
}

// A unit resolved to its expert.
struct UnitRef {
  bool shared, ok;
  int e, s, slot, rows;  // expert, slice, routed slot, token rows
  int tok[kMaxRows];     // token of each row
};

template <int NB, int NR, bool XF, int CU, int DP, bool CF>
__global__ void __launch_bounds__(kThreads) k_decode_step(StepArgs a) {
  extern __shared__ u32x4_t s_dyn[];  // x | phase scratch
  __shared__ int s_id[kMaxPicks], s_prow[kMaxPicks], s_pslot[kMaxPicks];  // per pick t*K + j
  __shared__ float s_pw[kMaxPicks];
  __shared__ float s_gl[kMaxPicks + 1];  // the down projections' globals: per pick, then the shared expert's
  __shared__ int s_rt[kMaxPicks];       // token of each packed row
  __shared__ int s_r0[kMaxPicks];       // first packed row of each slot
  __shared__ uint32_t s_bits[kMaxRows][MOE_MAX_EXPERTS / 32];  // each token's picked experts
  const DecodeLayerProblem &lp = a.lp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int32_t *err = lp.sync;
  int32_t *flags = lp.sync + 2;
  uint8_t *s_xb = (uint8_t *)s_dyn;    // x
  uint8_t *s_scr = s_xb + a.x_lds;     // phase scratch
  uint8_t *my_sc = (uint8_t *)s_dyn + a.sc_off + wave * kScW;  // this wavefront's scales of the unit
  const int n = lp.n_tokens, d = lp.d, E = lp.n_experts, K = lp.top_k, P = n * K, NE = n * E;
  const int n_units_max = a.ns + lp.max_slots * a.nr;

  // ---- the logits and x first: everything waits on them
  float lg[kLogitsPerThread];
#pragma unroll
  for (int i = 0; i < kLogitsPerThread; ++i) lg[i] = lp.logits[min(tid + kThreads * i, NE - 1)];
  const int xpr = XF ? d / 4 : d / 8;  // 16-byte pieces of one token's x
  u32x4_t xv[kXLoads];
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int c = tid + kThreads * i;
    if (c < n * xpr) xv[i] = *((const u32x4_t *)lp.x + c);
  }
  // this launch's count, requested after the shared expert's first weights
  // (below): used only when partial sums are stored and compared, so that no
  // wait for it holds back the weight requests
  int32_t epoch = 0;

  // ---- a unit's weights.  Pieces in a fixed order -- the up pieces, then
  //      the down block pairs -- and a window of kWin loads in flight: piece
  //      i + kWin is requested as piece i is used, so the compiler waits for
  //      each piece alone.  The unit's up pieces, (chunk, tile) with the tile
  //      fastest, are dealt round-robin to the wavefronts, so each wavefront
  //      keeps one tile (its index mod the tiles per chunk) and the counts
  //      differ by at most one.  No branches: an absent piece (past the
  //      chunks, tiles or block pairs) reloads a present one, which the
  //      caches hold, and is not used (requesting it past the buffer's extent
  //      instead, so that nothing is read, was measured slower).  Buffer loads
  //      over the expert's region: the per-lane part of an address is one
  //      register for all pieces, the rest a scalar offset.
  constexpr int TPC = 4 * NB;  // up tiles per chunk
  constexpr int SU = CU * TPC, S = SU + DP;
  static_assert(CU * 1024 <= kScUp && (DP * 8 + 63) / 64 * 1024 <= kScW - kScUp,
                "a wavefront's scale loads stay inside its LDS region");
  const int my_t = wave % TPC;  // this wavefront's up tile
  // CF (chunk-fastest; dch = 8 CU): up piece i of every wavefront is tile
  // i / CU, chunk wave + 8 (i % CU), so that in each round the wavefronts
  // read 8 adjacent chunks of one 16-row block and a workgroup's loads in
  // flight cover one contiguous stretch of its unit's blocks; each wavefront
  // then holds a partial sum of every tile.  Otherwise piece i is tile my_t,
  // chunk (wave + 8 i) / TPC (past the chunks: absent).
  auto up_tile = [&](int i) { return CF ? i / CU : my_t; };
  auto up_chunk = [&](int i) { return CF ? wave + kWaves * (i % CU) : (wave + kWaves * i) / TPC; };
  const int nq = lane >> 4, nn = lane & 15;                        // up: k-quarter, row
  const int dq = lane & 1, dr = (lane & 31) >> 1, dh = lane >> 5;  // down: slice half, row, block of the pair
  const int up_lc = (nq >> 1) * 512 + nn * 32 + (nq & 1) * 16;
  struct UnitSrc {
    __amdgpu_buffer_rsrc_t uc, us, dc, dsc;
    int nb_out, dnch, s;
  };
  auto unit_src = [&](const UnitRef &u) {
    const ProjProblem &up = u.shared ? lp.up[0] : lp.up[1];
    const ProjProblem &dn = u.shared ? lp.down[0] : lp.down[1];
    UnitSrc q;
    q.nb_out = up.n_out >> 4;
    q.dnch = (up.n_out + 127) >> 7;
    q.s = u.s;
    const size_t up_nblk = (size_t)(up.n_w >> 4);
    q.uc = make_rsrc(up.codes_packed + (size_t)u.e * up_nblk * a.dch * 1024, (uint32_t)(up_nblk * a.dch * 1024));
    q.us = make_rsrc(up.scales_packed + (size_t)u.e * up_nblk * a.dch * 128, (uint32_t)(up_nblk * a.dch * 128));
    q.dc = make_rsrc(dn.codes_packed + (size_t)u.e * a.dblk * q.dnch * 1024,
                     (uint32_t)((size_t)a.dblk * q.dnch * 1024));
    q.dsc = make_rsrc(dn.scales_packed + (size_t)u.e * a.dblk * q.dnch * 128,
                      (uint32_t)((size_t)a.dblk * q.dnch * 128));
    return q;
  };
  // piece i (a compile-time index) of the unit: 16 bytes of codes.  Its two
  // scales (the low byte for the first 16 k) are read from the wavefront's
  // LDS copy of the unit's scales, which start_unit requests with a few
  // buffer-to-LDS loads (a 2-byte load per piece cost about a sixth of the
  // stream's time: a request per piece for 128 bytes).
  struct Piece {
    u32x4_t w;
  };
  const int up_ls = (nq >> 1) * 64 + nn * 4 + (nq & 1) * 2;   // a lane's scales in a block-chunk
  const int dn_ls = dh * 64 + dr * 4 + dq * 2;                 // ... in a block pair's down scales
  auto load_piece = [&](const UnitSrc &q, int i) -> Piece {
    Piece p;
    if (i < SU) {
      const int tt = up_tile(i), c = min(up_chunk(i), a.dch - 1), blk = min(4 * q.s + (tt & 3), q.nb_out - 1);
      const int piece = ((tt >> 2) * q.nb_out + blk) * a.dch + c;
      p.w = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(q.uc, up_lc, piece * 1024, 0));
      return p;
    }
    const int jj = i - SU;
    const int pr = min(wave + kWaves * jj, (a.dblk - 1) >> 1);
    // block 2 pr + dh (the first block of a half-used last pair), row dr, half dq
    const bool whole = 2 * pr + 1 < a.dblk;
    const int lc = (whole ? dh * q.dnch * 1024 : 0) + dr * 32 + dq * 16;
    const int piece = 2 * pr * q.dnch + (q.s >> 1);
    p.w = __builtin_bit_cast(u32x4_t,
                             __builtin_amdgcn_raw_buffer_load_b128(q.dc, lc, piece * 1024 + (q.s & 1) * 512, 0));
    return p;
  };

  // the gather layout, in every wavefront's registers (lane = pick t K + j):
  // the pick's expert and token, its slot, whether it owns the slot (the
  // slot's lower token) and the slot's rows; and the number of slots
  int r_e = 0, r_t = 0, r_slot = 0, r_rows = 0, r_nact = 0;
  bool r_own = false;
  auto resolve = [&](int uidx, UnitRef &u) {
    u.shared = uidx < a.ns;
    if (u.shared) {
      u.ok = true;
      u.e = 0;
      u.s = uidx;
      u.slot = -1;
      u.rows = n;
      u.tok[0] = 0;
      u.tok[1] = 1;
    } else {  // from the layout registers: the lane of the pick that owns the slot
      const int v = uidx - a.ns;
      u.slot = v / a.nr;
      u.s = v - u.slot * a.nr;
      u.ok = u.slot < r_nact;
      const uint64_t m = __ballot(r_own && r_slot == u.slot);
      const int ol = m ? (int)__builtin_ctzll(m) : 0;
      u.e = min(max(__builtin_amdgcn_readlane(r_e, ol), 0), E - 1);
      u.rows = __builtin_amdgcn_readlane(r_rows, ol);
      u.tok[0] = __builtin_amdgcn_readlane(r_t, ol);
      u.tok[1] = 1;
    }
  };

  // ---- routing (the pages' rule: top-K by logit, the lower index first among
  //      equal logits; the weights a softmax over the picks, summed in slot
  //      order) on 64-bit keys ordered like the rule.  An expert's rank is the
  //      number of keys above its own, counted by 2^ps threads per expert.
  //      One pass over all of a token's keys when that is few comparisons per
  //      thread; else two: an expert's rank inside its group of 2^gs experts
  //      keeps each group's best min(K, 2^gs) as candidates, and a
  //      candidate's rank among its token's candidates is its slot, if below
  //      K.  The shapes of the passes come from the host (no divisions here:
  //      this runs once per step on the critical path).
  //  rank_pass: item (t, i), i < L, is key i of row t (stride Lp, zero-
  //  padded: key 0 is below every real key); its rank in its range (the
  //  row, or its group of 2^gs = 2^ps * share keys) is counted by 2^ps
  //  threads, each over a contiguous share (a multiple of 16) with 16-byte
  //  loads and no per-key tests; emit(t, i, cnt, key) for part 0.  (With 8
  //  wavefronts on 4 SIMDs every instruction costs about 8 cycles: this pass
  //  is kept short.)
  auto rank_pass = [&](const uint64_t *keys, int L, int Lp, int gs, int ps, int share, auto emit) {
    const int parts = 1 << ps, part = tid & (parts - 1);
    for (int pr0 = 0; pr0 < n * L; pr0 += kThreads >> ps) {
      const int pr = pr0 + (tid >> ps);
      const bool ok = pr < n * L;
      const int c = ok ? pr : 0, t = c >= L, i = c - t * L;
      const uint64_t *row = keys + t * Lp;
      const uint64_t my = row[i];
      const u32x4_t *src = (const u32x4_t *)(row + ((i >> gs) << gs) + part * share);
      int cnt = 0;
      for (int k = 0; k < share; k += 16, src += 8) {
        u32x4_t k8[8];
#pragma unroll
        for (int h = 0; h < 8; ++h) k8[h] = src[h];
#pragma unroll
        for (int h = 0; h < 8; ++h) {
          cnt += (((uint64_t)k8[h].y << 32) | k8[h].x) > my;
          cnt += (((uint64_t)k8[h].w << 32) | k8[h].z) > my;
        }
      }
      cnt = group_sum(cnt, parts);
      if (ok && part == 0) emit(t, i, cnt, my);
    }
  };
  auto route = [&]() {
    // key rows zero-padded to Ep (a multiple of the first pass's range)
    const int Ep = a.rk_ep, Kc = a.rk_kc, C = a.rk_c, Cp = a.rk_cp;
    uint64_t *s_key = (uint64_t *)s_scr;                                   // [n][Ep]
    uint64_t *s_cand = s_key + kMaxRows * kKeyRow;                         // [n][Cp]
    float *s_logit = (float *)(s_cand + kMaxRows * kKeyRow);               // [n][E]
    uint64_t *s_pick = (uint64_t *)(s_logit + kMaxRows * MOE_MAX_EXPERTS);  // [n][K]
#pragma unroll
    for (int i = 0; i < kLogitsPerThread; ++i) {
      if (kThreads * i >= NE) break;  // uniform
      const int c = tid + kThreads * i;
      if (c < NE) {
        const int t = c >= E, e = c - t * E;
        s_logit[c] = lg[i];
        s_key[t * Ep + e] = route_key(lg[i], e);
      }
    }
    for (int c = tid; c < n * (MOE_MAX_EXPERTS / 32); c += kThreads) (&s_bits[0][0])[c] = 0u;
    {  // the padding of each key row, and the candidate rows
      const int pad = Ep - E;
      for (int c = tid; c < n * pad; c += kThreads) {
        const int t = c >= pad;
        s_key[t * Ep + E + c - t * pad] = 0ull;
      }
      if (a.rk_two)
        for (int c = tid; c < n * Cp; c += kThreads) s_cand[c] = 0ull;
    }
    lds_barrier();
    auto pick = [&](int t, int cnt, uint64_t key) {  // slot cnt of token t; its expert's bit
      s_pick[t * K + cnt] = key;
      const int e = min(max(route_key_index(key), 0), E - 1);
      __hip_atomic_fetch_or(&s_bits[t][e >> 5], 1u << (e & 31), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    if (!a.rk_two) {
      rank_pass(s_key, E, Ep, 30, a.rk_p1, a.rk_s1, [&](int t, int, int cnt, uint64_t key) {
        if (cnt < K) pick(t, cnt, key);
      });
    } else {
      rank_pass(s_key, E, Ep, a.rk_gs, a.rk_p1, a.rk_s1, [&](int t, int i, int cnt, uint64_t key) {
        if (cnt < Kc) s_cand[t * Cp + (i >> a.rk_gs) * Kc + cnt] = key;
      });
      lds_barrier();
      rank_pass(s_cand, C, Cp, 30, a.rk_p2, a.rk_s2, [&](int t, int, int cnt, uint64_t key) {
        if (key != 0ull && cnt < K) pick(t, cnt, key);
      });
    }
    lds_barrier();
    // gather layout, from the picked-expert bitmaps, in every wavefront (no
    // barrier after it): rows grouped by expert in ascending id, tokens
    // ascending within an expert; a slot per distinct expert, in ascending id.
    // A pick's row is the number of picks (of both tokens) with a lower id,
    // plus one for the second token of an expert both picked; its slot the
    // number of distinct experts with a lower id.
    {
      const bool ok = lane < P;
      const int t = lane >= K;
      const int e = ok ? min(max(route_key_index(s_pick[lane]), 0), E - 1) : 0;
      const int ew = e >> 5;
      int below = 0, below_u = 0, nact = 0;
      uint32_t w0e = 0u, w1e = 0u;
      for (int w = 0; w < (E + 31) >> 5; ++w) {
        const uint32_t b0 = s_bits[0][w], b1 = n > 1 ? s_bits[1][w] : 0u;
        const uint32_t m = w < ew ? 0xFFFFFFFFu : (w == ew ? (1u << (e & 31)) - 1u : 0u);
        below += __builtin_popcount(b0 & m) + __builtin_popcount(b1 & m);
        below_u += __builtin_popcount((b0 | b1) & m);
        nact += __builtin_popcount(b0 | b1);
        if (w == ew) {
          w0e = b0;
          w1e = b1;
        }
      }
      const bool other = ((t ? w0e : w1e) >> (e & 31)) & 1u;  // the other token picked e too
      r_e = e;
      r_t = t;
      r_slot = below_u;
      r_own = ok && (t == 0 || !other);
      r_rows = 1 + (t == 0 && other);
      r_nact = nact;
      if (wave == 0 && ok) {  // the tables the reducer and the routing views read
        const int r = below + (t == 1 && other);
        s_id[lane] = e;
        s_prow[lane] = r;
        s_pslot[lane] = below_u;
        s_rt[r] = t;
        if (r_own) s_r0[below_u] = below;
      }
    }
  };
  // The routing weights (wavefront 0), off the critical path: read after
  // later barriers.  The down globals the reducer scales by are requested
  // here too and kept in registers until it runs, so their latency hides
  // under the units.
  float gl_pick = 0.f, gl_sh = 0.f;
  auto route_weights = [&]() {
    const float *s_logit = (const float *)((const uint64_t *)s_scr + 2 * kMaxRows * kKeyRow);
    if (wave == 0) {
      const bool ok = lane < P;
      gl_pick = ok ? lp.down[1].global[s_id[lane]] : 0.f;
      gl_sh = lp.has_shared ? lp.down[0].global[0] : 0.f;
      const int t = lane >= K;
      const float l = ok ? s_logit[t * E + s_id[lane]] : 0.f;
      const float l0 = t ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), K))
                         : __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 0));
      const float ex = ok ? expf(l - l0) : 0.f;
      float sum0 = 0.f, sum1 = 0.f;  // in slot order
      for (int j = 0; j < K; ++j) sum0 += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
      if (n > 1)
        for (int j = 0; j < K; ++j) sum1 += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), K + j));
      if (ok) s_pw[lane] = ex / (t ? sum1 : sum0);
    }
  };

  // ---- x into LDS as loaded (bf16 or fp32), zero-padded to whole chunks
  auto stage_x = [&]() {
    const int eb = XF ? 4 : 2;
    const int ppt = a.x_stride * eb / 16;  // 16-byte pieces per token in LDS
    for (int c = tid; c < n * ppt; c += kThreads) {
      const int t = c / ppt, p = c - t * ppt;
      if (p >= xpr) *(u32x4_t *)(s_xb + (size_t)c * 16) = u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) {
      const int c = tid + kThreads * i;
      if (c < n * xpr) {
        const int t = c / xpr, p = c - t * xpr;
        *(u32x4_t *)(s_xb + ((size_t)t * ppt + p) * 16) = xv[i];
      }
    }
  };

  // ---- one unit: up rows -> h slice (LDS) -> down partials (stored with
  //      the epoch).  ring holds the first kWin pieces on entry.
  auto run_unit = [&](const UnitRef &u, const UnitSrc &q, Piece (&ring)[kWin]) {
    const ProjProblem &up = u.shared ? lp.up[0] : lp.up[1];
    const int nout = up.n_out;
    const float gl_up = up.global[u.e];
    const int R = u.rows;
    float acc[NR];  // tile up_tile(i), per row
#pragma unroll
    for (int r = 0; r < NR; ++r) acc[r] = 0.f;
    u32x4_t x4[NR][4];
    f32x4_t x8[NR][8];
    f32x4_t hq[NR][8];
    uint64_t *part = (uint64_t *)lp.part + (size_t)(u.shared ? u.s : a.ns + u.slot * a.nr + u.s) * kMaxRows * d;
    float *s_up = (float *)s_scr;                         // up_part_floats(NB): the partial sums
    float *s_usum = s_up + up_part_floats(NB);            // [4 NB][kMaxRows][16]
    float *s_h = s_usum + 4 * NB * kMaxRows * 16;         // [kMaxRows][64]
#pragma unroll
    for (int i = 0; i < S; ++i) {
      // one piece at a time: without the barrier the scheduler hoists later
      // pieces' decode and LDS reads, and runs out of registers
      __builtin_amdgcn_sched_barrier(0);
      const u32x4_t w = ring[i % kWin].w;
      if (i + kWin < S) ring[i % kWin] = load_piece(q, i + kWin);
      if (i < SU) {  // ---- up piece: chunk c of tile up_tile(i)
        const int c = up_chunk(i);
        if (c < a.dch) {  // uniform (always with CF)
          const int k0 = 128 * c + 32 * nq;
#pragma unroll
          for (int r = 0; r < NR; ++r) {  // this chunk's x, all rows
            if constexpr (XF) {
              const f32x4_t *xs = (const f32x4_t *)(s_xb + ((size_t)u.tok[r] * a.x_stride + k0) * 4);
#pragma unroll
              for (int e = 0; e < 8; ++e) x8[r][e] = xs[e];
            } else {
              const u32x4_t *xs = (const u32x4_t *)(s_xb + ((size_t)u.tok[r] * a.x_stride + k0) * 2);
#pragma unroll
              for (int e = 0; e < 4; ++e) x4[r][e] = xs[e];
            }
          }
          float s0, s1;
          e4m3x2_to_f32(*(const uint16_t *)(my_sc + (CF ? i : c) * 128 + up_ls), s0, s1);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (r >= R) break;  // uniform
            if constexpr (XF) {
              acc[r] = fmaf(s0, dot16v(w.x, w.y, x8[r][0], x8[r][1], x8[r][2], x8[r][3]), acc[r]);
              acc[r] = fmaf(s1, dot16v(w.z, w.w, x8[r][4], x8[r][5], x8[r][6], x8[r][7]), acc[r]);
            } else {
              acc[r] = fmaf(s0, dot16_bf16(w.x, w.y, x4[r][0], x4[r][1]), acc[r]);
              acc[r] = fmaf(s1, dot16_bf16(w.z, w.w, x4[r][2], x4[r][3]), acc[r]);
            }
          }
        }
        if constexpr (CF) {
          if (i % CU == CU - 1) {  // the wavefront's last piece of tile i / CU: its sums over the k-quarters
            const int tt = i / CU;
#pragma unroll
            for (int r = 0; r < NR; ++r) {
              float v = acc[r];
              v += __shfl_xor(v, 16);
              v += __shfl_xor(v, 32);
              if (nq == 0) s_up[((tt * kWaves + wave) * kMaxRows + r) * 16 + nn] = v;
              acc[r] = 0.f;
            }
          }
        }
      }
      if (i == SU - 1) {  // ---- the up sums of the wavefronts and k-quarters of a tile, in a fixed order -> h
        if constexpr (!CF) {
#pragma unroll
          for (int r = 0; r < kMaxRows; ++r) s_up[(r * kWaves + wave) * 64 + lane] = r < NR ? acc[r < NR ? r : 0] : 0.f;
        }
        lds_barrier();
        if (tid < TPC * kMaxRows * 16) {  // (tile t, row r, column n): tid = (t kMaxRows + r) 16 + n
          const int tr = tid >> 4, t = tr / kMaxRows, r = tr - t * kMaxRows;
          float sum = 0.f;
          if constexpr (CF) {  // rows past NR are never read
#pragma unroll
            for (int wv = 0; wv < kWaves; ++wv) sum += s_up[((t * kWaves + wv) * kMaxRows + r) * 16 + (tid & 15)];
          } else {
            const float *pp = s_up + r * kThreads + (tid & 15);
#pragma unroll
            for (int wv = t; wv < kWaves; wv += TPC)
#pragma unroll
              for (int qq = 0; qq < 4; ++qq) sum += pp[wv * 64 + qq * 16];
          }
          s_usum[tid] = sum;
        }
        lds_barrier();
        if (tid < kMaxRows * kSlice) {
          const int r = tid >> 6, cl = tid & 63, t = cl >> 4, nrow = cl & 15;
          float h = 0.f;
          if (r < R && kSlice * u.s + cl < nout) {
            const float ga = s_usum[(t * kMaxRows + r) * 16 + nrow];
            const float gb = NB > 1 ? s_usum[((t + 4) * kMaxRows + r) * 16 + nrow] : 0.f;
            h = epilogue<NB == 2 ? EPI_SWIGLU : EPI_RELU2>(gl_up, ga, gb);
          }
          s_h[tid] = h;
        }
        lds_barrier();
        // this lane's 32 hidden values of each row
#pragma unroll
        for (int r = 0; r < NR; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) hq[r][e] = ((const f32x4_t *)(s_h + r * kSlice + 32 * dq))[e];
      }
      if (i >= SU) {  // ---- down block pair
        const int jj = i - SU, pr = wave + kWaves * jj, blk = 2 * pr + dh;
        if (2 * pr < a.dblk) {  // uniform
          float s0, s1;
          e4m3x2_to_f32(*(const uint16_t *)(my_sc + kScUp + jj * 128 + dn_ls), s0, s1);
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            if (r >= R) break;  // uniform
            float v = fmaf(s0, dot16v(w.x, w.y, hq[r][0], hq[r][1], hq[r][2], hq[r][3]), 0.f);
            v = fmaf(s1, dot16v(w.z, w.w, hq[r][4], hq[r][5], hq[r][6], hq[r][7]), v);
            v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
            if (dq == 0 && blk < a.dblk)
              __hip_atomic_store(part + (size_t)r * d + 16 * blk + dr,
                                 ((uint64_t)((uint32_t)epoch + 1u) << 32) | (uint64_t)__float_as_uint(v), __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      }
    }
    lds_barrier();  // the scratch serves the next unit
  };

  // ---- this workgroup's units.  The shared expert's units need no routing:
  //      their workgroups compute them first and route afterwards; the others
  //      route, then compute theirs.
  Piece ring[kWin];
  auto start_unit = [&](const UnitRef &u, UnitSrc &q) {
    q = unit_src(u);
    // this wavefront's scales, into its LDS region: the up scales its pieces
    // read (CF: the block-chunk of each piece; else its tile's block for every
    // chunk, dch x 128 contiguous bytes), then its block pairs' down scales
    // (the unit's 64-wide half of one chunk: 64 bytes per block)
    if constexpr (CF) {  // the block-chunk (128 bytes) of each of its SU = 8 CU pieces: CU x 1 KB
#pragma unroll
      for (int k = 0; k < CU; ++k) {
        const int pi = 8 * k + (lane >> 3), tt = pi / CU, c = wave + kWaves * (pi % CU);
        const int blk = min(4 * q.s + (tt & 3), q.nb_out - 1);
        load16_to_lds(q.us, my_sc + k * 1024, (((tt >> 2) * q.nb_out + blk) * a.dch + c) * 128 + (lane & 7) * 16);
      }
    } else {
      const int blk = min(4 * q.s + (my_t & 3), q.nb_out - 1);
      const int base = ((my_t >> 2) * q.nb_out + blk) * a.dch * 128, nbytes = a.dch * 128;
#pragma unroll
      for (int k = 0; k < CU; ++k) {  // dch <= 8 CU chunks: CU x 1 KB
        const int off = (k * 64 + lane) * 16;
        load16_to_lds(q.us, my_sc + k * 1024, off < nbytes ? base + off : kOob);
      }
    }
    {
#pragma unroll
      for (int k = 0; k < (DP * 8 + 63) / 64; ++k) {  // DP pairs x 2 blocks x 4 lanes of 16 bytes
        const int g = k * 64 + lane, jj = g >> 3, hb = (g >> 2) & 1;
        const int pr = min(wave + kWaves * jj, (a.dblk - 1) >> 1);
        const int b = 2 * pr + (2 * pr + 1 < a.dblk ? hb : 0);  // the first block of a half-used last pair
        const int off = (b * q.dnch + (q.s >> 1)) * 128 + (q.s & 1) * 64 + (g & 3) * 16;
        load16_to_lds(q.dsc, my_sc + kScUp + k * 1024, g < DP * 8 ? off : kOob);
      }
    }
#pragma unroll
    for (int i = 0; i < kWin; ++i) ring[i] = load_piece(q, i);
  };
  const bool pre = (int)blockIdx.x < a.ns;
  if (pre) {  // one block from the requests to the unit, so each wait counts the loads in flight
    UnitRef u;
    UnitSrc q;
    resolve(blockIdx.x, u);
    start_unit(u, q);
    epoch = __hip_atomic_load(&flags[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    stage_x();
    lds_barrier();
    run_unit(u, q, ring);
  } else {
    epoch = __hip_atomic_load(&flags[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  route();
  const int n_units = a.ns + r_nact * a.nr;
  bool weighted = false;
  for (int ui = blockIdx.x + (pre ? a.grid : 0); ui < n_units; ui += a.grid) {
    UnitRef u;
    UnitSrc q;
    resolve(ui, u);
    if (!u.ok) continue;  // uniform
    start_unit(u, q);
    if (!weighted) {  // while the first pieces stream in
      route_weights();
      if (!pre) stage_x();
      lds_barrier();
      weighted = true;
    }
    run_unit(u, q, ring);
  }
  if (!weighted) {
    route_weights();
    lds_barrier();  // wavefront 0's layout tables, for the reducer
  }

  // ---- reduce and combine output columns [16 cb, 16 cb + 16): each thread
  //      loads kSumGroup slices of two columns of one term (the shared
  //      expert, then the picks), until all carry this launch's epoch.
  //      (Dealing the column blocks first to the workgroups that finish early,
  //      with 32-column blocks so that fewer workgroups reduce, was measured
  //      slower: a poll round over twice the loads takes longer.)
  constexpr int G2 = kRedCols / 2;  // two-column groups of a block
  const int terms = 1 + K;
  const int items = n * terms * G2 * a.sgroups;
  f32x2_t *s_yp = (f32x2_t *)s_scr;                                       // [n][terms][G2][sgroups]
  float *s_y = (float *)(s_yp + kMaxRows * (1 + MOE_MAX_TOPK) * G2 * a.sgroups);  // [n][terms][kRedCols]
  const __amdgpu_buffer_rsrc_t pr =
      coherent_rsrc(lp.part, (size_t)n_units_max * kMaxRows * d * sizeof(uint64_t));
  if (wave == 0) {  // read after the first barrier below
    if (lane < P) s_gl[lane] = gl_pick;
    if (lane == 0) s_gl[kMaxPicks] = gl_sh;
  }
  for (int cb = blockIdx.x; cb < d / kRedCols; cb += a.grid) {
    for (int it = tid; it < items; it += kThreads) {
      const int sg = it % a.sgroups, g = (it / a.sgroups) % G2, tt = it / (a.sgroups * G2);
      const int t = tt / terms, term = tt - t * terms;
      int base, count, row;
      if (term == 0) {
        base = 0;
        count = lp.has_shared ? a.ns : 0;
        row = t;
      } else {
        const int pick = t * K + term - 1, sl = s_pslot[pick];
        base = a.ns + sl * a.nr;
        count = a.nr;
        row = s_prow[pick] - s_r0[sl];
      }
      const int s_lo = sg * kSumGroup;
      u32x4_t v[kSumGroup];
      uint32_t off[kSumGroup];
#pragma unroll
      for (int i = 0; i < kSumGroup; ++i) {
        const int sl2 = min(s_lo + i, max(count - 1, 0));
        off[i] = (uint32_t)((((size_t)(base + sl2) * kMaxRows + row) * d + kRedCols * cb + 2 * g) * 8);
        v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(pr, off[i], 0, kSc1));
      }
      for (int spins = 0;; ++spins) {
        bool ready = true;
#pragma unroll
        for (int i = 0; i < kSumGroup; ++i)
          if (s_lo + i < count) ready &= v[i].y == (uint32_t)epoch + 1u && v[i].w == (uint32_t)epoch + 1u;
        if (ready) break;
        if (spins >= kSpinLimit) {
          __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        // a compiler barrier: nothing in this loop writes memory, so without
        // one the repeated loads of the same addresses may be merged with the
        // first ones, and the loop would test the same stale values
        asm volatile("" ::: "memory");
#pragma unroll
        for (int i = 0; i < kSumGroup; ++i)
          v[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(pr, off[i], 0, kSc1));
      }
      f32x2_t acc2 = {0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kSumGroup; ++i)
        if (s_lo + i < count) {
          acc2.x += __uint_as_float(v[i].x);
          acc2.y += __uint_as_float(v[i].z);
        }
      s_yp[it] = acc2;
    }
    lds_barrier();
    for (int c = tid; c < n * terms * kRedCols; c += kThreads) {
      const int col = c % kRedCols, tt = c / kRedCols, t = tt / terms, term = tt - t * terms;
      const float gl = term == 0 ? s_gl[kMaxPicks] : s_gl[t * K + term - 1];
      const f32x2_t *pp = s_yp + (size_t)(tt * G2 + (col >> 1)) * a.sgroups;
      float y = 0.f;
      for (int sg = 0; sg < a.sgroups; ++sg) y += pp[sg][col & 1];
      s_y[c] = gl * y;
    }
    lds_barrier();
    if (tid < n * kRedCols) {
      const int t = tid / kRedCols, col = kRedCols * cb + tid % kRedCols;
      const float *yt = s_y + (size_t)t * terms * kRedCols + tid % kRedCols;
      float accw = 0.f;
      for (int j = 0; j < K; ++j) {
        const float y = yt[(1 + j) * kRedCols];
        accw = fmaf(s_pw[t * K + j], y, accw);
        lp.yg[(size_t)s_prow[t * K + j] * d + col] = y;
      }
      lp.out[(size_t)t * d + col] = lp.has_shared ? yt[0] + accw : accw;
    }
    lds_barrier();
  }
  if (tid == 0) __hip_atomic_store(&flags[blockIdx.x], epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // workgroup 0: the routing and layout views
  if (blockIdx.x == 0) {
    if (tid < P) {
      lp.ids[tid] = s_id[tid];
      lp.topk_w[tid] = s_pw[tid];
      lp.rows[tid] = s_prow[tid];
      lp.row_token[tid] = s_rt[tid];
    }
    for (int e = tid; e <= E; e += kThreads) {
      int below = 0;
      for (int q = 0; q < P; ++q) below += s_id[q] < e;
      lp.offsets[e] = below;
    }
    if (tid == 0) __hip_atomic_fetch_add(lp.sync + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

__global__ void k_zero_words(int32_t *w, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) w[i] = 0;
}

__global__ void k_zero_words_long(int32_t *w, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) w[i] = 0;
}

// Bytes of the phase scratch: routing (keys, candidates, logits, picks); one
// unit's up sums and h slice.
size_t scratch_bytes(int NB) {
  const size_t route = (size_t)kMaxRows * kKeyRow * 16 + (size_t)kMaxRows * MOE_MAX_EXPERTS * 4 + (size_t)kMaxPicks * 8;
  const size_t up = ((size_t)up_part_floats(NB) + (size_t)4 * NB * kMaxRows * 16 + (size_t)kMaxRows * kSlice) * 4;
  return std::max(route, up);
}

template <int NB, int NR, bool XF, int CU, int DP, bool CF>
hipError_t launch_one(StepArgs &a, size_t lds, hipStream_t stream) {
  static int occ = -1;  // same code object on every device
  static size_t occ_lds = 0, static_lds = 0;
  if (occ < 0) {
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, (const void *)k_decode_step<NB, NR, XF, CU, DP, CF>) != hipSuccess)
      return hipErrorInvalidValue;
    static_lds = attr.sharedSizeBytes;
  }
  if (lds + static_lds > (size_t)kLdsLimit) return hipErrorNotSupported;
  if (occ < 0 || occ_lds != lds) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, k_decode_step<NB, NR, XF, CU, DP, CF>, kThreads, lds) !=
        hipSuccess)
      return hipErrorInvalidValue;
    occ = o;
    occ_lds = lds;
  }
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidValue;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidValue;
  // every workgroup must be resident at once
  if ((long)occ * cus < a.grid) return hipErrorNotSupported;
  hipLaunchKernelGGL((k_decode_step<NB, NR, XF, CU, DP, CF>), dim3(a.grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

// Register tiles by d_model class: up chunk iterations CU = ceil(d / 1024),
// down block-pair iterations DP = 4 CU (8 wavefronts); fp32 x for d_model <=
// 1024 only (its x tiles take twice the registers).
template <int NB, int NR, bool XF, int CU, int DP>
hipError_t launch_cf(StepArgs &a, size_t lds, hipStream_t stream) {
  // SwiGLU units whose up chunks fill the wavefronts' rounds exactly (dch = 8 CU)
  // take their up pieces chunk-fastest
  if constexpr (NB == 2)
    if (a.dch == 8 * CU) return launch_one<NB, NR, XF, CU, DP, true>(a, lds, stream);
  return launch_one<NB, NR, XF, CU, DP, false>(a, lds, stream);
}

template <int NB, int NR>
hipError_t launch_class(StepArgs &a, size_t lds, hipStream_t stream) {
  const int cls = (a.lp.d + 1023) / 1024;
  if (a.lp.x_f32) return cls <= 1 ? launch_cf<NB, NR, true, 1, 4>(a, lds, stream) : hipErrorNotSupported;
  if (cls <= 1) return launch_cf<NB, NR, false, 1, 4>(a, lds, stream);
  if (cls <= 2) return launch_cf<NB, NR, false, 2, 8>(a, lds, stream);
  if constexpr (NB == 1) {
    if (cls <= 3) return launch_cf<NB, NR, false, 3, 12>(a, lds, stream);
  }
  return hipErrorNotSupported;
}

}  // namespace

size_t decode_layer_sync_words() { return (size_t)kSyncWords; }

bool decode_layer_takes(int n_tokens, int top_k, int d_model) {
  return n_tokens >= 1 && n_tokens <= kMaxRows && top_k >= 1 && n_tokens * top_k <= kMaxPicks &&
         d_model >= 16 && d_model <= kMaxD;
}

size_t decode_layer_part_bytes(int n_tokens, int n_experts, int top_k, int d_model, int d_ff, int shared_d_ff) {
  if (!decode_layer_takes(n_tokens, top_k, d_model)) return 0;
  const long slots = std::min<long>(n_experts, (long)n_tokens * top_k);
  const long units = (shared_d_ff + kSlice - 1) / kSlice + slots * ((d_ff + kSlice - 1) / kSlice);
  return (size_t)units * kMaxRows * d_model * sizeof(uint64_t);
}

hipError_t decode_layer_init(int32_t *sync, void *part, size_t part_bytes, hipStream_t stream) {
  hipLaunchKernelGGL(k_zero_words, dim3((kSyncWords + 255) / 256), dim3(256), 0, stream, sync, kSyncWords);
  if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
  const long words = (long)(part_bytes / 4);
  if (part && words > 0) {
    const long blocks = std::min<long>((words + 255) / 256, 65535);
    hipLaunchKernelGGL(k_zero_words_long, dim3((unsigned)blocks), dim3(256), 0, stream, (int32_t *)part, words);
  }
  return hipGetLastError();
}

hipError_t launch_decode_layer(const DecodeLayerProblem &lp, hipStream_t stream) {
  StepArgs a{};
  a.lp = lp;
  const int d = lp.d, n = lp.n_tokens, K = lp.top_k, E = lp.n_experts;
  const bool swiglu = lp.act == EPI_SWIGLU;
  // the shared expert is relu^2: with a gated routed FFN it keeps its own launches
  if (!decode_layer_takes(n, K, d) || (swiglu && lp.has_shared) || d % 32 != 0) return hipErrorNotSupported;
  if (E < K || E > MOE_MAX_EXPERTS || lp.n_rows != n * K) return hipErrorNotSupported;
  if (lp.max_slots != std::min(E, lp.n_rows)) return hipErrorNotSupported;
  if (!lp.part) return hipErrorNotSupported;
  // it reads the repacked weights
  for (int i = 0; i < 2; ++i) {
    if (i == 0 && !lp.has_shared) continue;
    const ProjProblem &u = lp.up[i], &w = lp.down[i];
    if (!u.codes_packed || !u.scales_packed || !w.codes_packed || !w.scales_packed) return hipErrorNotSupported;
    if (u.k != d || w.n_w != d || w.n_out != d || w.k != u.n_out) return hipErrorNotSupported;
    if (u.n_out % 32 != 0 || u.n_w != (i == 1 && swiglu ? 2 : 1) * u.n_out) return hipErrorNotSupported;
  }
  if ((long)n * d * (lp.x_f32 ? 4 : 2) > (long)kXLoads * kThreads * 16) return hipErrorNotSupported;
  a.ns = lp.has_shared ? (lp.fs + kSlice - 1) / kSlice : 0;
  a.nr = (lp.f + kSlice - 1) / kSlice;
  a.dch = (d + 127) / 128;
  a.dblk = d / 16;
  // routing: the ranking passes with the fewest 16-key steps per thread (a
  // pass over items with 2^ps threads each, each comparing `share` keys of a
  // range of 2^ps * share; one extra step per barrier)
  {
    auto rup = [](int v, int m) { return (v + m - 1) / m * m; };
    auto plan = [&](int items, int range, int &ps, int &share) {  // returns steps per thread
      ps = 0;
      while (ps < 4 && (items << (ps + 1)) <= kThreads && (16 << (ps + 1)) <= rup(range, 16)) ++ps;
      share = rup(range, 16 << ps) >> ps;
      return (long)((items + (kThreads >> ps) - 1) / (kThreads >> ps)) * (share / 16);
    };
    int p, sh;
    long best = plan(n * E, E, p, sh);
    a.rk_two = 0;
    a.rk_p1 = p;
    a.rk_s1 = sh;
    a.rk_ep = sh << p;
    a.rk_gs = 0;
    a.rk_kc = a.rk_c = a.rk_cp = 0;
    a.rk_p2 = a.rk_s2 = 0;
    for (int gs = 4; (1 << gs) < E; ++gs) {
      const int G = 1 << gs, kc = std::min(K, G), C = ((E + G - 1) / G) * kc;
      if (C >= E) continue;
      int p1, s1, p2, s2;
      const long c1 = plan(n * E, G, p1, s1);
      if ((s1 << p1) != G) continue;  // the first pass's ranges must be the groups
      const long c2 = plan(n * C, C, p2, s2);
      if ((long)rup(C, 16) > kKeyRow || (long)(s2 << p2) > kKeyRow) continue;
      if (c1 + c2 + 1 < best) {
        best = c1 + c2 + 1;
        a.rk_two = 1;
        a.rk_gs = gs;
        a.rk_kc = kc;
        a.rk_c = C;
        a.rk_cp = s2 << p2;
        a.rk_ep = rup(E, G);
        a.rk_p1 = p1;
        a.rk_s1 = s1;
        a.rk_p2 = p2;
        a.rk_s2 = s2;
      }
    }
    if (a.rk_ep > kKeyRow) return hipErrorNotSupported;
  }
  a.sgroups = (std::max(a.ns, a.nr) + kSumGroup - 1) / kSumGroup;
  a.x_stride = a.dch * 128;
  a.x_lds = (int)((size_t)n * a.x_stride * (lp.x_f32 ? 4 : 2));
  const size_t reduce = (size_t)kMaxRows * (1 + MOE_MAX_TOPK) * (kRedCols / 2) * a.sgroups * 8 +
                        (size_t)kMaxRows * (1 + MOE_MAX_TOPK) * kRedCols * 4;
  a.sc_off = (int)((size_t)a.x_lds + std::max(scratch_bytes(swiglu ? 2 : 1), reduce));
  a.sc_off = (a.sc_off + 15) / 16 * 16;
  const size_t lds = (size_t)a.sc_off + (size_t)kWaves * kScW;
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidValue;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidValue;
  a.grid = cus;
  if (a.grid > kMaxGrid || a.grid < 1) return hipErrorNotSupported;
  // the reducer addresses the partial sums with 32-bit byte offsets
  const long units = a.ns + (long)lp.max_slots * a.nr;
  if (units * kMaxRows * d * 8 > 0x7FFFFFF0L) return hipErrorNotSupported;
  if (swiglu) return n == 1 ? launch_class<2, 1>(a, lds, stream) : launch_class<2, 2>(a, lds, stream);
  return n == 1 ? launch_class<1, 1>(a, lds, stream) : launch_class<1, 2>(a, lds, stream);
}

}  // namespace moe
