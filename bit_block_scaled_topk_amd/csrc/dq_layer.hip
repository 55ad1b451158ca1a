// dq_layer.hip -- a whole decode step (one or two tokens) of the MoE layer in
// ONE persistent launch: routing, the gather layout, the shared and routed
// experts' up projections (+ activation), their down projections, and the
// WeightedRowSum combine (gllm PR #91, "What changes"; Glq v0.2.13, "Remaining
// gap to bf16-native": a single-launch parallel-experts kernel is the way past
// per-expert launches).
//
// Work is split into 16-column tiles: every up tile of the shared expert and of
// each active routed expert, then every down tile.  One workgroup per CU (all
// resident).  Workgroups [0, gs) take the shared expert's tiles and the others
// the routed experts' (gs in proportion to the bytes), each a contiguous range
// of equal count.  Each workgroup requests all of its weights before it
// computes anything, so the whole weight stream is in flight at once and no
// tile waits out its own memory latency:
//   0  the logits and x, then the routing; the shared expert's workgroups
//      request their weights (step 1) before they route, the others after
//      (they need the picks).
//   1  up tiles' weights into registers, down tiles' weights into LDS (direct
//      global->LDS copies); wait.
//   2  compute the up tiles, store h (fp32); publish.
//   3  for each down tile: wait for its expert's h, copy those h rows into LDS
//      (once per expert), compute, store.
//   4  count the down tiles; the last producer of a 16-column block of the
//      output computes the combine for that block.
//
// With one or two tokens a 16-row matrix-core tile would be mostly padding, so
// the dot products run on the vector ALUs in fp32.  Half-wavefront hf of
// wavefront w owns row 2w + hf of every tile (one output column) and its lane
// c the 32-element k-groups c, c + 32, ...: the 32 lanes of a half read 512
// contiguous bytes of one weight row per load, from HBM (up tiles) or from LDS
// without bank conflicts (down tiles).  The FP4 converter gives the exact e2m1
// values, each 16-element block's sum is scaled by its e4m3 scale, and the 32
// lanes' sums are added by a fixed butterfly, so no workgroup-wide reduction
// is needed.  Activations staged in LDS (x for two tokens or fp32 x, and h)
// are transposed so that consecutive k-groups are 16 bytes apart.
//
// Results handed from one workgroup to another (h, the routed outputs yg, the
// shared expert's output) are stored and loaded with device-coherent accesses
// (relaxed agent-scope atomic stores and sc1 loads, which write through and
// read past the per-XCD L2s), and a tile is counted only after its stores have
// completed (s_waitcnt vmcnt(0)).  So no workgroup writes back or invalidates a
// whole L2: an agent-scope fence costs tens of nanoseconds, serialised per
// XCD, per call.
//
// Routing comes first and is done by every workgroup for itself (one or two
// tokens: a wavefront per token, top-K then softmax over the picks), followed
// by the packed-row layout of the gather (expert ascending, token ascending
// within an expert), kept in LDS; workgroup 0 also stores the routing and
// layout views.  So a step is this one launch.
//
// Flags and counters live at the start of the caller's workspace; they are
// zeroed once (decode_layer_init) and each launch leaves them ready for the
// next, so no launch has to clear them:
//   up_flag[w]  workgroup w's launch count: w reads its own flag e at start
//               (every flag holds the same count between launches) and stores
//               e + 1 once its up tiles are stored; a down tile of an expert
//               waits until the flags of the workgroups that own that
//               expert's up tiles read e + 1 (plain flags, one per workgroup:
//               counters that hundreds of workgroups increment serialise on
//               one address).
//   ct_done[c]  down tiles finished for output column block c (one counter per
//               64 bytes); the workgroup that finishes the last of them resets
//               it to zero and computes out = shared + sum_j w_j * y_j for
//               those 16 columns, j in order.
// Every wait is bounded (kSpinLimit sleeps); on expiry the error word is set
// (it stays set) and the workgroup goes on, so the kernel always finishes and
// every flag and counter still ends as described.  No workgroup waits before
// it has published all of its up tiles, so every wait ends once the whole grid
// is resident (the host checks that with the occupancy query).
#include <algorithm>

#include "launch.hpp"
#include "nvfp4_device.hpp"

namespace moe {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSpinLimit = 1 << 22;
constexpr int kSc1 = 16;               // cache-policy bit of a buffer load: device-coherent access
constexpr int kLdsLimit = 160 * 1024;  // LDS of one CU
constexpr int kStaticLds = 11 * 1024;  // the kernel's own LDS arrays (checked exactly at launch)
constexpr int kMaxUp = 4;              // up tiles one workgroup holds in registers
constexpr int kMaxDown = 64;           // down tiles of one workgroup
constexpr int kMaxRows = 2;            // token rows of the vector dot products
constexpr int kXChunks = 4;            // 16-byte chunks of x per thread
constexpr int kHReg = 2;               // one token: h k-group iterations kept in registers
constexpr int kMaxGrid = 1024;         // workgroups (one per CU)
constexpr int kCtStride = 16;          // words between column counters: one counter per 64 bytes (atomics
                                       // to one cache line serialise)
constexpr int kMaxCt = 1024;           // column blocks: d <= 16384
constexpr int kMaxPicks = kMaxRows * MOE_MAX_TOPK;  // routed rows of a step (<= 64: one wavefront)
constexpr int kSyncWords = 2 + kMaxGrid + kMaxCt * kCtStride;
constexpr int kLogitsPerThread = kMaxRows * MOE_MAX_EXPERTS / kThreads;

struct LayerArgs {
  DecodeLayerProblem lp;
  int up_tiles[2];      // 16-column tiles per expert of the up projections
  int down_tiles;       // d / 16
  int n_up, n_down;     // tiles in the two lists
  long down_bytes[2];   // LDS bytes of one down tile's weights (shared, routed)
  int grid;
  int gs;               // workgroups [0, gs) take the shared expert's tiles, the rest the routed ones
  int x_lds, h_lds;     // LDS bytes of x and of one expert's h (fp32)
  int us_lds, us_blk;   // LDS bytes of the up tiles' scales, and of one 16-row block of them
};

struct Tile {
  int prob;  // 0 shared, 1 routed
  int slot;
  int tile;
};

// i-th tile of the up list: the shared expert's tiles, then slot by slot.
__device__ __forceinline__ Tile up_tile(const LayerArgs &a, int i) {
  const int ups = a.lp.has_shared ? a.up_tiles[0] : 0;
  if (i < ups) return Tile{0, 0, i};
  const int r = i - ups, s = r / a.up_tiles[1];
  return Tile{1, s, r - s * a.up_tiles[1]};
}

__device__ __forceinline__ Tile down_tile(const LayerArgs &a, int i) {
  const int ds = a.lp.has_shared ? a.down_tiles : 0;
  if (i < ds) return Tile{0, 0, i};
  const int r = i - ds, s = r / a.down_tiles;
  return Tile{1, s, r - s * a.down_tiles};
}

// Item range [first, last) of member v of a group of g that splits n items.
__host__ __device__ __forceinline__ void split_range(int v, int g, int n, int &first, int &last) {
  first = (int)((long)v * n / g);
  last = (int)((long)(v + 1) * n / g);
}

// The member of a group of g splitting n items that holds item i.
__host__ __device__ __forceinline__ int split_owner(int i, int n, int g) {
  int w = (int)((long)i * g / n);
  while (w + 1 < g && (long)(w + 1) * n / g <= i) ++w;
  while (w > 0 && (long)w * n / g > i) --w;
  return w;
}

// Tile ranges of workgroup w in a list of n_sh shared-expert tiles followed by
// n - n_sh routed ones: workgroups [0, gs) split the shared tiles, the others
// the routed tiles (both with equal counts; the tiles of a group are alike).
__host__ __device__ __forceinline__ void group_range(int w, int grid, int gs, int n_sh, int n, int &first,
                                                     int &last) {
  if (w < gs) {
    split_range(w, gs, n_sh, first, last);
  } else {
    split_range(w - gs, grid - gs, n - n_sh, first, last);
    first += n_sh;
    last += n_sh;
  }
}

__host__ __device__ __forceinline__ int group_owner(int i, int grid, int gs, int n_sh, int n) {
  return i < n_sh ? split_owner(i, n_sh, gs) : gs + split_owner(i - n_sh, n - n_sh, grid - gs);
}

__host__ __device__ __forceinline__ long round_kb(long b) { return (b + 1023) / 1024 * 1024; }

// LDS bytes of one down tile's weights: 16 code rows, then 16 scale rows.
__host__ __device__ __forceinline__ long down_tile_bytes(int k) {
  return round_kb(16L * (k / 2)) + round_kb(16L * (k / 16));
}

// The fields of one projection that a tile reads.  Tiles pick the shared or
// the routed view with selects: indexing the argument struct by a run-time
// value would make the compiler read it from memory inside the tile loop.
struct ProbView {
  const uint8_t *codes, *scales;
  const float *global;
  const int32_t *row_map;
  float *h;  // fp32 h of this expert group (up: written; down: read)
  int n_w, k, n_out, known_rows, ldh;
};

__device__ __forceinline__ ProbView view_of(const ProjProblem &p, float *h, int ldh) {
  return ProbView{p.codes, p.scales, p.global, p.row_map, h, p.n_w, p.k, p.n_out, p.known_rows, ldh};
}

__device__ __forceinline__ ProbView pick(bool first, const ProbView &a, const ProbView &b) {
  ProbView r;
  r.codes = first ? a.codes : b.codes;
  r.scales = first ? a.scales : b.scales;
  r.global = first ? a.global : b.global;
  r.row_map = first ? a.row_map : b.row_map;
  r.h = first ? a.h : b.h;
  r.n_w = first ? a.n_w : b.n_w;
  r.k = first ? a.k : b.k;
  r.n_out = first ? a.n_out : b.n_out;
  r.known_rows = first ? a.known_rows : b.known_rows;
  r.ldh = first ? a.ldh : b.ldh;
  return r;
}

// A lane's codes of one up tile: k-group iterations i = 0..KI-1 of NB rows
// (NB = 2 for SwiGLU: the gate row and the up row).  (The tile's scales are
// copied to LDS: 16 contiguous rows, a few 16-byte loads per tile instead of a
// 2-byte load per lane and group.)
template <int NB, int KI>
struct RowW {
  u32x4_t wq[NB][KI];
};

// Issue the code loads of this lane's k-groups of one up tile (no waits): lane
// c of half hf reads k-groups c + 32 i of row 2 * wave + hf; the 32 lanes of a
// half read 512 contiguous bytes per load.  Groups past the row repeat its
// last group (their scale is zeroed where they are used).
template <int NB, int KI>
__device__ __forceinline__ void issue_rows(const ProbView &p, int e, int tile, int lane, int wave, RowW<NB, KI> &R) {
  const int c = lane & 31;
  const int G = p.k >> 5;
  const int col = min(tile * 16 + 2 * wave + (lane >> 5), p.n_out - 1);
  const size_t crow = (size_t)(p.k >> 1);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const size_t wr = (size_t)e * p.n_w + (size_t)col + (size_t)b * p.n_out;
    const uint8_t *wrow = p.codes + wr * crow;
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int gc = min(c + 32 * i, G - 1);
      R.wq[b][i] = *(const u32x4_t *)(wrow + (size_t)gc * 16);
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_cvoid;

// Copy `bytes` (a multiple of 16) to LDS dst with direct loads: each
// instruction of wavefront w moves 64 16-byte chunks (lane l: chunk cw + l,
// cw = 64 w + 512 j); lanes past the end reload the last chunk into the
// rounding (dst is rounded up to whole 1 KB).  COH: device-coherent (sc1) loads
// through `rsrc` at byte offset src_off; else plain loads from src.
template <bool COH>
__device__ __forceinline__ void copy_to_lds(const uint8_t *src, __amdgpu_buffer_rsrc_t rsrc, uint32_t src_off,
                                            long bytes, uint8_t *dst, int wave, int lane) {
  const int total = (int)(bytes >> 4);
  for (int cw = wave * 64; cw < total; cw += kThreads) {
    const int c = min(cw + lane, total - 1);
    lds_void *d = (lds_void *)(dst + (size_t)cw * 16);
    if (COH)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, d, 16, src_off + (uint32_t)c * 16, 0, 0, kSc1);
    else
      __builtin_amdgcn_global_load_lds((global_cvoid *)(src + (size_t)c * 16), d, 16, 0, 0);
  }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void *base, size_t bytes) {
  const int n = bytes > 0x7FFFFFF0u ? (int)0x7FFFFFF0u : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// Workgroup barrier for LDS only: unlike __syncthreads it does not wait for
// this wavefront's outstanding global loads and stores.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ void memory_done() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every copy, load and store of this wavefront has completed
  __syncthreads();
}

// 16 e2m1 codes (two words, element 0 in the low nibble of byte 0) times 16
// fp32 activations: four chains of four elements in order, then
// (c0 + c1) + (c2 + c3) -- four independent chains keep the FMA pipeline busy.
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

__device__ __forceinline__ float dot16(uint32_t w0, uint32_t w1, const float *x) {
  return dot16v(w0, w1, *(const f32x4_t *)(x), *(const f32x4_t *)(x + 4), *(const f32x4_t *)(x + 8),
                *(const f32x4_t *)(x + 12));
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

// 16-byte chunk t (0..7) of k-group g of row r of an activation staged in
// LDS (G k-groups per row): consecutive groups are 16 bytes apart, so the
// lanes of a half-wavefront read consecutive chunks.
__device__ __forceinline__ int tchunk(int r, int t, int g, int G) { return (r * 8 + t) * G + g; }

// acc + s0 * (codes 0..15 . x 0..15) + s1 * (codes 16..31 . x 16..31), x from
// row r of a transposed LDS activation.
__device__ __forceinline__ float dot32_lds(const u32x4_t &w, float s0, float s1, const f32x4_t *xs, int r, int g,
                                           int G, float acc) {
  acc = fmaf(s0, dot16v(w.x, w.y, xs[tchunk(r, 0, g, G)], xs[tchunk(r, 1, g, G)], xs[tchunk(r, 2, g, G)],
                        xs[tchunk(r, 3, g, G)]),
             acc);
  return fmaf(s1, dot16v(w.z, w.w, xs[tchunk(r, 4, g, G)], xs[tchunk(r, 5, g, G)], xs[tchunk(r, 6, g, G)],
                         xs[tchunk(r, 7, g, G)]),
              acc);
}

// Sum over the 32 lanes of a half-wavefront, by a fixed butterfly: every lane
// ends with the same bits.
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o, 32);
  return v;
}

// The output of a column from its sums: gl * a (EPI_F32), relu(gl * a)^2, or
// silu(gl * a) * (gl * b) (SwiGLU, a the gate row).
template <int EPI>
__device__ __forceinline__ float epilogue(float gl, float a, float b) {
  if (EPI == EPI_F32) return gl * a;
  if (EPI == EPI_RELU2) {
    float u = gl * a;
    u = u > 0.f ? u : 0.f;
    return u * u;
  }
  const float av = gl * a, bv = gl * b;
  return (av / (1.0f + expf(-av))) * bv;
}

// Wavefront-wide wait until flags[w_lo .. w_hi] all read `target` (lane l
// polls w_lo + l, + 64, ...).  Bounded: on expiry the error word is set.
__device__ __forceinline__ void wait_flags(const int32_t *flags, int w_lo, int w_hi, int32_t target, int lane,
                                           int32_t *err) {
  for (int base = w_lo; base <= w_hi; base += 64) {
    const int w = base + lane;
    int spins = 0;
    while (!__all(w > w_hi || __hip_atomic_load(flags + w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == target)) {
      if (++spins > kSpinLimit) {
        if (lane == 0) __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
      }
      __builtin_amdgcn_s_sleep(2);
    }
  }
}

// NB: weight rows per lane of an up tile (2 for SwiGLU); KU: k-group iterations
// of an up tile per lane; X_F32: x is fp32 (else bf16); XREG: one token with
// bf16 x -- each lane keeps its k-groups of x, and of an expert's h, in
// registers, loaded once (activations from LDS would be read once per tile by
// all 16 column lanes, which the LDS bandwidth cannot sustain).
template <int NB, int KU, int EPI_UP, bool X_F32, bool XREG>
__global__ void __launch_bounds__(kThreads) k_decode_layer(LayerArgs a) {
  extern __shared__ u32x4_t s_dyn[];  // x [n][d] f32 | h [rows][k] f32 | down weights
  __shared__ int s_e[kMaxPicks], s_r0[kMaxPicks], s_rows[kMaxPicks];  // per slot: expert, first row, rows
  __shared__ int s_id[kMaxPicks], s_prow[kMaxPicks];                      // per pick t*K+j: expert, packed row
  __shared__ float s_pw[kMaxPicks];                                        // ... and routing weight
  __shared__ float s_lsel[kMaxPicks];                                      // ... and logit
  __shared__ __attribute__((aligned(16))) float s_logit[kMaxRows * MOE_MAX_EXPERTS];  // [n][E rounded up to 4]
  __shared__ int s_rt[kMaxPicks];                                          // token of each packed row
  __shared__ int s_nact;
  __shared__ float s_dgl[kMaxDown];  // globals of this workgroup's down tiles
  __shared__ int s_last[kMaxDown];   // 1: this workgroup combines that tile's 16 columns
  const DecodeLayerProblem &lp = a.lp;
  const int tid = threadIdx.x, lane = tid & 63, c32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rowl = 2 * wave + (lane >> 5);  // this lane's row of every tile
  int32_t *err = lp.sync;
  int32_t *up_flag = lp.sync + 2;
  int32_t *ct_done = up_flag + kMaxGrid;
  f32x4_t *s_x = (f32x4_t *)s_dyn;  // transposed (tchunk)
  f32x4_t *s_h = (f32x4_t *)((uint8_t *)s_dyn + a.x_lds);
  uint8_t *s_us = (uint8_t *)s_dyn + a.x_lds + a.h_lds;  // [kMaxUp][NB] 16-row blocks of up scales
  uint8_t *s_w = s_us + a.us_lds;                          // down tiles: codes, then scales
  const int n = lp.n_tokens;
  const int Gx = lp.d >> 5;  // k-groups of x

  // this workgroup's tiles: the shared expert's (blockIdx.x < gs) or routed ones
  const int ups = lp.has_shared ? a.up_tiles[0] : 0;
  const int n_sd = lp.has_shared ? a.down_tiles : 0;
  const bool shared_wg = blockIdx.x < a.gs;
  int u_first, u_last, d_first, d_last;
  group_range(blockIdx.x, a.grid, a.gs, ups, a.n_up, u_first, u_last);
  group_range(blockIdx.x, a.grid, a.gs, n_sd, a.n_down, d_first, d_last);

  // the logits first: routing is the first step on the critical path
  const int E = lp.n_experts, K = lp.top_k, P = n * K, NE = n * E;
  const int Epad = (E + 3) & ~3;
  float lg[kLogitsPerThread];
#pragma unroll
  for (int i = 0; i < kLogitsPerThread; ++i) {
    const int c = tid + kThreads * i;
    lg[i] = lp.logits[min(c, NE - 1)];
  }

  // x: XREG: this lane's k-groups into registers (bf16), else all of x
  // (written to LDS as fp32 after the wait)
  u32x4_t xv[XREG ? 1 : kXChunks];
  u32x4_t xb[XREG ? KU : 1][4];
  const int x_chunks = X_F32 ? n * lp.d / 4 : n * lp.d / 8;
  if constexpr (XREG) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int g = min(c32 + 32 * i, Gx - 1);
#pragma unroll
      for (int t = 0; t < 4; ++t) xb[i][t] = *((const u32x4_t *)lp.x + g * 4 + t);
    }
  } else {
#pragma unroll
    for (int j = 0; j < kXChunks; ++j) {
      const int c = tid + kThreads * j;
      if (c < x_chunks) xv[j] = *((const u32x4_t *)lp.x + c);
    }
  }

  // this launch's count: the value every flag holds until its owner finishes
  // its up tiles (read early, used late)
  const int32_t epoch = __hip_atomic_load(&up_flag[blockIdx.x], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // the four projections, read once
  const ProbView U0 = view_of(lp.up[0], lp.h[0], lp.fs), U1 = view_of(lp.up[1], lp.h[1], lp.f);
  const ProbView D0 = view_of(lp.down[0], lp.h[0], lp.fs), D1 = view_of(lp.down[1], lp.h[1], lp.f);
  int n_active = 0;  // distinct routed experts, once routed
  auto expert_of = [&](const Tile &t, const ProbView &p, int &e, int &r0, int &rows) -> bool {
    if (t.prob == 0) {
      e = 0;
      r0 = 0;
      rows = p.known_rows;
      return true;
    }
    if (t.slot >= n_active) return false;
    e = s_e[t.slot];
    r0 = s_r0[t.slot];
    rows = s_rows[t.slot];
    return true;
  };

  // ---- 1. up weights (registers), each up tile's global and token rows, then
  //         the down weights (LDS) and globals
  //  The loads are issued without branches (an absent tile loads expert 0's
  //  first tile), and nothing loaded is used before the wait: a value merged
  //  across branches, or used at once, makes the compiler wait for every load
  //  issued before it.
  RowW<NB, KU> RU[kMaxUp];
  float ugl[kMaxUp];
  int utok[kMaxUp][kMaxRows];  // token of each row of the tile's expert
  bool uok[kMaxUp];
  float dgl = 0.f;  // thread i: global of down tile d_first + i
  auto route = [&]() {
    // routing (the pages' rule: top-K by logit, the lower index first among
    // equal logits, weights a softmax over the picks).  The rank of expert e
    // among token t's logits is the number of experts that beat it; the experts
    // of rank < K are the picks, slot = rank.  Threads split each expert's
    // comparisons into `parts` interleaved 16-byte chunks of LDS.
#pragma unroll
    for (int i = 0; i < kLogitsPerThread; ++i) {
      const int c = tid + kThreads * i;
      if (c < NE) {
        const int t = c >= E, e = c - t * E;
        s_logit[t * Epad + e] = lg[i];
      }
    }
    {  // padding: -inf at an index past E never beats an expert
      const int padw = Epad - E;
      if (padw > 0 && tid < n * padw) {
        const int t = tid >= padw;
        s_logit[t * Epad + E + tid - t * padw] = -__builtin_inff();
      }
    }
    lds_barrier();
    {
      int parts = 1;
      while (parts < 16 && 2 * parts * NE <= kThreads) parts <<= 1;
      const int part = tid & (parts - 1);
      for (int pr = tid / parts; pr - tid / parts < NE; pr += kThreads / parts) {
        const bool ok = pr < NE;
        const int t = ok && pr >= E, e = ok ? pr - t * E : 0;
        const float *row = s_logit + t * Epad;
        const float v = row[e];
        int cnt = 0;
        for (int c = part; 4 * c < E; c += parts) {
          const f32x4_t w4 = *(const f32x4_t *)(row + 4 * c);
          const int e0 = 4 * c;
          cnt += (w4.x > v) | ((w4.x == v) & (e0 < e));
          cnt += (w4.y > v) | ((w4.y == v) & (e0 + 1 < e));
          cnt += (w4.z > v) | ((w4.z == v) & (e0 + 2 < e));
          cnt += (w4.w > v) | ((w4.w == v) & (e0 + 3 < e));
        }
        for (int o = 1; o < parts; o <<= 1) cnt += __shfl_xor(cnt, o, 64);
        if (ok && part == 0 && cnt < K) {
          s_id[t * K + cnt] = e;
          s_lsel[t * K + cnt] = v;
        }
      }
    }
    lds_barrier();
    // weights and gather layout (picks in wavefront 0, P <= 64): rows grouped by
    // expert in ascending id, tokens ascending within an expert; a slot per
    // distinct expert, in ascending id
    if (wave == 0) {
      const bool ok = lane < P;
      const int t = lane >= K;
      const int e = ok ? s_id[lane] : 0x7FFFFFFF;
      const float l = ok ? s_lsel[lane] : 0.f;
      const float l0 = s_lsel[ok ? t * K : 0];
      const float ex = ok ? expf(l - l0) : 0.f;
      float sum0 = 0.f, sum1 = 0.f;  // in slot order
      for (int j = 0; j < K; ++j) {
        sum0 += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), j));
        if (n > 1) sum1 += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ex), K + j));
      }
      // other: the other token picked e too
      int other = 0;
      for (int q = 0; q < P; ++q) other |= ((q >= K) != t) & (__builtin_amdgcn_readlane(e, q) == e);
      const unsigned long long both = __ballot(ok && t == 0 && other);  // token 0's picks shared with token 1
      int below = 0, dup_below = 0;
      for (int q = 0; q < P; ++q) {
        const int eq = __builtin_amdgcn_readlane(e, q);
        below += eq < e;
        dup_below += (int)((both >> q) & 1ull) & (eq < e);
      }
      if (ok) {
        s_pw[lane] = ex / (t ? sum1 : sum0);
        const int r = below + (t == 1 && other);
        s_prow[lane] = r;
        s_rt[r] = t;
        if (t == 0 || !other) {
          const int slot = below - dup_below;
          s_e[slot] = e;
          s_r0[slot] = below;
          s_rows[slot] = 1 + (t == 0 && other);
        }
      }
      if (lane == 0) s_nact = P - __popcll(both);
    }
    lds_barrier();
    n_active = s_nact;
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
  };
  auto issue = [&]() {
#pragma unroll
    for (int u = 0; u < kMaxUp; ++u) {
      const int ui = min(u_first + u, a.n_up - 1);
      const Tile t = up_tile(a, ui);
      const ProbView p = pick(t.prob == 0, U0, U1);
      int e = 0, r0 = 0, rows = 0;
      uok[u] = u_first + u < u_last && expert_of(t, p, e, r0, rows);
      if (!uok[u]) e = 0, r0 = 0;
      issue_rows<NB, KU>(p, e, uok[u] ? t.tile : 0, lane, wave, RU[u]);
      if (uok[u]) {
        const __amdgpu_buffer_rsrc_t none = coherent_rsrc(lp.x, 16);  // unused by plain copies
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const size_t row0 = (size_t)e * p.n_w + (size_t)t.tile * 16 + (size_t)b * p.n_out;
          copy_to_lds<false>(p.scales + row0 * (p.k / 16), none, 0, 16L * (p.k / 16),
                             s_us + (size_t)(u * NB + b) * a.us_blk, wave, lane);
        }
      }
      ugl[u] = p.global[e];
#pragma unroll
      for (int r = 0; r < kMaxRows; ++r) utok[u][r] = s_rt[min(r0 + r, P - 1)];
    }
    // thread i: the global of down tile d_first + i
    if (tid < d_last - d_first) {
      const Tile t = down_tile(a, d_first + tid);
      const ProbView p = pick(t.prob == 0, D0, D1);
      int e, r0, rows;
      if (expert_of(t, p, e, r0, rows)) dgl = p.global[e];
    }
  };
  // the down tiles' weights into LDS
  auto issue_down = [&]() {
    long off = 0;
    const __amdgpu_buffer_rsrc_t none = coherent_rsrc(lp.x, 16);  // unused by plain copies
    for (int i = d_first; i < d_last; ++i) {
      const Tile t = down_tile(a, i);
      const ProbView p = pick(t.prob == 0, D0, D1);
      int e, r0, rows;
      if (!expert_of(t, p, e, r0, rows)) continue;
      const size_t row0 = (size_t)e * p.n_w + (size_t)t.tile * 16;
      const long cb = 16L * (p.k / 2), sb = 16L * (p.k / 16);
      copy_to_lds<false>(p.codes + row0 * (p.k / 2), none, 0, cb, s_w + off, wave, lane);
      copy_to_lds<false>(p.scales + row0 * (p.k / 16), none, 0, sb, s_w + off + round_kb(cb), wave, lane);
      off += round_kb(cb) + round_kb(sb);
    }
  };
  // The shared expert's tiles need no routing: their workgroups request their
  // weights first and route while they stream in.
  if (shared_wg) {
    issue();
    issue_down();
    route();
  } else {
    route();
    issue();
    issue_down();
  }
  memory_done();
  if (tid < d_last - d_first) s_dgl[tid] = dgl;
#pragma unroll
  for (int j = 0; j < (XREG ? 0 : kXChunks); ++j) {
    const int c = tid + kThreads * j;
    if (c >= x_chunks) break;
    if (X_F32) {
      const int e0 = 4 * c, r = e0 / lp.d, col = e0 - r * lp.d;
      s_x[tchunk(r, (col & 31) >> 2, col >> 5, Gx)] = __builtin_bit_cast(f32x4_t, xv[j]);
    } else {
      const int e0 = 8 * c, r = e0 / lp.d, col = e0 - r * lp.d;
      f32x4_t lo, hi;  // bf16 -> f32: the bits in the upper half
      lo.x = __uint_as_float(xv[j].x << 16);
      lo.y = __uint_as_float(xv[j].x & 0xFFFF0000u);
      lo.z = __uint_as_float(xv[j].y << 16);
      lo.w = __uint_as_float(xv[j].y & 0xFFFF0000u);
      hi.x = __uint_as_float(xv[j].z << 16);
      hi.y = __uint_as_float(xv[j].z & 0xFFFF0000u);
      hi.z = __uint_as_float(xv[j].w << 16);
      hi.w = __uint_as_float(xv[j].w & 0xFFFF0000u);
      s_x[tchunk(r, (col & 31) >> 2, col >> 5, Gx)] = lo;
      s_x[tchunk(r, ((col & 31) >> 2) + 1, col >> 5, Gx)] = hi;
    }
  }
  lds_barrier();

  // ---- 2. up tiles; publish them once their h stores have completed
#pragma unroll
  for (int u = 0; u < kMaxUp; ++u) {
    if (!uok[u]) continue;  // uniform
    const Tile t = up_tile(a, u_first + u);
    const ProbView p = pick(t.prob == 0, U0, U1);
    int e, r0, rows;
    expert_of(t, p, e, r0, rows);
    float acc[kMaxRows][NB];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r)
#pragma unroll
      for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int g = c32 + 32 * i, gc = min(g, Gx - 1);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        float s0, s1;
        e4m3x2_to_f32(*(const uint16_t *)(s_us + (size_t)(u * NB + b) * a.us_blk + rowl * (Gx * 2) + gc * 2), s0,
                      s1);
        if (g >= Gx) s0 = s1 = 0.f;  // a repeated group
        const u32x4_t w = RU[u].wq[b][i];
        if constexpr (XREG) {
          acc[0][b] = fmaf(s0, dot16_bf16(w.x, w.y, xb[i][0], xb[i][1]), acc[0][b]);
          acc[0][b] = fmaf(s1, dot16_bf16(w.z, w.w, xb[i][2], xb[i][3]), acc[0][b]);
        } else {
#pragma unroll
          for (int r = 0; r < kMaxRows; ++r) {
            if (r >= rows) break;  // uniform
            // x row: token r for the shared expert, the row's token for a routed one
            const int xr = t.prob == 0 ? r : max(utok[u][r], 0);
            acc[r][b] = dot32_lds(w, s0, s1, s_x, xr, gc, Gx, acc[r][b]);
          }
        }
      }
      // one k-group's activations in registers at a time
      if constexpr (!XREG) __builtin_amdgcn_sched_barrier(0);
    }
    const int col = t.tile * 16 + rowl;
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) {
      if (r >= rows) break;  // uniform
      const float v0 = half_sum(acc[r][0]);
      const float v1 = NB > 1 ? half_sum(acc[r][NB - 1]) : 0.f;
      if (c32 == 0 && col < p.n_out)
        __hip_atomic_store(p.h + (size_t)(r0 + r) * p.ldh + col, epilogue<EPI_UP>(ugl[u], v0, v1), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  memory_done();
  if (tid == 0) __hip_atomic_store(&up_flag[blockIdx.x], epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- 3. down tiles, each once its expert's h is complete
  long off = 0;
  int staged = -1;  // problem slot whose h is in LDS
  bool use_hreg = false;
  f32x4_t hreg[XREG ? kHReg : 1][8];  // XREG: this lane's k-groups of the staged h
  for (int i = d_first; i < d_last; ++i) {
    const Tile t = down_tile(a, i);
    const ProbView p = pick(t.prob == 0, D0, D1);
    int e, r0, rows;
    if (!expert_of(t, p, e, r0, rows)) continue;
    const int G = p.k >> 5;
    const int pslot = t.prob == 0 ? 0 : 1 + t.slot;
    if (pslot != staged) {
      if (wave == 0) {
        // the owners of this expert's up tiles
        const int u0 = t.prob == 0 ? 0 : ups + t.slot * a.up_tiles[1];
        const int u1 = u0 + a.up_tiles[t.prob] - 1;
        wait_flags(up_flag, group_owner(u0, a.grid, a.gs, ups, a.n_up), group_owner(u1, a.grid, a.gs, ups, a.n_up),
                   epoch + 1, lane, err);
      }
      __syncthreads();  // also: every wavefront is done with the previous h
      // h rows [r0, r0 + rows), device-coherent loads, transposed into LDS
      const long hrows = t.prob == 0 ? n : lp.n_rows;
      const __amdgpu_buffer_rsrc_t hr = coherent_rsrc(p.h, (size_t)hrows * p.ldh * 4);
      const int cpr = p.k >> 2, nq = rows * cpr;  // 16-byte chunks per row, in all
      for (int q0 = 0; q0 < nq; q0 += kThreads * 2) {  // two loads in flight per thread
        u32x4_t v[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int q = min(q0 + kThreads * j + tid, nq - 1), r = q / cpr, rem = q - r * cpr;
          v[j] = __builtin_amdgcn_raw_buffer_load_b128(hr, (uint32_t)(((size_t)(r0 + r) * p.ldh) * 4 + rem * 16), 0,
                                                       kSc1);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int q = q0 + kThreads * j + tid, r = q / cpr, rem = q - r * cpr;
          if (q < nq) s_h[tchunk(r, rem & 7, rem >> 3, G)] = __builtin_bit_cast(f32x4_t, v[j]);
        }
      }
      lds_barrier();
      staged = pslot;
      use_hreg = XREG && G <= 32 * kHReg;
      if (XREG && use_hreg) {
#pragma unroll
        for (int ii = 0; ii < kHReg; ++ii) {
          const int gc = min(c32 + 32 * ii, G - 1);
#pragma unroll
          for (int t4 = 0; t4 < 8; ++t4) hreg[ii][t4] = s_h[tchunk(0, t4, gc, G)];
        }
      }
    }
    const long cb = round_kb(16L * (p.k / 2));
    const uint8_t *wrow = s_w + off + (size_t)rowl * (p.k / 2);
    const uint8_t *srow = s_w + off + cb + (size_t)rowl * (p.k / 16);
    float acc[kMaxRows];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) acc[r] = 0.f;
    if (XREG && use_hreg) {
#pragma unroll
      for (int ii = 0; ii < kHReg; ++ii) {
        if (32 * ii >= G) break;  // uniform
        const int g = c32 + 32 * ii, gc = min(g, G - 1);
        const u32x4_t w = *(const u32x4_t *)(wrow + gc * 16);
        float s0, s1;
        e4m3x2_to_f32(*(const uint16_t *)(srow + gc * 2), s0, s1);
        if (g >= G) s0 = s1 = 0.f;
        acc[0] = fmaf(s0, dot16v(w.x, w.y, hreg[ii][0], hreg[ii][1], hreg[ii][2], hreg[ii][3]), acc[0]);
        acc[0] = fmaf(s1, dot16v(w.z, w.w, hreg[ii][4], hreg[ii][5], hreg[ii][6], hreg[ii][7]), acc[0]);
      }
    } else {
      for (int g0 = 0; g0 < G; g0 += 32) {
        const int g = g0 + c32, gc = min(g, G - 1);
        const u32x4_t w = *(const u32x4_t *)(wrow + gc * 16);
        float s0, s1;
        e4m3x2_to_f32(*(const uint16_t *)(srow + gc * 2), s0, s1);
        if (g >= G) s0 = s1 = 0.f;
#pragma unroll
        for (int r = 0; r < kMaxRows; ++r) {
          if (r >= rows) break;  // uniform
          acc[r] = dot32_lds(w, s0, s1, s_h, r, gc, G, acc[r]);
        }
      }
    }
    float *dst = t.prob == 0 ? lp.out : lp.yg;
    const int col = t.tile * 16 + rowl;
    const float gl = s_dgl[i - d_first];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) {
      if (r >= rows) break;  // uniform
      const float v = half_sum(acc[r]);
      if (c32 == 0 && col < p.n_out)
        __hip_atomic_store(dst + (size_t)(r0 + r) * lp.d + col, gl * v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    off += cb + round_kb(16L * (p.k / 16));
  }

  // ---- 4. count the down tiles once their stores have completed; the last
  //         producer of a 16-column block computes its combine, in slot order
  //         (one thread per tile and per output element: the round trips
  //         overlap instead of following one another)
  memory_done();
  const int nd_mine = d_last - d_first;
  for (int i = tid; i < nd_mine; i += kThreads) {
    const Tile t = down_tile(a, d_first + i);
    int last = 0;
    if (t.prob == 0 || t.slot < n_active) {
      int32_t *ct = &ct_done[t.tile * kCtStride];
      const int old = __hip_atomic_fetch_add(ct, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last = old == lp.has_shared + n_active - 1;
      if (last) __hip_atomic_store(ct, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // ready for the next launch
    }
    s_last[i] = last;
  }
  __syncthreads();
  {
    for (int j2 = tid; j2 < nd_mine * n * 16; j2 += kThreads) {
      const int i = j2 / (n * 16), rem = j2 - i * (n * 16);
      if (!s_last[i]) continue;
      const int tok = rem >> 4, c = down_tile(a, d_first + i).tile * 16 + (rem & 15);
      if (c >= lp.d) continue;
      float *o = lp.out + (size_t)tok * lp.d + c;
      const float sh = lp.has_shared ? __hip_atomic_load(o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0.f;
      float accw = 0.f;
      // the routed outputs in groups of eight: their loads in flight together
      for (int j0 = 0; j0 < K; j0 += 8) {
        float y[8];
        int ok[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int j = j0 + jj;
          ok[jj] = j < K;
          y[jj] = ok[jj] ? __hip_atomic_load(lp.yg + (size_t)s_prow[tok * K + j] * lp.d + c, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT)
                         : 0.f;
        }
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          if (ok[jj]) accw = fmaf(s_pw[tok * K + j0 + jj], y[jj], accw);
      }
      *o = lp.has_shared ? sh + accw : accw;
    }
  }
}

__global__ void k_zero_words(int32_t *w, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) w[i] = 0;
}

template <int NB, int KU, int EPI, bool XF, bool XR>
hipError_t launch_one(LayerArgs &a, size_t lds, hipStream_t stream) {
  static int occ = -1;  // same code object on every device
  static size_t occ_lds = 0, static_lds = 0;
  if (occ < 0) {
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, (const void *)k_decode_layer<NB, KU, EPI, XF, XR>) != hipSuccess)
      return hipErrorInvalidValue;
    static_lds = attr.sharedSizeBytes;
  }
  if (lds + static_lds > (size_t)kLdsLimit) return hipErrorNotSupported;
  if (occ < 0 || occ_lds != lds) {
    int o = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&o, k_decode_layer<NB, KU, EPI, XF, XR>, kThreads, lds) !=
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
  hipLaunchKernelGGL((k_decode_layer<NB, KU, EPI, XF, XR>), dim3(a.grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int NB, int KU, int EPI>
hipError_t launch_x(LayerArgs &a, bool xreg, size_t lds, hipStream_t stream) {
  if (xreg) return launch_one<NB, KU, EPI, false, true>(a, lds, stream);
  return a.lp.x_f32 ? launch_one<NB, KU, EPI, true, false>(a, lds, stream)
                    : launch_one<NB, KU, EPI, false, false>(a, lds, stream);
}

}  // namespace

size_t decode_layer_sync_words() { return (size_t)kSyncWords; }

bool decode_layer_takes(int n_tokens, int top_k, int d_model) {
  return n_tokens >= 1 && n_tokens <= kMaxRows && top_k >= 1 && n_tokens * top_k <= kMaxPicks &&
         d_model >= 16 && (d_model + 15) / 16 <= kMaxCt;
}

hipError_t decode_layer_init(int32_t *sync, hipStream_t stream) {
  hipLaunchKernelGGL(k_zero_words, dim3((kSyncWords + 255) / 256), dim3(256), 0, stream, sync, kSyncWords);
  return hipGetLastError();
}

hipError_t launch_decode_layer(const DecodeLayerProblem &lp, hipStream_t stream) {
  LayerArgs a;
  a.lp = lp;
  const int d = lp.d, n = lp.n_tokens;
  a.up_tiles[0] = (lp.up[0].n_out + 15) / 16;
  a.up_tiles[1] = (lp.up[1].n_out + 15) / 16;
  a.down_tiles = (d + 15) / 16;
  a.n_up = (lp.has_shared ? a.up_tiles[0] : 0) + lp.max_slots * a.up_tiles[1];
  a.n_down = (lp.has_shared ? a.down_tiles : 0) + lp.max_slots * a.down_tiles;
  const bool swiglu = lp.act == EPI_SWIGLU;
  // the shared expert is relu^2: with a gated routed FFN it keeps its own launches
  if (!decode_layer_takes(n, lp.top_k, d) || (swiglu && lp.has_shared) || d % 32 != 0) return hipErrorNotSupported;
  // it reads the canonical layout: weights given only as repacked copies take
  // the per-step launches
  for (int i = 0; i < 2; ++i) {
    if (i == 0 && !lp.has_shared) continue;
    if (!lp.up[i].codes || !lp.up[i].scales || !lp.down[i].codes || !lp.down[i].scales) return hipErrorNotSupported;
  }
  if (lp.n_experts < lp.top_k || lp.n_experts > MOE_MAX_EXPERTS || lp.n_rows != n * lp.top_k)
    return hipErrorNotSupported;
  if (lp.max_slots != (lp.n_experts < lp.n_rows ? lp.n_experts : lp.n_rows)) return hipErrorNotSupported;
  if ((long)n * d * (lp.x_f32 ? 4 : 2) > 16L * kThreads * kXChunks) return hipErrorNotSupported;
  // k-group iterations of an up tile per lane (32 lanes per row)
  const int ku = (d / 32 + 31) / 32;
  long h_lds = 0;
  a.down_bytes[0] = 0;
  for (int i = 0; i < 2; ++i) {
    if (i == 0 && !lp.has_shared) continue;
    if (lp.up[i].k != d || lp.down[i].n_out != d || lp.down[i].k % 32 != 0) return hipErrorNotSupported;
    a.down_bytes[i] = down_tile_bytes(lp.down[i].k);
    const long hb = round_kb((long)n * lp.down[i].k * 4);
    h_lds = hb > h_lds ? hb : h_lds;
  }
  // coherent loads of h use 32-bit byte offsets
  if ((long)lp.n_rows * lp.f * 4 > 0x7FFFFFF0L || (long)n * lp.fs * 4 > 0x7FFFFFF0L) return hipErrorNotSupported;
  const int n_sd = lp.has_shared ? a.down_tiles : 0;
  const int ups = lp.has_shared ? a.up_tiles[0] : 0;
  // one token, bf16 x: x in registers
  const bool xreg = n == 1 && !lp.x_f32;
  a.x_lds = xreg ? 0 : (int)round_kb((long)n * d * 4);
  a.h_lds = (int)h_lds;
  a.us_blk = (int)round_kb(16L * (d / 16));
  a.us_lds = kMaxUp * (swiglu ? 2 : 1) * a.us_blk;
  for (int i = 0; i < 2; ++i)  // whole 16-row tiles
    if (lp.up[i].n_out % 16 != 0 || lp.down[i].n_out % 16 != 0) return hipErrorNotSupported;
  // one workgroup per CU
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidValue;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidValue;
  a.grid = cus;
  if (a.grid > kMaxGrid || a.grid < 2) return hipErrorNotSupported;
  // Workgroups for the shared expert in proportion to its bytes (it is
  // requested while the others route); the nearest split that fits.
  const long wb_sh = lp.has_shared ? (long)a.up_tiles[0] * down_tile_bytes(lp.up[0].k) + (long)n_sd * a.down_bytes[0]
                                   : 0;
  const long wb_rt = (long)lp.max_slots * ((long)a.up_tiles[1] * down_tile_bytes(lp.up[1].k) * (swiglu ? 2 : 1) +
                                           (long)a.down_tiles * a.down_bytes[1]);
  const int gs0 = lp.has_shared ? (int)((a.grid * wb_sh + (wb_sh + wb_rt) / 2) / (wb_sh + wb_rt)) : 0;
  // the largest share of a group of g splitting n items
  auto most = [](int n_items, int g) { return g > 0 ? (n_items + g - 1) / g : 0; };
  long w_lds = -1;
  for (int dg = 0; dg < a.grid && w_lds < 0; ++dg) {
    for (int sgn = 0; sgn < 2 && w_lds < 0; ++sgn) {
      if (sgn == 1 && dg == 0) continue;
      const int gs = lp.has_shared ? gs0 + (sgn ? -dg : dg) : 0;
      if (lp.has_shared && (gs < 1 || gs > a.grid - 1)) continue;
      const int gr = a.grid - gs;
      const int up_most = std::max(most(ups, gs), most(a.n_up - ups, gr));
      const int dn_most = std::max(most(n_sd, gs), most(a.n_down - n_sd, gr));
      const long worst =
          std::max((long)most(n_sd, gs) * a.down_bytes[0], (long)most(a.n_down - n_sd, gr) * a.down_bytes[1]);
      if (up_most <= kMaxUp && dn_most <= kMaxDown && a.x_lds + a.h_lds + a.us_lds + worst + kStaticLds <= kLdsLimit) {
        a.gs = gs;
        w_lds = worst;
      }
    }
    if (!lp.has_shared) break;
  }
  if (w_lds < 0) return hipErrorNotSupported;
  const long lds = a.x_lds + a.h_lds + a.us_lds + w_lds;  // the kernel's static LDS is added in launch_one
  if (lds > kLdsLimit) return hipErrorNotSupported;
  if (swiglu) {
    if (ku <= 1) return launch_x<2, 1, EPI_SWIGLU>(a, xreg, (size_t)lds, stream);
    if (ku <= 2) return launch_x<2, 2, EPI_SWIGLU>(a, xreg, (size_t)lds, stream);
    if (ku <= 4) return launch_x<2, 4, EPI_SWIGLU>(a, xreg, (size_t)lds, stream);
    return hipErrorNotSupported;
  }
  if (ku <= 1) return launch_x<1, 1, EPI_RELU2>(a, xreg, (size_t)lds, stream);
  if (ku <= 2) return launch_x<1, 2, EPI_RELU2>(a, xreg, (size_t)lds, stream);
  if (ku <= 3) return launch_x<1, 3, EPI_RELU2>(a, xreg, (size_t)lds, stream);
  if (ku <= 4) return launch_x<1, 4, EPI_RELU2>(a, xreg, (size_t)lds, stream);
  return hipErrorNotSupported;
}

}  // namespace moe
