// dq_layer.hip -- the expert FFN of a decode step (one or two tokens) in ONE
// persistent launch: the shared and routed experts' up projections (+
// activation), their down projections, and the WeightedRowSum combine (gllm PR
// #91, "What changes"; Glq v0.2.13, "Remaining gap to bf16-native": a
// single-launch parallel-experts kernel is the way past per-expert launches).
//
// Work is split into 16-column tiles: every up tile of the shared expert and of
// each active routed expert, then every down tile.  One workgroup per CU (all
// resident); workgroup w owns a contiguous range of the up tiles (equal counts)
// and a contiguous range of the down tiles (equal bytes).  Each workgroup
// requests all of its weights before it computes anything, so the whole weight
// stream is in flight at once and no tile waits out its own memory latency:
//   1  x (registers, then LDS as fp32), its up tiles' weights (registers), its
//      down tiles' weights (direct global->LDS copies); wait.
//   2  compute the up tiles, store h (fp32); count each on its expert's
//      counter.
//   3  for each down tile: wait for its expert's h, copy those h rows into LDS
//      (once per expert), compute, store.
//   4  count the down tiles; the last producer of a 16-column block of the
//      output computes the combine for that block.
// (Vector memory results return in issue order, so step 2 could not start
// before the down weights land anyway.)
//
// With one or two tokens a 16-row matrix-core tile would be mostly padding, so
// the dot products run on the vector ALUs in fp32: lane (n = lane%16, q =
// lane/16) owns column n of the tile and, per iteration, k-group gb + 4i + q of
// its wavefront's slice of K; the FP4 converter gives the exact e2m1 values;
// each 16-element block's partial sum is scaled by its e4m3 scale; the four
// q-lanes and then the eight wavefronts are summed in a fixed order.
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
#include "launch.hpp"
#include "nvfp4_device.hpp"
#include "route_device.hpp"

namespace moe {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kSpinLimit = 1 << 22;
constexpr int kSc1 = 16;               // cache-policy bit of a buffer load: device-coherent access
constexpr int kLdsLimit = 160 * 1024;  // LDS of one CU
constexpr int kMaxUp = 4;              // up tiles one workgroup holds in registers
constexpr int kMaxDown = 64;           // down tiles of one workgroup
constexpr int kMaxRows = 2;            // token rows of the vector dot products
constexpr int kXChunks = 4;            // 16-byte chunks of x per thread
constexpr int kKD = 2;                 // k-group iterations of a down tile with h in registers
constexpr int kKDMax = 4;              // ... with the rest read from LDS (one-token path)
constexpr int kBatch = 4;              // one-token tiles whose sums are reduced together
constexpr int kMaxGrid = 1024;         // workgroups (one per CU)
constexpr int kCtStride = 16;          // words between column counters: one counter per 64 bytes (atomics
                                       // to one cache line serialise)
constexpr int kMaxCt = 1024;           // column blocks: d <= 16384
constexpr int kMaxPicks = kMaxRows * MOE_MAX_TOPK;  // routed rows of a step (<= 64: one wavefront)
constexpr int kSyncWords = 2 + kMaxGrid + kMaxCt * kCtStride;

struct LayerArgs {
  DecodeLayerProblem lp;
  int up_tiles[2];      // 16-column tiles per expert of the up projections
  int down_tiles;       // d / 16
  int n_up, n_down;     // tiles in the two lists
  long down_bytes[2];   // LDS bytes of one down tile's weights (shared, routed)
  long down_total;      // LDS bytes of the whole down list
  int grid;
  int x_lds, h_lds;     // LDS bytes of x and of one expert's h (fp32)
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

// Byte offset of down tile i in the list (shared tiles first).
__host__ __device__ __forceinline__ long down_prefix(int i, int n_shared_tiles, const long *bytes) {
  return i <= n_shared_tiles ? (long)i * bytes[0]
                             : (long)n_shared_tiles * bytes[0] + (long)(i - n_shared_tiles) * bytes[1];
}

// First down tile whose offset is >= byte position pos.
__host__ __device__ __forceinline__ int down_first_at(long pos, int n_shared_tiles, int n_down, const long *bytes) {
  const long sb = (long)n_shared_tiles * bytes[0];
  long t;
  if (pos <= sb)
    t = bytes[0] > 0 ? (pos + bytes[0] - 1) / bytes[0] : 0;
  else
    t = n_shared_tiles + (pos - sb + bytes[1] - 1) / bytes[1];
  return (int)(t < n_down ? t : n_down);
}

// Down tiles [first, last) of workgroup w: those whose offsets fall in
// [w * total / G, (w + 1) * total / G).
__host__ __device__ __forceinline__ void down_range(int w, int grid, int n_shared_tiles, int n_down,
                                                    const long *bytes, long total, int &first, int &last) {
  first = down_first_at(total * w / grid, n_shared_tiles, n_down, bytes);
  last = down_first_at(total * (w + 1) / grid, n_shared_tiles, n_down, bytes);
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

template <int NB, int KNI>
struct WRegs {
  u32x4_t wq[NB][KNI];
  uint32_t sc[NB][KNI];
};

// Issue the weight loads of this lane's k-groups of one up tile (no waits).
// NB = 2 (SwiGLU): rows col and col + n_out (gate and up) per lane.
template <int NB, int KNI>
__device__ __forceinline__ void issue_weights(const ProbView &p, int e, int tile, int lane, int wave,
                                              WRegs<NB, KNI> &R) {
  const int nl = lane & 15, q = lane >> 4;
  const int G = p.k >> 5;
  const int gpw = (G + kWaves - 1) / kWaves;
  const int gb = wave * gpw;
  const int ge = min(G, gb + gpw);
  const int col = min(tile * 16 + nl, p.n_out - 1);
  const size_t crow = (size_t)(p.k >> 1), srow = (size_t)(p.k >> 4);
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const size_t wr = (size_t)e * p.n_w + (size_t)col + (size_t)b * p.n_out;
    const uint8_t *wrow = p.codes + wr * crow;
    const uint8_t *sptr = p.scales + wr * srow;
#pragma unroll
    for (int i = 0; i < KNI; ++i) {
      const int gc = max(min(gb + 4 * i + q, ge - 1), 0);
      R.wq[b][i] = *(const u32x4_t *)(wrow + (size_t)gc * 16);
      R.sc[b][i] = *(const uint16_t *)(sptr + (size_t)gc * 2);
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

__device__ __forceinline__ void memory_done() {
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): every copy, load and store of this wavefront has completed
  __syncthreads();
}

// Weights of a tile for one k-group: from registers (up tiles) or from the LDS
// copy of the tile (down tiles: 16 code rows of k/2 bytes, then 16 scale rows
// of k/16 bytes).
template <int NB, int KNI>
struct RegB {
  const WRegs<NB, KNI> &R;
  __device__ __forceinline__ void get(int b, int i, int, u32x4_t &wq, uint32_t &sc) const {
    wq = R.wq[b][i];
    sc = R.sc[b][i];
  }
};
struct LdsB {
  const uint8_t *codes, *scales;  // this lane's row
  __device__ __forceinline__ void get(int, int, int g, u32x4_t &wq, uint32_t &sc) const {
    wq = *(const u32x4_t *)(codes + g * 16);
    sc = *(const uint16_t *)(scales + g * 2);
  }
};

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

// Sum a tile's per-lane partials in a fixed order -- the four q-lanes
// ((q0 + q1) + (q2 + q3)), then the wavefronts 0 + 1 + ... + 7 -- and store
// output row r (< rows) at dst[(r0 + r) * ldo + column] (device-coherent):
// gl * sum, or its activation (EPI_RELU2 / EPI_SWIGLU).  Ends with a
// workgroup barrier.
template <int NB, int EPI>
__device__ __forceinline__ void reduce_store(float (&acc)[kMaxRows][NB], int rows, int n_out, float gl, int tile,
                                             float *dst, long ldo, int r0, int lane, int wave, float *s_red) {
  const int nl = lane & 15, q = lane >> 4;
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float v = acc[r][b];
      v += __shfl_xor(v, 16, 64);
      v += __shfl_xor(v, 32, 64);
      if (q == 0) s_red[((wave * kMaxRows + r) * NB + b) * 16 + nl] = v;
    }
  __syncthreads();
  if (wave == 0 && lane < 16) {
    const int col = tile * 16 + nl;
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) {
      if (r >= rows) break;
      float sum[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        sum[b] = s_red[(r * NB + b) * 16 + nl];
        for (int w = 1; w < kWaves; ++w) sum[b] += s_red[((w * kMaxRows + r) * NB + b) * 16 + nl];
      }
      float v;
      if (EPI == EPI_F32) {
        v = gl * sum[0];
      } else if (EPI == EPI_RELU2) {
        float u = gl * sum[0];
        u = u > 0.f ? u : 0.f;
        v = u * u;
      } else {
        const float av = gl * sum[0];
        const float bv = gl * sum[NB - 1];
        v = (av / (1.0f + expf(-av))) * bv;
      }
      if (col < n_out)
        __hip_atomic_store(dst + (size_t)(r0 + r) * ldo + col, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();  // s_red and the staged operands are reused next
}

// Lane (n, q) of wavefront w: k-group gb + 4i + q of the wavefront's slice.
struct KSlice {
  int gb, ge;
  __device__ __forceinline__ KSlice(int k, int wave) {
    const int G = k >> 5;
    const int gpw = (G + kWaves - 1) / kWaves;
    gb = wave * gpw;
    ge = min(G, gb + gpw);
  }
};

// One 16-column tile on the vector ALUs, activations from LDS: row r (< rows)
// of the tile is LDS row xrow[r] of xs (pitch ldx floats).  KNI > 0: at most
// KNI k-group iterations, unrolled (register weights); KNI == 0: a loop (LDS
// weights).
template <int NB, int KNI, int EPI, typename WSrc>
__device__ __forceinline__ void tile_dot(int k, int n_out, float gl, int rows, const int *xrow, const float *xs,
                                         int ldx, int tile, float *dst, long ldo, int r0, int lane, int wave,
                                         const WSrc &ws, float *s_red) {
  const int q = lane >> 4;
  const KSlice ks(k, wave);
  float acc[kMaxRows][NB];
#pragma unroll
  for (int r = 0; r < kMaxRows; ++r)
#pragma unroll
    for (int b = 0; b < NB; ++b) acc[r][b] = 0.f;
  auto body = [&](int i) {
    const int g = ks.gb + 4 * i + q;
    if (g >= ks.ge) return;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      u32x4_t wq;
      uint32_t sc;
      ws.get(b, i, g, wq, sc);
      float s0, s1;
      e4m3x2_to_f32(sc, s0, s1);
#pragma unroll
      for (int r = 0; r < kMaxRows; ++r) {
        if (r >= rows) break;  // uniform
        const float *x = xs + (size_t)xrow[r] * ldx + g * 32;
        acc[r][b] = fmaf(s0, dot16(wq[0], wq[1], x), acc[r][b]);
        acc[r][b] = fmaf(s1, dot16(wq[2], wq[3], x + 16), acc[r][b]);
      }
    }
  };
  if constexpr (KNI > 0) {
#pragma unroll
    for (int i = 0; i < KNI; ++i) {
      if (ks.gb + 4 * i >= ks.ge) break;  // uniform
      body(i);
    }
  } else {
    for (int i = 0; ks.gb + 4 * i < ks.ge; ++i) body(i);
  }
  reduce_store<NB, EPI>(acc, rows, n_out, gl, tile, dst, ldo, r0, lane, wave, s_red);
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

// Per-tile outputs of a batch (one token), for the threads that sum them (in
// LDS: written by thread 0 before the batch's first barrier).
struct BatchOut {
  float *dst[kBatch];
  float gl[kBatch];
  int col0[kBatch], n_out[kBatch], valid[kBatch];
};

// Sum the partials of a batch of up to kBatch one-token tiles and store them:
// every lane writes its partial per tile, then thread (t, n) adds the 32
// partials of column n of tile t in a fixed order (wavefronts 0..7, in each the
// q-lanes 0..3) and stores gl * sum, or its activation, device-coherently.  One
// LDS round and two barriers per batch instead of per tile.
template <int NB, int EPI>
__device__ __forceinline__ void reduce_store_batch(const float (&acc)[kBatch][NB], const BatchOut &bo, int tid,
                                                   int lane, int wave, float *s_red) {
#pragma unroll
  for (int t = 0; t < kBatch; ++t)
#pragma unroll
    for (int b = 0; b < NB; ++b) s_red[((t * NB + b) * kWaves + wave) * 64 + lane] = acc[t][b];
  __syncthreads();
  if (tid < kBatch * 16) {
    const int t = tid >> 4, nl = tid & 15;
    if (bo.valid[t]) {
      float sum[NB];
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const float *sr = s_red + (size_t)(t * NB + b) * kWaves * 64 + nl;
        float pv[kWaves * 4];  // all loads first: one LDS latency, not 32
#pragma unroll
        for (int w = 0; w < kWaves; ++w)
#pragma unroll
          for (int q = 0; q < 4; ++q) pv[w * 4 + q] = sr[w * 64 + q * 16];
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < kWaves * 4; ++j) v += pv[j];
        sum[b] = v;
      }
      const float gl = bo.gl[t];
      float v;
      if (EPI == EPI_F32) {
        v = gl * sum[0];
      } else if (EPI == EPI_RELU2) {
        float u = gl * sum[0];
        u = u > 0.f ? u : 0.f;
        v = u * u;
      } else {
        const float av = gl * sum[0];
        const float bv = gl * sum[NB - 1];
        v = (av / (1.0f + expf(-av))) * bv;
      }
      const int col = bo.col0[t] + nl;
      if (col < bo.n_out[t]) __hip_atomic_store(bo.dst[t] + col, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __syncthreads();  // s_red is reused next
}

// Partial sums of one up tile of a one-token step with bf16 x held in
// registers: xb[i] is the 32 bf16 values of this lane's i-th k-group.
template <int NB, int KU>
__device__ __forceinline__ void partial_xreg(int k, const u32x4_t (&xb)[KU][4], int lane, int wave,
                                             const WRegs<NB, KU> &R, float (&acc)[NB]) {
  const int q = lane >> 4;
  const KSlice ks(k, wave);
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = 0.f;
#pragma unroll
  for (int i = 0; i < KU; ++i) {
    if (ks.gb + 4 * i >= ks.ge) break;  // uniform
    if (ks.gb + 4 * i + q >= ks.ge) continue;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      float s0, s1;
      e4m3x2_to_f32(R.sc[b][i], s0, s1);
      acc[b] = fmaf(s0, dot16_bf16(R.wq[b][i][0], R.wq[b][i][1], xb[i][0], xb[i][1]), acc[b]);
      acc[b] = fmaf(s1, dot16_bf16(R.wq[b][i][2], R.wq[b][i][3], xb[i][2], xb[i][3]), acc[b]);
    }
  }
}

// Partial sum of one down tile of a one-token step: this lane's first KD
// k-groups of h (fp32) are held in registers (xh[i]: 32 floats), later ones are
// read from the staged h in LDS; weights from LDS.
template <int KD>
__device__ __forceinline__ float partial_hreg(int k, const f32x4_t (&xh)[KD][8], const float *s_h, int lane,
                                              int wave, const LdsB &ws) {
  const int q = lane >> 4;
  const KSlice ks(k, wave);
  float acc = 0.f;
  u32x4_t wqs[kKDMax];  // every k-group's weights first: one LDS latency per tile
  uint32_t scs[kKDMax];
#pragma unroll
  for (int i = 0; i < kKDMax; ++i) ws.get(0, i, max(min(ks.gb + 4 * i + q, ks.ge - 1), 0), wqs[i], scs[i]);
#pragma unroll
  for (int i = 0; i < kKDMax; ++i) {
    if (ks.gb + 4 * i >= ks.ge) break;  // uniform
    const int g = ks.gb + 4 * i + q;
    if (g >= ks.ge) continue;
    const u32x4_t wq = wqs[i];
    float s0, s1;
    e4m3x2_to_f32(scs[i], s0, s1);
    if (i < KD) {
      acc = fmaf(s0, dot16v(wq[0], wq[1], xh[i][0], xh[i][1], xh[i][2], xh[i][3]), acc);
      acc = fmaf(s1, dot16v(wq[2], wq[3], xh[i][4], xh[i][5], xh[i][6], xh[i][7]), acc);
    } else {
      acc = fmaf(s0, dot16(wq[0], wq[1], s_h + g * 32), acc);
      acc = fmaf(s1, dot16(wq[2], wq[3], s_h + g * 32 + 16), acc);
    }
  }
  return acc;
}

// The workgroup whose up range [w n_up / G, (w + 1) n_up / G) holds tile i.
__device__ __forceinline__ int up_owner(int i, int n_up, int grid) {
  int w = (int)((long)i * grid / n_up);
  while (w + 1 < grid && (long)(w + 1) * n_up / grid <= i) ++w;
  while (w > 0 && (long)w * n_up / grid > i) --w;
  return w;
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
  __shared__ int s_id[kMaxPicks], s_prow[kMaxPicks], s_both[kMaxPicks];   // per pick t*K+j: expert, packed row
  __shared__ float s_pw[kMaxPicks];                                        // ... and routing weight
  __shared__ int s_rt[kMaxPicks];                                          // token of each packed row
  __shared__ int s_nact;
  __shared__ float s_dgl[kMaxDown];  // globals of this workgroup's down tiles
  __shared__ int s_last[kMaxDown];   // 1: this workgroup combines that tile's 16 columns
  __shared__ float s_red[XREG ? kBatch * NB * kWaves * 64 : kWaves * kMaxRows * NB * 16];
  __shared__ BatchOut s_bo;
  const DecodeLayerProblem &lp = a.lp;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int32_t *err = lp.sync;
  int32_t *up_flag = lp.sync + 2;
  int32_t *ct_done = up_flag + kMaxGrid;
  float *s_x = (float *)s_dyn;
  float *s_h = (float *)((uint8_t *)s_dyn + a.x_lds);
  uint8_t *s_w = (uint8_t *)s_dyn + a.x_lds + a.h_lds;
  const int n = lp.n_tokens;

  // this workgroup's tiles
  const int u_first = (int)((long)blockIdx.x * a.n_up / a.grid);
  const int u_last = (int)((long)(blockIdx.x + 1) * a.n_up / a.grid);
  const int n_sd = lp.has_shared ? a.down_tiles : 0;
  int d_first, d_last;
  down_range(blockIdx.x, a.grid, n_sd, a.n_down, a.down_bytes, a.down_total, d_first, d_last);

  // x: issued first; XREG: this lane's k-groups into registers, else all of x
  // (written to LDS as fp32 after the wait)
  u32x4_t xv[XREG ? 1 : kXChunks];
  u32x4_t xb[XREG ? KU : 1][4];
  const int x_chunks = X_F32 ? n * lp.d / 4 : n * lp.d / 8;
  if constexpr (XREG) {
    const KSlice ks(lp.d, wave);
#pragma unroll
    for (int i = 0; i < KU; ++i) {
      const int g = max(min(ks.gb + 4 * i + (lane >> 4), ks.ge - 1), 0);
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

  // routing: wavefront t picks token t's top-K experts and their weights
  const int E = lp.n_experts, K = lp.top_k, P = n * K;
  if (wave < n) {
    int my_id;
    float my_w;
    route_one_token_any(lp.logits + (size_t)wave * E, E, K, lane, my_id, my_w);
    if (lane < K) {
      s_id[wave * K + lane] = my_id;
      s_pw[wave * K + lane] = my_w;
    }
  }
  __syncthreads();
  // gather layout (picks in wavefront 0, P <= 64): rows grouped by expert in
  // ascending id, tokens ascending within an expert; a slot per distinct
  // expert, in ascending id.  s_both[p]: token 0's pick p is also token 1's.
  if (tid < P) {
    const int e = s_id[tid], t = tid >= K;
    int other = 0;
    for (int q = t ? 0 : K; q < (t ? K : P); ++q) other |= s_id[q] == e;
    s_both[tid] = t == 0 && other;
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the flags are written
    __builtin_amdgcn_wave_barrier();
    int below = 0, dup_below = 0, n_dup = 0;
    for (int q = 0; q < P; ++q) {
      const int eq = s_id[q], bq = q < K ? s_both[q] : 0;
      below += eq < e;
      dup_below += bq && eq < e;
      n_dup += bq;
    }
    const int r = below + (t == 1 && other);
    s_prow[tid] = r;
    s_rt[r] = t;
    if (t == 0 || !other) {
      const int slot = below - dup_below;
      s_e[slot] = e;
      s_r0[slot] = below;
      s_rows[slot] = 1 + (t == 0 && other);
    }
    if (tid == 0) s_nact = P - n_dup;
  }
  __syncthreads();
  const int n_active = s_nact;

  // the four projections, read once
  const ProbView U0 = view_of(lp.up[0], lp.h[0], lp.fs), U1 = view_of(lp.up[1], lp.h[1], lp.f);
  const ProbView D0 = view_of(lp.down[0], lp.h[0], lp.fs), D1 = view_of(lp.down[1], lp.h[1], lp.f);
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
  WRegs<NB, KU> RU[kMaxUp];
  float ugl[kMaxUp];
  int utok[kMaxUp][kMaxRows];  // token of each row of the tile's expert
  bool uok[kMaxUp];
#pragma unroll
  for (int u = 0; u < kMaxUp; ++u) {
    const int ui = min(u_first + u, a.n_up - 1);
    const Tile t = up_tile(a, ui);
    const ProbView p = pick(t.prob == 0, U0, U1);
    int e = 0, r0 = 0, rows = 0;
    uok[u] = u_first + u < u_last && expert_of(t, p, e, r0, rows);
    if (!uok[u]) e = 0, r0 = 0;
    issue_weights<NB, KU>(p, e, uok[u] ? t.tile : 0, lane, wave, RU[u]);
    ugl[u] = p.global[e];
#pragma unroll
    for (int r = 0; r < kMaxRows; ++r) utok[u][r] = s_rt[min(r0 + r, P - 1)];
  }
  float dgl = 0.f;  // thread i: global of down tile d_first + i
  {
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
      if (tid == i - d_first) dgl = p.global[e];
    }
  }
  // workgroup 0: the routing and layout views, while the weights stream in
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
  memory_done();
  if (tid < d_last - d_first) s_dgl[tid] = dgl;
#pragma unroll
  for (int j = 0; j < (XREG ? 0 : kXChunks); ++j) {
    const int c = tid + kThreads * j;
    if (c >= x_chunks) break;
    if (X_F32) {
      *((u32x4_t *)s_x + c) = xv[j];
    } else {
      f32x4_t lo, hi;  // bf16 -> f32: the bits in the upper half
      lo.x = __uint_as_float(xv[j].x << 16);
      lo.y = __uint_as_float(xv[j].x & 0xFFFF0000u);
      lo.z = __uint_as_float(xv[j].y << 16);
      lo.w = __uint_as_float(xv[j].y & 0xFFFF0000u);
      hi.x = __uint_as_float(xv[j].z << 16);
      hi.y = __uint_as_float(xv[j].z & 0xFFFF0000u);
      hi.z = __uint_as_float(xv[j].w << 16);
      hi.w = __uint_as_float(xv[j].w & 0xFFFF0000u);
      *((f32x4_t *)s_x + 2 * c) = lo;
      *((f32x4_t *)s_x + 2 * c + 1) = hi;
    }
  }
  __syncthreads();

  // ---- 2. up tiles; count them once their h stores have completed
  if constexpr (XREG) {
    static_assert(kMaxUp <= kBatch, "the up tiles form one batch");
    float uacc[kBatch][NB];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (tid == 0) s_bo.valid[u] = 0;
#pragma unroll
      for (int b = 0; b < NB; ++b) uacc[u][b] = 0.f;
      if (u >= kMaxUp || !uok[u]) continue;
      const Tile t = up_tile(a, u_first + u);
      const ProbView p = pick(t.prob == 0, U0, U1);
      int e, r0, rows;
      expert_of(t, p, e, r0, rows);
      partial_xreg<NB, KU>(p.k, xb, lane, wave, RU[u], uacc[u]);
      if (tid == 0) {
        s_bo.valid[u] = 1;
        s_bo.dst[u] = p.h + (size_t)r0 * p.ldh;
        s_bo.gl[u] = ugl[u];
        s_bo.col0[u] = t.tile * 16;
        s_bo.n_out[u] = p.n_out;
      }
    }
    reduce_store_batch<NB, EPI_UP>(uacc, s_bo, tid, lane, wave, s_red);
  }
#pragma unroll
  for (int u = 0; u < kMaxUp; ++u) {
    if (XREG || !uok[u]) continue;
    const Tile t = up_tile(a, u_first + u);
    const ProbView p = pick(t.prob == 0, U0, U1);
    int e, r0, rows;
    expert_of(t, p, e, r0, rows);
    {
      int xr[kMaxRows];  // x rows: tokens 0..n-1 for the shared expert, row_token for a routed one
#pragma unroll
      for (int r = 0; r < kMaxRows; ++r) xr[r] = t.prob == 0 ? r : max(utok[u][r], 0);
      tile_dot<NB, KU, EPI_UP>(p.k, p.n_out, ugl[u], rows, xr, s_x, lp.d, t.tile, p.h, p.ldh, r0, lane, wave,
                               RegB<NB, KU>{RU[u]}, s_red);
    }
  }
  memory_done();
  if (tid == 0) __hip_atomic_store(&up_flag[blockIdx.x], epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  // ---- 3. down tiles, each once its expert's h is complete
  long off = 0;
  int staged = -1;  // problem slot whose h is in LDS
  const int hrow[kMaxRows] = {0, 1};
  f32x4_t hreg[XREG ? kKD : 1][8];  // XREG: this lane's k-groups of the staged h
  // XREG: down tiles of one expert are summed in batches
  float dacc[kBatch][1];
#pragma unroll
  for (int c = 0; c < kBatch; ++c) dacc[c][0] = 0.f;
  int nb = 0;
  auto flush = [&]() {
    if (nb == 0) return;
    if (tid == 0)  // slots past nb hold no tile of this batch
      for (int c = nb; c < kBatch; ++c) s_bo.valid[c] = 0;
    reduce_store_batch<1, EPI_F32>(dacc, s_bo, tid, lane, wave, s_red);
    nb = 0;
  };
  for (int i = d_first; i < d_last; ++i) {
    const Tile t = down_tile(a, i);
    const ProbView p = pick(t.prob == 0, D0, D1);
    int e, r0, rows;
    if (!expert_of(t, p, e, r0, rows)) continue;
    const int pslot = t.prob == 0 ? 0 : 1 + t.slot;
    if (pslot != staged) {
      if (XREG) flush();
      if (wave == 0) {
        // the owners of this expert's up tiles
        const int ups = lp.has_shared ? a.up_tiles[0] : 0;
        const int u0 = t.prob == 0 ? 0 : ups + t.slot * a.up_tiles[1];
        const int u1 = u0 + a.up_tiles[t.prob] - 1;
        wait_flags(up_flag, up_owner(u0, a.n_up, a.grid), up_owner(u1, a.n_up, a.grid), epoch + 1, lane, err);
      }
      __syncthreads();
      const long ldh = p.ldh;
      const long hrows = t.prob == 0 ? n : lp.n_rows;
      const __amdgpu_buffer_rsrc_t hr = coherent_rsrc(p.h, (size_t)hrows * ldh * 4);
      copy_to_lds<true>(nullptr, hr, (uint32_t)((size_t)r0 * ldh * 4), (long)rows * ldh * 4, (uint8_t *)s_h, wave,
                        lane);
      memory_done();
      staged = pslot;
      if constexpr (XREG) {
        const KSlice ks(p.k, wave);
#pragma unroll
        for (int i = 0; i < kKD; ++i) {
          const int g = max(min(ks.gb + 4 * i + (lane >> 4), ks.ge - 1), 0);
#pragma unroll
          for (int t4 = 0; t4 < 8; ++t4) hreg[i][t4] = *((const f32x4_t *)s_h + g * 8 + t4);
        }
      }
    }
    const long cb = round_kb(16L * (p.k / 2));
    const LdsB bsrc{s_w + off + (size_t)(lane & 15) * (p.k / 2), s_w + off + cb + (size_t)(lane & 15) * (p.k / 16)};
    float *dst = t.prob == 0 ? lp.out : lp.yg;
    if constexpr (XREG) {
      const float pv = partial_hreg<kKD>(p.k, hreg, s_h, lane, wave, bsrc);
      const float gl = s_dgl[i - d_first];
#pragma unroll
      for (int c = 0; c < kBatch; ++c)
        if (c == nb) dacc[c][0] = pv;
      if (tid == 0) {
        s_bo.valid[nb] = 1;
        s_bo.dst[nb] = dst + (size_t)r0 * lp.d;
        s_bo.gl[nb] = gl;
        s_bo.col0[nb] = t.tile * 16;
        s_bo.n_out[nb] = p.n_out;
      }
      if (++nb == kBatch) flush();
    } else {
      tile_dot<1, 0, EPI_F32>(p.k, p.n_out, s_dgl[i - d_first], rows, hrow, s_h, p.k, t.tile, dst, lp.d, r0, lane,
                              wave, bsrc, s_red);
    }
    off += cb + round_kb(16L * (p.k / 16));
  }
  if (XREG) flush();

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
  if (lp.n_experts < lp.top_k || lp.n_experts > MOE_MAX_EXPERTS || lp.n_rows != n * lp.top_k)
    return hipErrorNotSupported;
  if (lp.max_slots != (lp.n_experts < lp.n_rows ? lp.n_experts : lp.n_rows)) return hipErrorNotSupported;
  if ((long)n * d * (lp.x_f32 ? 4 : 2) > 16L * kThreads * kXChunks) return hipErrorNotSupported;
  // k-group iterations of an up tile per lane
  const int ku = ((d / 32 + kWaves - 1) / kWaves + 3) / 4;
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
  a.down_total = down_prefix(a.n_down, n_sd, a.down_bytes);
  // one token, bf16 x, every down tile within kKD iterations: activations in registers
  bool xreg = n == 1 && !lp.x_f32;
  for (int i = 0; i < 2; ++i)
    if ((i == 1 || lp.has_shared) && ((lp.down[i].k / 32 + kWaves - 1) / kWaves + 3) / 4 > kKDMax) xreg = false;
  a.x_lds = xreg ? 0 : (int)round_kb((long)n * d * 4);
  a.h_lds = (int)h_lds;
  // one workgroup per CU
  int cus = 0, dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidValue;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return hipErrorInvalidValue;
  a.grid = cus;
  if (a.grid > kMaxGrid || (a.n_up + a.grid - 1) / a.grid > kMaxUp) return hipErrorNotSupported;
  long w_lds = 0;
  for (int g = 0; g < a.grid; ++g) {
    int f, l;
    down_range(g, a.grid, n_sd, a.n_down, a.down_bytes, a.down_total, f, l);
    const long b = down_prefix(l, n_sd, a.down_bytes) - down_prefix(f, n_sd, a.down_bytes);
    w_lds = b > w_lds ? b : w_lds;
    if (l - f > kMaxDown) return hipErrorNotSupported;
  }
  const long lds = a.x_lds + a.h_lds + w_lds;  // the kernel's static LDS is added in launch_one
  if (lds > kLdsLimit) return hipErrorNotSupported;
  if (swiglu) {
    if (ku <= 2) return launch_x<2, 2, EPI_SWIGLU>(a, xreg, (size_t)lds, stream);
    if (ku <= 4) return launch_x<2, 4, EPI_SWIGLU>(a, xreg, (size_t)lds, stream);
    return hipErrorNotSupported;
  }
  if (ku <= 2) return launch_x<1, 2, EPI_RELU2>(a, xreg, (size_t)lds, stream);
  if (ku <= 3) return launch_x<1, 3, EPI_RELU2>(a, xreg, (size_t)lds, stream);
  if (ku <= 4) return launch_x<1, 4, EPI_RELU2>(a, xreg, (size_t)lds, stream);
  return hipErrorNotSupported;
}

}  // namespace moe
