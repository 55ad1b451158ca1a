/*
 * moe_oracle.c -- plain, slow CPU reference for the NVFP4 MoE expert-FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the benchmark's CPU-baseline leg
 * use it.  It shares no code, header, table or helper with the HIP library.
 *
 * What it follows (page titles and sections of the source pages):
 *   [gllm#91]  "perf: gather tokens per MoE expert, run large NVFP4 GEMMs on bf16
 *              tensor cores #91" -- sections "What the profile showed",
 *              "What changes", "bf16 NVFP4 GEMM (CUDA)", "Testing".
 *   [glq]      "Glq v0.2.13" release notes -- "v3b" (relu^2 activation of the
 *              non-gated NemotronH experts).
 *   [tf#2265]  "nvfp4 experts cuda: decode kernels stall on load latency ..." --
 *              "What ncu shows" (the gate-up expert).
 *
 * Arithmetic: every floating-point value is carried in IEEE double and every sum
 * runs in one fixed, documented order, so the result does not depend on the
 * number of threads.  Each output element is produced by exactly one thread.
 * The functions ending in _f32 (at the end of the file) evaluate the same steps
 * in binary32 with fused multiply-adds in one fixed order instead; the double
 * ones are the exact values those round towards.
 *
 * Readings of points the pages leave open (each is stated where it is used):
 *   - e2m1 value set: OCP Microscaling spec, E2M1 (sign, 2 exponent bits with
 *     bias 1, 1 mantissa bit).  Code 8 is -0.
 *   - e4m3 block scale: OCP E4M3FN (bias 7, max 448, S.1111.111 = NaN, no inf).
 *   - block = 16 consecutive elements along the input (k) axis of an output row.
 *   - codes are stored [rows][cols/2], element 2i in the low nibble of byte i;
 *     scales are stored [rows][cols/16].
 *   - dequantised weight = global * e4m3(scale) * e2m1(code).
 *   - routing: top-K by logit (ties: lower expert index first), slot order is
 *     descending logit, weights = softmax over the K picked logits.
 *   - rows inside an expert's group are in ascending token order.
 */
#include <errno.h>
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_EINVAL 1
#define ORC_ERANGE 2
#define ORC_ENOMEM 3

/* ------------------------------------------------------------------------- */
/* Formats                                                                    */
/* ------------------------------------------------------------------------- */

/* e2m1 magnitudes for codes 0..7 (OCP MX E2M1); bit 3 is the sign.
 * [gllm#91] "bf16 NVFP4 GEMM (CUDA)": NVFP4 weights are e2m1 codes. */
static const double E2M1_MAGNITUDE[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1(unsigned code) {
  double m = E2M1_MAGNITUDE[code & 7u];
  return (code & 8u) ? -m : m;
}

/* OCP E4M3FN byte -> value.  [gllm#91] "bf16 NVFP4 GEMM (CUDA)": one e4m3 block
 * scale per block. */
double orc_e4m3(unsigned byte) {
  unsigned s = (byte >> 7) & 1u, e = (byte >> 3) & 15u, m = byte & 7u;
  double v;
  if (e == 15u && m == 7u) return NAN;
  if (e == 0u)
    v = ldexp((double)m, -9);            /* subnormal: m/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
  return s ? -v : v;
}

/* Dequantise one NVFP4 tensor [rows, cols] into doubles.
 * with_global != 0: value = global * scale * code (the format's definition);
 * with_global == 0: value = scale * code (the unpack that drops the per-tensor
 * global, [gllm#91] "bf16 NVFP4 GEMM (CUDA)").  Every such product is exact in
 * double (at most 24 + 4 + 2 significant bits). */
int orc_dequant(const uint8_t *codes, const uint8_t *scales, float global, int rows,
                int cols, int with_global, double *out) {
  if (rows < 0 || cols < 0 || (cols % 16) != 0) return ORC_EINVAL;
  for (int r = 0; r < rows; ++r) {
    for (int k = 0; k < cols; ++k) {
      uint8_t byte = codes[(size_t)r * (cols / 2) + k / 2];
      unsigned code = (k % 2 == 0) ? (byte & 15u) : (byte >> 4);
      double s = orc_e4m3(scales[(size_t)r * (cols / 16) + k / 16]);
      double v = s * orc_e2m1(code);
      if (with_global) v = (double)global * v;
      out[(size_t)r * cols + k] = v;
    }
  }
  return ORC_OK;
}

/* Round a double to the nearest bfloat16 value, ties to even (8 significant
 * bits, exponent range of binary32, subnormal quantum 2^-133).  Used only in
 * the bf16-activation mode that mirrors [gllm#91] "bf16 NVFP4 GEMM (CUDA)":
 * "the activation is rounded to bf16". */
double orc_round_bf16(double v) {
  if (v == 0.0 || !isfinite(v)) return v;
  int e;
  (void)frexp(v, &e);               /* |v| = f * 2^e, f in [0.5, 1) */
  int q = e - 8;                    /* quantum exponent for 8 significant bits */
  if (q < -133) q = -133;
  double r = nearbyint(ldexp(v, -q)); /* default rounding mode: to nearest even */
  double out = ldexp(r, q);
  if (fabs(out) > 3.3895313892515355e38) out = (v > 0) ? INFINITY : -INFINITY;
  return out;
}

/* ------------------------------------------------------------------------- */
/* A tiny parallel-for: [0, n) split into contiguous slices, one per thread.   */
/* ------------------------------------------------------------------------- */

typedef void (*orc_body_fn)(void *ctx, long i0, long i1);
typedef struct { orc_body_fn fn; void *ctx; long i0, i1; } orc_slice;

static void *orc_slice_main(void *p) {
  orc_slice *s = (orc_slice *)p;
  s->fn(s->ctx, s->i0, s->i1);
  return NULL;
}

static void orc_parallel_for(long n, int threads, orc_body_fn fn, void *ctx) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  if ((long)threads > n) threads = (int)(n > 0 ? n : 1);
  if (threads == 1) { fn(ctx, 0, n); return; }
  pthread_t tid[256];
  orc_slice sl[256];
  int started[256];
  for (int t = 0; t < threads; ++t) {
    sl[t].fn = fn; sl[t].ctx = ctx;
    sl[t].i0 = n * t / threads; sl[t].i1 = n * (t + 1) / threads;
    started[t] = (pthread_create(&tid[t], NULL, orc_slice_main, &sl[t]) == 0);
    if (!started[t]) fn(ctx, sl[t].i0, sl[t].i1);
  }
  for (int t = 0; t < threads; ++t)
    if (started[t]) pthread_join(tid[t], NULL);
}

/* ------------------------------------------------------------------------- */
/* Routing                                                                    */
/* ------------------------------------------------------------------------- */

/* Per token: the K experts with the largest logits, by repeated selection
 * (strictly larger wins, so among equal logits the lower expert index is taken
 * first), slot j = j-th largest.  Weights: softmax over the K picked logits,
 * w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0), the sum taken over i = 0..K-1 in
 * order.  The pages route with topK (gllm#91 "What the profile showed": topK 6)
 * and the per-pick weights are what WeightedRowSum consumes. */
int orc_route_topk(const float *logits, int n, int E, int K, int32_t *ids, double *w) {
  if (n < 0 || E < 1 || K < 1 || K > E) return ORC_EINVAL;
  unsigned char *taken = (unsigned char *)malloc((size_t)E);
  double *ex = (double *)malloc(sizeof(double) * (size_t)K);
  if (!taken || !ex) { free(taken); free(ex); return ORC_ENOMEM; }
  for (int t = 0; t < n; ++t) {
    const float *l = logits + (size_t)t * E;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < K; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (taken[e]) continue;
        if (best < 0 || l[e] > l[best]) best = e;
      }
      taken[best] = 1;
      ids[(size_t)t * K + j] = best;
    }
    double m = (double)l[ids[(size_t)t * K]];
    double sum = 0.0;
    for (int j = 0; j < K; ++j) {
      ex[j] = exp((double)l[ids[(size_t)t * K + j]] - m);
      sum += ex[j];
    }
    for (int j = 0; j < K; ++j) w[(size_t)t * K + j] = ex[j] / sum;
  }
  free(taken); free(ex);
  return ORC_OK;
}

/* The router logits that routing ranks: logits[t][e] = sum_k x[t][k] * W_r[e][k]
 * (the router's linear layer, x . W_r^T), k ascending, in double.  The
 * linked PR "perf: cut host overhead from long prefills (routing, matmul
 * scratch)" of [gllm#91] is about this step before routing. */
int orc_router_logits(const double *x, int n, int d, const double *wr, int E, double *logits) {
  if (n < 0 || d < 1 || E < 1) return ORC_EINVAL;
  for (int t = 0; t < n; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int k = 0; k < d; ++k) acc += x[(size_t)t * d + k] * wr[(size_t)e * d + k];
      logits[(size_t)t * E + e] = acc;
    }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Gather                                                                     */
/* ------------------------------------------------------------------------- */

/* [gllm#91] "What changes": n*topK rows, one per (token, picked expert) pair,
 * the rows of each expert contiguous.  count_e -> exclusive offsets;
 * then walking tokens in ascending order (and slots j ascending), the pick
 * (t, j) of expert e gets row off_e + (number of earlier picks of e).
 * rows[t*K + j] = that row, row_token[row] = t.  An expert id outside [0, E)
 * is an error (nothing is written). */
int orc_gather_layout(const int32_t *ids, int n, int K, int E, int32_t *offsets,
                      int32_t *row_token, int32_t *rows) {
  if (n < 0 || K < 1 || E < 1) return ORC_EINVAL;
  for (long i = 0; i < (long)n * K; ++i)
    if (ids[i] < 0 || ids[i] >= E) return ORC_ERANGE;
  int32_t *cursor = (int32_t *)calloc((size_t)E, sizeof(int32_t));
  if (!cursor) return ORC_ENOMEM;
  for (int e = 0; e <= E; ++e) offsets[e] = 0;
  for (long i = 0; i < (long)n * K; ++i) offsets[ids[i] + 1] += 1;
  for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
  for (int t = 0; t < n; ++t) {
    for (int j = 0; j < K; ++j) {
      int e = ids[(size_t)t * K + j];
      int32_t r = offsets[e] + cursor[e]++;
      rows[(size_t)t * K + j] = r;
      row_token[r] = t;
    }
  }
  free(cursor);
  return ORC_OK;
}

/* [gllm#91] "What changes": the inputs are gathered by a single row lookup,
 * xg[r] = x[row_token[r]], copied bit for bit. */
int orc_gather_copy(const void *x, int elem_bytes, int n, int d, const int32_t *row_token,
                    int R, void *xg) {
  size_t row_bytes = (size_t)elem_bytes * (size_t)d;
  for (int r = 0; r < R; ++r) {
    int t = row_token[r];
    if (t < 0 || t >= n) return ORC_ERANGE;
    memcpy((char *)xg + (size_t)r * row_bytes, (const char *)x + (size_t)t * row_bytes, row_bytes);
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* Expert FFN                                                                 */
/* ------------------------------------------------------------------------- */

#define ORC_ACT_RELU2 0
#define ORC_ACT_SWIGLU 1

/* act = relu^2: h = max(u, 0)^2  ([glq] "v3b": relu^2 for non-gated NemotronH;
 *   [gllm#91] "What changes": up -> relu^2 -> down).
 * act = swiglu: up rows [0, f) are the gate a, rows [f, 2f) the up half b;
 *   h = silu(a) * b with silu(a) = a / (1 + exp(-a))  ([tf#2265] "What ncu
 *   shows": the gated experts' fused gate-up projection). */
typedef struct {
  const double *x;          /* [n_rows, d] activations (already in double) */
  const int32_t *row_list;  /* rows of this expert: x row indices */
  const double *wu;         /* [up_rows, d] dequantised up weight */
  const double *wd;         /* [d_out, f] dequantised down weight */
  int d, f, d_out, act, bf16_act;
  double *out;              /* [n_rows, d_out] */
} orc_ffn_ctx;

static void orc_ffn_rows(void *p, long i0, long i1) {
  orc_ffn_ctx *c = (orc_ffn_ctx *)p;
  int up_rows = (c->act == ORC_ACT_SWIGLU) ? 2 * c->f : c->f;
  double *u = (double *)malloc(sizeof(double) * (size_t)up_rows);
  double *h = (double *)malloc(sizeof(double) * (size_t)c->f);
  double *xr = (double *)malloc(sizeof(double) * (size_t)c->d);
  if (!u || !h || !xr) { free(u); free(h); free(xr); return; }
  for (long i = i0; i < i1; ++i) {
    int r = c->row_list[i];
    for (int k = 0; k < c->d; ++k) {
      double v = c->x[(size_t)r * c->d + k];
      xr[k] = c->bf16_act ? orc_round_bf16(v) : v;
    }
    /* up projection: u[n] = sum_k x[k] * Wu[n,k], k ascending */
    for (int nn = 0; nn < up_rows; ++nn) {
      const double *wrow = c->wu + (size_t)nn * c->d;
      double acc = 0.0;
      for (int k = 0; k < c->d; ++k) acc += xr[k] * wrow[k];
      u[nn] = acc;
    }
    for (int nn = 0; nn < c->f; ++nn) {
      double hv;
      if (c->act == ORC_ACT_SWIGLU) {
        double a = u[nn], b = u[c->f + nn];
        hv = (a / (1.0 + exp(-a))) * b;
      } else {
        double a = u[nn] > 0.0 ? u[nn] : 0.0;
        hv = a * a;
      }
      h[nn] = c->bf16_act ? orc_round_bf16(hv) : hv;
    }
    /* down projection: y[m] = sum_k h[k] * Wd[m,k], k ascending */
    for (int m = 0; m < c->d_out; ++m) {
      const double *wrow = c->wd + (size_t)m * c->f;
      double acc = 0.0;
      for (int k = 0; k < c->f; ++k) acc += h[k] * wrow[k];
      c->out[(size_t)r * c->d_out + m] = acc;
    }
  }
  free(u); free(h); free(xr);
}

typedef struct {
  const uint8_t *codes, *scales;
  float global;
  int rows, cols;
  double *out;
} orc_deq_ctx;

static void orc_deq_rows(void *p, long i0, long i1) {
  orc_deq_ctx *c = (orc_deq_ctx *)p;
  (void)orc_dequant(c->codes + (size_t)i0 * (c->cols / 2), c->scales + (size_t)i0 * (c->cols / 16),
                    c->global, (int)(i1 - i0), c->cols, 1, c->out + (size_t)i0 * c->cols);
}

/* Expert FFN over packed rows grouped by expert ([gllm#91] "What changes":
 * an expert's up -> relu^2 -> down touches the rows routed to it and no
 * others).
 *   x       [n_rows, d] in double; rows [offsets[e], offsets[e+1]) belong to e
 *   up      codes [E][up_rows][d/2], scales [E][up_rows][d/16], globals [E]
 *           up_rows = f (relu^2) or 2f (swiglu)
 *   down    codes [E][d_out][f/2], scales [E][d_out][f/16], globals [E]
 *   out     [n_rows, d_out]: y = g_dn * ... computed from the dequantised weights
 * bf16_act != 0 rounds x and h to bf16 before their sums (the precision the
 * MFMA path documents); bf16_act == 0 is the exact definition. */
int orc_expert_ffn(const double *x, int n_rows, int d, const int32_t *offsets, int E,
                   const uint8_t *up_codes, const uint8_t *up_scales, const float *up_global,
                   const uint8_t *dn_codes, const uint8_t *dn_scales, const float *dn_global,
                   int f, int d_out, int act, int bf16_act, int threads, double *out) {
  if (n_rows < 0 || d < 16 || f < 16 || d_out < 1 || E < 1 || (d % 16) || (f % 16)) return ORC_EINVAL;
  if (act != ORC_ACT_RELU2 && act != ORC_ACT_SWIGLU) return ORC_EINVAL;
  if (offsets[0] != 0 || offsets[E] != n_rows) return ORC_EINVAL;
  for (int e = 0; e < E; ++e)
    if (offsets[e + 1] < offsets[e]) return ORC_EINVAL;
  int up_rows = (act == ORC_ACT_SWIGLU) ? 2 * f : f;
  double *wu = (double *)malloc(sizeof(double) * (size_t)up_rows * d);
  double *wd = (double *)malloc(sizeof(double) * (size_t)d_out * f);
  int32_t *row_list = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_rows > 0 ? n_rows : 1));
  if (!wu || !wd || !row_list) { free(wu); free(wd); free(row_list); return ORC_ENOMEM; }
  for (int r = 0; r < n_rows; ++r) row_list[r] = r;
  for (int e = 0; e < E; ++e) {
    int r0 = offsets[e], r1 = offsets[e + 1];
    if (r1 == r0) continue;
    orc_deq_ctx du = {up_codes + (size_t)e * up_rows * (d / 2), up_scales + (size_t)e * up_rows * (d / 16),
                      up_global[e], up_rows, d, wu};
    orc_parallel_for(up_rows, threads, orc_deq_rows, &du);
    orc_deq_ctx dd = {dn_codes + (size_t)e * d_out * (f / 2), dn_scales + (size_t)e * d_out * (f / 16),
                      dn_global[e], d_out, f, wd};
    orc_parallel_for(d_out, threads, orc_deq_rows, &dd);
    orc_ffn_ctx c = {x, row_list + r0, wu, wd, d, f, d_out, act, bf16_act, out};
    orc_parallel_for(r1 - r0, threads, orc_ffn_rows, &c);
  }
  free(wu); free(wd); free(row_list);
  return ORC_OK;
}

/* One projection only, y = A * W^T with W dequantised (global included):
 * y[r, n] = sum_k a[r,k] * W[n,k], k ascending.  Experts as in orc_expert_ffn.
 * This is the single NVFP4 matmul that [gllm#91] "Testing" holds to the f32
 * tolerance with bf16-exact activations. */
typedef struct {
  const double *a; const double *w; int k, nout; const int32_t *row_list; double *out;
} orc_lin_ctx;

static void orc_lin_rows(void *p, long i0, long i1) {
  orc_lin_ctx *c = (orc_lin_ctx *)p;
  for (long i = i0; i < i1; ++i) {
    int r = c->row_list[i];
    for (int nn = 0; nn < c->nout; ++nn) {
      double acc = 0.0;
      for (int k = 0; k < c->k; ++k) acc += c->a[(size_t)r * c->k + k] * c->w[(size_t)nn * c->k + k];
      c->out[(size_t)r * c->nout + nn] = acc;
    }
  }
}

int orc_linear(const double *a, int n_rows, int k, const int32_t *offsets, int E,
               const uint8_t *codes, const uint8_t *scales, const float *global, int nout,
               int threads, double *out) {
  if (n_rows < 0 || k < 16 || (k % 16) || nout < 1 || E < 1) return ORC_EINVAL;
  if (offsets[0] != 0 || offsets[E] != n_rows) return ORC_EINVAL;
  double *w = (double *)malloc(sizeof(double) * (size_t)nout * k);
  int32_t *row_list = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_rows > 0 ? n_rows : 1));
  if (!w || !row_list) { free(w); free(row_list); return ORC_ENOMEM; }
  for (int r = 0; r < n_rows; ++r) row_list[r] = r;
  for (int e = 0; e < E; ++e) {
    int r0 = offsets[e], r1 = offsets[e + 1];
    if (r1 < r0) { free(w); free(row_list); return ORC_EINVAL; }
    if (r1 == r0) continue;
    orc_deq_ctx dq = {codes + (size_t)e * nout * (k / 2), scales + (size_t)e * nout * (k / 16),
                      global[e], nout, k, w};
    orc_parallel_for(nout, threads, orc_deq_rows, &dq);
    orc_lin_ctx c = {a, w, k, nout, row_list + r0, out};
    orc_parallel_for(r1 - r0, threads, orc_lin_rows, &c);
  }
  free(w); free(row_list);
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* WeightedRowSum                                                              */
/* ------------------------------------------------------------------------- */

/* [gllm#91] "What changes": WeightedRowSum(dst, src, rows, weights) computes
 * dst[i] += sum_j w[i,j] * src[rows[i,j]] in a fixed j order.  Here the j-sum
 * starts at 0, runs j = 0..K-1, and is added to dst once at the end.  A row
 * index outside [0, n_src) is an error and nothing is written ("bounds are
 * checked", [gllm#91] "Testing"). */
int orc_weighted_row_sum(double *dst, const double *src, int n_src, const int32_t *rows,
                         const double *w, int n, int K, int d) {
  if (n < 0 || K < 1 || d < 0 || n_src < 0) return ORC_EINVAL;
  for (long i = 0; i < (long)n * K; ++i)
    if (rows[i] < 0 || rows[i] >= n_src) return ORC_ERANGE;
  for (int i = 0; i < n; ++i) {
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      for (int j = 0; j < K; ++j)
        acc += w[(size_t)i * K + j] * src[(size_t)rows[(size_t)i * K + j] * d + c];
      dst[(size_t)i * d + c] += acc;
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------------- */
/* The same steps in binary32, each sum in one fixed order                     */
/* ------------------------------------------------------------------------- */

/* The workload describes its CPU reference as fp32 accumulation in a fixed
 * order.  These functions are that evaluation, written out step by step:
 *   q = e4m3(scale) * e2m1(code)      exact in binary32 (2 + 4 significant
 *                                     bits, [gllm#91] "bf16 NVFP4 GEMM (CUDA)")
 *   F(a, b): acc = 0; for k ascending: acc = fmaf(a_k, b_k, acc)
 *   projection  out = global * F(a_row, q_row)   (the global applied once,
 *                                     after the dot product, as alpha)
 *   relu^2      h = max(u, 0); h = h * h
 *   swiglu      h = (a / (1 + expf(-a))) * b
 *   WeightedRowSum  acc = 0; for j ascending: acc = fmaf(w_ij, src_rj, acc);
 *                   dst = dst + acc          ([gllm#91] "What changes")
 * The file is built with -ffp-contract=off, so every other multiply and add
 * rounds on its own; fmaf is the C library's correctly rounded one. */

static float orc_q32(const uint8_t *codes, const uint8_t *scales, int cols, int r, int k) {
  uint8_t byte = codes[(size_t)r * (cols / 2) + k / 2];
  unsigned code = (k % 2 == 0) ? (byte & 15u) : (byte >> 4);
  return (float)(orc_e4m3(scales[(size_t)r * (cols / 16) + k / 16]) * orc_e2m1(code));
}

static float orc_dot32(const float *a, const float *b, int k) {
  float acc = 0.0f;
  for (int i = 0; i < k; ++i) acc = fmaf(a[i], b[i], acc);
  return acc;
}

typedef struct {
  const uint8_t *codes, *scales;
  int rows, cols;
  float *out;
} orc_deq32_ctx;

static void orc_deq32_rows(void *p, long i0, long i1) {
  orc_deq32_ctx *c = (orc_deq32_ctx *)p;
  for (long r = i0; r < i1; ++r)
    for (int k = 0; k < c->cols; ++k) c->out[(size_t)r * c->cols + k] = orc_q32(c->codes, c->scales, c->cols, (int)r, k);
}

typedef struct {
  const float *x; const int32_t *row_list; const float *qu, *qd;
  float gu, gd; int d, f, d_out, act; float *out;
} orc_ffn32_ctx;

static void orc_ffn32_rows(void *p, long i0, long i1) {
  orc_ffn32_ctx *c = (orc_ffn32_ctx *)p;
  int up_rows = (c->act == ORC_ACT_SWIGLU) ? 2 * c->f : c->f;
  float *u = (float *)malloc(sizeof(float) * (size_t)up_rows);
  float *h = (float *)malloc(sizeof(float) * (size_t)c->f);
  if (!u || !h) { free(u); free(h); return; }
  for (long i = i0; i < i1; ++i) {
    int r = c->row_list[i];
    const float *xr = c->x + (size_t)r * c->d;
    for (int nn = 0; nn < up_rows; ++nn) u[nn] = c->gu * orc_dot32(xr, c->qu + (size_t)nn * c->d, c->d);
    for (int nn = 0; nn < c->f; ++nn) {
      if (c->act == ORC_ACT_SWIGLU) {
        float a = u[nn], b = u[c->f + nn];
        float s = a / (1.0f + expf(-a));
        h[nn] = s * b;
      } else {
        float a = u[nn] > 0.0f ? u[nn] : 0.0f;
        h[nn] = a * a;
      }
    }
    for (int m = 0; m < c->d_out; ++m)
      c->out[(size_t)r * c->d_out + m] = c->gd * orc_dot32(h, c->qd + (size_t)m * c->f, c->f);
  }
  free(u); free(h);
}

/* orc_expert_ffn in binary32 (arguments as there, x and out in float). */
int orc_expert_ffn_f32(const float *x, int n_rows, int d, const int32_t *offsets, int E,
                       const uint8_t *up_codes, const uint8_t *up_scales, const float *up_global,
                       const uint8_t *dn_codes, const uint8_t *dn_scales, const float *dn_global,
                       int f, int d_out, int act, int threads, float *out) {
  if (n_rows < 0 || d < 16 || f < 16 || d_out < 1 || E < 1 || (d % 16) || (f % 16)) return ORC_EINVAL;
  if (act != ORC_ACT_RELU2 && act != ORC_ACT_SWIGLU) return ORC_EINVAL;
  if (offsets[0] != 0 || offsets[E] != n_rows) return ORC_EINVAL;
  for (int e = 0; e < E; ++e)
    if (offsets[e + 1] < offsets[e]) return ORC_EINVAL;
  int up_rows = (act == ORC_ACT_SWIGLU) ? 2 * f : f;
  float *qu = (float *)malloc(sizeof(float) * (size_t)up_rows * d);
  float *qd = (float *)malloc(sizeof(float) * (size_t)d_out * f);
  int32_t *row_list = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_rows > 0 ? n_rows : 1));
  if (!qu || !qd || !row_list) { free(qu); free(qd); free(row_list); return ORC_ENOMEM; }
  for (int r = 0; r < n_rows; ++r) row_list[r] = r;
  for (int e = 0; e < E; ++e) {
    int r0 = offsets[e], r1 = offsets[e + 1];
    if (r1 == r0) continue;
    orc_deq32_ctx du = {up_codes + (size_t)e * up_rows * (d / 2), up_scales + (size_t)e * up_rows * (d / 16),
                        up_rows, d, qu};
    orc_parallel_for(up_rows, threads, orc_deq32_rows, &du);
    orc_deq32_ctx dd = {dn_codes + (size_t)e * d_out * (f / 2), dn_scales + (size_t)e * d_out * (f / 16),
                        d_out, f, qd};
    orc_parallel_for(d_out, threads, orc_deq32_rows, &dd);
    orc_ffn32_ctx c = {x, row_list + r0, qu, qd, up_global[e], dn_global[e], d, f, d_out, act, out};
    orc_parallel_for(r1 - r0, threads, orc_ffn32_rows, &c);
  }
  free(qu); free(qd); free(row_list);
  return ORC_OK;
}

typedef struct {
  const float *a; const float *q; float g; int k, nout; const int32_t *row_list; float *out;
} orc_lin32_ctx;

static void orc_lin32_rows(void *p, long i0, long i1) {
  orc_lin32_ctx *c = (orc_lin32_ctx *)p;
  for (long i = i0; i < i1; ++i) {
    int r = c->row_list[i];
    for (int nn = 0; nn < c->nout; ++nn)
      c->out[(size_t)r * c->nout + nn] = c->g * orc_dot32(c->a + (size_t)r * c->k, c->q + (size_t)nn * c->k, c->k);
  }
}

/* orc_linear in binary32. */
int orc_linear_f32(const float *a, int n_rows, int k, const int32_t *offsets, int E,
                   const uint8_t *codes, const uint8_t *scales, const float *global, int nout,
                   int threads, float *out) {
  if (n_rows < 0 || k < 16 || (k % 16) || nout < 1 || E < 1) return ORC_EINVAL;
  if (offsets[0] != 0 || offsets[E] != n_rows) return ORC_EINVAL;
  float *q = (float *)malloc(sizeof(float) * (size_t)nout * k);
  int32_t *row_list = (int32_t *)malloc(sizeof(int32_t) * (size_t)(n_rows > 0 ? n_rows : 1));
  if (!q || !row_list) { free(q); free(row_list); return ORC_ENOMEM; }
  for (int r = 0; r < n_rows; ++r) row_list[r] = r;
  for (int e = 0; e < E; ++e) {
    int r0 = offsets[e], r1 = offsets[e + 1];
    if (r1 < r0) { free(q); free(row_list); return ORC_EINVAL; }
    if (r1 == r0) continue;
    orc_deq32_ctx dq = {codes + (size_t)e * nout * (k / 2), scales + (size_t)e * nout * (k / 16), nout, k, q};
    orc_parallel_for(nout, threads, orc_deq32_rows, &dq);
    orc_lin32_ctx c = {a, q, global[e], k, nout, row_list + r0, out};
    orc_parallel_for(r1 - r0, threads, orc_lin32_rows, &c);
  }
  free(q); free(row_list);
  return ORC_OK;
}

/* WeightedRowSum in binary32: for each output element the j-sum is a chain of
 * fmaf from a zero accumulator, j = 0..K-1, then one add onto dst.  A row
 * index outside [0, n_src) is an error and nothing is written. */
int orc_weighted_row_sum_f32(float *dst, const float *src, int n_src, const int32_t *rows,
                             const float *w, int n, int K, int d) {
  if (n < 0 || K < 1 || d < 0 || n_src < 0) return ORC_EINVAL;
  for (long i = 0; i < (long)n * K; ++i)
    if (rows[i] < 0 || rows[i] >= n_src) return ORC_ERANGE;
  for (int i = 0; i < n; ++i) {
    for (int c = 0; c < d; ++c) {
      float acc = 0.0f;
      for (int j = 0; j < K; ++j)
        acc = fmaf(w[(size_t)i * K + j], src[(size_t)rows[(size_t)i * K + j] * d + c], acc);
      dst[(size_t)i * d + c] = dst[(size_t)i * d + c] + acc;
    }
  }
  return ORC_OK;
}
