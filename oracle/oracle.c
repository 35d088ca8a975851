/*
 * CPU oracle for the small-batch W4A16 sigmoid-routed MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU baseline leg of
 * the benchmark do.  It shares no code, header, table or constant with the
 * GPU library.
 *
 * What it computes is the plain definition of the layer, per token, in FP64
 * from BF16 inputs, with one BF16 round-to-nearest-even at each stated
 * rounding point.  Sources (page titles as printed on the pages):
 *   - "Day-0 Support for Flint on vLLM" (Chinese translation), section
 *     "Model architecture": 256 experts, sigmoid top-6, plus a shared expert;
 *     the NVFP4 checkpoint is GGUF with NVIDIA NVFP4 blocks in another byte
 *     order, run weight-only (W4A16) with BF16 activations; kernels follow
 *     the reference implementation's rounding points.
 *   - same page, section "Optimizations": the router and expert GEMVs read
 *     only the selected experts' weights; norm and SiLU kernels follow the
 *     reference rounding.
 *   - "vLLM Flint" (English commentary), section "Only 14 of 49 layers
 *     retain full-history KV": 49 pre-norm layers, hidden size 2048.
 *   - the same two pages on attention: 35 layers attend over a 513-token
 *     sliding window with RoPE, 14 over the full context without positional
 *     encoding; GQA with 32 query and 4 KV heads; per-head Q/K RMSNorm;
 *     learned attention sinks; BF16 KV cache of 28 KiB per token over the
 *     14 full layers (head_dim 128); the Q/K norm, RoPE and KV write are one
 *     fused step, decode attention handles sinks and the window.
 * Readings where the pages are silent (rounding points, tie-break, router
 * bias, renormalisation, shared-expert weight, SwiGLU orientation, NVFP4
 * value, GGUF block byte order, RMSNorm form) are listed in the design notes
 * and restated at each function below.
 *
 * Pins: every function here is checked by the CPU tests against values fixed
 * outside this file (format definitions and a library decoder, hand-worked
 * rounding ties, closed forms, top-k invariants, permutation equivariance,
 * a brute-force dense MoE with a one-hot gate, and NVFP4 == BF16 at
 * power-of-two tensor scales); the attention functions against closed
 * forms, rotations written as complex products, and torch's float64
 * scaled-dot-product attention with GQA heads repeated, the window as a mask
 * and the sink as an extra key.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

static double g_e2m1[16];
static double g_e4m3[256];
static int g_ready = 0;

/* E2M1 (OCP Microscaling FP4): sign bit 3, exponent bits 2..1 (bias 1),
 * mantissa bit 0.  Exponent 0 is subnormal: m * 0.5. */
static double e2m1_def(int code) {
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double v = (e == 0) ? 0.5 * m : (1.0 + 0.5 * m) * ldexp(1.0, e - 1);
  return s ? -v : v;
}

/* E4M3FN (OCP 8-bit floating point): sign bit 7, exponent bits 6..3 (bias
 * 7), mantissa bits 2..0.  Exponent 0 is subnormal: m/8 * 2^-6.  The codes
 * S.1111.111 are NaN; there is no infinity. */
static double e4m3_def(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? (m / 8.0) * ldexp(1.0, -6) : (1.0 + m / 8.0) * ldexp(1.0, e - 7);
  return s ? -v : v;
}

static void tables_init(void) {
  if (g_ready) return;
  for (int c = 0; c < 16; ++c) g_e2m1[c] = e2m1_def(c);
  for (int c = 0; c < 256; ++c) g_e4m3[c] = e4m3_def(c);
  g_ready = 1;
}

double oracle_e2m1_value(int32_t code) { tables_init(); return g_e2m1[code & 15]; }
double oracle_e4m3_value(int32_t code) { tables_init(); return g_e4m3[code & 255]; }

/* BF16 bits -> value (exact). */
double oracle_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

/* One correctly rounded BF16 rounding of an FP64 value: round to nearest,
 * ties to even, directly from the FP64 value (no intermediate FP32), with
 * gradual underflow and overflow to infinity. */
uint16_t oracle_bf16_round(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (a >= 0x1p128) return sign | 0x7F80;
  int e;
  frexp(a, &e);          /* a = f * 2^e with f in [0.5, 1) */
  int q = e - 8;         /* weight of the 8th significant bit */
  if (q < -133) q = -133; /* BF16 subnormal spacing */
  double r = ldexp(nearbyint(ldexp(a, -q)), q); /* nearbyint: ties to even */
  if (r >= 0x1p128) return sign | 0x7F80;
  float f = (float)r; /* exact: r has at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return sign | (uint16_t)(u >> 16);
}

static inline double bf16r(double v) { return oracle_bf16_value(oracle_bf16_round(v)); }

/* oracle_bf16_round over n values. */
void oracle_bf16_round_array(const double *v, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(v[i]);
}

/* ------------------------------------------------------------------ */
/* Weight matrices                                                     */
/* ------------------------------------------------------------------ */

enum { OR_W_BF16 = 0, OR_W_NVFP4 = 1 };

/* A weight matrix [rows][cols], W[r][c] multiplies input element c.
 *   BF16: rows*cols bf16 values, row-major.
 *   NVFP4 (GGUF-like block order, one reading of "NVIDIA NVFP4 blocks in a
 *   different byte order"): row-major over rows; each row is cols/16 blocks
 *   of 9 bytes = [E4M3 scale][8 nibble bytes]; nibble byte j holds element j
 *   of the block in its low nibble and element j+8 in its high nibble.
 *   Element value = E2M1[q] * E4M3[s] * tensor_scale. */
typedef struct {
  const uint8_t *data;
  int64_t rows, cols;
  int wtype;
  double tscale;
} omat;

static int64_t omat_bytes(int wtype, int64_t rows, int64_t cols) {
  return wtype == OR_W_BF16 ? rows * cols * 2 : rows * (cols / 16) * 9;
}

/* Dot product of row r with x, in FP64.  Each weight value is exact in FP64
 * (at most 30 significant bits for NVFP4), each product with a BF16 input is
 * exact; only the running sum rounds.  Counts NaN scale bytes met. */
static double row_dot(const omat *m, int64_t r, const double *x, int64_t *nan_count) {
  double acc = 0.0;
  if (m->wtype == OR_W_BF16) {
    const uint16_t *w = (const uint16_t *)(const void *)m->data + r * m->cols;
    for (int64_t c = 0; c < m->cols; ++c) acc += oracle_bf16_value(w[c]) * x[c];
    return acc;
  }
  const uint8_t *row = m->data + r * (m->cols / 16) * 9;
  for (int64_t b = 0; b < m->cols / 16; ++b) {
    const uint8_t *blk = row + b * 9;
    double s = g_e4m3[blk[0]];
    if (isnan(s)) ++*nan_count;
    for (int j = 0; j < 8; ++j) {
      double lo = g_e2m1[blk[1 + j] & 15] * s * m->tscale;
      double hi = g_e2m1[blk[1 + j] >> 4] * s * m->tscale;
      acc += lo * x[b * 16 + j];
      acc += hi * x[b * 16 + j + 8];
    }
  }
  return acc;
}

/* Decode a whole GGUF-like NVFP4 matrix to FP64 (for tests); returns the
 * number of NaN scale bytes. */
int64_t oracle_decode_nvfp4(const uint8_t *src, int64_t rows, int64_t cols, double tensor_scale, double *out) {
  tables_init();
  int64_t nan_count = 0;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t b = 0; b < cols / 16; ++b) {
      const uint8_t *blk = src + (r * (cols / 16) + b) * 9;
      double s = g_e4m3[blk[0]];
      if (isnan(s)) ++nan_count;
      for (int j = 0; j < 8; ++j) {
        out[r * cols + b * 16 + j] = g_e2m1[blk[1 + j] & 15] * s * tensor_scale;
        out[r * cols + b * 16 + j + 8] = g_e2m1[blk[1 + j] >> 4] * s * tensor_scale;
      }
    }
  return nan_count;
}

/* A dense projection on the same NVFP4 weights (the small-batch dense
 * GEMV of "Day-0 Support for Flint on vLLM", section "Optimizations", for
 * the layers outside the MoE blocks): for each of T tokens,
 *   y_n = BF16( sum_k W[n][k] x_k ),  W = E2M1 * E4M3 block scale * S,
 * in FP64 from the BF16 inputs, one rounding at the end (the same rounding
 * point as the expert GEMVs).  src: GGUF-like NVFP4 bytes [rows][cols];
 * x [T][cols] and y [T][rows] BF16 bits.  Returns the number of NaN scale
 * bytes met (0 for a valid matrix). */
int64_t oracle_gemv_nvfp4(const uint8_t *src, int64_t rows, int64_t cols, double tensor_scale, const uint16_t *x,
                          int32_t T, uint16_t *y) {
  tables_init();
  int64_t nan_count = 0;
  omat W = {src, rows, cols, OR_W_NVFP4, tensor_scale};
  double *xv = (double *)malloc(sizeof(double) * (size_t)cols);
  for (int32_t t = 0; t < T; ++t) {
    for (int64_t c = 0; c < cols; ++c) xv[c] = oracle_bf16_value(x[(int64_t)t * cols + c]);
    for (int64_t n = 0; n < rows; ++n) {
      int64_t nan_row = 0;
      y[(int64_t)t * rows + n] = oracle_bf16_round(row_dot(&W, n, xv, &nan_row));
      if (t == 0) nan_count += nan_row;
    }
  }
  free(xv);
  return nan_count;
}

/* ------------------------------------------------------------------ */
/* The layer                                                           */
/* ------------------------------------------------------------------ */

/* Layer description and weights.  Expert e's matrices are at offset
 * e * (bytes of one matrix) in the stacked arrays. */
typedef struct {
  int32_t hidden, inter, shared_inter, n_experts, top_k, wtype;
  double norm_eps;          /* used when norm_gain != NULL */
  int32_t residual;         /* 1: output x + layer(x) */
  const uint16_t *norm_gain;   /* [H] bf16 or NULL (no pre-norm) */
  const uint16_t *router_w;    /* [E][H] bf16 */
  const float *router_b;       /* [E] or NULL (zero) */
  const uint8_t *w_gate, *w_up, *w_down; /* [E] x ([I][H], [I][H], [H][I]) */
  const float *w_scale;        /* [E][3] tensor scales (NVFP4) */
  const uint8_t *sh_gate, *sh_up, *sh_down; /* [Is][H], [Is][H], [H][Is] */
  const float *sh_scale;       /* [3] */
} oracle_layer;

/* One SwiGLU expert on xn (FP64 values of BF16 numbers), written as
 * y = BF16(Wd . h), h_n = BF16(SiLU(g_n) * u_n), g = BF16(Wg . xn),
 * u = BF16(Wu . xn).  Reading: SiLU(g) = g / (1 + exp(-g)) on the rounded g,
 * the product with u rounded once; W stored [out][in]. */
static void expert_ffn(const omat *g, const omat *u, const omat *d, const double *xn, double *y,
                       int64_t *nan_count) {
  int64_t I = g->rows, H = d->rows;
  double *h = (double *)malloc(sizeof(double) * (size_t)I);
  for (int64_t n = 0; n < I; ++n) {
    double gn = bf16r(row_dot(g, n, xn, nan_count));
    double un = bf16r(row_dot(u, n, xn, nan_count));
    double silu = gn / (1.0 + exp(-gn));
    h[n] = bf16r(silu * un);
  }
  for (int64_t m = 0; m < H; ++m) y[m] = bf16r(row_dot(d, m, h, nan_count));
  free(h);
}

typedef struct {
  double logit;
  int32_t e;
} cand;

/* Order: larger logit first; equal logits -> lower expert index first. */
static int cand_cmp(const void *pa, const void *pb) {
  const cand *a = (const cand *)pa, *b = (const cand *)pb;
  if (a->logit > b->logit) return -1;
  if (a->logit < b->logit) return 1;
  return (a->e < b->e) ? -1 : (a->e > b->e);
}

static double sigmoid(double l) { return 1.0 / (1.0 + exp(-l)); }

/*
 * One token through the layer.
 *  x [H] bf16 in; out [H] bf16 out.
 *  forced_idx [k] or NULL: when given, use these experts (in this order)
 *    instead of selecting; used to re-evaluate flagged near-tie tokens with
 *    the GPU's choice.
 *  idx_out [k], w_out [k] (score-descending), flag_out: 1 when the k-th and
 *    (k+1)-th sigmoid scores differ by less than 1e-5, logits_out [E] or NULL.
 * Steps:
 *  1. xn = x, or with a pre-norm gain g: xn_k = BF16(x_k / sqrt(mean(x^2) +
 *     eps) * g_k)  (RMSNorm, one rounding after the gain).
 *  2. l_e = sum_k Wr[e][k] xn_k + b_e   (router logits, not rounded).
 *  3. s_e = 1 / (1 + exp(-l_e))         (sigmoid scores).
 *  4. pick the k experts with the largest l (ties: lower index first); the
 *     set equals that of the largest s since the sigmoid is increasing.
 *  5. w_j = s_idx_j / sum_j' s_idx_j'   (renormalised to sum 1).
 *  6. y_e = SwiGLU expert (see expert_ffn) for each selected e and for the
 *     shared expert.
 *  7. o_m = BF16(sum_j w_j y_idx_j[m] + y_shared[m]); the shared expert is
 *     added with weight 1 outside the renormalisation.
 *  8. residual: out_m = BF16(x_m + o_m); otherwise out = o.
 * Returns 0, or -1 if a NaN E4M3 scale byte was met in a matrix it read.
 */
int32_t oracle_moe_token(const oracle_layer *L, const uint16_t *x, const int32_t *forced_idx,
                         uint16_t *out, int32_t *idx_out, double *w_out, int32_t *flag_out, double *logits_out) {
  tables_init();
  const int64_t H = L->hidden, I = L->inter, Is = L->shared_inter, E = L->n_experts;
  const int32_t k = (E > 0) ? L->top_k : 0;
  int64_t nan_count = 0;
  double *xv = (double *)malloc(sizeof(double) * (size_t)H);
  double *xn = (double *)malloc(sizeof(double) * (size_t)H);
  double *acc = (double *)calloc((size_t)H, sizeof(double));
  double *y = (double *)malloc(sizeof(double) * (size_t)H);
  for (int64_t i = 0; i < H; ++i) xv[i] = oracle_bf16_value(x[i]);

  /* 1. pre-norm */
  if (L->norm_gain) {
    double ss = 0.0;
    for (int64_t i = 0; i < H; ++i) ss += xv[i] * xv[i];
    double inv = 1.0 / sqrt(ss / (double)H + L->norm_eps);
    for (int64_t i = 0; i < H; ++i) xn[i] = bf16r(xv[i] * inv * oracle_bf16_value(L->norm_gain[i]));
  } else {
    memcpy(xn, xv, sizeof(double) * (size_t)H);
  }

  if (flag_out) *flag_out = 0;
  if (E > 0) {
    /* 2-3. router */
    cand *c = (cand *)malloc(sizeof(cand) * (size_t)E);
    omat R = {(const uint8_t *)(const void *)L->router_w, E, H, OR_W_BF16, 1.0};
    for (int64_t e = 0; e < E; ++e) {
      c[e].logit = row_dot(&R, e, xn, &nan_count) + (L->router_b ? (double)L->router_b[e] : 0.0);
      c[e].e = (int32_t)e;
      if (logits_out) logits_out[e] = c[e].logit;
    }
    double *logit_of = (double *)malloc(sizeof(double) * (size_t)E);
    for (int64_t e = 0; e < E; ++e) logit_of[e] = c[e].logit;
    /* 4. select */
    qsort(c, (size_t)E, sizeof(cand), cand_cmp);
    if (flag_out && E > k && sigmoid(c[k - 1].logit) - sigmoid(c[k].logit) < 1e-5) *flag_out = 1;
    int32_t *sel = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
    for (int32_t j = 0; j < k; ++j) sel[j] = forced_idx ? forced_idx[j] : c[j].e;
    /* 5. weights */
    double ssum = 0.0;
    for (int32_t j = 0; j < k; ++j) ssum += sigmoid(logit_of[sel[j]]);
    /* 6-7. selected experts, accumulated in selection order */
    int64_t bg = omat_bytes(L->wtype, I, H), bd = omat_bytes(L->wtype, H, I);
    for (int32_t j = 0; j < k; ++j) {
      int32_t e = sel[j];
      double wj = sigmoid(logit_of[e]) / ssum;
      double sg = L->w_scale ? L->w_scale[3 * e + 0] : 1.0;
      double su = L->w_scale ? L->w_scale[3 * e + 1] : 1.0;
      double sd = L->w_scale ? L->w_scale[3 * e + 2] : 1.0;
      omat G = {L->w_gate + e * bg, I, H, L->wtype, sg};
      omat U = {L->w_up + e * bg, I, H, L->wtype, su};
      omat D = {L->w_down + e * bd, H, I, L->wtype, sd};
      expert_ffn(&G, &U, &D, xn, y, &nan_count);
      for (int64_t m = 0; m < H; ++m) acc[m] += wj * y[m];
      if (idx_out) idx_out[j] = e;
      if (w_out) w_out[j] = wj;
    }
    free(sel);
    free(logit_of);
    free(c);
  }
  if (Is > 0) {
    double sg = L->sh_scale ? L->sh_scale[0] : 1.0;
    double su = L->sh_scale ? L->sh_scale[1] : 1.0;
    double sd = L->sh_scale ? L->sh_scale[2] : 1.0;
    omat G = {L->sh_gate, Is, H, L->wtype, sg};
    omat U = {L->sh_up, Is, H, L->wtype, su};
    omat D = {L->sh_down, H, Is, L->wtype, sd};
    expert_ffn(&G, &U, &D, xn, y, &nan_count);
    for (int64_t m = 0; m < H; ++m) acc[m] += y[m];
  }
  for (int64_t m = 0; m < H; ++m) {
    double o = bf16r(acc[m]);
    out[m] = L->residual ? oracle_bf16_round(xv[m] + o) : oracle_bf16_round(o);
  }
  free(y);
  free(acc);
  free(xn);
  free(xv);
  return nan_count ? -1 : 0;
}

/* T independent tokens (decode batch or prefill: tokens do not interact).
 * x [T][H], out [T][H], idx/w [T][k], flags [T], logits [T][E] (nullable),
 * forced [T][k] (nullable).  Returns the number of tokens that met a NaN
 * scale. */
int32_t oracle_moe_tokens(const oracle_layer *L, const uint16_t *x, int32_t T, const int32_t *forced,
                          uint16_t *out, int32_t *idx, double *w, int32_t *flags, double *logits) {
  int32_t bad = 0;
  const int64_t H = L->hidden;
  const int32_t k = (L->n_experts > 0) ? L->top_k : 0;
  for (int32_t t = 0; t < T; ++t) {
    int32_t rc = oracle_moe_token(L, x + (int64_t)t * H, forced ? forced + (int64_t)t * k : NULL,
                                  out + (int64_t)t * H, idx ? idx + (int64_t)t * k : NULL,
                                  w ? w + (int64_t)t * k : NULL, flags ? flags + t : NULL,
                                  logits ? logits + (int64_t)t * L->n_experts : NULL);
    if (rc) ++bad;
  }
  return bad;
}

/* The same T tokens over n_threads host threads.  Tokens do not interact,
 * so each one is computed start to finish by one thread (token t by thread
 * t % n_threads) exactly as oracle_moe_tokens computes it: the results are
 * bit-identical for any thread count.  Returns as oracle_moe_tokens. */
typedef struct {
  const oracle_layer *L;
  const uint16_t *x;
  int32_t T, first, stride;
  const int32_t *forced;
  uint16_t *out;
  int32_t *idx;
  double *w;
  int32_t *flags;
  double *logits;
  int32_t bad;
} tok_job;

static void *tok_worker(void *p) {
  tok_job *j = (tok_job *)p;
  const int64_t H = j->L->hidden, E = j->L->n_experts;
  const int32_t k = (E > 0) ? j->L->top_k : 0;
  for (int32_t t = j->first; t < j->T; t += j->stride) {
    int32_t rc = oracle_moe_token(j->L, j->x + (int64_t)t * H, j->forced ? j->forced + (int64_t)t * k : NULL,
                                  j->out + (int64_t)t * H, j->idx ? j->idx + (int64_t)t * k : NULL,
                                  j->w ? j->w + (int64_t)t * k : NULL, j->flags ? j->flags + t : NULL,
                                  j->logits ? j->logits + (int64_t)t * E : NULL);
    if (rc) ++j->bad;
  }
  return NULL;
}

int32_t oracle_moe_tokens_mt(const oracle_layer *L, const uint16_t *x, int32_t T, const int32_t *forced,
                             uint16_t *out, int32_t *idx, double *w, int32_t *flags, double *logits,
                             int32_t n_threads) {
  tables_init(); /* before any thread reads the tables */
  if (n_threads < 1) n_threads = 1;
  if (n_threads > T) n_threads = T > 0 ? T : 1;
  tok_job *jobs = (tok_job *)calloc((size_t)n_threads, sizeof(tok_job));
  pthread_t *th = (pthread_t *)calloc((size_t)n_threads, sizeof(pthread_t));
  for (int32_t i = 0; i < n_threads; ++i) {
    tok_job j = {L, x, T, i, n_threads, forced, out, idx, w, flags, logits, 0};
    jobs[i] = j;
  }
  /* thread 0's share runs on the calling thread; a thread that cannot be
   * started has its share run here too */
  for (int32_t i = 1; i < n_threads; ++i) {
    if (pthread_create(&th[i], NULL, tok_worker, &jobs[i]) != 0) {
      tok_worker(&jobs[i]);
      jobs[i].stride = 0; /* ran here: nothing to join */
    }
  }
  tok_worker(&jobs[0]);
  int32_t bad = jobs[0].bad;
  for (int32_t i = 1; i < n_threads; ++i) {
    if (jobs[i].stride) pthread_join(th[i], NULL);
    bad += jobs[i].bad;
  }
  free(th);
  free(jobs);
  return bad;
}


/* ------------------------------------------------------------------ */
/* Attention of a decode token ("Day-0 Support for Flint on vLLM",     */
/* sections "Model architecture" and "Optimizations")                  */
/* ------------------------------------------------------------------ */

/* Shape of one attention layer: GQA with n_q query heads and n_kv K/V
 * heads of head_dim (query head h reads K/V head h / (n_q / n_kv)).
 * window: 0 = the whole context; W = the last W positions, the current one
 * included (the pages' 513-token sliding window).  rope: 1 = RoPE on q and
 * k (the sliding-window layers), 0 = none (the full-context layers). */
typedef struct {
  int32_t n_q, n_kv, head_dim, window, rope;
  double rope_theta, norm_eps;
} oracle_attn;

/* Per-head RMSNorm with a gain shared by the heads, rounded once:
 * out_d = BF16(x_d / sqrt(mean(x^2) + eps) * g_d). */
static void head_rmsnorm(const double *x, const uint16_t *g, int32_t D, double eps, double *out) {
  double ss = 0.0;
  for (int32_t d = 0; d < D; ++d) ss += x[d] * x[d];
  double inv = 1.0 / sqrt(ss / (double)D + eps);
  for (int32_t d = 0; d < D; ++d) out[d] = bf16r(x[d] * inv * oracle_bf16_value(g[d]));
}

/* RoPE, rotate-half form (a reading: the pages say only "RoPE"): element d
 * < D/2 pairs with d + D/2, rotated by the angle pos * theta^(-2d/D):
 *   (a, b) -> BF16(a cos - b sin), BF16(b cos + a sin). */
static void head_rope(double *x, int32_t D, int64_t pos, double theta) {
  for (int32_t d = 0; d < D / 2; ++d) {
    double ang = (double)pos * pow(theta, -2.0 * (double)d / (double)D);
    double c = cos(ang), sn = sin(ang);
    double a = x[d], b = x[d + D / 2];
    x[d] = bf16r(a * c - b * sn);
    x[d + D / 2] = bf16r(b * c + a * sn);
  }
}

/* Q/K norm, RoPE and the K/V to be cached, for one token.
 *  qkv [(n_q + 2 n_kv) * D] BF16: q heads, then k heads, then v heads.
 *  q_out [n_q * D], k_out [n_kv * D], v_out [n_kv * D] BF16.
 * q and k: per-head RMSNorm with q_gain / k_gain [D], then RoPE at pos
 * when the layer has it; v is stored as given. */
void oracle_attn_prep(const oracle_attn *A, const uint16_t *qkv, int64_t pos, const uint16_t *q_gain,
                      const uint16_t *k_gain, uint16_t *q_out, uint16_t *k_out, uint16_t *v_out) {
  const int32_t D = A->head_dim;
  double *x = (double *)malloc(sizeof(double) * (size_t)D);
  double *y = (double *)malloc(sizeof(double) * (size_t)D);
  for (int32_t h = 0; h < A->n_q + A->n_kv; ++h) {
    const int q = h < A->n_q;
    const uint16_t *src = qkv + (int64_t)h * D;
    for (int32_t d = 0; d < D; ++d) x[d] = oracle_bf16_value(src[d]);
    head_rmsnorm(x, q ? q_gain : k_gain, D, A->norm_eps, y);
    if (A->rope) head_rope(y, D, pos, A->rope_theta);
    uint16_t *dst = q ? q_out + (int64_t)h * D : k_out + (int64_t)(h - A->n_q) * D;
    for (int32_t d = 0; d < D; ++d) dst[d] = oracle_bf16_round(y[d]);
  }
  for (int64_t i = 0; i < (int64_t)A->n_kv * D; ++i) v_out[i] = qkv[(int64_t)(A->n_q + A->n_kv) * D + i];
  free(y);
  free(x);
}

/* Decode attention of one token at position pos over its cache.
 *  q [n_q * D] BF16 (normed, roped);
 *  k_cache, v_cache [slots][n_kv][D] BF16; position p lives in slot
 *  p % slots (slots >= the positions attended: the whole context for a
 *  full layer, at least the window for a sliding one);
 *  sinks [n_q] FP32 learned logits, or NULL (none);
 *  out [n_q * D] BF16.
 * Per query head h (K/V head g = h / (n_q / n_kv)), over the positions
 * lo..pos, lo = 0 or pos - window + 1 (not below 0):
 *   s_i = (q_h . k_i) / sqrt(D),  m = max(max_i s_i, sink_h),
 *   out = BF16( sum_i e^(s_i - m) v_i / (sum_i e^(s_i - m) + e^(sink_h - m)) ),
 * the sink taking part in the normalisation only (a reading of "learned
 * attention sinks"). */
void oracle_attn_decode(const oracle_attn *A, const uint16_t *q, const uint16_t *k_cache, const uint16_t *v_cache,
                        int64_t slots, int64_t pos, const float *sinks, uint16_t *out) {
  const int32_t D = A->head_dim, G = A->n_q / A->n_kv;
  int64_t lo = 0;
  if (A->window > 0 && pos - A->window + 1 > 0) lo = pos - A->window + 1;
  const int64_t n = pos - lo + 1;
  double *s = (double *)malloc(sizeof(double) * (size_t)n);
  double *acc = (double *)malloc(sizeof(double) * (size_t)D);
  const double scale = 1.0 / sqrt((double)D);
  for (int32_t h = 0; h < A->n_q; ++h) {
    const int32_t g = h / G;
    double m = sinks ? (double)sinks[h] : -INFINITY;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t slot = (lo + i) % slots;
      const uint16_t *k = k_cache + (slot * A->n_kv + g) * D;
      double dot = 0.0;
      for (int32_t d = 0; d < D; ++d) dot += oracle_bf16_value(q[(int64_t)h * D + d]) * oracle_bf16_value(k[d]);
      s[i] = dot * scale;
      if (s[i] > m) m = s[i];
    }
    double den = sinks ? exp((double)sinks[h] - m) : 0.0;
    for (int32_t d = 0; d < D; ++d) acc[d] = 0.0;
    for (int64_t i = 0; i < n; ++i) {
      const int64_t slot = (lo + i) % slots;
      const uint16_t *v = v_cache + (slot * A->n_kv + g) * D;
      const double p = exp(s[i] - m);
      den += p;
      for (int32_t d = 0; d < D; ++d) acc[d] += p * oracle_bf16_value(v[d]);
    }
    for (int32_t d = 0; d < D; ++d) out[(int64_t)h * D + d] = oracle_bf16_round(acc[d] / den);
  }
  free(acc);
  free(s);
}
