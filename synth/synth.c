/*
 * Seeded synthetic inputs for the W4A16 sigmoid-routed MoE layer.
 *
 * This module only *produces* inputs: BF16 activations and weights drawn
 * from N(0, sigma), NVFP4 weight matrices quantised from such draws and
 * written in the GGUF-like block order the checkpoint is described as
 * using, and the Zipf-style per-expert router offset.  It performs none of
 * the layer's arithmetic.  Both the CPU oracle and the GPU path consume the
 * bytes it writes, so the quantiser below cannot affect parity.
 *
 * Randomness: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC'11), a counter-based generator, so any
 * single tensor (layer, expert, projection) can be regenerated on its own.
 * One counter value yields four 32-bit words: (w0,w1) -> u1 and (w2,w3) -> u2,
 * two 53-bit uniforms in (0,1), which Box-Muller turns into two normals.
 *
 * Format facts used by the quantiser (from the OCP 8-bit and Microscaling
 * format specifications; the pages only say "NVIDIA NVFP4 blocks"):
 *   E2M1 magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3.
 *   E4M3 (FN variant): bias 7, subnormals m/8 * 2^-6, max 448, S.1111.111 NaN.
 * The GGUF-like source block (one reading of "different byte order"):
 *   16 elements along K -> 9 bytes: [E4M3 scale][8 nibble bytes], nibble
 *   byte j holds element j in its low nibble and element j+8 in its high one.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------- Philox4x32-10 ---------------- */
#define PHILOX_M0 0xD2511F53u
#define PHILOX_M1 0xCD9E8D57u
#define PHILOX_W0 0x9E3779B9u
#define PHILOX_W1 0xBB67AE85u

static inline void mulhilo(uint32_t a, uint32_t b, uint32_t *hi, uint32_t *lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

static void philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int r = 0; r < 10; ++r) {
    uint32_t hi0, lo0, hi1, lo1;
    mulhilo(PHILOX_M0, c0, &hi0, &lo0);
    mulhilo(PHILOX_M1, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += PHILOX_W0;
    k1 += PHILOX_W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Exported so a test can check the generator against the published
 * known-answer vectors of Philox4x32-10. */
void synth_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  philox4x32_10(ctr, key, out);
}

/* Two standard normals from counter i of stream (a, b) under key seed. */
static inline void normal_pair(uint64_t seed, uint32_t a, uint32_t b, uint64_t i, double *z0, double *z1) {
  uint32_t ctr[4] = {(uint32_t)i, (uint32_t)(i >> 32), a, b};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  philox4x32_10(ctr, key, w);
  /* 53-bit uniforms in (0, 1): never exactly 0, so log() is finite. */
  uint64_t m1 = (((uint64_t)w[0] << 32) | w[1]) >> 11;
  uint64_t m2 = (((uint64_t)w[2] << 32) | w[3]) >> 11;
  double u1 = ((double)m1 + 0.5) * (1.0 / 9007199254740992.0);
  double u2 = ((double)m2 + 0.5) * (1.0 / 9007199254740992.0);
  double r = sqrt(-2.0 * log(u1));
  double t = 6.283185307179586476925286766559 * u2;
  *z0 = r * cos(t);
  *z1 = r * sin(t);
}

/* sigma * N(0,1) samples, element i of stream (a, b). */
static void fill_normal(uint64_t seed, uint32_t a, uint32_t b, double sigma, int64_t n, double *out) {
  int64_t pairs = (n + 1) / 2;
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t p = 0; p < pairs; ++p) {
    double z0, z1;
    normal_pair(seed, a, b, (uint64_t)p, &z0, &z1);
    out[2 * p] = sigma * z0;
    if (2 * p + 1 < n) out[2 * p + 1] = sigma * z1;
  }
}

void synth_normal_f64(uint64_t seed, uint32_t a, uint32_t b, double sigma, int64_t n, double *out) {
  fill_normal(seed, a, b, sigma, n, out);
}

/* float -> bf16 bits, round to nearest even (inputs are finite here). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

/* BF16(sigma * N(0,1)) as raw bf16 bits. */
void synth_normal_bf16(uint64_t seed, uint32_t a, uint32_t b, double sigma, int64_t n, uint16_t *out) {
  int64_t pairs = (n + 1) / 2;
#pragma omp parallel for schedule(static) if (n > 65536)
  for (int64_t p = 0; p < pairs; ++p) {
    double z0, z1;
    normal_pair(seed, a, b, (uint64_t)p, &z0, &z1);
    out[2 * p] = f32_to_bf16_rne((float)(sigma * z0));
    if (2 * p + 1 < n) out[2 * p + 1] = f32_to_bf16_rne((float)(sigma * z1));
  }
}

/* ---------------- NVFP4 quantiser (test-data only) ---------------- */

/* E4M3FN value of a non-NaN code, written from the format definition. */
static double e4m3_value(int code) {
  int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp(8.0 + m, e - 10);
  return s ? -v : v;
}

/* Positive E4M3FN values are increasing in their code 0x00..0x7E. */
static double g_e4m3_pos[127];
static int g_e4m3_ready = 0;

static void e4m3_table_init(void) {
  if (g_e4m3_ready) return;
  for (int c = 0; c < 127; ++c) g_e4m3_pos[c] = e4m3_value(c);
  g_e4m3_ready = 1;
}

/* Nearest E4M3FN code for v >= 0, ties to even code, saturating at 448. */
static int e4m3_encode_pos(double v) {
  if (v >= g_e4m3_pos[126]) return 126;
  int lo = 0, hi = 126; /* g[lo] <= v < g[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (g_e4m3_pos[mid] <= v) lo = mid; else hi = mid;
  }
  double dl = v - g_e4m3_pos[lo], dh = g_e4m3_pos[hi] - v;
  if (dl < dh) return lo;
  if (dh < dl) return hi;
  return (lo & 1) ? hi : lo;
}

/* Nearest E2M1 code for real t, ties to the even code, saturating at 6.
 * The comparisons are the midpoints between neighbouring magnitudes; at a
 * midpoint the even code wins (strict '>' keeps the lower, even code, '>='
 * moves on to the upper, even code). */
static int e2m1_encode(double t) {
  double a = fabs(t);
  int c = (a > 0.25) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5) + (a > 5.0);
  int sign = (t < 0.0 && c != 0) ? 1 : 0;
  return (sign << 3) | c;
}

/* Exported for the generator's own tests. */
int synth_e2m1_encode(double t) { return e2m1_encode(t); }
int synth_e4m3_encode_pos(double v) { e4m3_table_init(); return e4m3_encode_pos(v); }

/* Quantise a rows x cols real matrix (row-major, cols % 16 == 0) into the
 * GGUF-like block order.  tensor_scale = amax / (6 * 448), or the next power
 * of two above it when pow2_tensor_scale is set.  Block scale code =
 * E4M3(amax_blk / (6 * tensor_scale)); element code = E2M1(w / (s * S)).
 * All-zero blocks get scale code 0 and element codes 0. */
void synth_quantize_nvfp4(const double *w, int64_t rows, int64_t cols, int pow2_tensor_scale,
                          uint8_t *gguf_out, float *tensor_scale_out) {
  double amax = 0.0;
  for (int64_t i = 0; i < rows * cols; ++i) amax = fmax(amax, fabs(w[i]));
  double S = amax / (6.0 * 448.0);
  if (S == 0.0) S = 1.0;
  if (pow2_tensor_scale) S = ldexp(1.0, (int)ceil(log2(S)));
  S = (double)(float)S; /* the tensor scale is stored as FP32 */
  *tensor_scale_out = (float)S;
  e4m3_table_init();
  int64_t nblk = cols / 16;
#pragma omp parallel for schedule(static) if (rows * cols > 65536)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t bk = 0; bk < nblk; ++bk) {
      const double *src = w + r * cols + bk * 16;
      uint8_t *dst = gguf_out + (r * nblk + bk) * 9;
      double ab = 0.0;
      for (int i = 0; i < 16; ++i) ab = fmax(ab, fabs(src[i]));
      int sc = (ab == 0.0) ? 0 : e4m3_encode_pos(ab / (6.0 * S));
      double sv = e4m3_value(sc);
      uint8_t q[16];
      for (int i = 0; i < 16; ++i) q[i] = (sv == 0.0) ? 0 : (uint8_t)e2m1_encode(src[i] / (sv * S));
      dst[0] = (uint8_t)sc;
      for (int j = 0; j < 8; ++j) dst[1 + j] = (uint8_t)(q[j] | (q[j + 8] << 4));
    }
  }
}

/* NVFP4(N(0, sigma)) matrix of stream (a, b) in GGUF-like order. */
int synth_nvfp4_normal(uint64_t seed, uint32_t a, uint32_t b, double sigma, int64_t rows, int64_t cols,
                       int pow2_tensor_scale, uint8_t *gguf_out, float *tensor_scale_out) {
  double *tmp = (double *)malloc(sizeof(double) * (size_t)(rows * cols));
  if (!tmp) return -1;
  fill_normal(seed, a, b, sigma, rows * cols, tmp);
  synth_quantize_nvfp4(tmp, rows, cols, pow2_tensor_scale, gguf_out, tensor_scale_out);
  free(tmp);
  return 0;
}

/* Zipf(alpha)-style router offset: rank = seeded permutation of 1..E,
 * b_e = -beta * alpha * ln(rank_e), then mean-centred.  The permutation is a
 * Fisher-Yates shuffle driven by Philox stream (0, 0x5A1F) of seed. */
void synth_zipf_offset(uint64_t seed, int32_t n_experts, double alpha, double beta, float *out) {
  int32_t *rank = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_experts);
  for (int32_t i = 0; i < n_experts; ++i) rank[i] = i + 1;
  for (int32_t i = n_experts - 1; i > 0; --i) {
    uint32_t ctr[4] = {(uint32_t)i, 0u, 0u, 0x5A1Fu};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    philox4x32_10(ctr, key, w);
    uint64_t r64 = ((uint64_t)w[0] << 32) | w[1];
    int32_t j = (int32_t)(r64 % (uint64_t)(i + 1));
    int32_t t = rank[i];
    rank[i] = rank[j];
    rank[j] = t;
  }
  double mean = 0.0;
  double *v = (double *)malloc(sizeof(double) * (size_t)n_experts);
  for (int32_t i = 0; i < n_experts; ++i) {
    v[i] = -beta * alpha * log((double)rank[i]);
    mean += v[i];
  }
  mean /= (double)n_experts;
  for (int32_t i = 0; i < n_experts; ++i) out[i] = (float)(v[i] - mean);
  free(v);
  free(rank);
}

/* BF16(1 + sigma * N(0,1)): per-channel gains of a pre-norm. */
void synth_gain_bf16(uint64_t seed, uint32_t a, uint32_t b, double sigma, int64_t n, uint16_t *out) {
  double *tmp = (double *)malloc(sizeof(double) * (size_t)n);
  fill_normal(seed, a, b, sigma, n, tmp);
  for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne((float)(1.0 + tmp[i]));
  free(tmp);
}

/* n_mats NVFP4(N(0, sigma)) matrices of rows x cols, matrix i drawn from
 * stream (a, b0 + i * b_stride), written back to back in GGUF-like order;
 * tensor scale of matrix i -> scales_out[i * scale_stride].  Parallel over
 * matrices. */
int synth_nvfp4_normal_stack(uint64_t seed, uint32_t a, uint32_t b0, uint32_t b_stride, int64_t n_mats,
                             double sigma, int64_t rows, int64_t cols, int pow2_tensor_scale,
                             uint8_t *out, float *scales_out, int64_t scale_stride) {
  e4m3_table_init();
  int64_t mbytes = rows * (cols / 16) * 9;
  int err = 0;
#pragma omp parallel
  {
    double *tmp = (double *)malloc(sizeof(double) * (size_t)(rows * cols));
    if (!tmp) {
#pragma omp atomic write
      err = -1;
    }
#pragma omp for schedule(dynamic, 1)
    for (int64_t i = 0; i < n_mats; ++i) {
      if (!tmp) continue;
      uint32_t b = b0 + (uint32_t)i * b_stride;
      int64_t n = rows * cols;
      for (int64_t p = 0; p < (n + 1) / 2; ++p) {
        double z0, z1;
        normal_pair(seed, a, b, (uint64_t)p, &z0, &z1);
        tmp[2 * p] = sigma * z0;
        if (2 * p + 1 < n) tmp[2 * p + 1] = sigma * z1;
      }
      /* serial quantiser per matrix (the outer loop is the parallel one) */
      double amax = 0.0;
      for (int64_t j = 0; j < n; ++j) amax = fmax(amax, fabs(tmp[j]));
      double S = amax / (6.0 * 448.0);
      if (S == 0.0) S = 1.0;
      if (pow2_tensor_scale) S = ldexp(1.0, (int)ceil(log2(S)));
      S = (double)(float)S;
      scales_out[i * scale_stride] = (float)S;
      uint8_t *dst0 = out + i * mbytes;
      int64_t nblk = cols / 16;
      for (int64_t r = 0; r < rows; ++r)
        for (int64_t bk = 0; bk < nblk; ++bk) {
          const double *src = tmp + r * cols + bk * 16;
          uint8_t *dst = dst0 + (r * nblk + bk) * 9;
          double ab = 0.0;
          for (int q = 0; q < 16; ++q) ab = fmax(ab, fabs(src[q]));
          int sc = (ab == 0.0) ? 0 : e4m3_encode_pos(ab / (6.0 * S));
          double sv = e4m3_value(sc);
          uint8_t qq[16];
          for (int q = 0; q < 16; ++q) qq[q] = (sv == 0.0) ? 0 : (uint8_t)e2m1_encode(src[q] / (sv * S));
          dst[0] = (uint8_t)sc;
          for (int j = 0; j < 8; ++j) dst[1 + j] = (uint8_t)(qq[j] | (qq[j + 8] << 4));
        }
    }
    free(tmp);
  }
  return err;
}

/* n_mats BF16(N(0, sigma)) matrices, matrix i from stream (a, b0 + i*b_stride). */
void synth_bf16_normal_stack(uint64_t seed, uint32_t a, uint32_t b0, uint32_t b_stride, int64_t n_mats,
                             double sigma, int64_t n_per_mat, uint16_t *out) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < n_mats; ++i) {
    uint32_t b = b0 + (uint32_t)i * b_stride;
    uint16_t *o = out + i * n_per_mat;
    for (int64_t p = 0; p < (n_per_mat + 1) / 2; ++p) {
      double z0, z1;
      normal_pair(seed, a, b, (uint64_t)p, &z0, &z1);
      o[2 * p] = f32_to_bf16_rne((float)(sigma * z0));
      if (2 * p + 1 < n_per_mat) o[2 * p + 1] = f32_to_bf16_rne((float)(sigma * z1));
    }
  }
}
