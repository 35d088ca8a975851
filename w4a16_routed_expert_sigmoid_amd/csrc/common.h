// Internal definitions shared by the library's HIP kernels and host code.
//
// Runtime NVFP4 layout of one matrix W[N][K] (N % 8 == 0, K % 32 == 0),
// written by the load-time repack:
//   nibble plane  N * K/2 bytes, row-major; byte i of row n holds element
//                 2i in its low nibble and element 2i+1 in its high nibble,
//                 so a 16-byte load is one 32-element "chunk" of a row.
//   scale plane   N/8 * K/32 tiles of 16 bytes; tile (g, c) holds the two
//                 E4M3 block scales of chunk c for rows 8g..8g+7 as
//                 [row 0: block 2c, block 2c+1][row 1: ...]...[row 7: ...],
//                 so one 16-byte load serves one lane's 8 rows of a chunk.
// A lane of a GEMV owns (8-row group, chunk) pairs: 8 nibble loads and one
// scale load of 16 bytes each, all coalesced across the lanes of a wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxBatch = 8;   // decode path: up to eight tokens
constexpr int kMaxTopK = 8;
constexpr int kMaxExperts = 1024;

__host__ __device__ inline int64_t nvfp4_nibble_bytes(int64_t n, int64_t k) { return n * k / 2; }
__host__ __device__ inline int64_t nvfp4_matrix_bytes(int64_t n, int64_t k) { return n * k / 2 + n * k / 16; }

// Lanes that share one row: all 64 when a row has >= 64 chunks (each lane
// then walks chunks lane, lane+64, ...), else the chunk count, which must
// be a power of two.
__host__ __device__ inline int lanes_per_row(int k) {
  int c = k / 32;
  return c >= kWave ? kWave : c;
}

__host__ inline bool k_tileable(int64_t k) {
  if (k <= 0 || k % 32) return false;
  int64_t c = k / 32;
  return c >= kWave || (c & (c - 1)) == 0;
}

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// FP32 -> BF16 bits, round to nearest even (finite and infinite inputs;
// NaN stays NaN).
__device__ inline uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ inline float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// E4M3FN byte -> FP32: exponent field e (bias 7), mantissa m; e == 0 is
// subnormal m * 2^-9; S.1111.111 is NaN.
__device__ inline float e4m3_to_f32(uint32_t c) {
  uint32_t em = c & 0x7fu;
  float v = (em >= 8u) ? __uint_as_float((em << 20) + 0x3c000000u) : (float)em * 0x1p-9f;
  if (em == 0x7fu) v = __uint_as_float(0x7fc00000u);
  return __uint_as_float(__float_as_uint(v) | ((c & 0x80u) << 24));
}

// Two FP4 (E2M1) values of byte `sel` of w -> two BF16 (exact).
#define MOE_FP4X2_TO_BF16X2(w, sel) __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((w), 1.0f, (sel))

// acc + a.x*b.x + a.y*b.y with BF16 inputs and FP32 accumulation.
__device__ inline float dot2_bf16(bf16x2 a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(bf16x2, b), acc, false);
}

__device__ inline float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                         acc, false);
}

// acc + sum of the 8 FP4 elements of w (element 2i in the low nibble of
// byte i) times 8 BF16 activations x[0..3] (two per word, low half first).
__device__ inline float dot8_fp4_bf16(uint32_t w, uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                      float acc) {
  acc = dot2_bf16(MOE_FP4X2_TO_BF16X2(w, 0), x0, acc);
  acc = dot2_bf16(MOE_FP4X2_TO_BF16X2(w, 1), x1, acc);
  acc = dot2_bf16(MOE_FP4X2_TO_BF16X2(w, 2), x2, acc);
  acc = dot2_bf16(MOE_FP4X2_TO_BF16X2(w, 3), x3, acc);
  return acc;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ inline float group_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Device pointers of the decode workspace, carved from one caller buffer.
struct DecodeWs {
  uint32_t *counter;      // completion counter of the router kernel (kept 0)
  float *logits;          // [B][E]
  uint16_t *xn;           // [B][H] normalised input (pre-norm layers)
  int32_t *n_routed;      // number of distinct selected experts
  int32_t *entry_expert;  // [max_routed] expert id, ascending
  uint32_t *entry_mask;   // [max_routed] bit t: token t uses the expert
  float *entry_w;         // [max_routed][8] combine weight per token
  int32_t *topk_idx;      // [B][k] (used when the caller passes none)
  float *topk_w;          // [B][k]
  uint16_t *h;            // [(max_routed + 1)][B][Imax] SiLU(g)*u, BF16
  size_t bytes;
};

// Arguments of the decode kernels (passed by value).
struct DecodeArgs {
  int H, I, Is, E, k, B, residual, use_norm, max_routed, wtype;
  float eps;
  const uint16_t *x;
  uint16_t *y;
  const uint16_t *router_w;
  const float *router_b;
  const uint8_t *w_gate, *w_up, *w_down;
  const float *w_scale;
  const uint8_t *sh_gate, *sh_up, *sh_down;
  const float *sh_scale;
  const uint16_t *norm_gain;
  int32_t *out_idx;
  float *out_w;
  DecodeWs ws;
};

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_repack(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                         int32_t *nan_count, hipStream_t stream);
hipError_t launch_unpack(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                         hipStream_t stream);
hipError_t launch_dequant(const void *src, float *dst, int64_t rows, int64_t cols, int64_t n_mats,
                          const float *tensor_scale, hipStream_t stream);

}  // namespace moe
