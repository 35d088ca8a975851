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

#include <type_traits>

#include "shapes.h"

namespace moe {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// FP32 -> BF16 bits, round to nearest even, by gfx950's
// v_cvt_pk_bf16_f32.  Checked on the GPU against exact integer rounding
// (add 0x7fff plus the kept LSB, NaN quieted) over 16.7M inputs: every
// exponent with edge mantissas, halfway cases, denormals, infinities, NaNs
// and random patterns, with no difference in any bit.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// Two FP32 -> packed BF16 bits (lo in bits 0..15), same rounding.
__device__ inline uint32_t f32x2_to_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ inline float round_bf16(float f) { return bf16_to_f32(f32_to_bf16(f)); }

// E4M3FN byte (low 8 bits of c) -> FP32 with the hardware conversion; on
// gfx950 it decodes the OCP E4M3FN format (bias 7, subnormals, S.1111.111 =
// NaN), which the exhaustive code test checks against the format table.
__device__ inline float e4m3_to_f32(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

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

// 8 FP4 (one dword, element 2i in the low nibble of byte i) times the block
// scale s -> 8 BF16, an MFMA operand.  E2M1 x E4M3 has at most 6
// significant bits, so each FP32 product is exact in BF16 and its upper
// half is the BF16 value.
__device__ __forceinline__ bf16x8 dq8(uint32_t w, float s) {
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  u32x4 r;
  r.x = __builtin_amdgcn_perm(__float_as_uint(v0.y * s), __float_as_uint(v0.x * s), 0x07060302u);
  r.y = __builtin_amdgcn_perm(__float_as_uint(v1.y * s), __float_as_uint(v1.x * s), 0x07060302u);
  r.z = __builtin_amdgcn_perm(__float_as_uint(v2.y * s), __float_as_uint(v2.x * s), 0x07060302u);
  r.w = __builtin_amdgcn_perm(__float_as_uint(v3.y * s), __float_as_uint(v3.x * s), 0x07060302u);
  return __builtin_bit_cast(bf16x8, r);
}

// value of lane ^ O for a compile-time O: DPP within 16-lane rows (xor 1,
// 2, 4, 8), the gfx950 cross-row swaps for 16 and 32.  No LDS round trip.
// Every lane reads a valid lane with these patterns, so bound_ctrl and the
// old value never show; with them set, the compiler can fold the move into
// the VALU instruction that consumes it.
template <int CTRL>
__device__ inline float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
template <int CTRL>
__device__ inline uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
}

template <int O, typename T>
__device__ inline T xor_lane(T v) {
  static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16 || O == 32, "xor offset");
  if constexpr (O == 1) return dpp<0xB1>(v);                   // quad_perm [1,0,3,2]
  else if constexpr (O == 2) return dpp<0x4E>(v);              // quad_perm [2,3,0,1]
  else if constexpr (O == 4) return dpp<0x1B>(dpp<0x141>(v));  // row_half_mirror, quad_perm [3,2,1,0]
  else if constexpr (O == 8) return dpp<0x128>(v);             // row_ror:8
  else {
    const uint32_t u = __builtin_bit_cast(uint32_t, v);
    const bool hi = (threadIdx.x & O) != 0;
    if constexpr (O == 16) {
      const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      return __builtin_bit_cast(T, hi ? (uint32_t)r[0] : (uint32_t)r[1]);
    } else {
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      return __builtin_bit_cast(T, hi ? (uint32_t)r[0] : (uint32_t)r[1]);
    }
  }
}

// Max over the wave, in every lane.  Within 16-lane rows: the quad swaps,
// then rotations by 4 and 8 (each lane ends with its row's max; 0 is the
// identity of the unsigned max, so the rotations may fold into the max).
// Across rows: each lane pair of the row and half swaps holds the two
// partners' values, whose max is the pair's.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t m) {
  return max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, CTRL, 0xF, 0xF, true));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
  m = dpp_max_u32<0xB1>(m);   // quad_perm [1,0,3,2]
  m = dpp_max_u32<0x4E>(m);   // quad_perm [2,3,0,1]
  m = dpp_max_u32<0x124>(m);  // row_ror:4
  m = dpp_max_u32<0x128>(m);  // row_ror:8
  const auto r16 = __builtin_amdgcn_permlane16_swap(m, m, false, false);
  m = max((uint32_t)r16[0], (uint32_t)r16[1]);
  const auto r32 = __builtin_amdgcn_permlane32_swap(m, m, false, false);
  return max((uint32_t)r32[0], (uint32_t)r32[1]);
}

// xor_lane with an offset that is a compile-time constant after unrolling.
template <typename T>
__device__ inline T xor_lane_n(T v, int o) {
  switch (o) {
    case 1: return xor_lane<1>(v);
    case 2: return xor_lane<2>(v);
    case 4: return xor_lane<4>(v);
    case 8: return xor_lane<8>(v);
    case 16: return xor_lane<16>(v);
    default: return xor_lane<32>(v);
  }
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1, unrolled at
// compile time (so register arrays indexed by I stay in registers).
template <int I, int N>
struct StaticFor {
  template <typename F>
  __device__ static __forceinline__ void run(F &&f) {
    f(std::integral_constant<int, I>());
    StaticFor<I + 1, N>::run(f);
  }
};
template <int N>
struct StaticFor<N, N> {
  template <typename F>
  __device__ static __forceinline__ void run(F &&) {}
};

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ inline float group_sum(float v, int width) {
  if (width > 1) v += xor_lane<1>(v);
  if (width > 2) v += xor_lane<2>(v);
  if (width > 4) v += xor_lane<4>(v);
  if (width > 8) v += xor_lane<8>(v);
  if (width > 16) v += xor_lane<16>(v);
  if (width > 32) v += xor_lane<32>(v);
  return v;
}

// Sum of a double over aligned groups of `width` lanes (each half of the
// value moves with the 32-bit exchanges above).
template <int O>
__device__ inline double xor_lane_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint64_t lo = xor_lane<O>((uint32_t)u), hi = xor_lane<O>((uint32_t)(u >> 32));
  return __builtin_bit_cast(double, lo | (hi << 32));
}

__device__ inline double group_sum_f64(double v, int width) {
  if (width > 1) v += xor_lane_f64<1>(v);
  if (width > 2) v += xor_lane_f64<2>(v);
  if (width > 4) v += xor_lane_f64<4>(v);
  if (width > 8) v += xor_lane_f64<8>(v);
  if (width > 16) v += xor_lane_f64<16>(v);
  if (width > 32) v += xor_lane_f64<32>(v);
  return v;
}

// FP64 -> BF16 bits, correctly rounded to nearest even: first to FP32 with
// round-to-odd (round toward zero, then set the last bit when inexact),
// then FP32 -> BF16 to nearest even; FP32 keeps 16 more bits than BF16, so
// the two steps round once.
__device__ inline uint32_t f64_to_bf16(double d) {
  if (d != d) return 0x7fc0u;
  const float f = (float)d;
  uint32_t u = __float_as_uint(f);
  const double back = (double)f;
  if (back != d) {
    if (fabs(back) > fabs(d)) u -= 1u;  // one FP32 step toward zero
    u |= 1u;
  }
  return f32_to_bf16(__uint_as_float(u));
}

// SiLU(g) * u in FP32 from the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32, each about 1 ulp).  Callers round the result to
// BF16, where an FP32 error of a few ulps can only move a value that sits
// at a BF16 rounding midpoint.  Very negative g gives 2^x = inf and a
// (correctly) zero SiLU.
__device__ inline float silu_mul(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
  return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Pre-norm output of the 8 BF16 elements of a 16-byte piece of x and of the
// gain: BF16 of x * inv * g, rounded from the product as FP64 gives it (inv
// = 1/sqrt(mean(x^2) + eps) in FP64).  The FP32 product (x * inv_f) * g is
// within a few FP32 ulps of it, so it rounds the same way unless it lies
// within 16 ulps of a BF16 rounding midpoint (low 16 bits near 0x8000);
// those rare elements are redone in FP64.  Eight FP32 products, four packed
// conversions, and one branch per piece, taken only when some element needs
// the redo.
__device__ inline uint4 norm_piece_bf16(uint4 xv, uint4 gv, float inv_f, double inv) {
  const uint32_t xq[4] = {xv.x, xv.y, xv.z, xv.w}, gq[4] = {gv.x, gv.y, gv.z, gv.w};
  float p[8];
  uint32_t near = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t xb = (e & 1) ? (xq[e >> 1] >> 16) : (xq[e >> 1] & 0xffffu);
    const uint32_t gb = (e & 1) ? (gq[e >> 1] >> 16) : (gq[e >> 1] & 0xffffu);
    p[e] = bf16_to_f32(xb) * inv_f * bf16_to_f32(gb);
    near |= ((__float_as_uint(p[e]) & 0xffffu) - 0x7ff0u <= 0x20u ? 1u : 0u) << e;
  }
  uint32_t o[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) o[d] = f32x2_to_bf16x2(p[2 * d], p[2 * d + 1]);
  if (near) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if ((near >> e) & 1u) {
        const uint32_t xb = (e & 1) ? (xq[e >> 1] >> 16) : (xq[e >> 1] & 0xffffu);
        const uint32_t gb = (e & 1) ? (gq[e >> 1] >> 16) : (gq[e >> 1] & 0xffffu);
        const uint32_t r = f64_to_bf16((double)bf16_to_f32(xb) * inv * (double)bf16_to_f32(gb));
        o[e >> 1] = (e & 1) ? ((o[e >> 1] & 0xffffu) | (r << 16)) : ((o[e >> 1] & 0xffff0000u) | r);
      }
    }
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// Device pointers of the decode workspace, carved from one caller buffer.
struct DecodeWs {
  float *logits;          // [B][E]
  uint16_t *xn;           // [B][H] normalised input (pre-norm layers)
  int32_t *n_routed;      // number of distinct selected experts
  int32_t *entry_expert;  // [max_routed] expert id, ascending
  uint32_t *entry_mask;   // [max_routed] bit t: token t uses the expert
  float *entry_w;         // [max_routed][8] combine weight per token
  int32_t *topk_idx;      // [B][k] (used when the caller passes none)
  float *topk_w;          // [B][k]
  uint16_t *h;            // [(max_routed + 1)][B][Imax] SiLU(g)*u, BF16
  // One token (router, gate/up and down in one kernel).  Values one block
  // publishes for others travel in 64-bit words: the value in the low half,
  // the tag of the layer call that wrote it in the high half.  The sync
  // region (lines, logit words, h words) is zeroed by the first kernel of
  // every call; within a call, layer calls carry distinct tags.
  uint32_t *sync_lines;   // [kSyncLines][kXcdSlots][64]: word 0 of each 256-byte line is used
  uint64_t *sync_l;       // [E] logit words
  uint64_t *sync_h;       // [(k + 1) * Imax / 2] h words (two BF16 values each)
  uint64_t *sync_y;       // [H / 2] layer-output words of the persistent step (two BF16 each)
  float *xcd_l;           // [kXcdSlots][stage_l] per-XCD copy of the logits
  uint16_t *xcd_h;        // [kXcdSlots][stage_elems] per-XCD copy of h
  uint32_t *status;       // OR of kStatus* bits: bounded waits that gave up (zeroed per call)
  int64_t stage_l;        // E rounded up to 64
  int64_t stage_elems;    // (one-token max_routed + 1) * Imax, rounded up to 128
  size_t bytes;
};

// Arguments of the decode kernels (passed by value).
struct DecodeArgs {
  int H, I, Is, E, k, B, residual, use_norm, max_routed, wtype;
  float eps;
  uint32_t tag;  // one token: this layer call's position in the enqueuing call, from 1
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
  // zero0[0, zero_n) and zero1[0, zero_n): words the router kernel zeroes
  // for a later kernel of the same call (the small-tile prefill's expert
  // counts and cursors); NULL otherwise
  int32_t *zero0, *zero1;
  int zero_n;
};

// Arguments of the prefill kernels (passed by value).  Row space of the
// grouped GEMMs: rows [0, P) are the P = T*k (token, expert) pairs sorted
// by expert, rows [P, P + T) the shared expert's, in token order.
struct PrefillArgs {
  int T, H, I, Is, E, k, wtype, residual, use_norm, P, max_tiles;
  int tile_rows;  // rows per GEMM tile: kPrefillTileRows, or kPrefillSmallRows (small-tile kernels)
  int rsplit;     // K splits of the router GEMM: logits holds rsplit partial [T][E] arrays
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
  int32_t *out_idx;  // [T][k]
  float *out_w;      // [T][k]
  uint16_t *xn;      // [T][H] (pre-norm layers)
  float *logits;     // [T][E]
  int32_t *counts, *offsets, *cursors;  // [E + 1] each
  int32_t *n_tiles;
  PfTile *tiles;          // [max_tiles]
  int32_t *sorted_tok;    // [P] token of each sorted row
  int32_t *pair_pos;      // [T][k] row of each (token, k) pair
  uint16_t *h_rows;       // [P + T][max(I, Is)] SiLU(g)*u, BF16
  uint16_t *y_rows;       // [P + T][H] expert outputs, BF16
};

// Arguments of the dense NVFP4 projection (passed by value).
struct GemvArgs {
  const uint8_t *w;      // one NVFP4 matrix [N][K], runtime layout
  const float *scale;    // its FP32 tensor scale (device)
  const uint16_t *x;     // [B][K] BF16
  uint16_t *y;           // [B][N] BF16
  int N, K, B;
};
constexpr int kGemvThreads = 256;

hipError_t launch_gemv(const GemvArgs &g, hipStream_t stream);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t stream);

hipError_t launch_decode(const DecodeArgs &a, hipStream_t stream, hipEvent_t const *stage_events);
// The router of a batch of a.B tokens alone (one row of blocks per token):
// the pre-norm into ws.xn when the layer has one, the logits into
// ws.logits, and the zero0/zero1 words.  a.H <= kRouterTokenMaxHidden (a
// block stages its token in LDS).
constexpr int kRouterTokenMaxHidden = 16384;
hipError_t launch_router_tokens(const DecodeArgs &a, hipStream_t stream);

// The persistent one-token step: n_layers consecutive MoE layers of one
// shape in one launch.  a: the shapes and workspace of the first layer, x
// its input, y the last layer's output, tag the first layer's tag; L: each
// layer's weights; stage_*: the per-layer stage sets (slot l at base + l *
// slot_bytes).
struct PersistLayer {
  const uint16_t *router_w;
  const float *router_b;
  const uint8_t *w_gate, *w_up, *w_down;
  const float *w_scale;
  const uint8_t *sh_gate, *sh_up, *sh_down;
  const float *sh_scale;
  const uint16_t *norm_gain;
};
struct PersistArgs {
  DecodeArgs a;
  uint8_t *stages;
  int64_t slot_bytes, off_h, off_y;
  int n_layers;
  PersistLayer L[kPersistMaxLayers];
};
// Whether the persistent kernel's blocks for these shapes can all be
// resident at once on the current device (its hand-overs need that).
hipError_t persist_fits(const DecodeArgs &a, bool *fits);
hipError_t launch_step_b1(const PersistArgs &p, hipStream_t stream);
// Zeroes words [0, words) of a decode workspace (its status word and sync
// region) before a call's kernels run.
hipError_t launch_sync_clear(uint32_t *region, int64_t words, hipStream_t stream);
hipError_t launch_repack(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                         int32_t *nan_count, hipStream_t stream);
hipError_t launch_unpack(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                         hipStream_t stream);
hipError_t launch_dequant(const void *src, float *dst, int64_t rows, int64_t cols, int64_t n_mats,
                          const float *tensor_scale, hipStream_t stream);
hipError_t launch_probe_read(const void *src, int64_t bytes, int32_t blocks, uint32_t *sink, hipStream_t stream);

}  // namespace moe
