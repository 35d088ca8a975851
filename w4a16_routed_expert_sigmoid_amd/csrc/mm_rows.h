// Matrix-core building blocks shared by the small-batch decode kernels and
// the small-tile prefill kernels: branch-free buffer loads, and one block's
// product of a group of NVFP4 weight rows with up to 16 token rows.
#pragma once

#include "common.h"

namespace moe {

constexpr int kMmWaves = 8;

__device__ __forceinline__ uint32_t word_of(const uint4 &q, int s) {
  return s == 0 ? q.x : s == 1 ? q.y : s == 2 ? q.z : q.w;
}

// Buffer resource of a device range of `bytes` bytes (< 4 GiB) for the
// raw buffer loads: an offset at or past the range's end reads zeros and
// touches no memory, so a lane with nothing to load takes kBufNone instead
// of a branch around its load.  (Loads under branches, divergent or
// uniform, leave the compiler unable to count the ones in flight, and it
// then waits for all of them before the first use of any.)  Word 3 is the
// gfx9 data format for raw 32-bit access.
constexpr uint32_t kBufNone = 0x80000000u;

// An offset chosen by a lane condition, passed through an empty asm
// statement: the compiler cannot see the choice and so does not split the
// load into two loads under branches.
__device__ __forceinline__ uint32_t buf_off(bool ok, uint32_t off) {
  uint32_t v = ok ? off : kBufNone;
  asm("" : "+v"(v));
  return v;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}

__device__ __forceinline__ float buf_load4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}

// Rows [row0, row0 + 16 RG) of an N x K NVFP4 matrix pair (TWO: W1 gate
// and W2 up) or of one matrix W1, times up to 16 token rows of K BF16
// elements each, on v_mfma_f32_16x16x32_bf16: A = four (RG) 16-row weight
// tiles, dequantised once per element; B column c = the token row xrow of
// lane c (lane & 15; -1: none) of x (x_rows rows of x_stride elements).
// K is split over the block's kMmWaves waves, two 128-K super-steps per
// pass with all their loads issued first, and the K-partial sums meet in
// s_red.  out(t, n, bits) receives, for every column t in colmask and row
// n < N, BF16(SiLU(BF16(g S1)) BF16(u S2)) (TWO, RG <= 4) or BF16(y S1)
// (RG <= 8).  Called by
// every thread of the block; ends after the block's last read of s_red
// (a later call must pass a barrier before writing it: the first barrier
// below).
template <int RG, bool TWO, typename Out>
__device__ __forceinline__ void mm_rows(int K, const uint16_t *x, int x_rows, int x_stride, int xrow,
                                        const uint8_t *W1, const uint8_t *W2, float S1, float S2, int N, int row0,
                                        uint32_t colmask, float (&s_red)[kMmWaves][32][kWave], Out out) {
  static_assert(RG % 2 == 0 && (TWO ? RG <= 4 : RG <= 8), "the partial sums fit s_red");
  constexpr int RS = TWO ? 8 : 4;  // s_red rows per row group
  const int C = K / 32;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int r16 = lane & 15, p = lane >> 4;
  f32x4 acc[RG][2];
#pragma unroll
  for (int rg = 0; rg < RG; ++rg) acc[rg][0] = acc[rg][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int SS = (C + 3) / 4;
  // Two super-steps per pass, all their loads issued before any math, in
  // the order the math consumes them (tokens, then row group by row group;
  // raw buffer loads, a lane out of range reading zeros).
  const __amdgpu_buffer_rsrc_t xr = buf_rsrc(x, (int64_t)x_rows * x_stride * 2);
  const __amdgpu_buffer_rsrc_t gr = buf_rsrc(W1, nvfp4_matrix_bytes(N, K));
  const __amdgpu_buffer_rsrc_t ur = buf_rsrc(TWO ? W2 : W1, nvfp4_matrix_bytes(N, K));
  for (int ss0 = wave; ss0 < SS; ss0 += 2 * kMmWaves) {
    uint4 qg[2][RG], qu[2][RG], xv[2][4];
    uint32_t sg[2][RG], su[2][RG];
#pragma unroll
    for (int v = 0; v < 2; ++v) {
      const int ss = ss0 + v * kMmWaves;
      const int c = ss * 4 + p;
      const bool cok = ss < SS && c < C;
      const bool tok = cok && xrow >= 0;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        xv[v][s] = buf_load16(xr, buf_off(tok, (uint32_t)(xrow * x_stride + c * 32 + s * 8) * 2u));
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
        const int n = row0 + rg * 16 + r16;
        const bool ok = cok && n < N;
        const uint32_t qo = buf_off(ok, (uint32_t)(n * (K / 2) + c * 16));
        const uint32_t so = buf_off(ok, (uint32_t)(N * (K / 2) + ((n >> 3) * (K / 32) + c) * 16 + (n & 7) * 2));
        qg[v][rg] = buf_load16(gr, qo);
        sg[v][rg] = buf_load2(gr, so);
        if (TWO) {
          qu[v][rg] = buf_load16(ur, qo);
          su[v][rg] = buf_load2(ur, so);
        }
      }
    }
    // all loads of both super-steps issued before any math: the math of
    // the first waits for its own loads only, while the second's arrive
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const bf16x8 bx = __builtin_bit_cast(bf16x8, u32x4{xv[v][s].x, xv[v][s].y, xv[v][s].z, xv[v][s].w});
          const float scg = e4m3_to_f32((sg[v][rg] >> (8 * (s >> 1))) & 0xffu);
          acc[rg][0] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8(word_of(qg[v][rg], s), scg), bx, acc[rg][0], 0, 0, 0);
          if (TWO) {
            const float scu = e4m3_to_f32((su[v][rg] >> (8 * (s >> 1))) & 0xffu);
            acc[rg][1] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(dq8(word_of(qu[v][rg], s), scu), bx, acc[rg][1], 0, 0, 0);
          }
        }
      }
  }
  // K-partial sums of the waves, then the BF16 results.
  __syncthreads();  // the previous user of s_red has finished reading it
#pragma unroll
  for (int rg = 0; rg < RG; ++rg)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s_red[wave][rg * RS + i][lane] = acc[rg][0][i];
      if (TWO) s_red[wave][rg * RS + 4 + i][lane] = acc[rg][1][i];
    }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < RG / 2; ++k) {
    const int idx = tid + k * kMmWaves * kWave;  // (row group, value, lane)
    const int rg = idx >> 8, i = (idx >> 6) & 3, l = idx & 63;
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int w = 0; w < kMmWaves; ++w) {
      g += s_red[w][rg * RS + i][l];
      if (TWO) u += s_red[w][rg * RS + 4 + i][l];
    }
    const int t = l & 15, n = row0 + rg * 16 + (l >> 4) * 4 + i;
    if (n < N && ((colmask >> t) & 1u)) {
      if (TWO) {
        const float gg = round_bf16(g * S1), uu = round_bf16(u * S2);
        out(t, n, f32_to_bf16(silu_mul(gg, uu)));
      } else {
        out(t, n, f32_to_bf16(g * S1));
      }
    }
  }
}

}  // namespace moe
