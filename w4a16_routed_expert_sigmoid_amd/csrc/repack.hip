// Load-time lossless repack of NVFP4 matrices from the GGUF-like block order
// into the runtime layout, and its inverse.
//
// "Day-0 Support for Flint on vLLM", section "Model architecture": the
// checkpoint stores NVIDIA NVFP4 blocks in GGUF with a different byte order
// and is repacked without loss when loaded.  The exact GGUF order is not
// given on the pages; the source order read here is: per row, blocks of 16
// elements along K as 9 bytes [E4M3 scale][8 nibble bytes], nibble byte j
// holding element j (low nibble) and element j+8 (high nibble).
//
// One thread moves one (matrix, 8-row group, 32-element chunk) tile: 8 rows
// x 2 source blocks (144 bytes) -> 8 nibble rows of 16 bytes + one 16-byte
// scale tile.
#include "common.h"

namespace moe {

// Source block (8 nibble bytes, half-split order) -> 8 bytes of adjacent
// pairs (element 2i low, 2i+1 high).
__device__ inline uint64_t halfsplit_to_pairs(const uint8_t *nb) {
  uint8_t q[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    q[j] = nb[j] & 15u;
    q[j + 8] = nb[j] >> 4;
  }
  uint64_t out = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) out |= (uint64_t)(q[2 * i] | (q[2 * i + 1] << 4)) << (8 * i);
  return out;
}

__device__ inline void pairs_to_halfsplit(uint64_t v, uint8_t *nb) {
  uint8_t q[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint8_t b = (uint8_t)(v >> (8 * i));
    q[2 * i] = b & 15u;
    q[2 * i + 1] = b >> 4;
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) nb[j] = (uint8_t)(q[j] | (q[j + 8] << 4));
}

__global__ void k_repack(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t cols, int64_t n_mats,
                         int32_t *nan_count) {
  const int64_t chunks = cols / 32, groups = rows / 8;
  const int64_t tiles = n_mats * groups * chunks;
  const int64_t mbytes = nvfp4_matrix_bytes(rows, cols);
  int nan = 0;
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < tiles; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = t % chunks, g = (t / chunks) % groups, m = t / (chunks * groups);
    const uint8_t *s = src + m * mbytes;
    uint8_t *d = dst + m * mbytes;
    uint8_t tile[16];
    for (int r = 0; r < 8; ++r) {
      const int64_t row = g * 8 + r;
      const uint8_t *b0 = s + (row * (cols / 16) + 2 * c) * 9;  // blocks 2c and 2c+1
      uint64_t lo = halfsplit_to_pairs(b0 + 1), hi = halfsplit_to_pairs(b0 + 10);
      uint64_t *dn = reinterpret_cast<uint64_t *>(d + row * (cols / 2) + c * 16);
      dn[0] = lo;
      dn[1] = hi;
      tile[2 * r] = b0[0];
      tile[2 * r + 1] = b0[9];
      nan += ((b0[0] & 0x7f) == 0x7f) + ((b0[9] & 0x7f) == 0x7f);
    }
    uint8_t *ds = d + rows * cols / 2 + (g * chunks + c) * 16;
    for (int q = 0; q < 16; ++q) ds[q] = tile[q];
  }
  if (nan_count && nan) atomicAdd(nan_count, nan);
}

__global__ void k_unpack(const uint8_t *src, uint8_t *dst, int64_t rows, int64_t cols, int64_t n_mats) {
  const int64_t chunks = cols / 32, groups = rows / 8;
  const int64_t tiles = n_mats * groups * chunks;
  const int64_t mbytes = nvfp4_matrix_bytes(rows, cols);
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < tiles; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = t % chunks, g = (t / chunks) % groups, m = t / (chunks * groups);
    const uint8_t *s = src + m * mbytes;
    uint8_t *d = dst + m * mbytes;
    const uint8_t *ss = s + rows * cols / 2 + (g * chunks + c) * 16;
    for (int r = 0; r < 8; ++r) {
      const int64_t row = g * 8 + r;
      const uint64_t *sn = reinterpret_cast<const uint64_t *>(s + row * (cols / 2) + c * 16);
      uint8_t *b0 = d + (row * (cols / 16) + 2 * c) * 9;
      b0[0] = ss[2 * r];
      pairs_to_halfsplit(sn[0], b0 + 1);
      b0[9] = ss[2 * r + 1];
      pairs_to_halfsplit(sn[1], b0 + 10);
    }
  }
}

// Runtime layout -> FP32 values E2M1 * E4M3 * tensor_scale, through the same
// conversions the GEMV kernels use (FP4 pair -> BF16 pair, E4M3 -> FP32).
__global__ void k_dequant(const uint8_t *src, float *dst, int64_t rows, int64_t cols, int64_t n_mats,
                          const float *tensor_scale) {
  const int64_t chunks = cols / 32, groups = rows / 8;
  const int64_t tiles = n_mats * groups * chunks;
  const int64_t mbytes = nvfp4_matrix_bytes(rows, cols);
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < tiles; t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = t % chunks, g = (t / chunks) % groups, m = t / (chunks * groups);
    const uint8_t *s = src + m * mbytes;
    const float S = tensor_scale ? tensor_scale[m] : 1.0f;
    const uint4 sc = *reinterpret_cast<const uint4 *>(s + rows * cols / 2 + (g * chunks + c) * 16);
    const uint32_t scw[4] = {sc.x, sc.y, sc.z, sc.w};
    for (int r = 0; r < 8; ++r) {
      const int64_t row = g * 8 + r;
      const uint4 nb = *reinterpret_cast<const uint4 *>(s + row * (cols / 2) + c * 16);
      const uint32_t nw[4] = {nb.x, nb.y, nb.z, nb.w};
      const uint32_t sword = scw[r >> 1] >> ((r & 1) * 16);
      const float s0 = e4m3_to_f32(sword & 0xffu), s1 = e4m3_to_f32((sword >> 8) & 0xffu);
      float *o = dst + (m * rows + row) * cols + c * 32;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const float bs = (d < 2 ? s0 : s1) * S;
        bf16x2 p0 = MOE_FP4X2_TO_BF16X2(nw[d], 0), p1 = MOE_FP4X2_TO_BF16X2(nw[d], 1);
        bf16x2 p2 = MOE_FP4X2_TO_BF16X2(nw[d], 2), p3 = MOE_FP4X2_TO_BF16X2(nw[d], 3);
        o[d * 8 + 0] = (float)p0.x * bs;
        o[d * 8 + 1] = (float)p0.y * bs;
        o[d * 8 + 2] = (float)p1.x * bs;
        o[d * 8 + 3] = (float)p1.y * bs;
        o[d * 8 + 4] = (float)p2.x * bs;
        o[d * 8 + 5] = (float)p2.y * bs;
        o[d * 8 + 6] = (float)p3.x * bs;
        o[d * 8 + 7] = (float)p3.y * bs;
      }
    }
  }
}

static int grid_for(int64_t tiles, int block) {
  int64_t g = (tiles + block - 1) / block;
  return (int)(g < 65536 ? (g > 0 ? g : 1) : 65536);
}

hipError_t launch_repack(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                         int32_t *nan_count, hipStream_t stream) {
  const int64_t tiles = n_mats * (rows / 8) * (cols / 32);
  hipLaunchKernelGGL(k_repack, dim3(grid_for(tiles, 256)), dim3(256), 0, stream, (const uint8_t *)src,
                     (uint8_t *)dst, rows, cols, n_mats, nan_count);
  return hipGetLastError();
}

hipError_t launch_unpack(const void *src, void *dst, int64_t rows, int64_t cols, int64_t n_mats,
                         hipStream_t stream) {
  const int64_t tiles = n_mats * (rows / 8) * (cols / 32);
  hipLaunchKernelGGL(k_unpack, dim3(grid_for(tiles, 256)), dim3(256), 0, stream, (const uint8_t *)src,
                     (uint8_t *)dst, rows, cols, n_mats);
  return hipGetLastError();
}

hipError_t launch_dequant(const void *src, float *dst, int64_t rows, int64_t cols, int64_t n_mats,
                          const float *tensor_scale, hipStream_t stream) {
  const int64_t tiles = n_mats * (rows / 8) * (cols / 32);
  hipLaunchKernelGGL(k_dequant, dim3(grid_for(tiles, 256)), dim3(256), 0, stream, (const uint8_t *)src, dst,
                     rows, cols, n_mats, tensor_scale);
  return hipGetLastError();
}

}  // namespace moe
