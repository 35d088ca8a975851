// Measurement kernel: one streaming read of a device buffer, the practical
// HBM read ceiling the decode kernels are compared with (and a read of
// known size to scale the hardware traffic counters by).
#include "common.h"

namespace moe {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 4;

// Every 16-byte piece of src read exactly once (grid-stride, kProbeUnroll
// independent loads in flight per lane), folded into one word that is
// stored only if it equals a constant, so no load can be dropped.
__global__ __launch_bounds__(kProbeThreads) void k_probe_read(const u32x4 *src, int64_t n16, uint32_t *sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4 v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x9E3779B9u) *sink = acc;
}

hipError_t launch_probe_read(const void *src, int64_t bytes, int32_t blocks, uint32_t *sink, hipStream_t stream) {
  hipLaunchKernelGGL(k_probe_read, dim3(blocks), dim3(kProbeThreads), 0, stream,
                     reinterpret_cast<const u32x4 *>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
