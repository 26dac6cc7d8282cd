// Streaming-read kernel: the achievable HBM read bandwidth on this device, measured
// next to the decode kernel (16-byte loads, a few KB in flight per wave).
#include "fp4kv_internal.h"

namespace fp4kv {

__global__ __launch_bounds__(256) void stream_read(const uint4 *src, size_t n16, uint32_t *sink) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * 4;
  for (size_t i = (size_t)blockIdx.x * 256 * 4 + threadIdx.x; i < n16; i += stride) {
    uint4 v0 = src[i];
    uint4 v1 = i + 256 < n16 ? src[i + 256] : uint4{0, 0, 0, 0};
    uint4 v2 = i + 512 < n16 ? src[i + 512] : uint4{0, 0, 0, 0};
    uint4 v3 = i + 768 < n16 ? src[i + 768] : uint4{0, 0, 0, 0};
    acc ^= v0.x ^ v0.y ^ v0.z ^ v0.w ^ v1.x ^ v1.y ^ v1.z ^ v1.w;
    acc ^= v2.x ^ v2.y ^ v2.z ^ v2.w ^ v3.x ^ v3.y ^ v3.z ^ v3.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int k = 0; k < 256; k++) r ^= red[k];
    sink[blockIdx.x] = r;
  }
}

// Plain copy of n16 16-byte words (the known-size reference for the HBM traffic counters).
__global__ __launch_bounds__(256) void stream_copy(const uint4 *src, uint4 *dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

hipError_t launch_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t s) {
  size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  stream_copy<<<(unsigned)blocks, 256, 0, s>>>((const uint4 *)src, (uint4 *)dst, n16);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s) {
  size_t n16 = bytes / 16;
  size_t blocks = (n16 + 1023) / 1024;
  if (blocks > 4096) blocks = 4096;
  stream_read<<<(unsigned)blocks, 256, 0, s>>>((const uint4 *)src, n16, sink);
  return hipGetLastError();
}

}  // namespace fp4kv
