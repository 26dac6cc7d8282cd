// Streaming-read kernel: the achievable HBM read bandwidth on this device, measured
// next to the decode kernel (16-byte loads, a few KB in flight per wave).
#include "decode_common.h"

namespace fp4kv {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Eight non-temporal 16-byte loads in flight per thread (the fastest plain streaming
// read measured on MI355X); a ragged end is read by the bounds-checked tail loop.
__global__ __launch_bounds__(256) void stream_read(const uint4 *src, size_t n16, uint32_t *sink) {
  constexpr int U = 8;
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x;
  for (; i + 256 * (U - 1) < n16; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; u++) v[u] = __builtin_nontemporal_load((const u32x4 *)(src + i + 256 * u));
#pragma unroll
    for (int u = 0; u < U; u++) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += 256) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)(src + i));
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
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

// E2M1 codes of x / 2^e (the conversion divides by its scale operand) with the hardware conversion the decode kernels use for the
// probabilities (v_cvt_scalef32_pk_fp4_f32, the same call sequence as their packing): thread i
// converts x[8 i .. 8 i + 7] into one word, byte j = code(x[2 j]) | code(x[2 j + 1]) << 4.
__global__ __launch_bounds__(256) void pack_e2m1(const float *x, size_t n8, float scale, uint32_t *out) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const float *p = x + 8 * i;
  out[i] = pack8(p, p + 4, scale);
}

hipError_t launch_pack_e2m1(const float *x, size_t n, int scale_exp, uint8_t *out, hipStream_t s) {
  const size_t n8 = n / 8;
  pack_e2m1<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(x, n8, ldexpf(1.0f, scale_exp), (uint32_t *)out);
  return hipGetLastError();
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
  size_t blocks = (n16 + 2047) / 2048;
  if (blocks > 2048) blocks = 2048;
  stream_read<<<(unsigned)blocks, 256, 0, s>>>((const uint4 *)src, n16, sink);
  return hipGetLastError();
}

}  // namespace fp4kv
