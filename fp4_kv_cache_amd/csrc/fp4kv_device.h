// Device-side scalar codecs and helpers shared by the gfx950 kernels.
//
// Formats: E2M1 elements and E8M0 scales as in the OCP Microscaling (MX) v1.0
// specification, E4M3 ("FN") scales as in the OCP 8-bit floating point
// specification; NVFP4 = 16-element blocks with an E4M3 scale and an fp32
// tensor scale.  Every quantization decision below is taken with single IEEE
// binary32 operations in a fixed order (the library is built with
// -ffp-contract=off), so that codes and scales are reproducible bit for bit.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4kv {

constexpr int kFmtNV = 0;
constexpr int kFmtMX = 1;

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Load element i of an fp32 or bf16 array as fp32 (bf16 -> fp32 is exact).
__device__ __forceinline__ float load_elem(const void *p, long i, int bf16) {
  return bf16 ? bf16_to_f32(((const uint16_t *)p)[i]) : ((const float *)p)[i];
}

// E2M1 conversions by the hardware (v_cvt_scalef32_pk_fp4_f32 / v_cvt_scalef32_pk_f32_fp4 with
// scale 1).  Encode: round to nearest with ties to the even code, saturation at +-6, the sign
// from y's sign bit (-0.0 gives code 8) -- the format's definition, which the GPU tests check
// against the oracle's encoder at every rounding threshold, its fp32 neighbours, the grid,
// values past 6, zeros and subnormals, both signs.  Decode: exact.
__device__ __forceinline__ uint32_t e2m1_enc_hw(float y) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y, y, 1.0f, 0) & 0xFu;
}
// byte = code(y0) | code(y1) << 4
__device__ __forceinline__ uint32_t e2m1_enc2_hw(float y0, float y1) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, y0, y1, 1.0f, 0) & 0xFFu;
}
__device__ __forceinline__ float e2m1_dec_hw(uint32_t c) { return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0)[0]; }
// dec(enc(y)): y rounded onto the E2M1 grid
__device__ __forceinline__ float e2m1_round_hw(float y) { return e2m1_dec_hw(e2m1_enc_hw(y)); }

// E4M3 byte -> fp32 (exact).  0x7F / 0xFF decode to NaN.
__device__ __forceinline__ float e4m3_dec(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0.001953125f;
  if (e == 15u && m == 7u) v = __uint_as_float(0x7FC00000u);
  return (c & 0x80u) ? -v : v;
}

// Non-negative fp32 -> E4M3 byte, round to nearest with ties to the even code,
// saturating at 448 (code 0x7E, so the NaN pattern is never produced).
__device__ __forceinline__ uint32_t e4m3_enc_sat(float t) {
  if (!(t < 448.0f)) return 0x7Eu;
  if (t < 0.015625f) return (uint32_t)rintf(t * 512.0f);  // multiples of 2^-9; 8 is code 0x08
  int e = (int)((__float_as_uint(t) >> 23) & 0xFFu) - 127;
  uint32_t q = (uint32_t)rintf(ldexpf(t, 3 - e));           // in [8, 16]
  if (q == 16u) { e += 1; q = 8u; }
  uint32_t code = ((uint32_t)(e + 7) << 3) | (q - 8u);
  return code > 0x7Eu ? 0x7Eu : code;
}

// ceil(log2 t) for t > 0 finite or +inf, clamped to [lo, hi]; t == 0 gives lo.
__device__ __forceinline__ int ceil_log2_clamp(float t, int lo, int hi) {
  uint32_t b = __float_as_uint(t);
  uint32_t ef = (b >> 23) & 0xFFu;
  if (ef == 0u) return lo;                       // zero or subnormal: below 2^-126
  int e = (int)ef - 127 + ((b & 0x7FFFFFu) ? 1 : 0);
  return e < lo ? lo : (e > hi ? hi : e);
}

// MX shared exponent floor(log2 amax) - 2, clamped to [-127, 127]; amax == 0 (or
// subnormal, whose floor(log2) is below -126) gives -127.
__device__ __forceinline__ int mx_exp(float amax) {
  uint32_t ef = (__float_as_uint(amax) >> 23) & 0xFFu;
  if (ef == 0u) return -127;
  int e = (int)ef - 127 - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Cache layout: byte offset of the MXFP4 key scale of (token t of the page, channel
// block q) inside its page and KV head.  The eight scales one decode lane needs (rows
// t, t+4, ..., t+28 of a 32-token span) are contiguous.
__device__ __forceinline__ int mx_kscale_off(int t, int q) {
  return (((t >> 5) * 4 + (t & 3)) * 4 + q) * 8 + ((t & 31) >> 2);
}

// Cache layout: byte offset of the value scale of (channel c, token block j) inside its
// page and KV head (head_dim 128), with J = min(P, 32) / B blocks per 32-token span.
// A decode lane's scales (channels c % 16 + 16 k, k = 0..7, over one span) are contiguous.
__device__ __forceinline__ int vscale_off(int c, int j, int J) {
  return ((j / J) * 16 + (c & 15)) * 8 * J + (c >> 4) * J + j % J;
}

// 2^e as fp32 for e in [-126, 127].
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

}  // namespace fp4kv
