// Helpers shared by the decode kernels (gfx950): MFMA wrappers, cross-lane reductions,
// FP4 packing of probabilities, page lookup and streamed 16-byte loads.
#pragma once
#include "fp4kv_device.h"
#include "fp4kv_internal.h"

namespace fp4kv {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

template <int OPA, int OPB>
__device__ __forceinline__ v4f mfma4(const v8i &a, const v8i &b, v4f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 4, 4, OPA, sa, OPB, sb);
}

// lane l <- lane (l ^ 8) inside each row of 16 (row_ror:8)
__device__ __forceinline__ float xlane8(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false));
}
// lane l <- lane (l ^ 1) (quad_perm [1,0,3,2])
__device__ __forceinline__ float xlane1(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
}
// {x(l), x(l^16)} and {x(l), x(l^32)} pairs
__device__ __forceinline__ float max_x16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_x32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_x16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_x32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Four E2M1 conversions of consecutive token pairs into one dword:
// nibbles (x0[0..3], x1[0..3]) = tokens 4i..4i+3, 4i+4..4i+7, divided by the power of two `sc`.
template <int SEL>
__device__ __forceinline__ uint32_t cvt_pk(uint32_t old, float a, float b, float sc) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, sc, SEL);
}
__device__ __forceinline__ uint32_t pack8(const float *x0, const float *x1, float sc) {
  uint32_t w = 0u;
  w = cvt_pk<0>(w, x0[0], x0[1], sc);
  w = cvt_pk<1>(w, x0[2], x0[3], sc);
  w = cvt_pk<2>(w, x1[0], x1[1], sc);
  w = cvt_pk<3>(w, x1[2], x1[3], sc);
  return w;
}

// Physical page of logical page lp of sequence b, clamped to the sequence's last page
// (tokens past the end are masked, but their loads must stay inside the pool); a page
// id outside the pool is clamped into it, so a bad table reads wrong data, not memory
// outside the cache.
// A sequence's length clamped to [0, max_pages * P] (the tokens the block table can name).
__device__ __forceinline__ int seq_len_clamped(const DecodeArgs &a, int b) {
  const int L = a.seq_lens[b];
  return L < 0 ? 0 : min(L, a.max_pages * a.page_size);
}

__device__ __forceinline__ int phys_page(const DecodeArgs &a, int b, int lp, int last_lp) {
  int pg = a.block_table[(long)b * a.max_pages + (lp < last_lp ? lp : last_lp)];
  return pg < 0 ? 0 : (pg >= a.num_pages ? a.num_pages - 1 : pg);
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte load of streamed cache data: read once per step, so marked non-temporal.
__device__ __forceinline__ uint4 ld16(const uint8_t *p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
  return uint4{v[0], v[1], v[2], v[3]};
}

// byte k (compile-time after unrolling) of a 16-byte register group
__device__ __forceinline__ uint32_t byte_of(const uint4 &u, int k) {
  const uint32_t w = k < 4 ? u.x : (k < 8 ? u.y : (k < 12 ? u.z : u.w));
  return (w >> (8 * (k & 3))) & 0xFFu;
}

}  // namespace fp4kv
