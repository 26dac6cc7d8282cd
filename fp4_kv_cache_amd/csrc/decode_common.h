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

// An E4M3 scale S on the E8M0-scaled MFMA: S = t0 + t1 - t2 with t0, t1, t2 powers of two or
// zero, each applied by one MFMA pass whose scale byte is that power (byte 0 = 2^-127 for an
// absent term: its products fall below fp32 resolution).  The third term is always the
// subtracted one, so its pass runs on operands with flipped sign bits for every row alike.
// In units of 2^(E-3), a normal S = 2^E (8 + m) / 8 is
//   8, 8+1, 8+2, 8+4-1, 8+4, 16+1-4, 16-2, 16-1   (m = 0 .. 7),
// a subnormal S = m 2^-9 is 1, 2, 2+1, 4, 4+1, 4+2, 8-1.  Bytes 0 and 1 hold the added terms,
// byte 2 the subtracted one (E8M0 exponent + 127).  Codes 0x7F and above give no term.
constexpr uint32_t e4m3_pass_word(int c) {
  if (c < 0 || c >= 0x7F) return 0u;
  const int ef = c >> 3, m = c & 7;
  // exponents (relative to the unit) of t0, t1, t2; -99 = absent
  constexpr int kAbs = -99;
  const int unit = ef != 0 ? ef - 7 - 3 : -9;
  int e0 = kAbs, e1 = kAbs, e2 = kAbs;
  if (ef != 0) {
    constexpr int t0[8] = {3, 3, 3, 3, 3, 4, 4, 4};
    constexpr int t1[8] = {kAbs, 0, 1, 2, 2, 0, kAbs, kAbs};
    constexpr int t2[8] = {kAbs, kAbs, kAbs, 0, kAbs, 2, 1, 0};
    e0 = t0[m], e1 = t1[m], e2 = t2[m];
  } else {
    constexpr int t0[8] = {kAbs, 0, 1, 1, 2, 2, 2, 3};
    constexpr int t1[8] = {kAbs, kAbs, kAbs, 0, kAbs, 0, 1, kAbs};
    constexpr int t2[8] = {kAbs, kAbs, kAbs, kAbs, kAbs, kAbs, kAbs, 0};
    e0 = t0[m], e1 = t1[m], e2 = t2[m];
  }
  auto byte = [unit](int e) -> uint32_t { return e == kAbs ? 0u : (uint32_t)(unit + e + 127); };
  return byte(e0) | (byte(e1) << 8) | (byte(e2) << 16);
}

namespace detail {
constexpr double pow2c(int e) {
  double r = 1.0;
  for (; e > 0; e--) r *= 2.0;
  for (; e < 0; e++) r *= 0.5;
  return r;
}
// every finite non-negative E4M3 code: t0 + t1 - t2 is the scale itself
constexpr bool pass_words_are_exact() {
  for (int c = 0; c < 0x7F; c++) {
    const uint32_t w = e4m3_pass_word(c);
    double s = 0.0;
    for (int k = 0; k < 3; k++) {
      const int b = (int)((w >> (8 * k)) & 0xFFu);
      if (b == 0) continue;
      s += (k == 2 ? -1.0 : 1.0) * pow2c(b - 127);
    }
    if ((w >> 24) != 0u) return false;
    const int ef = c >> 3, m = c & 7;
    const double want = ef != 0 ? pow2c(ef - 7) * (8 + m) / 8.0 : pow2c(-6) * m / 8.0;
    if (s != want) return false;
  }
  return e4m3_pass_word(0x7F) == 0u && e4m3_pass_word(0x80) == 0u;
}
static_assert(pass_words_are_exact(), "E4M3 pass words must sum to the scale");
}  // namespace detail

// Sign bits of the eight E2M1 codes of a word: the operand of the subtracted term's pass.
constexpr uint32_t kFp4SignBits = 0x88888888u;

// Ablation study only (normalized P): P.V of one 16-token parity when the P block scale is a
// general E4M3 value like the value scale -- both as signed-digit passes, 3 x 3 MFMAs; a term
// takes the sign-flipped P when exactly one of its two digits is the subtracted one.
template <int DV, int DP>
__device__ __forceinline__ v4f pv_term(const v8i &av, const v8i &p, const v8i &pn, v4f c, int lv, int lp) {
  return mfma4<DV, DP>(av, ((DV == 2) != (DP == 2)) ? pn : p, c, lv, lp);
}
__device__ __forceinline__ v4f pv_general(const v8i &av, const v8i &p, const v8i &pn, v4f c, int lv, int lp) {
  c = pv_term<0, 0>(av, p, pn, c, lv, lp);
  c = pv_term<0, 1>(av, p, pn, c, lv, lp);
  c = pv_term<0, 2>(av, p, pn, c, lv, lp);
  c = pv_term<1, 0>(av, p, pn, c, lv, lp);
  c = pv_term<1, 1>(av, p, pn, c, lv, lp);
  c = pv_term<1, 2>(av, p, pn, c, lv, lp);
  c = pv_term<2, 0>(av, p, pn, c, lv, lp);
  c = pv_term<2, 1>(av, p, pn, c, lv, lp);
  return pv_term<2, 2>(av, p, pn, c, lv, lp);
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
// The two E2M1 codes of byte SEL of w, times the power of two `sc` (exact): hardware decode.
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2f dec_pk(uint32_t w, int sel, float sc) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, sc, 3);
  }
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

// ---------------- balanced partition of the work ----------------
// The work of one launch is the list of all 128-token tiles of all (sequence, KV head)
// units (MLA: one latent head, so a unit is a sequence), in the order u = b * Hkv + kvh,
// tiles in sequence order within a unit.  Wave i of
// the W waves that get work takes tiles [floor(i T / W), floor((i+1) T / W)) of this list
// (T tiles in all), so every wave streams the same number of tiles however ragged the
// sequence lengths are.  A wave whose range crosses unit boundaries writes one partial
// per unit it touches, into slot i + u: the ranges are ordered like the units, so no two
// (wave, unit) pairs share a slot and the slots of one unit are consecutive.  A batch with
// fewer tiles than planned waves gets one tile per wave (it is latency-bound).
constexpr int kMinTilesPerWave = 1;

// A sequence's tiles of 128 tokens.
__device__ __forceinline__ int seq_tiles(const DecodeArgs &a, int b) { return (seq_len_clamped(a, b) + 127) >> 7; }

__device__ __forceinline__ long uni_l(long v) {
  const int lo = __builtin_amdgcn_readfirstlane((int)(unsigned)(v & 0xffffffffL));
  const int hi = __builtin_amdgcn_readfirstlane((int)(v >> 32));
  return (long)(((unsigned long)(unsigned)hi << 32) | (unsigned)lo);
}

// The wave's share: the current unit (b, kvh) with its n tiles starting at flattened
// index ustart, and the flattened range [x, x1) still to do; L is sequence b's length.
struct Share {
  long x, x1, ustart, total;
  int b, kvh, n, waves, L;
};

// Wave count W and total T as every kernel of a launch computes them.
__device__ __forceinline__ void work_total(const DecodeArgs &a, int lane, long &total, int &waves) {
  long t = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64)
    if (b0 + lane < a.batch) t += seq_tiles(a, b0 + lane);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o);
  total = uni_l(t * a.hkv);
  const long useful = (total + kMinTilesPerWave - 1) / kMinTilesPerWave;
  waves = (int)(useful < (long)a.n_waves ? useful : (long)a.n_waves);
}

// Wave that holds flattened tile x.
__device__ __forceinline__ long owner_of(long x, long total, int waves) {
  return ((x + 1) * waves + total - 1) / total - 1;
}

// Finds the wave's share; false when it has no tiles.
__device__ inline bool find_share(const DecodeArgs &a, int wave, int lane, Share &s) {
  if (a.batch <= 64) {
    // one pass: lane b holds sequence b's length; the total is the scan's last entry
    const int len = lane < a.batch ? seq_len_clamped(a, lane) : 0;
    const int t = (len + 127) >> 7;
    int incl = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    s.total = uni_l((long)__shfl(incl, 63) * a.hkv);
    const long useful = (s.total + kMinTilesPerWave - 1) / kMinTilesPerWave;
    s.waves = (int)(useful < (long)a.n_waves ? useful : (long)a.n_waves);
    if (wave >= s.waves) return false;
    const long T = s.total, W = s.waves;
    s.x = wave * T / W;
    s.x1 = (wave + 1) * T / W;
    const unsigned long long m = __ballot((long)incl * a.hkv > s.x);
    const int j = __builtin_ctzll(m);   // m != 0: x < T
    const int n = __builtin_amdgcn_readfirstlane(__shfl(t, j));
    const long before = uni_l((long)__shfl(incl, j) - n);   // tiles of sequences < b
    s.b = j;
    s.n = n;
    s.L = __builtin_amdgcn_readfirstlane(__shfl(len, j));
    s.kvh = (int)((s.x - before * a.hkv) / n);
    s.ustart = before * a.hkv + (long)s.kvh * n;
    return true;
  }
  work_total(a, lane, s.total, s.waves);
  if (wave >= s.waves) return false;
  const long T = s.total, W = s.waves;
  s.x = wave * T / W;
  s.x1 = (wave + 1) * T / W;
  // the sequence whose units hold tile x: scan the tile counts 64 sequences at a time
  long carry = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int len = b0 + lane < a.batch ? seq_len_clamped(a, b0 + lane) : 0;
    const int t = (len + 127) >> 7;
    int incl = t;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o);
      if (lane >= o) incl += v;
    }
    const unsigned long long m = __ballot((carry + incl) * a.hkv > s.x);
    if (m) {
      const int j = __builtin_ctzll(m);
      const int n = __builtin_amdgcn_readfirstlane(__shfl(t, j));
      const long before = uni_l(carry + __shfl(incl, j) - n);   // tiles of sequences < b
      s.b = b0 + j;
      s.n = n;
      s.L = __builtin_amdgcn_readfirstlane(__shfl(len, j));
      s.kvh = (int)((s.x - before * a.hkv) / n);
      s.ustart = before * a.hkv + (long)s.kvh * n;
      return true;
    }
    carry += __shfl(incl, 63);
  }
  return false;   // not reached: x < T
}

// Moves a share past the unit that ends at flattened tile uend to the next unit that has
// tiles; false when the share ends there.
__device__ inline bool next_unit(const DecodeArgs &a, Share &s, long uend) {
  if (s.x1 <= uend) return false;
  s.x = s.ustart = uend;
  if (++s.kvh == a.hkv) {
    s.kvh = 0;
    do {
      if (++s.b >= a.batch) return false;
      s.L = seq_len_clamped(a, s.b);
      s.n = (s.L + 127) >> 7;
    } while (s.n == 0);
  }
  return true;
}

}  // namespace fp4kv
