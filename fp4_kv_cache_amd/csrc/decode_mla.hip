// Paged FP4 decode attention for MLA on gfx950: all query heads share one latent head
// that serves as key and value, plus an unquantized bf16 rope part of the key.
//
// Method ("BitDecoding-FP4: Native FP4 KV Cache Decoding via Algorithm-System
// Co-Design", Article Summary: the design covers GQA and MLA models; "BitDecoding-FP4 :
// décodage natif du KV cache FP4", Analyse approfondie): dual-residual FP4 query,
// stacked query rows sharing each latent tile, transposed softmax with fused
// underflow-aware FP4 probability quantization.
//
// Mapping onto CDNA4, NVFP4 latent (one workgroup of eight waves = one (sequence, split) for
// four groups of 16 query heads; per group one wave for Q.K^T and softmax, one for P.V):
//  * The latent is quantized in 16-token x 16-channel tiles with an E4M3 scale each.  For
//    Q.K^T the latent codes are widened to fp16 with their tile scale (code * S has at
//    most six significant bits, so the fp16 value is exact) and the dual-residual query
//    rows are fp16 as well (FP4 code times a power-of-two block scale, exact); the
//    contraction runs on v_mfma_f32_16x16x32_f16 with exact products and fp32
//    accumulation, so the logit is the exact dot up to the matrix core's fp32
//    summation order.  The rope part runs on the bf16 MFMA.
//  * MFMA K index -> channel: lane group q (lanes 16q..16q+15) takes channels
//    128q + 8s .. 128q + 8s + 7 in K-step s, so each lane reads 64 contiguous bytes of
//    its token's latent row per token group.
//  * Token rows of the Q.K^T A operand are ordered like the GQA kernel (row 4q + r of
//    token group i = tile token 32q + 4i + r), so the D layout is the P.V B operand.
//  * P.V: the value operand (16 channels x 128 tokens) is read transposed from the same
//    token-major tile in LDS, and the tile scale goes through the same binary expansion
//    into E8M0 passes as the GQA value scale (four mantissa-bit passes x two token parities).
//  * The merge kernel un-rotates and un-smooths the merged latent output:
//    out = (o H / 512) * q_smooth.
#include "decode_common.h"

namespace fp4kv {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef __bf16 bh8 __attribute__((ext_vector_type(8)));

constexpr int kMlaD = 512;        // latent channels
constexpr int kMlaR = 64;         // rope channels
constexpr int kMlaHeads = 16;     // query heads per wave

// Eight FP4 codes (the nibbles of w, low first) -> fp16 code * S, S given as an fp16 pair.
template <int SEL>
__device__ __forceinline__ h2 fp4x2_f16(uint32_t w) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}
__device__ __forceinline__ h8 fp4x8_f16(uint32_t w, h2 s) {
  const h2 a = fp4x2_f16<0>(w) * s, b = fp4x2_f16<1>(w) * s, c = fp4x2_f16<2>(w) * s, d = fp4x2_f16<3>(w) * s;
  return h8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ v4f mfma_f16(const h8 &a, const h8 &b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ v4f mfma_bf16(const bh8 &a, const bh8 &b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bh8 as_bh8(const uint4 &u) {
  bh8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// E4M3 scale byte -> fp16 pair (exact: E4M3 values are fp16 values)
__device__ __forceinline__ h2 e4m3_h2(uint32_t byte) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)byte, false);
  const _Float16 h = (_Float16)f[0];
  return h2{h, h};
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at lds + 16 l (lds is
// wave-uniform; inactive lanes write nothing).  Written as inline assembly because the compiler
// would make every LDS read it cannot prove disjoint from a pending LDS load wait for it, which
// defeats loading the next tile while the current one is read; the kernel waits for its own
// loads (vmcnt) before the barrier that hands a tile to the other waves.  M0 holds the LDS base
// (one wait state between writing M0 and the load).
__device__ __forceinline__ void lds_load16(const void *g, const void *lds) {
  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(base)), "v"(g) : "memory");
}
__device__ __forceinline__ void wait_lds_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Transposed 4-bit LDS read: within each group of 16 lanes, lane 16 g + j receives nibble j of
// the 8-byte rows addressed by lanes 16 g .. 16 g + 15, in lane order.
typedef int v2i __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v2i lds_read_tr4(const uint8_t *p) {
  return __builtin_amdgcn_ds_read_tr4_b64_v2i32((__attribute__((address_space(3))) v2i *)(p));
}

// One Walsh-Hadamard butterfly across lanes l and l ^ 16 (permlane16_swap) or l and l ^ 32
// (permlane32_swap): both return the pair as (value of the lane with the bit clear, value of
// the lane with it set) in both lanes; the first lane keeps the sum, the second the difference.
__device__ __forceinline__ float bfly_x16(float x, bool upper) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float lo = __uint_as_float(r[0]), hi = __uint_as_float(r[1]);
  return upper ? lo - hi : lo + hi;
}
__device__ __forceinline__ float bfly_x32(float x, bool upper) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float lo = __uint_as_float(r[0]), hi = __uint_as_float(r[1]);
  return upper ? lo - hi : lo + hi;
}

// Slot of 16-byte chunk c of a staged latent row r is c ^ swz_lat(r), of a rope row c ^ swz_rope(r):
// the 16 rows one Q.K^T operand read touches (tile tokens 32 a + b + 4 i, a, b < 4) and the 16
// consecutive rows one transposed P.V read touches then fall on distinct banks.
__device__ __forceinline__ int swz_lat(int r) { return (r & 15) ^ (((r >> 5) & 3) << 2); }
__device__ __forceinline__ int swz_rope(int r) { return ((r >> 1) & 1) | (((r >> 5) & 3) << 1); }

// MLA partials, NVFP4 latent.  A workgroup of eight waves serves one (sequence, split) for four
// groups of 16 query heads.  Waves 0-3 ("score" waves, one per head group) keep that group's
// Q1 / Q2 rows and compute Q.K^T over all 512 latent channels, the transposed softmax and the
// FP4 probabilities; waves 4-7 ("value" waves, one per head group) keep the group's running
// output and compute P.V one tile behind, taking the probabilities, their scales and the
// online-softmax rescale factor from LDS.  Each SIMD holds one wave of each kind, so the
// widening VALU work of one overlaps the matrix work of the other.  The workgroup stages
// each 128-token tile once in LDS -- latent codes (token-major), rope keys and tile scales --
// with direct LDS loads issued a whole tile ahead, and every wave reads its operands there:
//  * Q.K^T: the lane's 64 bytes of its token row, widened to fp16 with the tile scale (exact)
//    against the fp16 Q1 / Q2 rows on v_mfma_f32_16x16x32_f16; rope on the bf16 MFMA.
//  * P.V: the value operand (16 channels x 32 tokens per lane) is read from the same
//    token-major tile with the 4-bit transposed LDS read, so the cache holds the latent once;
//    the tile scale's binary expansion gives the E8M0 passes as in the GQA kernel.
// Iteration j: score waves on tile j, value waves on tile j - 1, direct loads of tile j + 1;
// latent tiles and scales are triple-buffered, rope double-buffered, the handoff double-buffered.
// Grid: one-dimensional, ids with equal residue mod 8 (one XCD) take the head-group quads of
// consecutive units.  Performance only: any placement gives the same result.
template <int P>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_partials(DecodeArgs a) {
  constexpr int D = kMlaD, R = kMlaR, HG = kMlaHeads;
  constexpr int NPT = P >= 128 ? 1 : 128 / P;
  constexpr int LAT = 128 * 256, ROPE = 128 * 128, SCL = 8 * 32;
  static_assert(P >= 16 && P % 16 == 0, "page size");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool scorer = wv < 4;                 // wave-uniform role
  const int nhg = a.hq / HG, ngrp = (nhg + 3) / 4;
  const int units = a.batch * a.n_split;
  int id = blockIdx.x;
  const int slot = id & 7;
  id >>= 3;
  const int grp = id % ngrp, ublk = id / ngrp;
  const int unit = ublk * 8 + slot;
  if (unit >= units) return;
  const int b = unit / a.n_split, split = unit % a.n_split;
  const int L = seq_len_clamped(a, b);
  const int ntiles = (L + 127) >> 7;
  const int tb = split * a.tiles_per_split;
  const int te = min(ntiles, tb + a.tiles_per_split);
  if (tb >= te) return;
  const int nt = te - tb;
  const int last_lp = min((L - 1) / P, a.max_pages - 1);
  const int hgl = wv & 3, hg = 4 * grp + hgl;
  const bool active = hg < nhg;               // wave-uniform: idle waves still load and sync
  const int h0 = (active ? hg : 0) * HG;

  __shared__ __align__(16) uint8_t lat[3 * LAT];
  __shared__ __align__(16) uint8_t rope[2 * ROPE];
  __shared__ __align__(16) uint8_t scl[3 * SCL];
  __shared__ __align__(16) uint4 hand[2][4][2][64];   // [tile & 1][group][part][lane]
  __shared__ uint32_t lut[256];
  __shared__ int pgl[kMaxSplitPages];

  for (int e = tid; e < nt * NPT; e += 512)
    pgl[e] = phys_page(a, b, ((tb + e / NPT) * 128) / P + e % NPT, last_lp);
  // E4M3 code -> four E8M0 pass bytes (binary expansion of the scale) for the P.V passes
  if (tid < 256) {
    const int c = tid;
    const int ef = (c >> 3) & 15, m = c & 7;
    const int E = (ef ? ef : 1) - 7 + 127;
    const uint32_t w = (ef ? (uint32_t)E : 0u) | ((m & 4) ? (uint32_t)(E - 1) << 8 : 0u) |
                       ((m & 2) ? (uint32_t)(E - 2) << 16 : 0u) | ((m & 1) ? (uint32_t)(E - 3) << 24 : 0u);
    lut[c] = c < 0x7F ? w : 0u;
  }
  __syncthreads();

  // Physical row (page * P + offset) of token r of relative tile j
  auto row_of = [&](int j, int r) -> long {
    const int pg = pgl[j * NPT + (NPT == 1 ? 0 : r / P)];
    return (long)pg * P + ((tb + j) * 128 + r) % P;
  };
  // Stage relative tile j: 32 latent, 16 rope and 1 scale instruction, spread over the waves
  auto stage_tile = [&](int j) {
    uint8_t *Lt = lat + (j % 3) * LAT;
    uint8_t *Rt = rope + (j & 1) * ROPE;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int g = 4 * wv + m;
      const int r = 4 * g + (lane >> 4);
      const int c = (lane & 15) ^ swz_lat(r);
      lds_load16(a.k_codes + row_of(j, r) * (D / 2) + 16 * c, Lt + 1024 * g);
    }
#pragma unroll
    for (int m = 0; m < 2; m++) {
      const int g = 2 * wv + m;
      const int r = 8 * g + (lane >> 3);
      const int c = (lane & 7) ^ swz_rope(r);
      lds_load16((const uint8_t *)a.k_rope + row_of(j, r) * (2 * R) + 16 * c, Rt + 1024 * g);
    }
    if (wv == 0 && lane < 16) {
      const int tr = lane >> 1;   // tile row (16 tokens): 32 scale bytes
      const int pg = pgl[j * NPT + (NPT == 1 ? 0 : 16 * tr / P)];
      const int off = (((tb + j) * 128 + 16 * tr) % P) / 16;
      lds_load16(a.k_scales + ((long)pg * (P / 16) + off) * 32 + 16 * (lane & 1), scl + (j % 3) * SCL);
    }
  };
  stage_tile(0);

  const int q4 = lane >> 4;        // lane group
  const int n = lane & 15;         // operand row / output column = head h0 + n
  const float gk = a.gk[0];
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  if (scorer) {
    // ---------------- score waves ----------------
    // Prologue: smoothing, rotation, dual-residual FP4 query.  Lane (n, q4) holds channels
    // 128 q4 .. + 127 of head h0 + n, the B-operand layout: K-step s, element j is channel
    // 128 q4 + 8 s + j.  Walsh-Hadamard stages 1 .. 64 in the lane, 128 and 256 with lanes
    // l ^ 16, l ^ 32 (the stage order of the oracle).
    h8 bq0[16], bq1[16];
    float qg0 = 0.0f, qg1 = 0.0f;
    if (active) {
      const long q0 = ((long)b * a.hq + h0 + n) * (D + R) + 128 * q4;
      float y[128];
      if (a.q_bf16) {
        const uint16_t *qp = (const uint16_t *)a.q + q0;
#pragma unroll
        for (int j = 0; j < 128; j++) y[j] = bf16_to_f32(qp[j]);
      } else {
        const float *qp = (const float *)a.q + q0;
#pragma unroll
        for (int j = 0; j < 128; j++) y[j] = qp[j];
      }
#pragma unroll
      for (int j = 0; j < 128; j++) y[j] = y[j] * a.qs[128 * q4 + j];
#pragma unroll
      for (int h = 1; h < 128; h <<= 1)
#pragma unroll
        for (int j = 0; j < 128; j++)
          if ((j & h) == 0) {
            const float x0 = y[j], x1 = y[j + h];
            y[j] = x0 + x1;
            y[j + h] = x0 - x1;
          }
#pragma unroll
      for (int j = 0; j < 128; j++) y[j] = bfly_x16(y[j], (lane & 16) != 0);
#pragma unroll
      for (int j = 0; j < 128; j++) y[j] = bfly_x32(y[j], (lane & 32) != 0);
      // dual-residual NVFP4: power-of-two block scales over 16 channels, G = row max / 1536.
      // The codes are kept packed (word s = channels 8 s .. 8 s + 7) with their block
      // exponents and widened to fp16 once the rotation registers are free.
      uint32_t qc[2][16];
      int qe[2][8];
#pragma unroll
      for (int k = 0; k < 2; k++) {
        float rmax = 0.0f;
#pragma unroll
        for (int j = 0; j < 128; j++) rmax = fmaxf(rmax, fabsf(y[j]));
        rmax = fmaxf(rmax, __shfl_xor(rmax, 16));
        rmax = fmaxf(rmax, __shfl_xor(rmax, 32));
        const float gq = rmax / 1536.0f;
        const float sixg = 6.0f * gq;
        const float inv6g = sixg != 0.0f ? 1.0f / sixg : 0.0f;
#pragma unroll
        for (int blk = 0; blk < 8; blk++) {
          float bmax = 0.0f;
#pragma unroll
          for (int i = 0; i < 16; i++) bmax = fmaxf(bmax, fabsf(y[16 * blk + i]));
          const bool valid = bmax > 0.0f && gq > 0.0f;
          const int e = ceil_log2_clamp(bmax * inv6g, -9, 8);
          const float S = pow2f(e);
          const float sg = S * gq;
          const float rr = (valid && sg != 0.0f) ? 1.0f / sg : 0.0f;   // invalid: every code is 0
          qe[k][blk] = e;
#pragma unroll
          for (int h = 0; h < 2; h++) {
            uint32_t w = 0u;
#pragma unroll
            for (int i = 0; i < 8; i++) {
              const int ch = 16 * blk + 8 * h + i;
              const float x = y[ch];
              const uint32_t c = e2m1_enc(x * rr);
              w |= c << (4 * i);
              y[ch] = x - (e2m1_dec(c) * S) * gq;
            }
            qc[k][2 * blk + h] = w;
          }
        }
        if (k == 0) qg0 = gq;
        else qg1 = gq;
      }
      // fp16 operands: code * 2^e, exact (the convert applies a power-of-two scale exactly)
#pragma unroll
      for (int st = 0; st < 16; st++) {
        const float s0 = pow2f(qe[0][st >> 1]), s1 = pow2f(qe[1][st >> 1]);
        const h2 a0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qc[0][st], s0, 0);
        const h2 a1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qc[0][st], s0, 1);
        const h2 a2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qc[0][st], s0, 2);
        const h2 a3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qc[0][st], s0, 3);
        bq0[st] = h8{a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
        const h2 b0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qc[1][st], s1, 0);
        const h2 b1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qc[1][st], s1, 1);
        const h2 b2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qc[1][st], s1, 2);
        const h2 b3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(qc[1][st], s1, 3);
        bq1[st] = h8{b0[0], b0[1], b1[0], b1[1], b2[0], b2[1], b3[0], b3[1]};
      }
    } else {
#pragma unroll
      for (int st = 0; st < 16; st++) {
        bq0[st] = h8{};
        bq1[st] = h8{};
      }
    }
    // rope query (bf16): K-step s, lane group q4, element j is rope channel 32 s + 8 q4 + j
    bh8 bqr[2];
    {
      const long qr = ((long)b * a.hq + h0 + n) * (D + R) + D + 8 * q4;
#pragma unroll
      for (int st = 0; st < 2; st++) {
        uint16_t hb[8];
        if (a.q_bf16) {
#pragma unroll
          for (int j = 0; j < 8; j++) hb[j] = ((const uint16_t *)a.q)[qr + 32 * st + j];
        } else {  // fp32 rope query rounded to bf16 (nearest even)
#pragma unroll
          for (int j = 0; j < 8; j++) {
            const uint32_t u = __float_as_uint(((const float *)a.q)[qr + 32 * st + j]);
            hb[j] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
          }
        }
        __builtin_memcpy(&bqr[st], hb, 16);
      }
    }
    const float a1 = (qg0 * gk) * a.coef, a2 = (qg1 * gk) * a.coef, cr = a.coef_rope;
    float m_run = -INFINITY, l_run = 0.0f, f_run = 1.0f;
    int nzero = 0;
    const float inv6gp = 1.0f / (6.0f * 0.0009765625f);   // fl32(1 / fl32(6 * 2^-10))
    const bool count_zero = a.zero_blocks != nullptr && active;
    const int trow = 32 * (n >> 2) + (n & 3);   // A-operand row: tile token trow + 4 i in group i

    wait_lds_loads();
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j <= nt; j++) {
      if (j + 1 < nt) stage_tile(j + 1);
      if (active && j < nt) {
        const uint8_t *Lt = lat + (j % 3) * LAT;
        const uint8_t *Rt = rope + (j & 1) * ROPE;
        const uint8_t *St = scl + (j % 3) * SCL;
        // ---- Q.K^T: 8 token groups of 16
        float s[8][4];
#pragma unroll
        for (int i = 0; i < 8; i++) {
          const int r = trow + 4 * i;
          const uint8_t *row = Lt + r * 256;
          const int sw = swz_lat(r);
          uint4 w4[4];
#pragma unroll
          for (int kk = 0; kk < 4; kk++) w4[kk] = *(const uint4 *)(row + (((4 * q4 + kk) ^ sw) << 4));
          const uint2 sc8 = *(const uint2 *)(St + (2 * (n >> 2) + (i >> 2)) * 32 + 8 * q4);
          const uint32_t ws[16] = {w4[0].x, w4[0].y, w4[0].z, w4[0].w, w4[1].x, w4[1].y, w4[1].z, w4[1].w,
                                   w4[2].x, w4[2].y, w4[2].z, w4[2].w, w4[3].x, w4[3].y, w4[3].z, w4[3].w};
          h2 sq[8];
#pragma unroll
          for (int k = 0; k < 8; k++) sq[k] = e4m3_h2(((k < 4 ? sc8.x : sc8.y) >> (8 * (k & 3))) & 0xFFu);
          v4f acc1 = zero, acc2 = zero, accr = zero;
#pragma unroll
          for (int st = 0; st < 16; st++) {
            const h8 av = fp4x8_f16(ws[st], sq[st >> 1]);
            acc1 = mfma_f16(av, bq0[st], acc1);
            acc2 = mfma_f16(av, bq1[st], acc2);
          }
          const uint8_t *rrow = Rt + r * 128;
          const int swr = swz_rope(r);
          accr = mfma_bf16(as_bh8(*(const uint4 *)(rrow + ((q4 ^ swr) << 4))), bqr[0], accr);
          accr = mfma_bf16(as_bh8(*(const uint4 *)(rrow + (((4 + q4) ^ swr) << 4))), bqr[1], accr);
#pragma unroll
          for (int rr = 0; rr < 4; rr++) {
            const float t12 = a1 * acc1[rr] + a2 * acc2[rr];
            s[i][rr] = t12 + cr * accr[rr];
          }
        }
        // ---- transposed softmax (lane (n, q4) holds tokens 32 q4 .. + 31 of head n)
        const int tok0 = (tb + j) * 128;
        if (tok0 + 128 > L) {
#pragma unroll
          for (int i = 0; i < 8; i++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++)
              if (tok0 + 32 * q4 + 4 * i + rr >= L) s[i][rr] = -INFINITY;
        }
        float bm0 = -INFINITY, bm1 = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int rr = 0; rr < 4; rr++) {
            bm0 = fmaxf(bm0, s[i][rr]);
            bm1 = fmaxf(bm1, s[i + 4][rr]);
          }
        const float mt = max_x32(max_x16(fmaxf(bm0, bm1)));
        float lt = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
          for (int rr = 0; rr < 4; rr++) {
            const float p = __builtin_amdgcn_exp2f(s[i][rr] - mt);
            s[i][rr] = p;
            lt = lt + p;
          }
        // ---- fused probability quantization (NVFP4, power-of-two block scales, G_P = 2^-10)
        uint32_t pk[4];
        int pbyte[2];
        const float am[2] = {__builtin_amdgcn_exp2f(bm0 - mt), __builtin_amdgcn_exp2f(bm1 - mt)};
#pragma unroll
        for (int pb = 0; pb < 2; pb++) {
          const int e = ceil_log2_clamp(am[pb] * inv6gp, -9, 8);
          const float ps = pow2f(e - 10);
          pbyte[pb] = e - 10 + 127;
          pk[2 * pb] = pack8(s[4 * pb], s[4 * pb + 1], ps);
          pk[2 * pb + 1] = pack8(s[4 * pb + 2], s[4 * pb + 3], ps);
        }
        if (count_zero) {
#pragma unroll
          for (int pb = 0; pb < 2; pb++)
            if (tok0 + 32 * q4 + 16 * pb < L && ((pk[2 * pb] | pk[2 * pb + 1]) & 0x77777777u) == 0u) nzero++;
        }
        // ---- online softmax: the value waves keep the output as o_run * f_run and rescale
        // it by gamma before adding this tile
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        const float beta = __builtin_amdgcn_exp2f(mt - m_new);
        l_run = fmaf(l_run, alpha, lt * beta);
        m_run = m_new;
        const float f_new = fmaxf(beta, 8.67361737988403547e-19f);   // 2^-60
        const float gamma = (alpha * f_run) * __builtin_amdgcn_rcpf(f_new);
        f_run = f_new;
        hand[j & 1][hgl][0][lane] = uint4{pk[0], pk[1], pk[2], pk[3]};
        hand[j & 1][hgl][1][lane] = uint4{(uint32_t)pbyte[0] | ((uint32_t)pbyte[1] << 8), __float_as_uint(gamma),
                                          __float_as_uint(f_run), 0u};
      }
      wait_lds_loads();
      __syncthreads();
    }
    if (!active) return;
    const float l_tot = sum_x32(sum_x16(l_run));
    if (q4 == 0) {
      const long rowi = ((long)b * a.hq + h0 + n) * a.n_split + split;
      *(float2 *)(a.ws_ml + rowi * 2) = float2{m_run, l_tot};
    }
    if (count_zero) {
      int z = nzero;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
      if (lane == 0 && z) atomicAdd(a.zero_blocks, z);
    }
  } else {
    // ---------------- value waves ----------------
    v4f o_run[32];
#pragma unroll
    for (int cg = 0; cg < 32; cg++) o_run[cg] = zero;
    float f_run = 1.0f;
    const int ra = 32 * q4 + n, rb = ra + 16;   // rows of the lane's two transposed reads
    const int swa = swz_lat(ra), swb = swz_lat(rb);
    wait_lds_loads();
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j <= nt; j++) {
      if (j + 1 < nt) stage_tile(j + 1);
      if (active && j >= 1) {
        const int jp = j - 1;
        const uint8_t *Lt = lat + (jp % 3) * LAT;
        const uint8_t *St = scl + (jp % 3) * SCL;
        const uint4 hp = hand[jp & 1][hgl][0][lane];
        const uint4 hs = hand[jp & 1][hgl][1][lane];
        const int pb0 = (int)(hs.x & 0xFFu), pb1 = (int)((hs.x >> 8) & 0xFFu);
        const float gamma = __uint_as_float(hs.y);
        f_run = __uint_as_float(hs.z);
#pragma unroll
        for (int cg = 0; cg < 32; cg++)
#pragma unroll
          for (int rr = 0; rr < 4; rr++) o_run[cg][rr] = o_run[cg][rr] * gamma;
        const v8i p0 = {(int)hp.x, (int)hp.y, 0, 0, 0, 0, 0, 0};
        const v8i p1 = {0, 0, (int)hp.z, (int)hp.w, 0, 0, 0, 0};
        const uint8_t *rowa = Lt + ra * 256, *rowb = Lt + rb * 256;
        // P.V: channels 16 cg + n, tokens 32 q4 .. + 31, in chunks of four channel groups; the
        // value operands and pass bytes of chunk i + 1 are read while chunk i computes
        const uint4 sa0 = *(const uint4 *)(St + (2 * q4) * 32), sa1 = *(const uint4 *)(St + (2 * q4) * 32 + 16);
        const uint4 sb0 = *(const uint4 *)(St + (2 * q4 + 1) * 32), sb1 = *(const uint4 *)(St + (2 * q4 + 1) * 32 + 16);
        v2i vt[2][4][2];
        int lt[2][4][2];
        auto read_vals = [&](int i, v2i (*o)[2], int (*l)[2]) {
#pragma unroll
          for (int k = 0; k < 4; k++) {
            const int cg = 4 * i + k;
            const int off = 8 * (cg & 1);
            o[k][0] = lds_read_tr4(rowa + (((cg >> 1) ^ swa) << 4) + off);
            o[k][1] = lds_read_tr4(rowb + (((cg >> 1) ^ swb) << 4) + off);
            l[k][0] = (int)lut[byte_of(cg < 16 ? sa0 : sa1, cg & 15)];
            l[k][1] = (int)lut[byte_of(cg < 16 ? sb0 : sb1, cg & 15)];
          }
        };
        read_vals(0, vt[0], lt[0]);
#pragma unroll
        for (int i = 0; i < 8; i++) {
          if (i < 7) read_vals(i + 1, vt[(i + 1) & 1], lt[(i + 1) & 1]);
#pragma unroll
          for (int k = 0; k < 4; k++) {
            const int cg = 4 * i + k;
            const v2i lo = vt[i & 1][k][0], hi = vt[i & 1][k][1];
            const v8i av = {lo[0], lo[1], hi[0], hi[1], 0, 0, 0, 0};
            const int l0 = lt[i & 1][k][0], l1 = lt[i & 1][k][1];
            v4f c = mfma4<0, 0>(av, p0, o_run[cg], l0, pb0);
            c = mfma4<1, 0>(av, p0, c, l0, pb0);
            c = mfma4<2, 0>(av, p0, c, l0, pb0);
            c = mfma4<3, 0>(av, p0, c, l0, pb0);
            c = mfma4<0, 0>(av, p1, c, l1, pb1);
            c = mfma4<1, 0>(av, p1, c, l1, pb1);
            c = mfma4<2, 0>(av, p1, c, l1, pb1);
            o_run[cg] = mfma4<3, 0>(av, p1, c, l1, pb1);
          }
        }
      }
      wait_lds_loads();
      __syncthreads();
    }
    if (!active) return;
    // split partials (latent output, still rotated)
    const long rowi = ((long)b * a.hq + h0 + n) * a.n_split + split;
    const float g = gk * f_run;
#pragma unroll
    for (int cg = 0; cg < 32; cg++) {
      float4 v = {o_run[cg][0] * g, o_run[cg][1] * g, o_run[cg][2] * g, o_run[cg][3] * g};
      *(float4 *)(a.ws_o + rowi * D + 16 * cg + 4 * q4) = v;
    }
  }
}

// MLA partials, MXFP4 latent.  The 32-token x 32-channel tiles carry E8M0 scales, which is
// the block-scaled MFMA's own scale granularity (32 K-elements per lane), so Q.K^T and P.V
// both run as native FP4 x FP4 MFMAs with both scales applied in hardware and no widening:
// per 16 tokens, four MFMAs per query pass over the 512 channels plus two bf16 MFMAs for the
// rope part; per tile, one MFMA per 16 output channels.  The workgroup structure is the NVFP4
// kernel's: eight waves for one (sequence, split) and four groups of 16 query heads, score
// waves 0-3 (Q.K^T, softmax, FP4 probabilities) and value waves 4-7 (P.V one tile behind,
// the value operand read transposed from the token-major tile), latent tiles, rope keys and
// scales staged once per workgroup in LDS with direct loads a tile ahead.
// The query is rotated and quantized directly in the B-operand layout: lane (n, q4) holds
// channels 128 st + 32 q4 + j (st = 0..3, j = 0..31), so the Walsh-Hadamard stages on
// channel bits 0-4 and 7-8 stay in the lane, bits 5 and 6 pair lanes l ^ 16 and l ^ 32,
// and every 32-channel MX block is one lane's own.
template <int P>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_partials_mx(DecodeArgs a) {
  constexpr int D = kMlaD, R = kMlaR, HG = kMlaHeads;
  constexpr int NPT = P >= 128 ? 1 : 128 / P;
  constexpr int LAT = 128 * 256, ROPE = 128 * 128, SCL = 4 * 16;
  static_assert(P >= 32 && P % 32 == 0, "page size");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool scorer = wv < 4;                 // wave-uniform role
  const int nhg = a.hq / HG, ngrp = (nhg + 3) / 4;
  const int units = a.batch * a.n_split;
  int id = blockIdx.x;
  const int slot = id & 7;
  id >>= 3;
  const int grp = id % ngrp, ublk = id / ngrp;
  const int unit = ublk * 8 + slot;
  if (unit >= units) return;
  const int b = unit / a.n_split, split = unit % a.n_split;
  const int L = seq_len_clamped(a, b);
  const int ntiles = (L + 127) >> 7;
  const int tb = split * a.tiles_per_split;
  const int te = min(ntiles, tb + a.tiles_per_split);
  if (tb >= te) return;
  const int nt = te - tb;
  const int last_lp = min((L - 1) / P, a.max_pages - 1);
  const int hgl = wv & 3, hg = 4 * grp + hgl;
  const bool active = hg < nhg;               // wave-uniform: idle waves still load and sync
  const int h0 = (active ? hg : 0) * HG;

  __shared__ __align__(16) uint8_t lat[3 * LAT];
  __shared__ __align__(16) uint8_t rope[2 * ROPE];
  __shared__ __align__(16) uint8_t scl[3 * SCL];
  __shared__ __align__(16) uint4 hand[2][4][2][64];   // [tile & 1][group][part][lane]
  __shared__ int pgl[kMaxSplitPages];

  for (int e = tid; e < nt * NPT; e += 512)
    pgl[e] = phys_page(a, b, ((tb + e / NPT) * 128) / P + e % NPT, last_lp);
  __syncthreads();

  auto row_of = [&](int j, int r) -> long {
    const int pg = pgl[j * NPT + (NPT == 1 ? 0 : r / P)];
    return (long)pg * P + ((tb + j) * 128 + r) % P;
  };
  // Stage relative tile j: 32 latent, 16 rope and 1 scale instruction, spread over the waves
  auto stage_tile = [&](int j) {
    uint8_t *Lt = lat + (j % 3) * LAT;
    uint8_t *Rt = rope + (j & 1) * ROPE;
#pragma unroll
    for (int m = 0; m < 4; m++) {
      const int g = 4 * wv + m;
      const int r = 4 * g + (lane >> 4);
      const int c = (lane & 15) ^ swz_lat(r);
      lds_load16(a.k_codes + row_of(j, r) * (D / 2) + 16 * c, Lt + 1024 * g);
    }
#pragma unroll
    for (int m = 0; m < 2; m++) {
      const int g = 2 * wv + m;
      const int r = 8 * g + (lane >> 3);
      const int c = (lane & 7) ^ swz_rope(r);
      lds_load16((const uint8_t *)a.k_rope + row_of(j, r) * (2 * R) + 16 * c, Rt + 1024 * g);
    }
    if (wv == 0 && lane < 4) {
      const int t = 32 * lane;   // token block (32 tokens): 16 scale bytes
      const int pg = pgl[j * NPT + (NPT == 1 ? 0 : t / P)];
      lds_load16(a.k_scales + ((long)pg * (P / 32) + (((tb + j) * 128 + t) % P) / 32) * 16, scl + (j % 3) * SCL);
    }
  };
  stage_tile(0);

  const int q4 = lane >> 4;        // lane group
  const int n = lane & 15;         // operand row / output column = head h0 + n
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  if (scorer) {
    // ---------------- score waves ----------------
    v8i bq[2][4];            // [pass][K-step]: FP4 codes of channels 128 st + 32 q4 .. + 31
    int qsb[2][4];           // their E8M0 scale bytes
    if (active) {
      // prologue: smoothing, rotation, dual-residual MXFP4 query
      const long q0 = ((long)b * a.hq + h0 + n) * (D + R) + 32 * q4;
      float y[4][32];
  #pragma unroll
      for (int st = 0; st < 4; st++) {
        if (a.q_bf16) {
          const uint16_t *qp = (const uint16_t *)a.q + q0 + 128 * st;
  #pragma unroll
          for (int j = 0; j < 32; j++) y[st][j] = bf16_to_f32(qp[j]);
        } else {
          const float *qp = (const float *)a.q + q0 + 128 * st;
  #pragma unroll
          for (int j = 0; j < 32; j++) y[st][j] = qp[j];
        }
  #pragma unroll
        for (int j = 0; j < 32; j++) y[st][j] = y[st][j] * a.qs[128 * st + 32 * q4 + j];
      }
      // stages h = 1 .. 16 (channel bits 0-4) in the lane
  #pragma unroll
      for (int h = 1; h < 32; h <<= 1)
  #pragma unroll
        for (int st = 0; st < 4; st++)
  #pragma unroll
          for (int j = 0; j < 32; j++)
            if ((j & h) == 0) {
              const float x0 = y[st][j], x1 = y[st][j + h];
              y[st][j] = x0 + x1;
              y[st][j + h] = x0 - x1;
            }
      // stages h = 32, 64 (channel bits 5, 6 = lane bits 4, 5)
  #pragma unroll
      for (int st = 0; st < 4; st++)
  #pragma unroll
        for (int j = 0; j < 32; j++) y[st][j] = bfly_x16(y[st][j], (lane & 16) != 0);
  #pragma unroll
      for (int st = 0; st < 4; st++)
  #pragma unroll
        for (int j = 0; j < 32; j++) y[st][j] = bfly_x32(y[st][j], (lane & 32) != 0);
      // stages h = 128, 256 (channel bits 7, 8 = the K-step index) in the lane
  #pragma unroll
      for (int hs = 1; hs < 4; hs <<= 1)
  #pragma unroll
        for (int st = 0; st < 4; st++)
          if ((st & hs) == 0) {
  #pragma unroll
            for (int j = 0; j < 32; j++) {
              const float x0 = y[st][j], x1 = y[st + hs][j];
              y[st][j] = x0 + x1;
              y[st + hs][j] = x0 - x1;
            }
          }
      // pass k quantizes the residual of pass k - 1: E8M0 per 32 channels, no tensor scale
  #pragma unroll
      for (int k = 0; k < 2; k++)
  #pragma unroll
        for (int st = 0; st < 4; st++) {
          float bmax = 0.0f;
  #pragma unroll
          for (int j = 0; j < 32; j++) bmax = fmaxf(bmax, fabsf(y[st][j]));
          const int e = mx_exp(bmax);
          uint32_t w[4] = {0u, 0u, 0u, 0u};
  #pragma unroll
          for (int j = 0; j < 32; j++) {
            const uint32_t c = e2m1_enc(ldexpf(y[st][j], -e));
            w[j / 8] |= c << (4 * (j % 8));
            y[st][j] = y[st][j] - ldexpf(e2m1_dec(c), e);
          }
          bq[k][st] = v8i{(int)w[0], (int)w[1], (int)w[2], (int)w[3], 0, 0, 0, 0};
          qsb[k][st] = e + 127;
        }
    } else {
#pragma unroll
      for (int k = 0; k < 2; k++)
#pragma unroll
        for (int st = 0; st < 4; st++) {
          bq[k][st] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          qsb[k][st] = 0;
        }
    }
    // rope query (bf16): K-step s, lane group q4, element j is rope channel 32 s + 8 q4 + j
    bh8 bqr[2];
    {
      const long qr = ((long)b * a.hq + h0 + n) * (D + R) + D + 8 * q4;
  #pragma unroll
      for (int st = 0; st < 2; st++) {
        uint16_t hb[8];
        if (a.q_bf16) {
  #pragma unroll
          for (int j = 0; j < 8; j++) hb[j] = ((const uint16_t *)a.q)[qr + 32 * st + j];
        } else {  // fp32 rope query rounded to bf16 (nearest even)
  #pragma unroll
          for (int j = 0; j < 8; j++) {
            const uint32_t u = __float_as_uint(((const float *)a.q)[qr + 32 * st + j]);
            hb[j] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
          }
        }
        __builtin_memcpy(&bqr[st], hb, 16);
      }
    }
    const float c1 = a.coef, cr = a.coef_rope;   // MXFP4: no tensor scales, a1 = a2 = c
    float m_run = -INFINITY, l_run = 0.0f, f_run = 1.0f;
    int nzero = 0;
    const bool count_zero = a.zero_blocks != nullptr && active;
    const int trow = 32 * (n >> 2) + (n & 3);   // A-operand row: tile token trow + 4 i in group i

    wait_lds_loads();
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j <= nt; j++) {
      if (j + 1 < nt) stage_tile(j + 1);
      if (active && j < nt) {
        const uint8_t *Lt = lat + (j % 3) * LAT;
        const uint8_t *Rt = rope + (j & 1) * ROPE;
        // E8M0 scales of the lane's token block (n / 4): its 16 channel blocks
        const uint4 scc = *(const uint4 *)(scl + (j % 3) * SCL + 16 * (n >> 2));
        // ---- Q.K^T: 8 token groups of 16; the operands of group i + 1 (four latent chunks,
        // two rope chunks) are read from LDS while group i computes
        float s[8][4];
        uint4 opd[2][6];
        auto read_ops = [&](int i, uint4 *o) {
          const int r = trow + 4 * i;
          const uint8_t *row = Lt + r * 256;
          const int sw = swz_lat(r);
#pragma unroll
          for (int st = 0; st < 4; st++) o[st] = *(const uint4 *)(row + (((4 * st + q4) ^ sw) << 4));
          const uint8_t *rrow = Rt + r * 128;
          const int swr = swz_rope(r);
          o[4] = *(const uint4 *)(rrow + ((q4 ^ swr) << 4));
          o[5] = *(const uint4 *)(rrow + (((4 + q4) ^ swr) << 4));
        };
        read_ops(0, opd[0]);
#pragma unroll
        for (int i = 0; i < 8; i++) {
          if (i < 7) read_ops(i + 1, opd[(i + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          const uint4 *o = opd[i & 1];
          v4f acc1 = zero, acc2 = zero, accr = zero;
#pragma unroll
          for (int st = 0; st < 4; st++) {
            const v8i av = {(int)o[st].x, (int)o[st].y, (int)o[st].z, (int)o[st].w, 0, 0, 0, 0};
            const int sa = (int)byte_of(scc, 4 * st + q4);
            acc1 = mfma4<0, 0>(av, bq[0][st], acc1, sa, qsb[0][st]);
            acc2 = mfma4<0, 0>(av, bq[1][st], acc2, sa, qsb[1][st]);
          }
          accr = mfma_bf16(as_bh8(o[4]), bqr[0], accr);
          accr = mfma_bf16(as_bh8(o[5]), bqr[1], accr);
#pragma unroll
          for (int rr = 0; rr < 4; rr++) {
            const float t12 = c1 * acc1[rr] + c1 * acc2[rr];
            s[i][rr] = t12 + cr * accr[rr];
          }
        }
        // ---- transposed softmax (lane (n, q4) holds tokens 32 q4 .. + 31 of head n)
        const int tok0 = (tb + j) * 128;
        if (tok0 + 128 > L) {
#pragma unroll
          for (int i = 0; i < 8; i++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++)
              if (tok0 + 32 * q4 + 4 * i + rr >= L) s[i][rr] = -INFINITY;
        }
        float bm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
          for (int rr = 0; rr < 4; rr++) bm = fmaxf(bm, s[i][rr]);
        const float mt = max_x32(max_x16(bm));
        float lt = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
          for (int rr = 0; rr < 4; rr++) {
            const float p = __builtin_amdgcn_exp2f(s[i][rr] - mt);
            s[i][rr] = p;
            lt = lt + p;
          }
        // ---- fused probability quantization (MXFP4: the lane's 32 tokens are one block)
        uint32_t pk[4];
        const int pe = mx_exp(__builtin_amdgcn_exp2f(bm - mt));
        const int pbyte = pe + 127;
        {
          const float ps = ldexpf(1.0f, pe);
#pragma unroll
          for (int w = 0; w < 4; w++) pk[w] = pack8(s[2 * w], s[2 * w + 1], ps);
        }
        if (count_zero && tok0 + 32 * q4 < L && ((pk[0] | pk[1] | pk[2] | pk[3]) & 0x77777777u) == 0u) nzero++;
        // ---- online softmax: the value waves keep the output as o_run * f_run
        const float m_new = fmaxf(m_run, mt);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        const float beta = __builtin_amdgcn_exp2f(mt - m_new);
        l_run = fmaf(l_run, alpha, lt * beta);
        m_run = m_new;
        const float f_new = fmaxf(beta, 8.67361737988403547e-19f);   // 2^-60
        const float gamma = (alpha * f_run) * __builtin_amdgcn_rcpf(f_new);
        f_run = f_new;
        hand[j & 1][hgl][0][lane] = uint4{pk[0], pk[1], pk[2], pk[3]};
        hand[j & 1][hgl][1][lane] = uint4{(uint32_t)pbyte, __float_as_uint(gamma), __float_as_uint(f_run), 0u};
      }
      wait_lds_loads();
      __syncthreads();
    }
    if (!active) return;
    const float l_tot = sum_x32(sum_x16(l_run));
    if (q4 == 0) {
      const long rowi = ((long)b * a.hq + h0 + n) * a.n_split + split;
      *(float2 *)(a.ws_ml + rowi * 2) = float2{m_run, l_tot};
    }
    if (count_zero) {
      int z = nzero;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
      if (lane == 0 && z) atomicAdd(a.zero_blocks, z);
    }
  } else {
    // ---------------- value waves ----------------
    v4f o_run[32];
#pragma unroll
    for (int cg = 0; cg < 32; cg++) o_run[cg] = zero;
    float f_run = 1.0f;
    const int ra = 32 * q4 + n, rb = ra + 16;   // rows of the lane's two transposed reads
    const int swa = swz_lat(ra), swb = swz_lat(rb);
    wait_lds_loads();
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j <= nt; j++) {
      if (j + 1 < nt) stage_tile(j + 1);
      if (active && j >= 1) {
        const int jp = j - 1;
        const uint8_t *Lt = lat + (jp % 3) * LAT;
        const uint4 hp = hand[jp & 1][hgl][0][lane];
        const uint4 hs = hand[jp & 1][hgl][1][lane];
        const int pbyte = (int)hs.x;
        const float gamma = __uint_as_float(hs.y);
        f_run = __uint_as_float(hs.z);
        // E8M0 scales of the lane's token block q4: its 16 channel blocks
        const uint4 sv = *(const uint4 *)(scl + (jp % 3) * SCL + 16 * q4);
#pragma unroll
        for (int cg = 0; cg < 32; cg++)
#pragma unroll
          for (int rr = 0; rr < 4; rr++) o_run[cg][rr] = o_run[cg][rr] * gamma;
        const v8i pv = {(int)hp.x, (int)hp.y, (int)hp.z, (int)hp.w, 0, 0, 0, 0};
        const uint8_t *rowa = Lt + ra * 256, *rowb = Lt + rb * 256;
        // P.V: channels 16 cg + n, tokens 32 q4 .. + 31, one MFMA per channel group with the
        // scale of (token block q4, channel block cg / 2)
        // value operands of channel groups 4 c .. 4 c + 3 are read while chunk c - 1 computes
        v2i vt[2][4][2];
        auto read_vals = [&](int c, v2i (*o)[2]) {
#pragma unroll
          for (int k = 0; k < 4; k++) {
            const int cg = 4 * c + k;
            const int off = 8 * (cg & 1);
            o[k][0] = lds_read_tr4(rowa + (((cg >> 1) ^ swa) << 4) + off);
            o[k][1] = lds_read_tr4(rowb + (((cg >> 1) ^ swb) << 4) + off);
          }
        };
        read_vals(0, vt[0]);
#pragma unroll
        for (int c = 0; c < 8; c++) {
          if (c < 7) read_vals(c + 1, vt[(c + 1) & 1]);
#pragma unroll
          for (int k = 0; k < 4; k++) {
            const int cg = 4 * c + k;
            const v2i lo = vt[c & 1][k][0], hi = vt[c & 1][k][1];
            const v8i av = {lo[0], lo[1], hi[0], hi[1], 0, 0, 0, 0};
            o_run[cg] = mfma4<0, 0>(av, pv, o_run[cg], (int)byte_of(sv, cg >> 1), pbyte);
          }
        }
      }
      wait_lds_loads();
      __syncthreads();
    }
    if (!active) return;
    // split partials (latent output, still rotated)
    const long rowi = ((long)b * a.hq + h0 + n) * a.n_split + split;
#pragma unroll
    for (int cg = 0; cg < 32; cg++) {
      float4 v = {o_run[cg][0] * f_run, o_run[cg][1] * f_run, o_run[cg][2] * f_run, o_run[cg][3] * f_run};
      *(float4 *)(a.ws_o + rowi * D + 16 * cg + 4 * q4) = v;
    }
  }
}

// Merge of one (sequence, query head) row: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// then un-rotated (Walsh-Hadamard over the 512 channels, / 512) and un-smoothed (* q_smooth).
// Lane l holds channels 8 l .. 8 l + 7.
constexpr int kMlaMergeFast = 8;   // splits per row that the merge loads all at once

__global__ __launch_bounds__(64) void mla_merge(DecodeArgs a) {
  constexpr int D = kMlaD;
  const int row = blockIdx.x, lane = threadIdx.x;
  const int b = row / a.hq;
  float4 *dst = (float4 *)(a.out + (long)row * D + 8 * lane);
  const float *ml = a.ws_ml + (long)row * a.n_split * 2;
  const float *o = a.ws_o + (long)row * a.n_split * D + 8 * lane;
  // up to kMlaMergeFast splits: every split row of the workspace is loaded together with the
  // sequence length, before the count of splits in use is known (rows past that count hold
  // stale values and are not used)
  const bool fast = a.n_split <= kMlaMergeFast;
  float2 mlf = float2{-INFINITY, 0.f};
  float4 u[kMlaMergeFast][2];
  if (fast) {
    if (lane < a.n_split) mlf = *(const float2 *)(ml + 2 * lane);
#pragma unroll
    for (int s = 0; s < kMlaMergeFast; s++) {
      u[s][0] = s < a.n_split ? *(const float4 *)(o + (long)s * D) : float4{0.f, 0.f, 0.f, 0.f};
      u[s][1] = s < a.n_split ? *(const float4 *)(o + (long)s * D + 4) : float4{0.f, 0.f, 0.f, 0.f};
    }
  }
  const int L = seq_len_clamped(a, b);
  const int ntiles = (L + 127) >> 7;
  const int nv = min((ntiles + a.tiles_per_split - 1) / a.tiles_per_split, a.n_split);
  if (nv == 0) {
    dst[0] = float4{0.f, 0.f, 0.f, 0.f};
    dst[1] = float4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (fast) {
    // the same operations in the same order as the general path below
    const float2 mlv = lane < nv ? mlf : float2{-INFINITY, 0.f};
    float M = mlv.x;
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k));
    const float wl = lane < nv ? __builtin_amdgcn_exp2f(mlv.x - M) : 0.f;
    den = lane < nv ? fmaf(wl, mlv.y, 0.f) : 0.f;
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) den += __shfl_xor(den, k);
#pragma unroll
    for (int s = 0; s < kMlaMergeFast; s++) {
      if (s < nv) {
        const float w = __shfl(wl, s);
        y[0] = fmaf(w, u[s][0].x, y[0]); y[1] = fmaf(w, u[s][0].y, y[1]);
        y[2] = fmaf(w, u[s][0].z, y[2]); y[3] = fmaf(w, u[s][0].w, y[3]);
        y[4] = fmaf(w, u[s][1].x, y[4]); y[5] = fmaf(w, u[s][1].y, y[5]);
        y[6] = fmaf(w, u[s][1].z, y[6]); y[7] = fmaf(w, u[s][1].w, y[7]);
      }
    }
  } else {
  float M = -INFINITY;
  for (int s = lane; s < nv; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k));
  for (int s = lane; s < nv; s += 64) den = fmaf(__builtin_amdgcn_exp2f(ml[2 * s] - M), ml[2 * s + 1], den);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) den += __shfl_xor(den, k);
  for (int s = 0; s < nv; s++) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);
    const float4 u0 = *(const float4 *)(o + (long)s * D), u1 = *(const float4 *)(o + (long)s * D + 4);
    y[0] = fmaf(w, u0.x, y[0]); y[1] = fmaf(w, u0.y, y[1]); y[2] = fmaf(w, u0.z, y[2]); y[3] = fmaf(w, u0.w, y[3]);
    y[4] = fmaf(w, u1.x, y[4]); y[5] = fmaf(w, u1.y, y[5]); y[6] = fmaf(w, u1.z, y[6]); y[7] = fmaf(w, u1.w, y[7]);
  }
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int j = 0; j < 8; j++) y[j] *= inv;
  // Walsh-Hadamard over 512 channels: stages 1, 2, 4 in the lane, 8 .. 256 across lanes
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int j = 0; j < 8; j++)
      if ((j & h) == 0) {
        const float x0 = y[j], x1 = y[j + h];
        y[j] = x0 + x1;
        y[j + h] = x0 - x1;
      }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const float x = __shfl_xor(y[j], m);
      y[j] = upper ? x - y[j] : y[j] + x;
    }
  }
  const float *qs = a.qs + 8 * lane;
#pragma unroll
  for (int j = 0; j < 8; j++) y[j] = y[j] * (1.0f / 512.0f) * qs[j];
  dst[0] = float4{y[0], y[1], y[2], y[3]};
  dst[1] = float4{y[4], y[5], y[6], y[7]};
}

hipError_t launch_mla_partials(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const int nhg = a.hq / kMlaHeads;
  if (a.fmt == kFmtMX) {
    const long units = (long)a.batch * a.n_split;
    const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * ((nhg + 3) / 4));
    switch (a.page_size) {
      case 32: mla_partials_mx<32><<<grid, 512, 0, s>>>(a); break;
      case 64: mla_partials_mx<64><<<grid, 512, 0, s>>>(a); break;
      case 128: mla_partials_mx<128><<<grid, 512, 0, s>>>(a); break;
      case 256: mla_partials_mx<256><<<grid, 512, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const long units = (long)a.batch * a.n_split;
  const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * ((nhg + 3) / 4));
  switch (a.page_size) {
    case 32: mla_partials<32><<<grid, 512, 0, s>>>(a); break;
    case 64: mla_partials<64><<<grid, 512, 0, s>>>(a); break;
    case 128: mla_partials<128><<<grid, 512, 0, s>>>(a); break;
    case 256: mla_partials<256><<<grid, 512, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_mla_merge(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  mla_merge<<<(unsigned)(a.batch * a.hq), 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace fp4kv
