// Paged FP4 decode attention for MLA on gfx950: all query heads share one latent head
// that serves as key and value, plus an unquantized bf16 rope part of the key.
//
// Method ("BitDecoding-FP4: Native FP4 KV Cache Decoding via Algorithm-System
// Co-Design", Article Summary: the design covers GQA and MLA models; "BitDecoding-FP4 :
// décodage natif du KV cache FP4", Analyse approfondie): dual-residual FP4 query,
// stacked query rows sharing each latent tile, transposed softmax with fused
// underflow-aware FP4 probability quantization.
//
// Mapping onto CDNA4 (one workgroup of two waves = one (sequence, group of 16 heads, split),
// each wave owning half of the 512 latent channels):
//  * The latent is quantized in 16-token x 16-channel tiles with an E4M3 scale each.  For
//    Q.K^T the latent codes are widened to fp16 with their tile scale (code * S has at
//    most six significant bits, so the fp16 value is exact) and the dual-residual query
//    rows are fp16 as well (FP4 code times a power-of-two block scale, exact); the
//    contraction runs on v_mfma_f32_16x16x32_f16 with exact products and fp32
//    accumulation.  Per-16-channel exact block terms summed in a fixed order (the
//    reading the GQA kernel reproduces bit for bit) would cost one fp32 FMA per
//    (token, query row, block) -- 8192 per token at 128 heads -- so here the block terms
//    are accumulated in the matrix core's fp32 order instead; the logits agree with
//    that reading to fp32 rounding.  The rope part runs on the bf16 MFMA.
//  * MFMA K index -> channel: lane group q (lanes 16q..16q+15) takes channels
//    128q + 8s .. 128q + 8s + 7 in K-step s, so each lane reads 64 contiguous bytes of
//    its token's latent row per token group.
//  * Token rows of the Q.K^T A operand are ordered like the GQA kernel (row 4q + r of
//    token group i = tile token 32q + 4i + r), so the D layout is the P.V B operand.
//  * P.V: the latent's channel-major copy is the A operand (16 channels x 128 tokens) and
//    the tile scale goes through the same binary expansion into E8M0 passes as the GQA
//    value scale (four mantissa-bit passes x two token parities).
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

// MLA partials.  A workgroup of two waves serves one (sequence, group of 16 query heads,
// split).  Wave hc owns latent channels 256 hc .. 256 hc + 255: it keeps its half of the
// Q1 / Q2 operands in registers, computes the Q1 and Q2 dot products over its channels,
// and accumulates P.V for its channels only.  The half dot products meet in LDS once per
// tile; both waves add them (addition is commutative, so both get the same sums), compute
// the 64-channel rope dot product in full, and form the same logits, softmax state and P.
// Grid: one-dimensional; the head groups of one (sequence, split) get ids with equal
// residue mod 8 so that they tend to share an XCD's L2 (they read the same latent tiles).
// Performance only: any placement gives the same result.
template <int P>
__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_partials(DecodeArgs a) {
  constexpr int D = kMlaD, R = kMlaR, HG = kMlaHeads;
  constexpr int DH = D / 2;                     // latent channels per wave
  constexpr int NPT = P >= 128 ? 1 : 128 / P;
  constexpr int NB = 2;                         // ring of token-group loads, NB - 1 ahead (NB divides 8)
  static_assert(P >= 16 && P % 16 == 0, "page size");
  const int tid = threadIdx.x, lane = tid & 63, hc = tid >> 6;
  const int nhg = a.hq / HG;
  const int units = a.batch * a.n_split;
  int id = blockIdx.x;
  const int slot = id & 7;
  id >>= 3;
  const int hg = id % nhg, ublk = id / nhg;
  const int unit = ublk * 8 + slot;
  if (unit >= units) return;
  const int b = unit / a.n_split, split = unit % a.n_split;
  const int L = a.seq_lens[b];
  const int ntiles = (L + 127) >> 7;
  const int tb = split * a.tiles_per_split;
  const int te = min(ntiles, tb + a.tiles_per_split);
  if (tb >= te) return;
  const int last_lp = min((L - 1) / P, a.max_pages - 1);
  const int h0 = hg * HG;

  // The query (exact fp16 Q1 / Q2 values, rows padded by 16 bytes) is staged here once;
  // afterwards the same bytes carry the half dot products the two waves exchange,
  // [wave][group][Q1 / Q2][lane] float4.
  constexpr int QH_BYTES = 2 * HG * (D + 8) * 2;
  constexpr int SX_BYTES = 2 * 8 * 2 * 64 * 16;
  __shared__ __align__(16) uint8_t stage[QH_BYTES > SX_BYTES ? QH_BYTES : SX_BYTES];
  _Float16 (*qh)[HG][D + 8] = reinterpret_cast<_Float16 (*)[HG][D + 8]>(stage);
  __shared__ float qg[2][HG];
  __shared__ uint32_t lut[256];
  __shared__ int pgl[kMaxSplitPages];

  for (int e = tid; e < (te - tb) * NPT; e += 128)
    pgl[e] = phys_page(a, b, ((tb + e / NPT) * 128) / P + e % NPT, last_lp);

  // ---------------- prologue: smoothing, rotation, dual-residual FP4 query ----------------
  // thread t: head r = t / 8, channels c0 = 64 * (t % 8) .. + 63
  {
    const int r = tid >> 3, c0 = 64 * (tid & 7);
    const long q0 = ((long)b * a.hq + h0 + r) * (D + R) + c0;
    float y[64];
    if (a.q_bf16) {
      const uint16_t *qp = (const uint16_t *)a.q + q0;
#pragma unroll
      for (int j = 0; j < 64; j++) y[j] = bf16_to_f32(qp[j]);
    } else {
      const float *qp = (const float *)a.q + q0;
#pragma unroll
      for (int j = 0; j < 64; j++) y[j] = qp[j];
    }
#pragma unroll
    for (int j = 0; j < 64; j++) y[j] = y[j] * a.qs[c0 + j];
    // Walsh-Hadamard stages h = 1 .. 32 inside the lane, 64, 128, 256 with lanes t ^ 1, ^ 2, ^ 4
#pragma unroll
    for (int h = 1; h < 64; h <<= 1)
#pragma unroll
      for (int j = 0; j < 64; j++)
        if ((j & h) == 0) {
          const float x0 = y[j], x1 = y[j + h];
          y[j] = x0 + x1;
          y[j + h] = x0 - x1;
        }
#pragma unroll
    for (int m = 1; m <= 4; m <<= 1) {
      const bool upper = (tid & m) != 0;
#pragma unroll
      for (int j = 0; j < 64; j++) {
        const float o = __shfl_xor(y[j], m);
        y[j] = upper ? o - y[j] : y[j] + o;
      }
    }
    // dual-residual NVFP4: power-of-two block scales over 16 channels, G = row max / 1536
#pragma unroll
    for (int k = 0; k < 2; k++) {
      float rmax = 0.0f;
#pragma unroll
      for (int j = 0; j < 64; j++) rmax = fmaxf(rmax, fabsf(y[j]));
      rmax = fmaxf(rmax, __shfl_xor(rmax, 1));
      rmax = fmaxf(rmax, __shfl_xor(rmax, 2));
      rmax = fmaxf(rmax, __shfl_xor(rmax, 4));
      const float gq = rmax / 1536.0f;
      const float sixg = 6.0f * gq;
      const float inv6g = sixg != 0.0f ? 1.0f / sixg : 0.0f;
#pragma unroll
      for (int blk = 0; blk < 4; blk++) {
        float bmax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) bmax = fmaxf(bmax, fabsf(y[16 * blk + i]));
        const bool valid = bmax > 0.0f && gq > 0.0f;
        const int e = ceil_log2_clamp(bmax * inv6g, -9, 8);
        const float S = pow2f(e);
        const float sg = S * gq;
        const float rr = (valid && sg != 0.0f) ? 1.0f / sg : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const float x = y[16 * blk + i];
          const uint32_t c = e2m1_enc(x * rr);
          const float qv = valid ? e2m1_dec(c) * S : 0.0f;
          qh[k][r][c0 + 16 * blk + i] = (_Float16)qv;
          y[16 * blk + i] = x - (e2m1_dec(c) * S) * gq;
        }
      }
      if ((tid & 7) == 0) qg[k][r] = gq;
    }
  }
  // E4M3 code -> four E8M0 pass bytes (binary expansion of the scale) for the P.V passes
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int c = tid + 128 * i;
    const int ef = (c >> 3) & 15, m = c & 7;
    const int E = (ef ? ef : 1) - 7 + 127;
    uint32_t w = (ef ? (uint32_t)E : 0u) | ((m & 4) ? (uint32_t)(E - 1) << 8 : 0u) |
                 ((m & 2) ? (uint32_t)(E - 2) << 16 : 0u) | ((m & 1) ? (uint32_t)(E - 3) << 24 : 0u);
    lut[c] = c < 0x7F ? w : 0u;
  }
  __syncthreads();

  const int q4 = lane >> 4;        // lane group
  const int n = lane & 15;         // operand row / output column = head h0 + n
  // B operands of this wave's channels: Q.K^T K-step st, lane group q4, element j is
  // latent channel DH hc + 64 q4 + 8 st + j (the lane's A operand holds the same channels)
  h8 bq0[8], bq1[8];
#pragma unroll
  for (int st = 0; st < 8; st++) {
    bq0[st] = *(const h8 *)&qh[0][n][DH * hc + 64 * q4 + 8 * st];
    bq1[st] = *(const h8 *)&qh[1][n][DH * hc + 64 * q4 + 8 * st];
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
  const float gk = a.gk[0];
  const float a1 = (qg[0][n] * gk) * a.coef, a2 = (qg[1][n] * gk) * a.coef, cr = a.coef_rope;
  float4 *sx = reinterpret_cast<float4 *>(stage);   // reused for the exchange (barrier in the loop)

  // ---------------- main loop over 128-token tiles ----------------
  float m_run = -INFINITY, l_run = 0.0f, f_run = 1.0f;
  v4f o_run[16];
#pragma unroll
  for (int cg = 0; cg < 16; cg++) o_run[cg] = v4f{0.f, 0.f, 0.f, 0.f};
  int nzero = 0;
  const float inv6gp = 1.0f / (6.0f * 0.0009765625f);   // fl32(1 / fl32(6 * 2^-10))
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const bool count_zero = a.zero_blocks != nullptr && hc == 0;

  // Loads run ahead of use: the latent and rope rows of token group i + NB - 1 (crossing
  // into the next tile) are issued while group i computes, and the next tile's key scales
  // while this tile's last groups compute.
  const int trow = 32 * (n >> 2) + (n & 3);   // A-operand row: tile token trow + 4 i in group i
  auto load_group = [&](int tile, int i, uint4 *w) {
    const bool live = tile < te;
    const int tl = live ? tile : te - 1;
    const int *pgt = pgl + (tl - tb) * NPT;
    const int t = trow + 4 * i;
    const int pg = pgt[NPT == 1 ? 0 : t / P];
    const long row = (long)pg * P + (tl * 128 + t) % P;
    const uint8_t *kb = a.k_codes + row * (D / 2) + (DH / 2) * hc + 32 * q4;
    const uint8_t *kr = (const uint8_t *)(a.k_rope + row * R + 8 * q4);
    w[0] = ld16(kb); w[1] = ld16(kb + 16); w[2] = ld16(kr); w[3] = ld16(kr + 64);
  };
  // tile scales (raw E4M3 bytes) of the lane's row tokens, token blocks of groups 0-3 and
  // 4-7, channel blocks 16 hc + 4 q4 .. + 3
  auto load_scales = [&](int tile, uint32_t *sc) {
    const int tl = tile < te ? tile : te - 1;
    const int *pgt = pgl + (tl - tb) * NPT;
#pragma unroll
    for (int hb = 0; hb < 2; hb++) {
      const int t = trow + 16 * hb;
      const int pg = pgt[NPT == 1 ? 0 : t / P];
      sc[hb] = *(const uint32_t *)(a.k_scales + ((long)pg * (P / 16) + ((tl * 128 + t) % P) / 16) * 32 +
                                   16 * hc + 4 * q4);
    }
  };
  uint4 gw[NB][4];
  uint32_t scn[2];
  load_scales(tb, scn);
#pragma unroll
  for (int i = 0; i < NB - 1; i++) load_group(tb, i, gw[i]);

#pragma unroll 1
  for (int tile = tb; tile < te; tile++) {
    const int tok0 = tile * 128;
    const int *pgt = pgl + (tile - tb) * NPT;
    const uint32_t scc[2] = {scn[0], scn[1]};   // this tile's key scales (scn is refilled ahead)
    // ---- Q.K^T: Q1 / Q2 over this wave's channels (to LDS), rope in full, 8 token groups of 16
    __syncthreads();   // the other wave has read the previous exchange (or the query stage)
    float4 *mine = sx + (hc * 16) * 64 + lane;
    float s[8][4];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      
      if (i + NB - 1 < 8) load_group(tile, i + NB - 1, gw[(i + NB - 1) % NB]);
      else load_group(tile + 1, i + NB - 1 - 8, gw[(i + NB - 1) % NB]);
      if (i == 4) load_scales(tile + 1, scn);
      
      const uint4 *w = gw[i % NB];
      const uint32_t ws[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
      h2 sq[4];
#pragma unroll
      for (int j = 0; j < 4; j++) sq[j] = e4m3_h2((scc[i >> 2] >> (8 * j)) & 0xFFu);
      v4f acc1 = zero, acc2 = zero, accr = zero;
#pragma unroll
      for (int st = 0; st < 8; st++) {
        const h8 av = fp4x8_f16(ws[st], sq[st >> 1]);
        acc1 = mfma_f16(av, bq0[st], acc1);
        acc2 = mfma_f16(av, bq1[st], acc2);
      }
      accr = mfma_bf16(as_bh8(w[2]), bqr[0], accr);
      accr = mfma_bf16(as_bh8(w[3]), bqr[1], accr);
      mine[64 * (2 * i)] = float4{acc1[0], acc1[1], acc1[2], acc1[3]};
      mine[64 * (2 * i + 1)] = float4{acc2[0], acc2[1], acc2[2], acc2[3]};
#pragma unroll
      for (int rr = 0; rr < 4; rr++) s[i][rr] = cr * accr[rr];
    }
    // ---- logits from the two halves' dot products: raw = half 0 + half 1 (the same sum in
    // both waves), s = (a1 raw1 + a2 raw2) + cr raw_rope
    __syncthreads();
    {
      const float4 *h0p = sx + lane, *h1p = sx + 16 * 64 + lane;
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const float4 x1 = h0p[64 * (2 * i)], y1 = h1p[64 * (2 * i)];
        const float4 x2 = h0p[64 * (2 * i + 1)], y2 = h1p[64 * (2 * i + 1)];
        const float r1[4] = {x1.x + y1.x, x1.y + y1.y, x1.z + y1.z, x1.w + y1.w};
        const float r2[4] = {x2.x + y2.x, x2.y + y2.y, x2.z + y2.z, x2.w + y2.w};
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
          const float t12 = a1 * r1[rr] + a2 * r2[rr];
          s[i][rr] = t12 + s[i][rr];
        }
      }
    }
    // P.V operands of this tile go out before the softmax
    const int tv = 32 * q4;
    const int pgv = pgt[NPT == 1 ? 0 : tv / P];
    const int tp = (tok0 + tv) % P;
    const uint8_t *srow = a.k_scales + ((long)pgv * (P / 16) + tp / 16) * 32 + 16 * hc;
    const uint8_t *vb = a.v_codes + ((long)pgv * D + DH * hc + n) * (P / 2) + tp / 2;
    uint4 vw[2][4];
    
    const uint4 sa = ld16(srow), sb = ld16(srow + 32);
#pragma unroll
    for (int j = 0; j < 4; j++) vw[0][j] = ld16(vb + (long)j * 16 * (P / 2));
    
    if (tok0 + 128 > L) {
#pragma unroll
      for (int i = 0; i < 8; i++)
#pragma unroll
        for (int rr = 0; rr < 4; rr++)
          if (tok0 + 32 * q4 + 4 * i + rr >= L) s[i][rr] = -INFINITY;
    }
    // ---- transposed softmax over the tile (lane (n, q4) holds tokens 32 q4 .. + 31 of head n)
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
    {
      const float am[2] = {__builtin_amdgcn_exp2f(bm0 - mt), __builtin_amdgcn_exp2f(bm1 - mt)};
#pragma unroll
      for (int pb = 0; pb < 2; pb++) {
        const int e = ceil_log2_clamp(am[pb] * inv6gp, -9, 8);
        const float ps = pow2f(e - 10);
        pbyte[pb] = e - 10 + 127;
        pk[2 * pb] = pack8(s[4 * pb], s[4 * pb + 1], ps);
        pk[2 * pb + 1] = pack8(s[4 * pb + 2], s[4 * pb + 3], ps);
      }
    }
    if (count_zero) {
#pragma unroll
      for (int pb = 0; pb < 2; pb++)
        if (tok0 + 32 * q4 + 16 * pb < L && ((pk[2 * pb] | pk[2 * pb + 1]) & 0x77777777u) == 0u) nzero++;
    }
    // ---- online rescale (running output kept as o_run * f_run, as in the GQA kernel)
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float beta = __builtin_amdgcn_exp2f(mt - m_new);
    l_run = fmaf(l_run, alpha, lt * beta);
    m_run = m_new;
    const float f_new = fmaxf(beta, 8.67361737988403547e-19f);   // 2^-60
    const float gamma = (alpha * f_run) * __builtin_amdgcn_rcpf(f_new);
    f_run = f_new;
#pragma unroll
    for (int cg = 0; cg < 16; cg++)
#pragma unroll
      for (int rr = 0; rr < 4; rr++) o_run[cg][rr] = o_run[cg][rr] * gamma;
    // ---- P.V over this wave's channels: channel-major latent (A: channels DH hc + 16 cg + n,
    // tokens 32 q4 .. + 31), batches of 4 channel groups, the next batch in flight
    const v8i p0 = {(int)pk[0], (int)pk[1], 0, 0, 0, 0, 0, 0};
    const v8i p1 = {0, 0, (int)pk[2], (int)pk[3], 0, 0, 0, 0};
#pragma unroll
    for (int bt = 0; bt < 4; bt++) {
      
      if (bt + 1 < 4) {
#pragma unroll
        for (int j = 0; j < 4; j++) vw[(bt + 1) & 1][j] = ld16(vb + (long)(4 * (bt + 1) + j) * 16 * (P / 2));
      }
      
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int cg = 4 * bt + j;
        const uint4 vc = vw[bt & 1][j];
        const v8i av = {(int)vc.x, (int)vc.y, (int)vc.z, (int)vc.w, 0, 0, 0, 0};
        const int l0 = (int)lut[byte_of(sa, cg)], l1 = (int)lut[byte_of(sb, cg)];
        v4f c = mfma4<0, 0>(av, p0, o_run[cg], l0, pbyte[0]);
        c = mfma4<1, 0>(av, p0, c, l0, pbyte[0]);
        c = mfma4<2, 0>(av, p0, c, l0, pbyte[0]);
        c = mfma4<3, 0>(av, p0, c, l0, pbyte[0]);
        c = mfma4<0, 0>(av, p1, c, l1, pbyte[1]);
        c = mfma4<1, 0>(av, p1, c, l1, pbyte[1]);
        c = mfma4<2, 0>(av, p1, c, l1, pbyte[1]);
        o_run[cg] = mfma4<3, 0>(av, p1, c, l1, pbyte[1]);
      }
    }
  }

  // ---------------- epilogue: split partials (latent output, still rotated) ----------------
  const float l_tot = sum_x32(sum_x16(l_run));
  {
    const long rowi = ((long)b * a.hq + h0 + n) * a.n_split + split;
    const float g = gk * f_run;
#pragma unroll
    for (int cg = 0; cg < 16; cg++) {
      float4 v = {o_run[cg][0] * g, o_run[cg][1] * g, o_run[cg][2] * g, o_run[cg][3] * g};
      *(float4 *)(a.ws_o + rowi * D + DH * hc + 16 * cg + 4 * q4) = v;
    }
    if (hc == 0 && q4 == 0) *(float2 *)(a.ws_ml + rowi * 2) = float2{m_run, l_tot};
  }
  if (count_zero) {
    int z = nzero;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
    if (lane == 0 && z) atomicAdd(a.zero_blocks, z);
  }
}

// MLA partials, MXFP4 latent.  The 32-token x 32-channel tiles carry E8M0 scales, which is
// the block-scaled MFMA's own scale granularity (32 K-elements per lane), so Q.K^T and P.V
// both run as native FP4 x FP4 MFMAs with both scales applied in hardware and no widening:
// per 16 tokens, four MFMAs per query pass over the 512 channels (the four products of one
// 128-channel step are summed by the matrix core, the steps chained on its accumulator)
// plus two bf16 MFMAs for the rope part; per tile, one MFMA per 16 output channels.
// One wave per (sequence, group of 16 query heads, split); lane (n, q4): head h0 + n.
// The query is rotated and quantized directly in the B-operand layout: lane (n, q4) holds
// channels 128 st + 32 q4 + j (st = 0..3, j = 0..31), so the Walsh-Hadamard stages on
// channel bits 0-4 and 7-8 stay in the lane, bits 5 and 6 pair lanes l ^ 16 and l ^ 32,
// and every 32-channel MX block is one lane's own.
template <int P>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 1))) void mla_partials_mx(DecodeArgs a) {
  constexpr int D = kMlaD, R = kMlaR, HG = kMlaHeads;
  constexpr int NPT = P >= 128 ? 1 : 128 / P;
  constexpr int NB = 2;                         // ring of token-group loads, NB - 1 ahead (NB divides 8)
  static_assert(P >= 32 && P % 32 == 0, "page size");
  const int lane = threadIdx.x;
  const int nhg = a.hq / HG;
  const int units = a.batch * a.n_split;
  int id = blockIdx.x;
  const int slot = id & 7;
  id >>= 3;
  const int hg = id % nhg, ublk = id / nhg;
  const int unit = ublk * 8 + slot;
  if (unit >= units) return;
  const int b = unit / a.n_split, split = unit % a.n_split;
  const int L = a.seq_lens[b];
  const int ntiles = (L + 127) >> 7;
  const int tb = split * a.tiles_per_split;
  const int te = min(ntiles, tb + a.tiles_per_split);
  if (tb >= te) return;
  const int last_lp = min((L - 1) / P, a.max_pages - 1);
  const int h0 = hg * HG;
  const int q4 = lane >> 4, n = lane & 15;

  __shared__ int pgl[kMaxSplitPages];
  for (int e = lane; e < (te - tb) * NPT; e += 64)
    pgl[e] = phys_page(a, b, ((tb + e / NPT) * 128) / P + e % NPT, last_lp);

  // ---------------- prologue: smoothing, rotation, dual-residual MXFP4 query ----------------
  v8i bq[2][4];            // [pass][K-step]: FP4 codes of channels 128 st + 32 q4 .. + 31
  int qsb[2][4];           // their E8M0 scale bytes
  {
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
    for (int m = 16; m <= 32; m <<= 1) {
      const bool upper = (lane & m) != 0;
#pragma unroll
      for (int st = 0; st < 4; st++)
#pragma unroll
        for (int j = 0; j < 32; j++) {
          const float o = __shfl_xor(y[st][j], m);
          y[st][j] = upper ? o - y[st][j] : y[st][j] + o;
        }
    }
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
  __syncthreads();

  // ---------------- main loop over 128-token tiles ----------------
  float m_run = -INFINITY, l_run = 0.0f, f_run = 1.0f;
  v4f o_run[32];
#pragma unroll
  for (int cg = 0; cg < 32; cg++) o_run[cg] = v4f{0.f, 0.f, 0.f, 0.f};
  int nzero = 0;
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const bool count_zero = a.zero_blocks != nullptr;

  const int trow = 32 * (n >> 2) + (n & 3);   // A-operand row: tile token trow + 4 i in group i
  auto load_group = [&](int tile, int i, uint4 *w) {
    const bool live = tile < te;
    const int tl = live ? tile : te - 1;
    const int *pgt = pgl + (tl - tb) * NPT;
    const int t = trow + 4 * i;
    const int pg = pgt[NPT == 1 ? 0 : t / P];
    const long row = (long)pg * P + (tl * 128 + t) % P;
    const uint8_t *kb = a.k_codes + row * (D / 2) + 16 * q4;
    const uint8_t *kr = (const uint8_t *)(a.k_rope + row * R + 8 * q4);
    w[0] = ld16(kb); w[1] = ld16(kb + 64); w[2] = ld16(kb + 128); w[3] = ld16(kb + 192);
    w[4] = ld16(kr); w[5] = ld16(kr + 64);
  };
  // E8M0 tile scales of the lane's row tokens (token block n / 4 of the tile): the 16
  // channel blocks of that token block
  auto load_scales = [&](int tile) -> uint4 {
    const int tl = tile < te ? tile : te - 1;
    const int *pgt = pgl + (tl - tb) * NPT;
    const int t = 32 * (n >> 2);
    const int pg = pgt[NPT == 1 ? 0 : t / P];
    return *(const uint4 *)(a.k_scales + ((long)pg * (P / 32) + ((tl * 128 + t) % P) / 32) * 16);
  };
  uint4 gw[NB][6];
  uint4 scn = load_scales(tb);
#pragma unroll
  for (int i = 0; i < NB - 1; i++) load_group(tb, i, gw[i]);

#pragma unroll 1
  for (int tile = tb; tile < te; tile++) {
    const int tok0 = tile * 128;
    const int *pgt = pgl + (tile - tb) * NPT;
    const uint4 scc = scn;
    // ---- Q.K^T over 8 token groups of 16
    float s[8][4];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if (i + NB - 1 < 8) load_group(tile, i + NB - 1, gw[(i + NB - 1) % NB]);
      else load_group(tile + 1, i + NB - 1 - 8, gw[(i + NB - 1) % NB]);
      if (i == 4) scn = load_scales(tile + 1);
      const uint4 *w = gw[i % NB];
      v4f acc1 = zero, acc2 = zero, accr = zero;
#pragma unroll
      for (int st = 0; st < 4; st++) {
        const v8i av = {(int)w[st].x, (int)w[st].y, (int)w[st].z, (int)w[st].w, 0, 0, 0, 0};
        const int sa = (int)byte_of(scc, 4 * st + q4);
        acc1 = mfma4<0, 0>(av, bq[0][st], acc1, sa, qsb[0][st]);
        acc2 = mfma4<0, 0>(av, bq[1][st], acc2, sa, qsb[1][st]);
      }
      accr = mfma_bf16(as_bh8(w[4]), bqr[0], accr);
      accr = mfma_bf16(as_bh8(w[5]), bqr[1], accr);
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        const float t12 = c1 * acc1[rr] + c1 * acc2[rr];
        s[i][rr] = t12 + cr * accr[rr];
      }
    }
    // P.V operands of this tile go out before the softmax
    const int tv = 32 * q4;
    const int pgv = pgt[NPT == 1 ? 0 : tv / P];
    const int tp = (tok0 + tv) % P;
    const uint4 sv = *(const uint4 *)(a.k_scales + ((long)pgv * (P / 32) + tp / 32) * 16);
    const uint8_t *vb = a.v_codes + ((long)pgv * D + n) * (P / 2) + tp / 2;
    uint4 vw[2][8];
#pragma unroll
    for (int j = 0; j < 8; j++) vw[0][j] = ld16(vb + (long)j * 16 * (P / 2));
    if (tok0 + 128 > L) {
#pragma unroll
      for (int i = 0; i < 8; i++)
#pragma unroll
        for (int rr = 0; rr < 4; rr++)
          if (tok0 + 32 * q4 + 4 * i + rr >= L) s[i][rr] = -INFINITY;
    }
    // ---- transposed softmax over the tile (lane (n, q4) holds tokens 32 q4 .. + 31 of head n)
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
    // ---- online rescale (running output kept as o_run * f_run)
    const float m_new = fmaxf(m_run, mt);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    const float beta = __builtin_amdgcn_exp2f(mt - m_new);
    l_run = fmaf(l_run, alpha, lt * beta);
    m_run = m_new;
    const float f_new = fmaxf(beta, 8.67361737988403547e-19f);   // 2^-60
    const float gamma = (alpha * f_run) * __builtin_amdgcn_rcpf(f_new);
    f_run = f_new;
#pragma unroll
    for (int cg = 0; cg < 32; cg++)
#pragma unroll
      for (int rr = 0; rr < 4; rr++) o_run[cg][rr] = o_run[cg][rr] * gamma;
    // ---- P.V: channel-major latent (A: channels 16 cg + n, tokens 32 q4 .. + 31), one MFMA
    // per channel group with the tile scale of (token block, channel block cg / 2)
    const v8i pv = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], 0, 0, 0, 0};
#pragma unroll
    for (int bt = 0; bt < 4; bt++) {
      if (bt + 1 < 4) {
#pragma unroll
        for (int j = 0; j < 8; j++) vw[(bt + 1) & 1][j] = ld16(vb + (long)(8 * (bt + 1) + j) * 16 * (P / 2));
      }
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int cg = 8 * bt + j;
        const uint4 vc = vw[bt & 1][j];
        const v8i av = {(int)vc.x, (int)vc.y, (int)vc.z, (int)vc.w, 0, 0, 0, 0};
        o_run[cg] = mfma4<0, 0>(av, pv, o_run[cg], (int)byte_of(sv, cg >> 1), pbyte);
      }
    }
  }

  // ---------------- epilogue: split partials (latent output, still rotated) ----------------
  const float l_tot = sum_x32(sum_x16(l_run));
  {
    const long rowi = ((long)b * a.hq + h0 + n) * a.n_split + split;
#pragma unroll
    for (int cg = 0; cg < 32; cg++) {
      float4 v = {o_run[cg][0] * f_run, o_run[cg][1] * f_run, o_run[cg][2] * f_run, o_run[cg][3] * f_run};
      *(float4 *)(a.ws_o + rowi * D + 16 * cg + 4 * q4) = v;
    }
    if (q4 == 0) *(float2 *)(a.ws_ml + rowi * 2) = float2{m_run, l_tot};
  }
  if (count_zero) {
    int z = nzero;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
    if (lane == 0 && z) atomicAdd(a.zero_blocks, z);
  }
}

// Merge of one (sequence, query head) row: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,
// then un-rotated (Walsh-Hadamard over the 512 channels, / 512) and un-smoothed (* q_smooth).
// Lane l holds channels 8 l .. 8 l + 7.
__global__ __launch_bounds__(64) void mla_merge(DecodeArgs a) {
  constexpr int D = kMlaD;
  const int row = blockIdx.x, lane = threadIdx.x;
  const int b = row / a.hq;
  const int L = a.seq_lens[b];
  const int ntiles = (L + 127) >> 7;
  const int nv = min((ntiles + a.tiles_per_split - 1) / a.tiles_per_split, a.n_split);
  float *dst = a.out + (long)row * D + 8 * lane;
  if (nv == 0) {
#pragma unroll
    for (int j = 0; j < 8; j++) dst[j] = 0.0f;
    return;
  }
  const float *ml = a.ws_ml + (long)row * a.n_split * 2;
  const float *o = a.ws_o + (long)row * a.n_split * D + 8 * lane;
  float M = -INFINITY;
  for (int s = lane; s < nv; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k));
  float den = 0.f;
  for (int s = lane; s < nv; s += 64) den = fmaf(__builtin_amdgcn_exp2f(ml[2 * s] - M), ml[2 * s + 1], den);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) den += __shfl_xor(den, k);
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < nv; s++) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);
    const float4 u0 = *(const float4 *)(o + (long)s * D), u1 = *(const float4 *)(o + (long)s * D + 4);
    y[0] = fmaf(w, u0.x, y[0]); y[1] = fmaf(w, u0.y, y[1]); y[2] = fmaf(w, u0.z, y[2]); y[3] = fmaf(w, u0.w, y[3]);
    y[4] = fmaf(w, u1.x, y[4]); y[5] = fmaf(w, u1.y, y[5]); y[6] = fmaf(w, u1.z, y[6]); y[7] = fmaf(w, u1.w, y[7]);
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
  for (int j = 0; j < 8; j++) dst[j] = y[j] * (1.0f / 512.0f) * qs[j];
}

hipError_t launch_mla_partials(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const int nhg = a.hq / kMlaHeads;
  if (a.fmt == kFmtMX) {
    const long units = (long)a.batch * a.n_split;
    const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * nhg);
    switch (a.page_size) {
      case 32: mla_partials_mx<32><<<grid, 64, 0, s>>>(a); break;
      case 64: mla_partials_mx<64><<<grid, 64, 0, s>>>(a); break;
      case 128: mla_partials_mx<128><<<grid, 64, 0, s>>>(a); break;
      case 256: mla_partials_mx<256><<<grid, 64, 0, s>>>(a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const long units = (long)a.batch * a.n_split;
  const unsigned grid = (unsigned)(((units + 7) / 8) * 8 * nhg);
  switch (a.page_size) {
    case 16: mla_partials<16><<<grid, 128, 0, s>>>(a); break;
    case 32: mla_partials<32><<<grid, 128, 0, s>>>(a); break;
    case 64: mla_partials<64><<<grid, 128, 0, s>>>(a); break;
    case 128: mla_partials<128><<<grid, 128, 0, s>>>(a); break;
    case 256: mla_partials<256><<<grid, 128, 0, s>>>(a); break;
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
