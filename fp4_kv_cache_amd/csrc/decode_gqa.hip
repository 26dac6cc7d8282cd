// Paged FP4 decode attention for GQA on gfx950: split-K partial kernel and merge kernel.
//
// Method ("BitDecoding-FP4: Native FP4 KV Cache Decoding via Algorithm-System
// Co-Design", Article Summary; "BitDecoding-FP4 : décodage natif du KV cache
// FP4", Analyse approfondie): the query is split into two FP4 tensors (the
// second holds the residual of the first); the query rows of one KV head are
// stacked so that one K/V tile load feeds all of them; the softmax is computed
// transposed and its probabilities are quantized to FP4 in registers, scaled so
// that E4M3 block scales keep long-context probabilities away from zero.
//
// Mapping onto CDNA4 (one wave = one workgroup = an equal share of all tiles of the batch):
//  * v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 operands: A = 16 tokens x 128
//    channels of K (lane l: token row l%16, channels 32*(l/16)..+31), B = the
//    stacked query rows, D lane l = column l%16, token rows 4*(l/16)..+3.
//    Token row 4q+r of token group i is tile token 32q + 4i + r, so after the 8
//    groups of a 128-token tile lane l holds 32 consecutive tokens
//    (32*(l/16)..+31) of its column -- exactly the K-slice the P.V MFMA takes
//    as its B operand.  The softmax works on this transposed layout and the
//    probabilities never leave registers.
//  * NVFP4 keys carry E4M3 block scales (16 channels) whose mantissa the
//    E8M0-scaled MFMA cannot take, over blocks half the MFMA's 32-element scale
//    group.  Each group of 16 tokens therefore runs as two parity passes (the
//    query operand keeps one 16-channel half of every lane group, the block its
//    exponent belongs to) times three signed-digit passes of the key scale
//    (S = t0 + t1 - t2, each term the A scale of one pass, the subtracted one
//    on sign-flipped key codes), six MFMAs on one accumulator: the exact
//    products code_K * S * code_Q * 2^eQ summed by the matrix core in fp32.
//    Columns: stacked row = 2 * virtual head + {Q1, Q2}, for both formats.
//  * MXFP4 keys (32-channel E8M0 blocks = one lane group) use one native MFMA
//    per 16 tokens with both scales in hardware.
//  * Probabilities: NVFP4 with power-of-two block scales and tensor scale 2^-10
//    over the tile-relative p = 2^(s - m_tile) (<= 1), converted with
//    v_cvt_scalef32_pk_fp4_f32 (exact power-of-two scaling, RNE); MXFP4 with
//    the MX exponent rule.
//  * NVFP4 values: the E4M3 block scale S_V = t0 + t1 - t2 (powers of two or
//    zeros) is applied as three E8M0 passes (an absent term uses scale byte 0,
//    2^-127, which contributes nothing; the subtracted one runs on P with
//    flipped signs) and two parity passes (16-token blocks inside a 32-token
//    lane group), accumulated in the MFMA.
#include "decode_common.h"

namespace fp4kv {


// One 128-token tile of keys or values in registers: 9 x 16 bytes per lane.
//   keys:   x[0..7] codes, lane row n -> token 32*(n/4) + 4i + n%4 (i = 0..7), channels
//           32*q4..+31; x[8] scales: NVFP4 the 8 block scales of tokens 2*lane, 2*lane+1
//           (staged through LDS), MXFP4 (x[8].x, x[8].y) the lane's 8 E8M0 scales, one per i.
//   values: x[0..7] codes, lane row n -> channel 16*cg + n (cg = 0..7), tokens 32*q4..+31;
//           x[8] the lane's value scales (see the layout notes at load_v).
// When `live` is false the load is a placeholder issued only to keep the wait counts
// static: every lane reads the same 16 bytes of the tile's first row.
struct Tile {
  uint4 x[9];
};

template <int FMT, int P>
__device__ __forceinline__ void load_k(const DecodeArgs &a, Tile &k, const int *pgt, int kvh, int tok0,
                                       int lane, bool live) {
  const int n = lane & 15, q4 = lane >> 4;
  const int tin = 32 * (n >> 2) + (n & 3);      // tile-relative token of row n, group 0
  if constexpr (P >= 32) {
    constexpr int NPT = P >= 128 ? 1 : 128 / P;
    const int pg = pgt[NPT == 1 ? 0 : tin / P];
    const long ph = (long)pg * a.hkv + kvh;
    const int t = (tok0 + tin) % P;
    const int lm = -(int)live;                  // all ones for a real load, zero for a placeholder
    const uint8_t *kb = a.k_codes + ph * (P * 64) + ((t * 64 + 16 * q4) & lm);
#pragma unroll
    for (int i = 0; i < 8; i++) k.x[i] = ld16(kb + 256 * i);
    if constexpr (FMT == kFmtMX) {
      // scale byte (token t, block q) at (((t/32)*4 + t%4)*4 + q)*8 + (t%32)/4
      const int off = (((t >> 5) * 4 + (n & 3)) * 4 + q4) * 8;
      const uint2 s = *(const uint2 *)(a.k_scales + ph * (P * 4) + (off & lm));
      k.x[8] = uint4{s.x, s.y, 0u, 0u};
    }
  } else {  // P == 16 (NVFP4 only): rows i < 4 in one page, i >= 4 in the next
    const int pg0 = pgt[tin / P], pg1 = pgt[tin / P + 1];
    const int t = tin % P;
    const int lo = (t * 64 + 16 * q4) & -(int)live;
    const uint8_t *k0 = a.k_codes + ((long)pg0 * a.hkv + kvh) * (P * 64) + lo;
    const uint8_t *k1 = a.k_codes + ((long)pg1 * a.hkv + kvh) * (P * 64) + lo;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      k.x[i] = ld16(k0 + 256 * i);
      k.x[i + 4] = ld16(k1 + 256 * i);
    }
  }
  if constexpr (FMT == kFmtNV) {
    constexpr int NPT = P >= 128 ? 1 : 128 / P;
    const int pg = pgt[NPT == 1 ? 0 : (2 * lane) / P];
    const uint8_t *sb = a.k_scales + ((long)pg * a.hkv + kvh) * (P * 8);
    k.x[8] = ld16(sb + ((((tok0 + 2 * lane) % P) * 8) & -(int)live));
  }
}

// Value scales of a page and KV head: the byte of (channel c, token block j) sits at
// ((j/J)*16 + c%16)*8*J + (c/16)*J + j%J with J = min(P, 32)/B blocks per 32-token span,
// so that lane (n, q4) finds the scales of channels n, 16+n, ..., 112+n over its 32
// tokens in one contiguous run (NVFP4 P >= 32: 16 bytes, MXFP4: 8 bytes, NVFP4 P == 16:
// 8 bytes in each of its two pages).
template <int FMT, int P>
__device__ __forceinline__ void load_v(const DecodeArgs &a, Tile &v, const int *pgt, int kvh, int tok0,
                                       int lane, bool live) {
  constexpr int D = 128;
  constexpr int B = FMT == kFmtNV ? 16 : 32;
  const int n = lane & 15, q4 = lane >> 4;
  if constexpr (P >= 32) {
    constexpr int NPT = P >= 128 ? 1 : 128 / P;
    constexpr int J = 32 / B;
    const int pg = pgt[NPT == 1 ? 0 : (32 * q4) / P];
    const long ph = (long)pg * a.hkv + kvh;
    const int t = (tok0 + 32 * q4) % P;
    const int lm = -(int)live;
    const uint8_t *cb = a.v_codes + ph * (D * P / 2) + ((n * (P / 2) + t / 2) & lm);
#pragma unroll
    for (int cg = 0; cg < 8; cg++) v.x[cg] = ld16(cb + cg * 16 * (P / 2));
    const uint8_t *sb = a.v_scales + ph * (D * P / B) + ((((t >> 5) * 16 + n) * 8 * J) & lm);
    if constexpr (FMT == kFmtNV) {
      v.x[8] = ld16(sb);
    } else {
      const uint2 s = *(const uint2 *)sb;
      v.x[8] = uint4{s.x, s.y, 0u, 0u};
    }
  } else {  // P == 16: the lane's 32 tokens span two pages
    const int pg0 = pgt[2 * q4], pg1 = pgt[2 * q4 + 1];
    const long p0 = (long)pg0 * a.hkv + kvh, p1 = (long)pg1 * a.hkv + kvh;
    const int lo = (n * 8) & -(int)live;
    const uint8_t *c0 = a.v_codes + p0 * (D * 8) + lo, *c1 = a.v_codes + p1 * (D * 8) + lo;
#pragma unroll
    for (int cg = 0; cg < 8; cg++) {
      const uint2 u0 = *(const uint2 *)(c0 + cg * 128), u1 = *(const uint2 *)(c1 + cg * 128);
      v.x[cg] = uint4{u0.x, u0.y, u1.x, u1.y};
    }
    const uint2 s0 = *(const uint2 *)(a.v_scales + p0 * D + lo);
    const uint2 s1 = *(const uint2 *)(a.v_scales + p1 * D + lo);
    v.x[8] = uint4{s0.x, s0.y, s1.x, s1.y};
  }
}


// NVFP4 key scales of a tile, staged as pass words [token][lane group] (uint2: blocks 2 q4 and
// 2 q4 + 1) with two entries of padding after every 32 tokens (LDS bank spread).
__device__ __forceinline__ int ksw_index(int tok, int q4) { return tok * 4 + q4 + 2 * (tok >> 5); }


// Query rows of one KV head: GV "virtual heads" = (query token j, query head g) pairs,
// v = j * group + g (one query token per sequence: v = g).  One 16-column MFMA holds 8 of
// them (Q1 and Q2 rows), so GV > 8 runs RS row sets on the same key/value tile registers.
template <int FMT, int GV>
constexpr int row_sets() { return (GV + 7) / 8; }

// MQ: several query tokens per sequence (causal rows); false compiles the one-token decode
// with every row seeing the whole sequence.
template <int FMT, int GV, int P, bool MQ>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(row_sets<FMT, GV>() == 1 ? 2 : 1, 2)))
void gqa_partials(DecodeArgs a) {
  constexpr int D = 128;
  constexpr int VS = 8;                        // virtual heads per row set
  constexpr int RS = row_sets<FMT, GV>();      // row sets
  constexpr int NR = 2 * (GV < VS ? GV : VS);  // stacked rows per set: (virtual head, Q1/Q2)
  constexpr int B = FMT == kFmtNV ? 16 : 32;   // scale block
  constexpr int NBLK = D / B;
  constexpr int NPT = P >= 128 ? 1 : 128 / P;  // pages touched by a 128-token tile
  constexpr int CAPG = kMaxSplitPages / NPT;   // tiles whose page ids the LDS window holds
  static_assert(RS <= 2, "at most two row sets");
  static_assert(P >= 16 && (P % B) == 0, "page size");

  const int lane = threadIdx.x;
  const int wave = blockIdx.x;
  Share sh;
  if (!find_share(a, wave, lane, sh)) return;

  __shared__ uint32_t qc[2][GV][D / 8];
  __shared__ int qe[2][GV][NBLK];
  __shared__ float qg[2][GV];
  __shared__ uint32_t lut[256];                // E4M3 value scale -> its three pass bytes
  __shared__ __align__(16) uint2 ksw[FMT == kFmtNV ? 128 * 4 + 8 : 2];   // NVFP4 key pass words
  // physical page ids of the segment's tiles: entry ((tile - tb) % CAPG) * NPT + j is logical
  // page tile * 128 / P + j (clamped to the sequence), so per-tile lookups are LDS reads; a
  // segment longer than CAPG tiles re-stages the window every CAPG tiles
  __shared__ int pgl[kMaxSplitPages];

  // E4M3 code -> its signed-digit pass bytes (t0 + t1 - t2), for NVFP4 values (read after the
  // first segment's barrier below)
#pragma unroll
  for (int i = 0; i < 4; i++) lut[lane + 64 * i] = e4m3_pass_word(lane + 64 * i);
  int nzero = 0;
  const bool count_zero = a.zero_blocks != nullptr;
  const int GQ = MQ ? a.group : GV, QL = MQ ? a.q_len : 1;   // query heads per KV head, tokens
  const int GVr = MQ ? GQ * QL : GV;           // virtual heads in use (<= GV)

  // one segment per (sequence, KV head) unit the wave's share touches
  for (;;) {
  const int b = sh.b, kvh = sh.kvh;
  const int L = sh.L;   // > 0: the unit has tiles
  const long uend = sh.ustart + sh.n;
  const int tb = (int)(sh.x - sh.ustart);
  const int te = (int)((sh.x1 < uend ? sh.x1 : uend) - sh.ustart);
  const int last_lp = min((L - 1) / P, a.max_pages - 1);
  __syncthreads();   // the previous segment has finished reading the staged query and page ids

  // The query rows of this KV head go out first, PG virtual heads per pass.  Lane l holds
  // EPL consecutive channels (c0 = EPL * (l % LPR)) of virtual head ps * PG + l / LPR.
  constexpr int PG = GV < (FMT == kFmtNV ? 8 : 16) ? GV : (FMT == kFmtNV ? 8 : 16);
  constexpr int NPASS = GV / PG;
  constexpr int LPR = 64 / PG;                 // lanes per virtual head
  constexpr int EPL = D / LPR;                 // channels per lane (2 PG)
  const int qr = lane / LPR, c0 = EPL * (lane % LPR);
  float y[EPL];
  auto load_q = [&](int ps) {
    const int v = ps * PG + qr;
    const bool in = !MQ || v < GVr;
    const int j = in ? v / GQ : 0, g = in ? v % GQ : 0;
    const long q0 = (((long)b * QL + j) * a.hq + kvh * GQ + g) * D + c0;
    if (a.q_bf16) {
      const uint16_t *qp = (const uint16_t *)a.q + q0;
#pragma unroll
      for (int i = 0; i < EPL; i++) y[i] = in ? bf16_to_f32(qp[i]) : 0.0f;
    } else {
      const float *qp = (const float *)a.q + q0;
#pragma unroll
      for (int i = 0; i < EPL; i++) y[i] = in ? qp[i] : 0.0f;
    }
    const float *sm = a.qs + kvh * D + c0;
#pragma unroll
    for (int i = 0; i < EPL; i++) y[i] = y[i] * sm[i];
  };
  load_q(0);
  // page ids of tiles t0 .. t0 + CAPG - 1 ((t0 - tb) a multiple of CAPG)
  auto stage_ids = [&](int t0) {
    const int cnt = min(CAPG, te - t0) * NPT;
    for (int e = lane; e < cnt; e += 64)
      pgl[e] = phys_page(a, b, ((t0 + e / NPT) * 128) / P + e % NPT, last_lp);
  };
  stage_ids(tb);
  __syncthreads();

  // the first tile's keys and values are in flight while the query is prepared
  Tile ta, tv;
  load_k<FMT, P>(a, ta, pgl, kvh, tb * 128, lane, true);
  load_v<FMT, P>(a, tv, pgl, kvh, tb * 128, lane, true);
  __builtin_amdgcn_sched_barrier(0);

  // ---------------- prologue: smoothing, rotation, dual-residual FP4 query ----------------
#pragma unroll
  for (int ps = 0; ps < NPASS; ps++) {
  if (ps > 0) load_q(ps);
  const int vq = ps * PG + qr;                 // this lane's virtual head
  // Walsh-Hadamard butterflies in the order of the stages h = 1, 2, ..., 64 (each output
  // a single rounded sum or difference): h < EPL inside the lane, h >= EPL with lane
  // l ^ (h / EPL), the lower lane taking x + x', the upper x' - x.
  if (!(kAblation && (a.abl & kAblNoRotation))) {
#pragma unroll
  for (int h = 1; h < EPL; h <<= 1)
#pragma unroll
    for (int j = 0; j < EPL; j++)
      if ((j & h) == 0) {
        const float x0 = y[j], x1 = y[j + h];
        y[j] = x0 + x1;
        y[j + h] = x0 - x1;
      }
#pragma unroll
  for (int h = EPL; h < D; h <<= 1) {
    const int m = h / EPL;
    const bool upper = (lane & m) != 0;
#pragma unroll
    for (int j = 0; j < EPL; j++) {
      const float o = __shfl_xor(y[j], m);
      y[j] = upper ? o - y[j] : y[j] + o;
    }
  }
  }
  // Dual-residual FP4 query: pass k quantizes the residual left by pass k - 1.  A block of
  // B channels spans B / EPL lanes; NVFP4 also needs the row maximum (all LPR lanes).
  constexpr int BL = B / EPL;                  // lanes per scale block
#pragma unroll
  for (int k = 0; k < 2; k++) {
    float bmax = 0.0f;
#pragma unroll
    for (int j = 0; j < EPL; j++) bmax = fmaxf(bmax, fabsf(y[j]));
#pragma unroll
    for (int o = 1; o < BL; o <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, o));
    uint32_t w[(EPL + 7) / 8];
#pragma unroll
    for (int i = 0; i < (EPL + 7) / 8; i++) w[i] = 0u;
    int e;
    float gq = 1.0f;
    if constexpr (FMT == kFmtNV) {
      float rmax = bmax;
#pragma unroll
      for (int o = BL; o < LPR; o <<= 1) rmax = fmaxf(rmax, __shfl_xor(rmax, o));
      gq = rmax / 1536.0f;
      const bool valid = bmax > 0.0f && gq > 0.0f;
      const float sixg = 6.0f * gq;
      const float inv6g = sixg != 0.0f ? 1.0f / sixg : 0.0f;
      e = ceil_log2_clamp(bmax * inv6g, -9, 8);
      const float S = pow2f(e);
      const float sg = S * gq;
      const float r = (valid && sg != 0.0f) ? 1.0f / sg : 0.0f;
#pragma unroll
      for (int j = 0; j < EPL; j++) {
        const uint32_t c = e2m1_enc_hw(y[j] * r);
        w[j / 8] |= c << (4 * (j % 8));
        y[j] = y[j] - (e2m1_dec_hw(c) * S) * gq;
      }
      if (!valid) e = -128;
    } else {
      e = mx_exp(bmax);
#pragma unroll
      for (int j = 0; j < EPL; j++) {
        const uint32_t c = e2m1_enc_hw(ldexpf(y[j], -e));
        w[j / 8] |= c << (4 * (j % 8));
        y[j] = y[j] - ldexpf(e2m1_dec_hw(c), e);
      }
    }
    // packed codes of channels c0 .. c0 + EPL - 1 (EPL / 2 bytes)
    if constexpr (EPL >= 8) {
#pragma unroll
      for (int i = 0; i < EPL / 8; i++) qc[k][vq][c0 / 8 + i] = w[i];
    } else if constexpr (EPL == 4) {
      ((uint16_t *)&qc[k][vq][0])[c0 / 4] = (uint16_t)w[0];
    } else {
      ((uint8_t *)&qc[k][vq][0])[c0 / 2] = (uint8_t)w[0];
    }
    if ((lane % BL) == 0) qe[k][vq][c0 / B] = e;
    if ((lane % LPR) == 0) qg[k][vq] = gq;
    if (kAblation && (a.abl & kAblSingleQ)) {   // single-pass query: the second pass sees zeros
#pragma unroll
      for (int j = 0; j < EPL; j++) y[j] = 0.0f;
    }
  }
  }   // passes
  __syncthreads();

  const int q4 = lane >> 4;        // lane group: channel block (A/B operands) or token group (D)
  const int n = lane & 15;         // operand row / output column
  // B operand (stacked query rows) and per-lane logit coefficients.  Per row set: column n
  // holds stacked row n: virtual head rs * VS + n / 2, query pass n & 1; its query token sees
  // Lrow tokens.  The lane holds the row's channels 32 q4 .. + 31.  NVFP4: one operand per
  // 16-channel parity (the other half zero), each with its block exponent (B scale byte p);
  // MXFP4: all 32 channels, one E8M0 scale.
  v8i bq[RS][2];
  int qsb[RS];
  float a_own[RS];
  int Lrow[RS];
  bool lrow[RS];                               // the column holds a row in use
  const int ncol = n;
#pragma unroll
  for (int rs = 0; rs < RS; rs++) {
    bq[rs][0] = bq[rs][1] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
    qsb[rs] = 127 | (127 << 8);
    a_own[rs] = 0.0f;
    const float gk = FMT == kFmtNV ? a.gk[kvh] : 1.0f;
    const int r = ncol;
    const int h = rs * VS + (r >> 1), k = r & 1;
    const bool live = r < NR && (!MQ || h < GVr);
    lrow[rs] = live;
    Lrow[rs] = MQ && live ? L - QL + 1 + h / GQ : L;
    if (live) {
      const uint32_t c0 = qc[k][h][4 * q4], c1 = qc[k][h][4 * q4 + 1];
      const uint32_t c2 = qc[k][h][4 * q4 + 2], c3 = qc[k][h][4 * q4 + 3];
      if constexpr (FMT == kFmtNV) {
        bq[rs][0] = v8i{(int)c0, (int)c1, 0, 0, 0, 0, 0, 0};
        bq[rs][1] = v8i{0, 0, (int)c2, (int)c3, 0, 0, 0, 0};
        const int e0 = qe[k][h][2 * q4], e1 = qe[k][h][2 * q4 + 1];   // -128: a block of zeros
        qsb[rs] = (e0 == -128 ? 127 : e0 + 127) | ((e1 == -128 ? 127 : e1 + 127) << 8);
      } else {
        bq[rs][0] = v8i{(int)c0, (int)c1, (int)c2, (int)c3, 0, 0, 0, 0};
        qsb[rs] = qe[k][h][q4] + 127;
      }
      a_own[rs] = (qg[k][h] * gk) * a.coef;
    }
  }
  const int Lmin = MQ ? L - QL + 1 : L;       // the shortest row's length
  // ablation study, normalized P: the row's max and softmax denominator from the first pass
  float vst[RS][2];
#pragma unroll
  for (int rs = 0; rs < RS; rs++) {
    vst[rs][0] = 0.0f;
    vst[rs][1] = 1.0f;
    if (kAblation && (a.abl & kAblVanillaP) && lrow[rs]) {
      const long row = (long)b * a.hq + kvh * GQ + rs * VS + (ncol >> 1);   // one query token
      vst[rs][0] = a.out[row * 128];
      vst[rs][1] = a.out[row * 128 + 1];
    }
  }

  // ---------------- main loop over 128-token tiles ----------------
  float m_run[RS], l_run[RS], f_run[RS];
  v4f o_run[RS][8];
#pragma unroll
  for (int rs = 0; rs < RS; rs++) {
    m_run[rs] = -INFINITY;
    l_run[rs] = 0.0f;
    f_run[rs] = 1.0f;
#pragma unroll
    for (int cg = 0; cg < 8; cg++) o_run[rs][cg] = v4f{0.f, 0.f, 0.f, 0.f};
  }
  const float inv6gp = 1.0f / (6.0f * 0.0009765625f);   // fl32(1 / fl32(6 * 2^-10))
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  // Tile `tile`: keys in kt, values in vt; the keys of tile + 1 are loaded into kn at the
  // start, the values of tile + 1 into vt once P.V has read it.
  auto body = [&](Tile &kt, Tile &vt, Tile &kn, int tile) {
    const int tok0 = tile * 128;
    if (tile + 1 < te && (tile + 1 - tb) % CAPG == 0) {
      // window edge: the ids of this tile were last read by the previous tile's loads
      stage_ids(tile + 1);
      __syncthreads();
    }
    {
      const bool live = tile + 1 < te;
      const int tn = live ? tile + 1 : tile;
      load_k<FMT, P>(a, kn, pgl + ((tn - tb) % CAPG) * NPT, kvh, tn * 128, lane, live);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FMT == kFmtNV) {
      // stage the tile's key scales as pass words: the lane holds the scale bytes of tokens
      // 2 lane and 2 lane + 1 (blocks 0..7 each)
      const uint32_t wv[4] = {kt.x[8].x, kt.x[8].y, kt.x[8].z, kt.x[8].w};
#pragma unroll
      for (int u = 0; u < 2; u++) {
        const int tok = 2 * lane + u;
#pragma unroll
        for (int hq = 0; hq < 2; hq++) {   // lane groups 2 hq, 2 hq + 1
          const uint32_t w = wv[2 * u + hq];
          *(uint4 *)&ksw[ksw_index(tok, 2 * hq)] =
              uint4{lut[w & 0xFFu], lut[(w >> 8) & 0xFFu], lut[(w >> 16) & 0xFFu], lut[w >> 24]};
        }
      }
      __syncthreads();
    }

    // ---- per row set: Q.K^T, softmax, P quantization, P.V on the same key / value tile
#pragma unroll
    for (int rs = 0; rs < RS; rs++) {
    // ---- Q.K^T: logits for (column n, tokens 32*q4 + 4i + rr)
    float s[8][4];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const v8i av = {(int)kt.x[i].x, (int)kt.x[i].y, (int)kt.x[i].z, (int)kt.x[i].w, 0, 0, 0, 0};
      if constexpr (FMT == kFmtNV) {
        // the key scales of the lane's row (token 32 (n / 4) + 4 i + n % 4), blocks 2 q4 + p,
        // as three signed-digit passes per parity p on one accumulator; the subtracted term's
        // passes take the key codes with flipped signs
        const uint2 w = ksw[ksw_index(32 * (n >> 2) + 4 * i + (n & 3), q4)];
        const v8i avn = {(int)(kt.x[i].x ^ kFp4SignBits), (int)(kt.x[i].y ^ kFp4SignBits),
                         (int)(kt.x[i].z ^ kFp4SignBits), (int)(kt.x[i].w ^ kFp4SignBits), 0, 0, 0, 0};
        v4f o = mfma4<0, 0>(av, bq[rs][0], zero, (int)w.x, qsb[rs]);
        o = mfma4<1, 0>(av, bq[rs][0], o, (int)w.x, qsb[rs]);
        o = mfma4<2, 0>(avn, bq[rs][0], o, (int)w.x, qsb[rs]);
        o = mfma4<0, 1>(av, bq[rs][1], o, (int)w.y, qsb[rs]);
        o = mfma4<1, 1>(av, bq[rs][1], o, (int)w.y, qsb[rs]);
        o = mfma4<2, 1>(avn, bq[rs][1], o, (int)w.y, qsb[rs]);
#pragma unroll
        for (int rr = 0; rr < 4; rr++) s[i][rr] = o[rr];
      } else {
        const v4f o = mfma4<0, 0>(av, bq[rs][0], zero, (int)byte_of(kt.x[8], i), qsb[rs]);
#pragma unroll
        for (int rr = 0; rr < 4; rr++) s[i][rr] = o[rr];
      }
    }
    // Q1/Q2 rows: s = fl32(a1*raw1) + fl32(a2*raw2); the neighbour column holds the other product
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        const float t1 = a_own[rs] * s[i][rr];
        s[i][rr] = t1 + xlane1(t1);
      }
    if (tok0 + 128 > Lmin) {   // past a row's own prefix (causal for several query tokens)
      const int Lr = Lrow[rs];
#pragma unroll
      for (int i = 0; i < 8; i++)
#pragma unroll
        for (int rr = 0; rr < 4; rr++)
          if (tok0 + 32 * q4 + 4 * i + rr >= Lr) s[i][rr] = -INFINITY;
    }
    uint32_t pk[4];
    int pbyte[2];
    uint32_t ppw[2] = {0u, 0u};   // normalized P, NVFP4: pass words of the P block scales
    if (kAblation && (a.abl & kAblVanillaP)) {
      // ablation study only: p = 2^(s - M) / den over the whole row (M, den from the first
      // pass), quantized with tensor scale 1: NVFP4 default E4M3 scale per 16 tokens, MXFP4
      // E8M0 per 32; the partial is the plain sum of P.V (the merge adds the unit's slots)
      const float Mr = vst[rs][0], dr = vst[rs][1];
      float am0 = 0.0f, am1 = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; i++)
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
          const float p = s[i][rr] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s[i][rr] - Mr) / dr;
          s[i][rr] = p;
          if (i < 4) am0 = fmaxf(am0, p);
          else am1 = fmaxf(am1, p);
        }
      if constexpr (FMT == kFmtNV) {
        const float am[2] = {am0, am1};
#pragma unroll
        for (int pb = 0; pb < 2; pb++) {
          const uint32_t c = e4m3_enc_sat(am[pb] / 6.0f);
          const float S = e4m3_dec(c);
          const float r = S != 0.0f ? 1.0f / S : 0.0f;
          float t[4][4];
#pragma unroll
          for (int j = 0; j < 4; j++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++) t[j][rr] = s[4 * pb + j][rr] * r;
          pk[2 * pb] = pack8(t[0], t[1], 1.0f);
          pk[2 * pb + 1] = pack8(t[2], t[3], 1.0f);
          ppw[pb] = lut[c];
          pbyte[pb] = 127;
        }
      } else {
        const int e = mx_exp(fmaxf(am0, am1));
        const float ps = ldexpf(1.0f, e);
        pbyte[0] = pbyte[1] = e + 127;
#pragma unroll
        for (int w = 0; w < 4; w++) pk[w] = pack8(s[2 * w], s[2 * w + 1], ps);
      }
      if (count_zero) {
        const bool rep = (ncol & 1) == 0 && lrow[rs];
        const int L = Lrow[rs];
        if (rep) {
          if constexpr (FMT == kFmtNV) {
#pragma unroll
            for (int pb = 0; pb < 2; pb++)
              if (tok0 + 32 * q4 + 16 * pb < L && ((pk[2 * pb] | pk[2 * pb + 1]) & 0x77777777u) == 0u) nzero++;
          } else {
            if (tok0 + 32 * q4 < L && ((pk[0] | pk[1] | pk[2] | pk[3]) & 0x77777777u) == 0u) nzero++;
          }
        }
      }
      m_run[rs] = 0.0f;                                  // weight 1 in the merge
      l_run[rs] = (tb == 0 && q4 == 0) ? 1.0f : 0.0f;    // the unit's first slot carries den = 1
    } else {
    // ---- transposed softmax over the tile; block maxima of the logits give the
    // probability block maxima (exp2 is monotone)
    float bm0 = -INFINITY, bm1 = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        bm0 = fmaxf(bm0, s[i][rr]);
        bm1 = fmaxf(bm1, s[i + 4][rr]);
      }
    const float mt = max_x32(max_x16(fmaxf(bm0, bm1)));
    // a tile holding none of the row's tokens (a shorter query row) contributes nothing
    const bool empty = MQ && mt == -INFINITY;
    const float mts = empty ? 0.0f : mt;
    float lt = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; i++)
#pragma unroll
      for (int rr = 0; rr < 4; rr++) {
        const float p = __builtin_amdgcn_exp2f(s[i][rr] - mts);
        s[i][rr] = p;
        lt = lt + p;
      }
    // ---- fused probability quantization into the P.V B operand
    if constexpr (FMT == kFmtNV) {
      const float am[2] = {__builtin_amdgcn_exp2f(bm0 - mts), __builtin_amdgcn_exp2f(bm1 - mts)};
#pragma unroll
      for (int pb = 0; pb < 2; pb++) {
        const int e = ceil_log2_clamp(am[pb] * inv6gp, -9, 8);
        const float ps = pow2f(e - 10);
        pbyte[pb] = e - 10 + 127;
        pk[2 * pb] = pack8(s[4 * pb], s[4 * pb + 1], ps);
        pk[2 * pb + 1] = pack8(s[4 * pb + 2], s[4 * pb + 3], ps);
      }
    } else {
      const float am = __builtin_amdgcn_exp2f(fmaxf(bm0, bm1) - mts);
      const int e = mx_exp(am);
      const float ps = ldexpf(1.0f, e);
      pbyte[0] = pbyte[1] = e + 127;
#pragma unroll
      for (int w = 0; w < 4; w++) pk[w] = pack8(s[2 * w], s[2 * w + 1], ps);
    }
    if (count_zero) {
      const bool rep = (ncol & 1) == 0 && lrow[rs];
      const int L = Lrow[rs];
      if (rep) {
        if constexpr (FMT == kFmtNV) {
#pragma unroll
          for (int pb = 0; pb < 2; pb++)
            if (tok0 + 32 * q4 + 16 * pb < L && ((pk[2 * pb] | pk[2 * pb + 1]) & 0x77777777u) == 0u) nzero++;
        } else {
          if (tok0 + 32 * q4 < L && ((pk[0] | pk[1] | pk[2] | pk[3]) & 0x77777777u) == 0u) nzero++;
        }
      }
    }
    // ---- online rescale.  The running output is kept as o_run * F (F per column): the
    // tile's P.V is accumulated by the MFMAs on top of o_run * gamma with the tile's own
    // weight as the new F, so no separate accumulator is needed.  A tile whose weight is
    // below 2^-60 is weighted 2^-60 (its contribution is below fp32 resolution either way).
    // An empty tile leaves the running state as it is (alpha 1, beta 0): a share whose first
    // tile is empty for a row would otherwise take exp2(-inf - -inf) = NaN.
    const float m_new = empty ? m_run[rs] : fmaxf(m_run[rs], mt);
    const float alpha = empty ? 1.0f : __builtin_amdgcn_exp2f(m_run[rs] - m_new);
    const float beta = empty ? 0.0f : __builtin_amdgcn_exp2f(mt - m_new);
    l_run[rs] = fmaf(l_run[rs], alpha, lt * beta);
    m_run[rs] = m_new;
    const float f_new = empty ? f_run[rs] : fmaxf(beta, 8.67361737988403547e-19f);   // 2^-60
    const float gamma = (alpha * f_run[rs]) * __builtin_amdgcn_rcpf(f_new);
    f_run[rs] = f_new;
#pragma unroll
    for (int cg = 0; cg < 8; cg++)
#pragma unroll
      for (int rr = 0; rr < 4; rr++) o_run[rs][cg][rr] = o_run[rs][cg][rr] * gamma;
    }   // method P
    // ---- P.V
    if constexpr (FMT == kFmtNV) {
      const v8i p0 = {(int)pk[0], (int)pk[1], 0, 0, 0, 0, 0, 0};
      const v8i p1 = {0, 0, (int)pk[2], (int)pk[3], 0, 0, 0, 0};
      // the subtracted term's passes take P with flipped signs
      const v8i p0n = {(int)(pk[0] ^ kFp4SignBits), (int)(pk[1] ^ kFp4SignBits), 0, 0, 0, 0, 0, 0};
      const v8i p1n = {0, 0, (int)(pk[2] ^ kFp4SignBits), (int)(pk[3] ^ kFp4SignBits), 0, 0, 0, 0};
#pragma unroll
      for (int cg = 0; cg < 8; cg++) {
        const v8i av = {(int)vt.x[cg].x, (int)vt.x[cg].y, (int)vt.x[cg].z, (int)vt.x[cg].w, 0, 0, 0, 0};
        // scale bytes of (channel 16*cg + n) for the lane's first and second 16 tokens
        const uint32_t b0 = P >= 32 ? byte_of(vt.x[8], 2 * cg) : byte_of(vt.x[8], cg);
        const uint32_t b1 = P >= 32 ? byte_of(vt.x[8], 2 * cg + 1) : byte_of(vt.x[8], 8 + cg);
        const int l0 = (int)lut[b0], l1 = (int)lut[b1];
        if (kAblation && (a.abl & kAblVanillaP)) {   // general E4M3 P block scales
          const v4f c = pv_general(av, p0, p0n, o_run[rs][cg], l0, (int)ppw[0]);
          o_run[rs][cg] = pv_general(av, p1, p1n, c, l1, (int)ppw[1]);
          continue;
        }
        v4f c = mfma4<0, 0>(av, p0, o_run[rs][cg], l0, pbyte[0]);
        c = mfma4<1, 0>(av, p0, c, l0, pbyte[0]);
        c = mfma4<2, 0>(av, p0n, c, l0, pbyte[0]);
        c = mfma4<0, 0>(av, p1, c, l1, pbyte[1]);
        c = mfma4<1, 0>(av, p1, c, l1, pbyte[1]);
        o_run[rs][cg] = mfma4<2, 0>(av, p1n, c, l1, pbyte[1]);
      }
    } else {
      const v8i pv = {(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3], 0, 0, 0, 0};
#pragma unroll
      for (int cg = 0; cg < 8; cg++) {
        const v8i av = {(int)vt.x[cg].x, (int)vt.x[cg].y, (int)vt.x[cg].z, (int)vt.x[cg].w, 0, 0, 0, 0};
        o_run[rs][cg] = mfma4<0, 0>(av, pv, o_run[rs][cg], (int)byte_of(vt.x[8], cg), pbyte[0]);
      }
    }
    }   // row sets
    __builtin_amdgcn_sched_barrier(0);
    {
      const bool live = tile + 1 < te;
      const int tn = live ? tile + 1 : tile;
      load_v<FMT, P>(a, vt, pgl + ((tn - tb) % CAPG) * NPT, kvh, tn * 128, lane, live);
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (FMT == kFmtNV) __syncthreads();   // key-scale stage is rewritten by the next tile
  };

  Tile tb2;
  for (int tile = tb; tile < te; tile += 2) {
    body(ta, tv, tb2, tile);
    if (tile + 1 < te) body(tb2, tv, ta, tile + 1);
  }

  // ---------------- epilogue: split partials ----------------
  const long u = (long)b * a.hkv + kvh;
  const long slot = wave + u;
#pragma unroll
  for (int rs = 0; rs < RS; rs++) {
    const float l_tot = sum_x32(sum_x16(l_run[rs]));
    const bool rep = (ncol & 1) == 0 && lrow[rs];
    if (rep) {
      const long rowi = slot * GVr + rs * VS + (ncol >> 1);   // one slot holds GVr partial rows
      const float gv = (FMT == kFmtNV ? a.gv[kvh] : 1.0f) * f_run[rs];
#pragma unroll
      for (int cg = 0; cg < 8; cg++) {
        float4 v = {o_run[rs][cg][0] * gv, o_run[rs][cg][1] * gv, o_run[rs][cg][2] * gv, o_run[rs][cg][3] * gv};
        *(float4 *)(a.ws_o + rowi * D + 16 * cg + 4 * q4) = v;
      }
      if (q4 == 0) *(float2 *)(a.ws_ml + rowi * 2) = float2{m_run[rs], l_tot};
    }
  }
  // the wave holding the unit's first tile records where the unit's partials are
  if (tb == 0 && lane == 0) {
    const long last = owner_of(uend - 1, sh.total, sh.waves);
    *(int2 *)(a.ws_meta + 2 * u) = int2{(int)slot, (int)(last - wave + 1)};
  }
  if (sh.x1 <= uend) break;
  // next unit with tiles
  sh.x = sh.ustart = uend;
  if (++sh.kvh == a.hkv) {
    sh.kvh = 0;
    do {
      if (++sh.b >= a.batch) break;
      sh.L = seq_len_clamped(a, sh.b);
      sh.n = (sh.L + 127) >> 7;
    } while (sh.n == 0);
    if (sh.b >= a.batch) break;   // not reached: the share ends inside the batch
  }
  }   // segments
  if (a.zero_blocks) {
    int z = nzero;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
    if (lane == 0 && z) atomicAdd(a.zero_blocks, z);
  }
}

// Measurement only: the partial kernel's reads without its arithmetic.  Same partition,
// same page-id staging, same tile loads in the same order (keys of tile t + 1 at the start
// of tile t, values of tile t + 1 after tile t's values are consumed); every word of every
// tile is folded (xor) into one word per lane, so the loads cannot be dropped and, for
// sequences of whole tiles, the xor of the sink is the xor of every cache byte read once.
// sink: W x 64 words.
template <int FMT, int P>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void gqa_read_only(DecodeArgs a,
                                                                                              uint32_t *sink) {
  constexpr int NPT = P >= 128 ? 1 : 128 / P;
  constexpr int CAPG = kMaxSplitPages / NPT;
  const int lane = threadIdx.x;
  const int wave = blockIdx.x;
  Share sh;
  if (!find_share(a, wave, lane, sh)) return;
  __shared__ int pgl[kMaxSplitPages];
  uint32_t acc = 0;
  auto fold = [&](const Tile &t) {
#pragma unroll
    for (int i = 0; i < 9; i++) acc ^= t.x[i].x ^ t.x[i].y ^ t.x[i].z ^ t.x[i].w;
  };
  for (;;) {
    const int b = sh.b, kvh = sh.kvh;
    const int L = sh.L;
    const long uend = sh.ustart + sh.n;
    const int tb = (int)(sh.x - sh.ustart);
    const int te = (int)((sh.x1 < uend ? sh.x1 : uend) - sh.ustart);
    const int last_lp = min((L - 1) / P, a.max_pages - 1);
    auto stage_ids = [&](int t0) {
      const int cnt = min(CAPG, te - t0) * NPT;
      for (int e = lane; e < cnt; e += 64)
        pgl[e] = phys_page(a, b, ((t0 + e / NPT) * 128) / P + e % NPT, last_lp);
    };
    __syncthreads();
    stage_ids(tb);
    __syncthreads();
    Tile kt, kn, vt;
    load_k<FMT, P>(a, kt, pgl, kvh, tb * 128, lane, true);
    load_v<FMT, P>(a, vt, pgl, kvh, tb * 128, lane, true);
    for (int tile = tb; tile < te; tile++) {
      if (tile + 1 < te && (tile + 1 - tb) % CAPG == 0) {
        stage_ids(tile + 1);
        __syncthreads();
      }
      const bool live = tile + 1 < te;
      const int tn = live ? tile + 1 : tile;
      load_k<FMT, P>(a, kn, pgl + ((tn - tb) % CAPG) * NPT, kvh, tn * 128, lane, live);
      fold(kt);
      fold(vt);
      load_v<FMT, P>(a, vt, pgl + ((tn - tb) % CAPG) * NPT, kvh, tn * 128, lane, live);
      kt = kn;
    }
    if (sh.x1 <= uend) break;
    sh.x = sh.ustart = uend;
    if (++sh.kvh == a.hkv) {
      sh.kvh = 0;
      do {
        if (++sh.b >= a.batch) break;
        sh.L = seq_len_clamped(a, sh.b);
        sh.n = (sh.L + 127) >> 7;
      } while (sh.n == 0);
      if (sh.b >= a.batch) break;
    }
  }
  sink[(long)wave * 64 + lane] = acc;
}

// One wave per (sequence, query head): out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s
// over the partials of the head's (sequence, KV head) unit.  Lanes first take one partial
// each for (m, l); the weights then go through LDS to the channel loop (lane = 2
// channels), whose loads are independent.
// Merge of one row whose nv <= N partials are all loaded at once (lane s also takes partial s's
// (m, l)); the same operations in the same order as the general path of gqa_merge.
template <int N>
__device__ __forceinline__ void merge_row_fast(const float *ml, const float *o, long sm, long so, int nv, int lane,
                                               float2 *dst) {
  float2 mlv = float2{-INFINITY, 0.f};
  if (lane < nv) mlv = *(const float2 *)(ml + sm * lane);
  float2 v[N];
#pragma unroll
  for (int s = 0; s < N; s++) v[s] = s < nv ? *((const float2 *)(o + so * s) + lane) : float2{0.f, 0.f};
  float M = mlv.x;
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k));
  if (!(M > -INFINITY)) { *dst = float2{0.f, 0.f}; return; }   // a query row with no tokens
  const float wl = lane < nv ? __builtin_amdgcn_exp2f(mlv.x - M) : 0.f;
  float den = lane < nv ? fmaf(wl, mlv.y, 0.f) : 0.f;
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) den += __shfl_xor(den, k);
  float n0 = 0.f, n1 = 0.f;
#pragma unroll
  for (int s = 0; s < N; s++) {
    if (s < nv) {
      const float w = __shfl(wl, s);
      n0 = fmaf(w, v[s].x, n0);
      n1 = fmaf(w, v[s].y, n1);
    }
  }
  *dst = float2{n0 / den, n1 / den};
}

__global__ __launch_bounds__(64) void gqa_merge(DecodeArgs a) {
  const int row = blockIdx.x, lane = threadIdx.x;   // row = (b * q_len + j) * hq + h
  const int G = a.group, GVr = a.group * a.q_len;
  const int b = row / (a.q_len * a.hq), rem = row % (a.q_len * a.hq);
  const int j = rem / a.hq, h = rem % a.hq;
  const long u = (long)b * a.hkv + h / G;
  float2 *dst = (float2 *)(a.out + (long)row * 128) + lane;
  // the unit's slot range is read together with its length (a unit without tiles has no
  // range: its meta words are not written and are not used)
  const int2 meta = *(const int2 *)(a.ws_meta + 2 * u);
  if (seq_tiles(a, b) == 0) { *dst = float2{0.f, 0.f}; return; }
  const int nv = meta.y;
  // first partial row; one slot holds GVr rows, virtual head j * G + h % G
  const long r0 = (long)meta.x * GVr + j * G + h % G;
  const float *ml = a.ws_ml + r0 * 2;
  const float *o = a.ws_o + r0 * 128;
  const long so = (long)GVr * 128, sm = 2L * GVr;  // strides between the unit's partials
  if (kAblation && (a.abl & kAblRowStats)) {
    // ablation study, first pass of normalized P: the row's max and softmax denominator
    float M = -INFINITY;
    for (int s = lane; s < nv; s += 64) M = fmaxf(M, ml[sm * s]);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k));
    float den = 0.f;
    if (M > -INFINITY)
      for (int s = lane; s < nv; s += 64) den = fmaf(__builtin_amdgcn_exp2f(ml[sm * s] - M), ml[sm * s + 1], den);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) den += __shfl_xor(den, k);
    if (lane == 0) *(float2 *)(a.out + (long)row * 128) = float2{M, den};
    return;
  }
  // every (m, l) pair and output partial of the row in flight at once, in three size classes (16, 32, 64)
  if (nv <= 16) { merge_row_fast<16>(ml, o, sm, so, nv, lane, dst); return; }
  if (nv <= 32) { merge_row_fast<32>(ml, o, sm, so, nv, lane, dst); return; }
  if (nv <= 64) { merge_row_fast<64>(ml, o, sm, so, nv, lane, dst); return; }
  __shared__ float wsh[256];
  float M = -INFINITY;
  for (int s = lane; s < nv; s += 64) M = fmaxf(M, ml[sm * s]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k));
  if (!(M > -INFINITY)) { *dst = float2{0.f, 0.f}; return; }   // a query row with no tokens
  float den = 0.f;
  for (int s = lane; s < nv; s += 64) den = fmaf(__builtin_amdgcn_exp2f(ml[sm * s] - M), ml[sm * s + 1], den);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) den += __shfl_xor(den, k);
  float n0 = 0.f, n1 = 0.f;
  for (int s0 = 0; s0 < nv; s0 += 256) {
    const int cnt = min(256, nv - s0);
    __syncthreads();
    for (int s = lane; s < cnt; s += 64) wsh[s] = __builtin_amdgcn_exp2f(ml[sm * (s0 + s)] - M);
    __syncthreads();
    int s = 0;
    for (; s + 4 <= cnt; s += 4) {
      const float2 v0 = *((const float2 *)(o + so * (s0 + s)) + lane);
      const float2 v1 = *((const float2 *)(o + so * (s0 + s + 1)) + lane);
      const float2 v2 = *((const float2 *)(o + so * (s0 + s + 2)) + lane);
      const float2 v3 = *((const float2 *)(o + so * (s0 + s + 3)) + lane);
      n0 = fmaf(wsh[s], v0.x, n0); n1 = fmaf(wsh[s], v0.y, n1);
      n0 = fmaf(wsh[s + 1], v1.x, n0); n1 = fmaf(wsh[s + 1], v1.y, n1);
      n0 = fmaf(wsh[s + 2], v2.x, n0); n1 = fmaf(wsh[s + 2], v2.y, n1);
      n0 = fmaf(wsh[s + 3], v3.x, n0); n1 = fmaf(wsh[s + 3], v3.y, n1);
    }
    for (; s < cnt; s++) {
      const float2 v = *((const float2 *)(o + so * (s0 + s)) + lane);
      n0 = fmaf(wsh[s], v.x, n0);
      n1 = fmaf(wsh[s], v.y, n1);
    }
  }
  *dst = float2{n0 / den, n1 / den};
}

template <int FMT, int GV, bool MQ>
static hipError_t launch_g(const DecodeArgs &a, dim3 grid, hipStream_t s) {
  switch (a.page_size) {
    case 16:
      if constexpr (FMT == kFmtNV) { gqa_partials<FMT, GV, 16, MQ><<<grid, 64, 0, s>>>(a); break; }
      return hipErrorInvalidValue;
    case 32: gqa_partials<FMT, GV, 32, MQ><<<grid, 64, 0, s>>>(a); break;
    case 64: gqa_partials<FMT, GV, 64, MQ><<<grid, 64, 0, s>>>(a); break;
    case 128: gqa_partials<FMT, GV, 128, MQ><<<grid, 64, 0, s>>>(a); break;
    case 256: gqa_partials<FMT, GV, 256, MQ><<<grid, 64, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Virtual heads (query tokens x query heads per KV head) rounded up to a compiled size: up
// to 16 (two row sets of 8); more row sets would not fit the register file next to the
// resident key / value tiles.
hipError_t launch_decode_partials(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_waves);
  if (a.q_len == 1) {   // one query token per sequence: virtual heads = query heads
    if (a.fmt == kFmtNV) {
      switch (a.group) {
        case 1: return launch_g<kFmtNV, 1, false>(a, grid, s);
        case 2: return launch_g<kFmtNV, 2, false>(a, grid, s);
        case 4: return launch_g<kFmtNV, 4, false>(a, grid, s);
        case 8: return launch_g<kFmtNV, 8, false>(a, grid, s);
        default: return hipErrorInvalidValue;
      }
    }
    switch (a.group) {
      case 1: return launch_g<kFmtMX, 1, false>(a, grid, s);
      case 2: return launch_g<kFmtMX, 2, false>(a, grid, s);
      case 4: return launch_g<kFmtMX, 4, false>(a, grid, s);
      case 8: return launch_g<kFmtMX, 8, false>(a, grid, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int gv = a.group * a.q_len;
  if (a.fmt == kFmtNV) {
    if (gv <= 2) return launch_g<kFmtNV, 2, true>(a, grid, s);
    if (gv <= 4) return launch_g<kFmtNV, 4, true>(a, grid, s);
    if (gv <= 8) return launch_g<kFmtNV, 8, true>(a, grid, s);
    if (gv <= 16) return launch_g<kFmtNV, 16, true>(a, grid, s);
    return hipErrorInvalidValue;
  }
  if (gv <= 2) return launch_g<kFmtMX, 2, true>(a, grid, s);
  if (gv <= 4) return launch_g<kFmtMX, 4, true>(a, grid, s);
  if (gv <= 8) return launch_g<kFmtMX, 8, true>(a, grid, s);
  if (gv <= 16) return launch_g<kFmtMX, 16, true>(a, grid, s);
  return hipErrorInvalidValue;
}

hipError_t launch_cache_read(const DecodeArgs &a, uint32_t *sink, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_waves);
  const bool nv = a.fmt == kFmtNV;
  switch (a.page_size) {
    case 16:
      if (nv) { gqa_read_only<kFmtNV, 16><<<grid, 64, 0, s>>>(a, sink); break; }
      return hipErrorInvalidValue;
    case 32: if (nv) gqa_read_only<kFmtNV, 32><<<grid, 64, 0, s>>>(a, sink); else gqa_read_only<kFmtMX, 32><<<grid, 64, 0, s>>>(a, sink); break;
    case 64: if (nv) gqa_read_only<kFmtNV, 64><<<grid, 64, 0, s>>>(a, sink); else gqa_read_only<kFmtMX, 64><<<grid, 64, 0, s>>>(a, sink); break;
    case 128: if (nv) gqa_read_only<kFmtNV, 128><<<grid, 64, 0, s>>>(a, sink); else gqa_read_only<kFmtMX, 128><<<grid, 64, 0, s>>>(a, sink); break;
    case 256: if (nv) gqa_read_only<kFmtNV, 256><<<grid, 64, 0, s>>>(a, sink); else gqa_read_only<kFmtMX, 256><<<grid, 64, 0, s>>>(a, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  gqa_merge<<<(unsigned)(a.batch * a.q_len * a.hq), 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace fp4kv
