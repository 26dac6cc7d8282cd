// KV-append quantizer kernels for gfx950.
//
// Keys follow Outlier-Aware Key Quantization ("BitDecoding-FP4: Native FP4 KV
// Cache Decoding via Algorithm-System Co-Design", Article Summary; "FP4 KV
// Cache Done Right", section "What is actually new in BitDecoding-FP4?"):
// static per-channel smoothing, a Hadamard rotation over head_dim, then a
// scale search per block under token-wise scaling ("BitDecoding-FP4 :
// décodage natif du KV cache FP4", Analyse approfondie: the search picks a
// better-fitted factor for each group).  The search window, objective and
// tie rule, the value blocking and the tail re-quantization are this
// library's readings of what the pages leave open:
//   * search: NVFP4 scale codes c0, c0+1, c0-1, c0-2, c0-3 (MXFP4 exponents
//     e0, e0+1, e0-1), objective sum of squared fp32 errors accumulated in
//     element order, first strictly smaller objective wins;
//   * values: channel-wise scales over page-aligned blocks of B tokens (the
//     P.V contraction runs over tokens), default scale, no search;
//   * the last, partly filled value block (MLA: latent tile) of a sequence is
//     re-quantized from the fp32 stage with absent tokens as +0.0.
// Every decision uses single fp32 operations in a fixed order (built with
// -ffp-contract=off), so codes and scales are reproducible bit for bit.
#include "fp4kv_device.h"
#include "fp4kv_internal.h"

namespace fp4kv {

// ---------------------------------------------------------------------------------------------
// Block encoders and scale search on arrays held in registers.

// Objective and codes of an NVFP4 block under scale code c and tensor scale G.
template <int N>
__device__ __forceinline__ float nv_block_err(const float *x, uint32_t c, float G) {
  float S = e4m3_dec(c);
  float sg = S * G;
  float r = (sg != 0.0f) ? 1.0f / sg : 0.0f;
  float err = 0.0f;
#pragma unroll
  for (int i = 0; i < N; i++) {
    float xh = (e2m1_round_hw(x[i] * r) * S) * G;
    float d = x[i] - xh;
    err = err + d * d;
  }
  return err;
}

template <int N>
__device__ __forceinline__ void nv_block_codes(const float *x, uint32_t c, float G, uint8_t *codes) {
  float S = e4m3_dec(c);
  float sg = S * G;
  float r = (sg != 0.0f) ? 1.0f / sg : 0.0f;
#pragma unroll
  for (int i = 0; i < N; i += 2)
    codes[i / 2] = (uint8_t)e2m1_enc2_hw(x[i] * r, x[i + 1] * r);
}

__device__ __forceinline__ uint32_t nv_default_scale(float amax, float G) {
  if (G == 0.0f) return 0u;
  float sixg = 6.0f * G;
  if (sixg == 0.0f) return 0u;
  return e4m3_enc_sat(amax / sixg);
}

// NVFP4 scale search (window of five codes around the default).
template <int N>
__device__ __forceinline__ uint32_t nv_search(const float *x, float G, bool search) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < N; i++) amax = fmaxf(amax, fabsf(x[i]));
  uint32_t c0 = nv_default_scale(amax, G);
  uint32_t best = c0;
  if (!search) return best;
  float best_err = nv_block_err<N>(x, c0, G);
  const int deltas[4] = {1, -1, -2, -3};
#pragma unroll
  for (int k = 0; k < 4; k++) {
    int c = (int)c0 + deltas[k];
    if (c < 0 || c > 0x7E) continue;
    float e = nv_block_err<N>(x, (uint32_t)c, G);
    if (e < best_err) { best_err = e; best = (uint32_t)c; }
  }
  return best;
}

template <int N>
__device__ __forceinline__ float mx_block_err(const float *x, int e) {
  float err = 0.0f;
#pragma unroll
  for (int i = 0; i < N; i++) {
    float xh = ldexpf(e2m1_round_hw(ldexpf(x[i], -e)), e);
    float d = x[i] - xh;
    err = err + d * d;
  }
  return err;
}

template <int N>
__device__ __forceinline__ void mx_block_codes(const float *x, int e, uint8_t *codes) {
#pragma unroll
  for (int i = 0; i < N; i += 2)
    codes[i / 2] = (uint8_t)e2m1_enc2_hw(ldexpf(x[i], -e), ldexpf(x[i + 1], -e));
}

// MXFP4 exponent search (e0, e0+1, e0-1).
template <int N>
__device__ __forceinline__ int mx_search(const float *x, bool search) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < N; i++) amax = fmaxf(amax, fabsf(x[i]));
  int e0 = mx_exp(amax);
  if (!search) return e0;
  int best = e0;
  float best_err = mx_block_err<N>(x, e0);
  const int deltas[2] = {1, -1};
#pragma unroll
  for (int k = 0; k < 2; k++) {
    int e = e0 + deltas[k];
    if (e < -127 || e > 127) continue;
    float er = mx_block_err<N>(x, e);
    if (er < best_err) { best_err = er; best = e; }
  }
  return best;
}

// Unnormalised Walsh-Hadamard transform of 128 values in registers; stages h = 1, 2, ..., 64.
__device__ __forceinline__ void fwht128(float *x) {
#pragma unroll
  for (int h = 1; h < 128; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 128; i++) {
      if (!(i & h)) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
}

// 8 consecutive elements (fp32 or bf16) starting at element index i (multiple of 8).
__device__ __forceinline__ void load8(const void *p, long i, int bf16, float *o) {
  if (bf16) {
    uint4 v = *(const uint4 *)((const uint16_t *)p + i);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      o[2 * k] = __uint_as_float(w[k] << 16);
      o[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    float4 a = *(const float4 *)((const float *)p + i);
    float4 b = *(const float4 *)((const float *)p + i + 4);
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
}

// ---------------------------------------------------------------------------------------------
// GQA keys: one thread per (new token, KV head); head_dim 128.

template <int FMT>
__global__ __launch_bounds__(128) void k_append_gqa(AppendArgs a) {
  constexpr int B = FMT == kFmtNV ? 16 : 32;
  constexpr int NB = 128 / B;
  long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (long)a.num_tokens * a.hkv) return;
  int tok = (int)(gid / a.hkv), h = (int)(gid % a.hkv);
  int slot = a.slots[tok];
  if (slot < 0 || slot >= a.num_pages * a.page_size) return;
  int page = slot / a.page_size, off = slot % a.page_size;

  float x[128];
  const long base = ((long)tok * a.hkv + h) * 128;
  const float *ksi = a.ksi + (long)h * 128;
#pragma unroll
  for (int c = 0; c < 128; c += 8) load8(a.k_new, base + c, a.bf16, x + c);
#pragma unroll
  for (int c = 0; c < 128; c++) x[c] = x[c] * ksi[c];
  if (!(kAblation && (a.abl & kAblNoRotation))) fwht128(x);
  const bool search = !(kAblation && (a.abl & kAblNoSearch));

  const float G = FMT == kFmtNV ? a.gk[h] : 1.0f;
  uint8_t codes[64];
  uint8_t sc[NB];
#pragma unroll
  for (int blk = 0; blk < NB; blk++) {
    if (FMT == kFmtNV) {
      uint32_t c = nv_search<B>(x + blk * B, G, search);
      nv_block_codes<B>(x + blk * B, c, G, codes + blk * B / 2);
      sc[blk] = (uint8_t)c;
    } else {
      int e = mx_search<B>(x + blk * B, search);
      mx_block_codes<B>(x + blk * B, e, codes + blk * B / 2);
      sc[blk] = (uint8_t)(e + 127);
    }
  }
  const long row = ((long)page * a.hkv + h) * a.page_size + off;
  uint4 *dst = (uint4 *)(a.k_codes + row * 64);
#pragma unroll
  for (int k = 0; k < 4; k++) {
    uint4 v;
    v.x = codes[16 * k + 0] | (codes[16 * k + 1] << 8) | (codes[16 * k + 2] << 16) | ((uint32_t)codes[16 * k + 3] << 24);
    v.y = codes[16 * k + 4] | (codes[16 * k + 5] << 8) | (codes[16 * k + 6] << 16) | ((uint32_t)codes[16 * k + 7] << 24);
    v.z = codes[16 * k + 8] | (codes[16 * k + 9] << 8) | (codes[16 * k + 10] << 16) | ((uint32_t)codes[16 * k + 11] << 24);
    v.w = codes[16 * k + 12] | (codes[16 * k + 13] << 8) | (codes[16 * k + 14] << 16) | ((uint32_t)codes[16 * k + 15] << 24);
    dst[k] = v;
  }
  if (NB == 8) {
    uint2 v;
    v.x = sc[0] | (sc[1] << 8) | (sc[2] << 16) | ((uint32_t)sc[3] << 24);
    v.y = sc[4 % NB] | (sc[5 % NB] << 8) | (sc[6 % NB] << 16) | ((uint32_t)sc[7 % NB] << 24);
    *(uint2 *)(a.k_scales + row * NB) = v;
  } else {
    uint8_t *sd = a.k_scales + ((long)page * a.hkv + h) * a.page_size * NB;
#pragma unroll
    for (int q = 0; q < NB; q++) sd[mx_kscale_off(off, q)] = sc[q];
  }
}

// ---------------------------------------------------------------------------------------------
// GQA keys, one wave per (new token, KV head): lane l holds channels 2l, 2l+1; the
// rotation's stages h >= 2 pair lane l with lane l ^ (h/2); then every (block,
// candidate) pair of the scale search gets its own lane (objective accumulated in
// element order), and one lane per block picks the first strictly smallest
// objective in candidate order.  Same arithmetic as k_append_gqa, at a fraction of
// its latency for decode-sized batches.

template <int FMT>
struct KWaveLds {
  static constexpr int B = FMT == kFmtNV ? 16 : 32;
  static constexpr int NB = 128 / B;
  static constexpr int NC = FMT == kFmtNV ? 5 : 3;
  float xs[128];
  float errs[NB][NC];
  int cands[NB][NC];
};

// One wave's key append for (token tok, KV head h).  Every lane of the workgroup reaches
// both barriers; `ok` false (no such pair, or a slot outside the cache) turns the wave's
// loads and stores off.
template <int FMT>
__device__ __forceinline__ void k_append_wave_body(const AppendArgs &a, int tok, int h, int lane, bool ok,
                                                   KWaveLds<FMT> &sh) {
  constexpr int B = KWaveLds<FMT>::B;
  constexpr int NB = KWaveLds<FMT>::NB;
  constexpr int NC = KWaveLds<FMT>::NC;
  float *xs = sh.xs;
  auto &errs = sh.errs;
  auto &cands = sh.cands;
  const int slot = ok ? a.slots[tok] : -1;
  ok = ok && slot >= 0 && slot < a.num_pages * a.page_size;
  const int page = ok ? slot / a.page_size : 0, off = ok ? slot % a.page_size : 0;
  const long base = ((long)tok * a.hkv + h) * 128 + 2 * lane;
  const float *ksi = a.ksi + (long)h * 128 + 2 * lane;
  float x0 = ok ? load_elem(a.k_new, base, a.bf16) * ksi[0] : 0.0f;
  float x1 = ok ? load_elem(a.k_new, base + 1, a.bf16) * ksi[1] : 0.0f;
  if (!(kAblation && (a.abl & kAblNoRotation))) {
    {
      const float p = x0 + x1, m = x0 - x1;
      x0 = p;
      x1 = m;
    }
#pragma unroll
    for (int hh = 2; hh < 128; hh <<= 1) {
      const int lb = hh >> 1;
      const float y0 = __shfl_xor(x0, lb), y1 = __shfl_xor(x1, lb);
      if (lane & lb) { x0 = y0 - x0; x1 = y1 - x1; }
      else { x0 = x0 + y0; x1 = x1 + y1; }
    }
  }
  xs[2 * lane] = x0;
  xs[2 * lane + 1] = x1;
  __syncthreads();
  const float G = FMT == kFmtNV && ok ? a.gk[h] : 1.0f;
  if (lane < NB * NC) {
    const int blk = lane / NC, k = lane % NC;
    float x[B];
#pragma unroll
    for (int i = 0; i < B; i++) x[i] = xs[blk * B + i];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < B; i++) amax = fmaxf(amax, fabsf(x[i]));
    float err = INFINITY;
    int cand;
    // (the ablation build's no-search switch leaves only the default candidate)
    const bool try_it = k == 0 || !(kAblation && (a.abl & kAblNoSearch));
    if constexpr (FMT == kFmtNV) {
      const int deltas[5] = {0, 1, -1, -2, -3};
      cand = (int)nv_default_scale(amax, G) + deltas[k];
      if (try_it && cand >= 0 && cand <= 0x7E) err = nv_block_err<B>(x, (uint32_t)cand, G);
    } else {
      const int deltas[3] = {0, 1, -1};
      cand = mx_exp(amax) + deltas[k];
      if (try_it && cand >= -127 && cand <= 127) err = mx_block_err<B>(x, cand);
    }
    errs[blk][k] = err;
    cands[blk][k] = cand;
  }
  __syncthreads();
  if (ok && lane < NB) {
    const int blk = lane;
    int best = cands[blk][0];
    float be = errs[blk][0];
#pragma unroll
    for (int k = 1; k < NC; k++)
      if (errs[blk][k] < be) { be = errs[blk][k]; best = cands[blk][k]; }
    float x[B];
#pragma unroll
    for (int i = 0; i < B; i++) x[i] = xs[blk * B + i];
    uint8_t codes[B / 2];
    uint8_t sbyte;
    if constexpr (FMT == kFmtNV) {
      nv_block_codes<B>(x, (uint32_t)best, G, codes);
      sbyte = (uint8_t)best;
    } else {
      mx_block_codes<B>(x, best, codes);
      sbyte = (uint8_t)(best + 127);
    }
    const long row = ((long)page * a.hkv + h) * a.page_size + off;
    uint8_t *dst = a.k_codes + row * 64 + blk * (B / 2);
#pragma unroll
    for (int j = 0; j < B / 2; j += 4)
      *(uint32_t *)(dst + j) = codes[j] | (codes[j + 1] << 8) | (codes[j + 2] << 16) | ((uint32_t)codes[j + 3] << 24);
    if constexpr (FMT == kFmtNV) a.k_scales[row * NB + blk] = sbyte;
    else a.k_scales[((long)page * a.hkv + h) * a.page_size * NB + mx_kscale_off(off, blk)] = sbyte;
  }
}

// ---------------------------------------------------------------------------------------------
// Token-block bookkeeping shared by the value and latent kernels.  Token i leads a
// block when it is the first token of its sequence in this batch or its position
// starts a block; the block's new tokens are i .. i + n_new - 1 and its first
// `first` positions were appended by earlier calls (their values are in the stage).
//
// The stage holds one open block per sequence, so inside one call only one workgroup may
// touch a sequence's stage rows: the workgroup of the sequence's first block in the batch
// (`chunk_first`).  It reads the rows earlier calls left (its `first` rows) and, once it has
// read them, writes the rows of the chunk's last block when that block stays incomplete --
// also when that block is a later one, whose own workgroup then leaves the stage alone.
// (Letting the later block's workgroup write would race with the first block's reads.)

struct BlockSpan {
  int seq, bstart, first, n_new, page, off0;
  bool ok;
  bool chunk_first;   // i is the first token of its sequence in the batch
  bool continues;     // the sequence's tokens go on past this block (i + n_new is one of them)
};

template <int B>
__device__ __forceinline__ BlockSpan block_span(const AppendArgs &a, int i) {
  BlockSpan sp;
  sp.ok = false;
  // the next token's id and position are read with this token's, so that one new token per
  // sequence (a decode step) costs a single round of loads
  const bool has_next = i + 1 < a.num_tokens;
  const int s_next = has_next ? a.seq_ids[i + 1] : -1, pos_next = has_next ? a.positions[i + 1] : 0;
  int s = a.seq_ids[i], pos = a.positions[i];
  bool leader = (i == 0) || (a.seq_ids[i - 1] != s) || (pos % B == 0);
  int slot = a.slots[i];
  if (!leader || s < 0 || s >= a.max_seqs || pos < 0 || slot < 0 || slot >= a.num_pages * a.page_size)
    return sp;
  sp.seq = s;
  sp.bstart = pos - pos % B;
  sp.first = pos - sp.bstart;
  int n = 1;
  if (has_next && s_next == s && pos_next < sp.bstart + B) {
    n = 2;
    while (i + n < a.num_tokens && a.seq_ids[i + n] == s && a.positions[i + n] < sp.bstart + B) n++;
  }
  sp.n_new = n;
  sp.chunk_first = (i == 0) || (a.seq_ids[i - 1] != s);
  sp.continues = i + n < a.num_tokens && a.seq_ids[i + n] == s;
  sp.page = slot / a.page_size;
  sp.off0 = (slot % a.page_size) - sp.first;
  // the block must sit inside the slot's page (slot and position disagree otherwise)
  sp.ok = sp.off0 >= 0 && (sp.off0 % B) == 0 && sp.off0 + B <= a.page_size;
  return sp;
}

// End of the chunk of sequence s that starts at batch index i0: the first index after i0
// whose token belongs to another sequence (or num_tokens).  The sequence's tokens are
// contiguous in the batch (a documented precondition), so "index j holds sequence s" is true
// up to the end and false after it; every round probes nthr evenly spaced indices of the open
// range and keeps the interval between the last true and the first false probe, so a chunk
// of n tokens takes about log(n) / log(nthr) rounds.  All nthr threads of the workgroup call it.
__device__ int chunk_end(const AppendArgs &a, int i0, int s, int tid, int nthr) {
  int lo = i0, hi = a.num_tokens;            // seq_ids[lo] == s; index hi counts as another sequence
  while (hi - lo > 1) {
    const int step = (hi - lo - 1 + nthr - 1) / nthr;   // >= 1; the last probe reaches hi - 1
    const long j = (long)lo + (long)step * (tid + 1);
    const int hit = j < hi && a.seq_ids[j] == s;
    const int cnt = __syncthreads_count(hit);
    lo = lo + step * cnt;
    hi = min(hi, lo + step);
  }
  return hi;
}

// The chunk's last block, seen from the chunk's first block (sp.continues): the batch index
// of its first token and its token count; false when it fills its block (nothing to stage)
// or the batch breaks the contiguity precondition.
struct TailSpan {
  int i, n;
};
template <int B>
__device__ bool chunk_tail(const AppendArgs &a, const BlockSpan &sp, int i0, int tid, int nthr, TailSpan &t) {
  const int i1 = chunk_end(a, i0, sp.seq, tid, nthr);
  const int pos_last = a.positions[i1 - 1];
  t.n = pos_last % B + 1;
  t.i = i1 - t.n;
  return t.n < B && t.i > i0 && a.positions[t.i] == pos_last - (t.n - 1);
}

// ---------------------------------------------------------------------------------------------
// GQA values: one workgroup per (leading token, KV head), one thread per channel.

template <int FMT>
__device__ __forceinline__ void v_append_body(const AppendArgs &a, int i, int h, int c) {
  constexpr int B = FMT == kFmtNV ? 16 : 32;
  const int d = 128;
  // the leading token's own value is read in the same round as the token bookkeeping
  const float v_lead = i < a.num_tokens ? load_elem(a.v_new, ((long)i * a.hkv + h) * d + c, a.bf16) : 0.0f;
  BlockSpan sp = block_span<B>(a, i);
  if (!sp.ok) return;
  // the workgroup of the chunk's first block stages the chunk's incomplete last block
  TailSpan tail{0, 0};
  const bool stage_tail = sp.chunk_first && sp.continues && chunk_tail<B>(a, sp, i, c, 128, tail);
  float *stage = a.stage + ((long)sp.seq * a.hkv + h) * B * d;
  float v[B];
#pragma unroll
  for (int k = 0; k < B; k++) {
    float x = 0.0f;
    if (k < sp.first) x = stage[k * d + c];
    else if (k == sp.first) x = v_lead;
    else if (k < sp.first + sp.n_new) x = load_elem(a.v_new, ((long)(i + k - sp.first) * a.hkv + h) * d + c, a.bf16);
    v[k] = x;
  }
  uint8_t codes[B / 2];
  uint32_t sbyte;
  if (FMT == kFmtNV) {
    const float G = a.gv[h];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < B; k++) amax = fmaxf(amax, fabsf(v[k]));
    uint32_t sc = nv_default_scale(amax, G);
    nv_block_codes<B>(v, sc, G, codes);
    sbyte = sc;
  } else {
    int e = mx_search<B>(v, false);
    mx_block_codes<B>(v, e, codes);
    sbyte = (uint32_t)(e + 127);
  }
  const long row = ((long)sp.page * a.hkv + h) * d + c;
  uint8_t *cdst = a.v_codes + row * (a.page_size / 2) + sp.off0 / 2;
#pragma unroll
  for (int k = 0; k < B / 2; k += 4)
    *(uint32_t *)(cdst + k) = codes[k] | (codes[k + 1] << 8) | (codes[k + 2] << 16) | ((uint32_t)codes[k + 3] << 24);
  const int J = (a.page_size < 32 ? a.page_size : 32) / B;
  a.v_scales[((long)sp.page * a.hkv + h) * d * (a.page_size / B) + vscale_off(c, sp.off0 / B, J)] = (uint8_t)sbyte;
  // this thread read its stage rows above, before it writes any (one thread per channel)
  if (sp.chunk_first && !sp.continues && sp.first + sp.n_new < B) {
#pragma unroll
    for (int k = 0; k < B; k++)
      if (k >= sp.first && k < sp.first + sp.n_new) stage[k * d + c] = v[k];
  }
  if (stage_tail) {
    for (int k = 0; k < tail.n; k++)
      stage[k * d + c] = load_elem(a.v_new, ((long)(tail.i + k) * a.hkv + h) * d + c, a.bf16);
  }
}

template <int FMT>
__global__ __launch_bounds__(128) void v_append_gqa(AppendArgs a) {
  v_append_body<FMT>(a, blockIdx.x, blockIdx.y, threadIdx.x);
}

// Keys and values of a decode-sized batch in one launch: blocks [0, nkb) hold two key
// waves each ((token, head) pairs 2 blk and 2 blk + 1 in token-major order), the blocks
// after them one value block each ((leading token, head) in token-major order).
template <int FMT>
__global__ __launch_bounds__(128) void kv_append_small(AppendArgs a, int nkb) {
  const int blk = blockIdx.x;
  if (blk < nkb) {
    __shared__ KWaveLds<FMT> sh[2];
    const int wv = threadIdx.x >> 6;
    const int pair = 2 * blk + wv;
    const bool ok = pair < a.num_tokens * a.hkv;
    k_append_wave_body<FMT>(a, ok ? pair / a.hkv : 0, ok ? pair % a.hkv : 0, threadIdx.x & 63, ok, sh[wv]);
  } else {
    const int u = blk - nkb;
    v_append_body<FMT>(a, u / a.hkv, u % a.hkv, threadIdx.x);
  }
}

// ---------------------------------------------------------------------------------------------
// MLA latent: one workgroup (512 threads) per (leading token) = one B-token tile row of
// the sequence.  The new tokens are smoothed and rotated over 512 channels in LDS, the
// earlier tokens of the tile come from the stage.  The scale search runs one thread per
// (B x B tile, candidate), each summing its objective in (token, channel) order; the
// first candidate with a strictly smaller objective wins, as in a sequential search.

constexpr int kNoCand = -(1 << 30);   // marks a scale candidate outside the code range
constexpr int kLatThreads = 512;      // threads of a latent-append workgroup

template <int FMT>
__global__ __launch_bounds__(kLatThreads) void latent_append(AppendArgs a) {
  constexpr int B = FMT == kFmtNV ? 16 : 32;
  constexpr int D = 512;
  constexpr int NT = D / B;                  // tiles of the row
  constexpr int NC = FMT == kFmtNV ? 5 : 3;  // scale candidates
  constexpr int DP = D + D / 16;             // row length with one pad word per 16 channels
  // channel ch of token k at xs[k][ch + ch / 16]: tile-strided reads fall in distinct banks
  __shared__ float xs[B][DP];
  __shared__ float errs[NC][NT];
  __shared__ int cand[NC][NT];
  __shared__ float rsc[NT];
  __shared__ int ebest[NT];
  const int i = blockIdx.x, tid = threadIdx.x;
  BlockSpan sp = block_span<B>(a, i);
  if (!sp.ok) return;
  float *stage = a.stage + (long)sp.seq * B * D;
  const float *ksi = a.ksi;
  auto X = [&](int k, int ch) -> float & { return xs[k][ch + (ch >> 4)]; };
  // earlier tokens of the tile from the stage, the new tokens, zeros after them: three loops
  // without branches inside, so that their loads are issued back to back
#pragma unroll 8
  for (int e = tid; e < sp.first * D; e += kLatThreads) X(e / D, e % D) = stage[e];
  for (int e = tid; e < sp.n_new * D; e += kLatThreads) {
    const int k = e / D, ch = e % D;
    X(sp.first + k, ch) = load_elem(a.k_new, (long)(i + k) * D + ch, a.bf16) * ksi[ch];
  }
  for (int e = (sp.first + sp.n_new) * D + tid; e < B * D; e += kLatThreads) X(e / D, e % D) = 0.0f;
  __syncthreads();
  // FWHT over the rows of the new tokens (stages h = 1, 2, ..., 256; none when the ablation
  // build switches the rotation off -- the barrier above already published the rows)
  const int hend = kAblation && (a.abl & kAblNoRotation) ? 1 : D;
  for (int h = 1; h < hend; h <<= 1) {
    for (int e = tid; e < sp.n_new * (D / 2); e += kLatThreads) {
      const int k = sp.first + e / (D / 2), w = e % (D / 2);
      int idx = (w / h) * 2 * h + (w % h);
      float p = X(k, idx), q = X(k, idx + h);
      X(k, idx) = p + q;
      X(k, idx + h) = p - q;
    }
    __syncthreads();
  }
  // stage the rotated new tokens when the tile stays incomplete and is the chunk's only one
  // (every stage read of this workgroup happened before the barriers above)
  if (sp.chunk_first && !sp.continues && sp.first + sp.n_new < B) {
    for (int e = tid; e < sp.n_new * D; e += kLatThreads) {
      const int k = sp.first + e / D, ch = e % D;
      stage[k * D + ch] = X(k, ch);
    }
  }
  // rope keys of the new tokens, copied unquantized
  for (int e = tid; e < sp.n_new * a.rope_dim; e += kLatThreads) {
    int k = e / a.rope_dim, r = e % a.rope_dim;
    a.k_rope[((long)sp.page * a.page_size + sp.off0 + sp.first + k) * a.rope_dim + r] =
        ((const uint16_t *)a.k_rope_new)[(long)(i + k) * a.rope_dim + r];
  }
  // ---- scale search.  Each tile's amax by TPT threads.  Then, chunk by chunk of each
  // tile's elements, every (candidate, tile, element) squared error by all threads into LDS,
  // and one thread per (candidate, tile) adding its chunk to a running sum in (token, channel)
  // order -- for every candidate the same fp32 operations in the same order as a sequential
  // search, with the candidates' sums running side by side.
  constexpr int TPT = kLatThreads / NT;      // threads per tile (NVFP4 16, MXFP4 32)
  constexpr int EPT = B * B / TPT;           // elements per thread and tile
  constexpr int CH = FMT == kFmtNV ? 64 : 256;    // elements per chunk of a tile
  constexpr int DDP = CH + 4;                // padded rows: 16-byte aligned, on distinct banks
  static_assert(NC * NT <= kLatThreads && (B * B) % CH == 0, "one summing thread per (candidate, tile)");
  __shared__ __attribute__((aligned(16))) float dd[NC][NT][DDP];
  __shared__ float tmax[NT];
  const float G = FMT == kFmtNV ? a.gk[0] : 1.0f;
  const int st_ct = tid / TPT, st_sub = tid % TPT;   // tile and element stride of this thread
  {
    float m = 0.0f;
#pragma unroll 8
    for (int j = 0; j < EPT; j++) {
      const int idx = st_sub + TPT * j;      // element idx = token * B + channel of the tile
      m = fmaxf(m, fabsf(X(idx / B, st_ct * B + idx % B)));
    }
#pragma unroll
    for (int o = TPT / 2; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));   // TPT consecutive lanes
    if (st_sub == 0) tmax[st_ct] = m;
  }
  __syncthreads();
  const bool summer = tid < NC * NT;
  const int s_kk = tid / NT, s_ct = tid % NT;   // the summing thread's (candidate, tile)
  if (summer) {
    const float amax = tmax[s_ct];
    int c;
    bool valid;
    if constexpr (FMT == kFmtNV) {
      const int deltas[5] = {0, 1, -1, -2, -3};
      c = (int)nv_default_scale(amax, G) + deltas[s_kk];
      valid = c >= 0 && c <= 0x7E;
    } else {
      const int deltas[3] = {0, 1, -1};
      c = mx_exp(amax) + deltas[s_kk];
      valid = c >= -127 && c <= 127;
    }
    // (the ablation build's no-search switch leaves only the default candidate)
    if (kAblation && s_kk > 0 && (a.abl & kAblNoSearch)) valid = false;
    cand[s_kk][s_ct] = valid ? c : kNoCand;
  }
  __syncthreads();
  // this thread's tile st_ct: every candidate's scale (an out-of-range candidate is evaluated
  // with a clamped code and its sum is never used)
  float c_s[NC], c_r[NC];
  int c_e[NC];
#pragma unroll
  for (int kk = 0; kk < NC; kk++) {
    const int c = cand[kk][st_ct];
    if constexpr (FMT == kFmtNV) {
      const float S = e4m3_dec((uint32_t)(c == kNoCand ? 0 : c)), sg = S * G;
      c_s[kk] = S;
      c_r[kk] = (sg != 0.0f) ? 1.0f / sg : 0.0f;
      c_e[kk] = 0;
    } else {
      c_s[kk] = c_r[kk] = 0.0f;
      c_e[kk] = c == kNoCand ? 0 : c;
    }
  }
  float err = 0.0f;
  for (int ch0 = 0; ch0 < B * B; ch0 += CH) {
#pragma unroll 4
    for (int j = 0; j < CH / TPT; j++) {
      const int e = st_sub + TPT * j, idx = ch0 + e;   // element idx = token * B + channel
      const float x = X(idx / B, st_ct * B + idx % B);
#pragma unroll
      for (int kk = 0; kk < NC; kk++) {
        float dx;
        if constexpr (FMT == kFmtNV) dx = x - (e2m1_round_hw(x * c_r[kk]) * c_s[kk]) * G;
        else dx = x - ldexpf(e2m1_round_hw(ldexpf(x, -c_e[kk])), c_e[kk]);
        dd[kk][st_ct][e] = dx * dx;
      }
    }
    __syncthreads();
    if (summer && cand[s_kk][s_ct] != kNoCand) {
      const float *row = dd[s_kk][s_ct];
#pragma unroll 8
      for (int e = 0; e < CH; e += 4) {
        const float4 v = *(const float4 *)(row + e);
        err = err + v.x;
        err = err + v.y;
        err = err + v.z;
        err = err + v.w;
      }
    }
    __syncthreads();
  }
  if (summer) errs[s_kk][s_ct] = err;
  __syncthreads();
  uint32_t sbyte_t = 0;
  if (tid < NT) {
    const int ct = tid;
    int best = cand[0][ct];               // the default candidate is always in range
    float best_err = errs[0][ct];
    for (int kk = 1; kk < NC; kk++)
      if (cand[kk][ct] != kNoCand && errs[kk][ct] < best_err) { best_err = errs[kk][ct]; best = cand[kk][ct]; }
    if constexpr (FMT == kFmtNV) {
      const float S = e4m3_dec((uint32_t)best), sg = S * G;
      rsc[ct] = (sg != 0.0f) ? 1.0f / sg : 0.0f;
      sbyte_t = (uint32_t)best;
    } else {
      ebest[ct] = best;
      sbyte_t = (uint32_t)(best + 127);
    }
    a.k_scales[((long)sp.page * (a.page_size / B) + sp.off0 / B) * NT + ct] = (uint8_t)sbyte_t;
  }
  __syncthreads();
  const long pbase = (long)sp.page * a.page_size;
  // token-major codes (the key operand, read transposed as the value operand): task = (token k,
  // tile ct), B / 2 bytes
  for (int e = tid; e < B * NT; e += kLatThreads) {
    const int k = e / NT, ct = e % NT;
    const float r = FMT == kFmtNV ? rsc[ct] : 0.0f;
    const int eb = FMT == kFmtNV ? 0 : ebest[ct];
    uint8_t *dst = a.k_codes + (pbase + sp.off0 + k) * (D / 2) + ct * (B / 2);
#pragma unroll
    for (int j = 0; j < B / 2; j += 4) {
      uint32_t w = 0;
#pragma unroll
      for (int u = 0; u < 8; u++) {
        const float x = X(k, ct * B + 2 * j + u);
        const uint32_t q = FMT == kFmtNV ? e2m1_enc_hw(x * r) : e2m1_enc_hw(ldexpf(x, -eb));
        w |= q << (4 * u);
      }
      *(uint32_t *)(dst + j) = w;
    }
  }
  // The chunk's first tile stages the chunk's incomplete last tile (a later tile of the same
  // call, whose own workgroup leaves the stage alone): its rows smoothed and rotated as above.
  if (!(sp.chunk_first && sp.continues)) return;
  TailSpan tail;
  if (!chunk_tail<B>(a, sp, i, tid, kLatThreads, tail)) return;
  __syncthreads();   // every thread is done reading xs
  for (int e = tid; e < tail.n * D; e += kLatThreads) {
    const int k = e / D, ch = e % D;
    X(k, ch) = load_elem(a.k_new, (long)(tail.i + k) * D + ch, a.bf16) * ksi[ch];
  }
  __syncthreads();
  for (int h = 1; h < hend; h <<= 1) {
    for (int e = tid; e < tail.n * (D / 2); e += kLatThreads) {
      const int k = e / (D / 2), w = e % (D / 2);
      const int idx = (w / h) * 2 * h + (w % h);
      const float p = X(k, idx), q = X(k, idx + h);
      X(k, idx) = p + q;
      X(k, idx + h) = p - q;
    }
    __syncthreads();
  }
  for (int e = tid; e < tail.n * D; e += kLatThreads) stage[e] = X(e / D, e % D);
}

// ---------------------------------------------------------------------------------------------

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.attn == FP4KV_GQA) {
    long n = (long)a.num_tokens * a.hkv;
    dim3 gk((unsigned)((n + 127) / 128)), gv((unsigned)a.num_tokens, (unsigned)a.hkv);
    // small batches (decode): one wave per (token, head) for latency, keys and values in
    // one launch; large ones (prefill): one thread per (token, head) for throughput.
    // Identical results.
    const bool wave = n <= 65536;
    if (wave) {   // one launch: key waves, then value blocks
      const int nkb = (int)((n + 1) / 2);
      const unsigned grid = (unsigned)(nkb + n);
      if (a.fmt == kFmtNV) kv_append_small<kFmtNV><<<grid, 128, 0, s>>>(a, nkb);
      else kv_append_small<kFmtMX><<<grid, 128, 0, s>>>(a, nkb);
    } else if (a.fmt == kFmtNV) {
      k_append_gqa<kFmtNV><<<gk, 128, 0, s>>>(a);
      v_append_gqa<kFmtNV><<<gv, 128, 0, s>>>(a);
    } else {
      k_append_gqa<kFmtMX><<<gk, 128, 0, s>>>(a);
      v_append_gqa<kFmtMX><<<gv, 128, 0, s>>>(a);
    }
  } else {
    if (a.fmt == kFmtNV) latent_append<kFmtNV><<<a.num_tokens, kLatThreads, 0, s>>>(a);
    else latent_append<kFmtMX><<<a.num_tokens, kLatThreads, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace fp4kv
