// Paged decode attention over a BF16 KV cache on gfx950: the comparison system the FP4 path
// is measured against ("FP4 KV Cache Done Right", section "How good are the results,
// really?": the serving gain over a BF16 KV cache).  Plain softmax attention -- no smoothing,
// rotation or quantization -- with the cache, the query and the probabilities in bfloat16 and
// every sum in fp32, on the same balanced split-K partition, partial layout and merge kernel
// as the FP4 GQA decode, so that the two differ only in what they read and multiply.
//
// Cache layout (head_dim 128, page size P, Hkv heads):
//   K bf16 [page][Hkv][P][128]   token-major: a lane's A operand is 16 contiguous bytes of a row
//   V bf16 [page][Hkv][128][P]   channel-major: a lane's A operand is 8 consecutive tokens of one
//                                channel (the P.V contraction runs over tokens)
//
// Mapping onto CDNA4 (one wave = one workgroup = an equal share of all 128-token tiles of the
// batch, processed as 64-token sub-tiles, the softmax tile):
//  * Q.K^T on v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 channels of K, B = the query heads of
//    the KV head (one per column); four MFMAs per 16 tokens.  Row 4 q + r of token group i is
//    sub-tile token 32 (i / 2) + 8 q + 4 (i % 2) + r, so after the four groups lane (n, q4)
//    holds tokens 32 c + 8 q4 .. + 7 (c = 0, 1) of column n: the P.V B operand.
//  * Transposed softmax over the sub-tile: two cross-lane steps for the max; the probabilities
//    are rounded to bf16 (nearest even) straight into the B operand.
//  * P.V on the same MFMA: A = 16 channels x 32 tokens of V, B = P; the running output is kept
//    as o * F with the online rescale folded into the accumulator (as in the FP4 kernel).
#include "decode_common.h"

namespace fp4kv {
namespace {

typedef __bf16 bh8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v4f mfma_bf16x32(const bh8 &a, const bh8 &b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bh8 as_bh8(const uint4 &u) {
  bh8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// fp32 -> bf16 bits, round to nearest with ties to even (finite inputs)
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) { return bf16_bits(lo) | (bf16_bits(hi) << 16); }

}  // namespace

// One wave per share of the balanced partition (find_share), G query heads per KV head.
template <int G, int P>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2))) void bf16_partials(DecodeArgs a) {
  constexpr int D = 128;
  constexpr int NPT = P >= 128 ? 1 : 128 / P;   // pages touched by a 128-token tile
  constexpr int CAPG = kMaxSplitPages / NPT;    // tiles whose page ids the LDS window holds
  static_assert(P >= 16 && P % 8 == 0 && G >= 1 && G <= 16, "shape");
  const int lane = threadIdx.x;
  const int wave = blockIdx.x;
  Share sh;
  if (!find_share(a, wave, lane, sh)) return;
  __shared__ int pgl[kMaxSplitPages];
  const int q4 = lane >> 4, n = lane & 15;
  const uint16_t *Kc = (const uint16_t *)a.k_codes;
  const uint16_t *Vc = (const uint16_t *)a.v_codes;
  const v4f zero = {0.f, 0.f, 0.f, 0.f};

  for (;;) {   // one segment per (sequence, KV head) unit the share touches
  const int b = sh.b, kvh = sh.kvh, L = sh.L;
  const long uend = sh.ustart + sh.n;
  const int tb = (int)(sh.x - sh.ustart);
  const int te = (int)((sh.x1 < uend ? sh.x1 : uend) - sh.ustart);
  const int last_lp = min((L - 1) / P, a.max_pages - 1);
  auto stage_ids = [&](int t0) {
    const int cnt = min(CAPG, te - t0) * NPT;
    for (int e = lane; e < cnt; e += 64)
      pgl[e] = phys_page(a, b, ((t0 + e / NPT) * 128) / P + e % NPT, last_lp);
  };
  __syncthreads();   // the previous segment has finished reading the page ids
  stage_ids(tb);
  __syncthreads();

  // query B operand of MFMA k: column n = query head kvh * G + n (n < G), channels 32 k + 8 q4 .. + 7
  bh8 bq[4];
  {
    const long q0 = ((long)b * a.hq + kvh * G + (n < G ? n : 0)) * D + 8 * q4;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      uint4 w = uint4{0u, 0u, 0u, 0u};
      if (n < G) {
        if (a.q_bf16) {
          w = *(const uint4 *)((const uint16_t *)a.q + q0 + 32 * k);
        } else {
          const float *qp = (const float *)a.q + q0 + 32 * k;
          w = uint4{pack_bf16(qp[0], qp[1]), pack_bf16(qp[2], qp[3]), pack_bf16(qp[4], qp[5]),
                    pack_bf16(qp[6], qp[7])};
        }
      }
      bq[k] = as_bh8(w);
    }
  }
  const float coef = a.coef;   // fl32(softmax_scale * fl32(log2 e))
  float m_run = -INFINITY, l_run = 0.0f, f_run = 1.0f;
  v4f o_run[8];
#pragma unroll
  for (int cg = 0; cg < 8; cg++) o_run[cg] = zero;

  for (int tile = tb; tile < te; tile++) {
    if (tile > tb && (tile - tb) % CAPG == 0) {   // page-id window edge
      __syncthreads();
      stage_ids(tile);
      __syncthreads();
    }
    const int *pgt = pgl + ((tile - tb) % CAPG) * NPT;
#pragma unroll 1
    for (int half = 0; half < 2; half++) {
      const int t0 = tile * 128 + 64 * half;   // first token of the sub-tile
      if (t0 >= L) break;
      // keys: group i, MFMA k -> row n's token, channels 32 k + 8 q4 .. + 7 (tokens past the
      // sequence read its last token; their logits are masked)
      uint4 kr[4][4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        int tok = t0 + 32 * (i >> 1) + 8 * (n >> 2) + 4 * (i & 1) + (n & 3);
        tok = tok < L ? tok : L - 1;
        const int rel = tok - tile * 128;
        const long row = ((long)pgt[NPT == 1 ? 0 : rel / P] * a.hkv + kvh) * P + tok % P;
        const uint16_t *kp = Kc + row * D + 8 * q4;
#pragma unroll
        for (int k = 0; k < 4; k++) kr[i][k] = ld16((const uint8_t *)(kp + 32 * k));
      }
      // values: chunk c, channel group cg -> channel 16 cg + n, tokens t0 + 32 c + 8 q4 .. + 7
      uint4 vr[2][8];
#pragma unroll
      for (int c = 0; c < 2; c++) {
        int tok = t0 + 32 * c + 8 * q4;
        tok = tok < L ? tok : ((L - 1) & ~7);
        const int rel = tok - tile * 128;
        const long pb = ((long)pgt[NPT == 1 ? 0 : rel / P] * a.hkv + kvh) * D;
        const uint16_t *vp = Vc + (pb + n) * P + tok % P;
#pragma unroll
        for (int cg = 0; cg < 8; cg++) vr[c][cg] = ld16((const uint8_t *)(vp + 16 * cg * P));
      }
      // ---- Q.K^T
      float s[4][4];
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v4f acc = zero;
#pragma unroll
        for (int k = 0; k < 4; k++) acc = mfma_bf16x32(as_bh8(kr[i][k]), bq[k], acc);
#pragma unroll
        for (int rr = 0; rr < 4; rr++) s[i][rr] = coef * acc[rr];
      }
      if (t0 + 64 > L) {
#pragma unroll
        for (int i = 0; i < 4; i++)
#pragma unroll
          for (int rr = 0; rr < 4; rr++)
            if (t0 + 32 * (i >> 1) + 8 * q4 + 4 * (i & 1) + rr >= L) s[i][rr] = -INFINITY;
        // values of tokens past the sequence may be anything: zero them (their P is 0)
#pragma unroll
        for (int c = 0; c < 2; c++) {
          const int tok = t0 + 32 * c + 8 * q4;
#pragma unroll
          for (int cg = 0; cg < 8; cg++) {
            uint32_t w[4] = {vr[c][cg].x, vr[c][cg].y, vr[c][cg].z, vr[c][cg].w};
#pragma unroll
            for (int j = 0; j < 4; j++) {
              const uint32_t keep_lo = tok + 2 * j < L ? 0x0000FFFFu : 0u;
              const uint32_t keep_hi = tok + 2 * j + 1 < L ? 0xFFFF0000u : 0u;
              w[j] &= keep_lo | keep_hi;
            }
            vr[c][cg] = uint4{w[0], w[1], w[2], w[3]};
          }
        }
      }
      // ---- transposed softmax over the 64 tokens of the sub-tile
      float bm = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int rr = 0; rr < 4; rr++) bm = fmaxf(bm, s[i][rr]);
      const float mt = max_x32(max_x16(bm));
      float lt = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int rr = 0; rr < 4; rr++) {
          const float p = __builtin_amdgcn_exp2f(s[i][rr] - mt);
          s[i][rr] = p;
          lt = lt + p;
        }
      // P as bf16 B operands: chunk c holds tokens 32 c + 8 q4 + j from groups 2 c (j < 4), 2 c + 1
      bh8 pbv[2];
#pragma unroll
      for (int c = 0; c < 2; c++)
        pbv[c] = as_bh8(uint4{pack_bf16(s[2 * c][0], s[2 * c][1]), pack_bf16(s[2 * c][2], s[2 * c][3]),
                              pack_bf16(s[2 * c + 1][0], s[2 * c + 1][1]),
                              pack_bf16(s[2 * c + 1][2], s[2 * c + 1][3])});
      // ---- online rescale (running output kept as o_run * F), as in the FP4 kernel
      const float m_new = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      const float beta = __builtin_amdgcn_exp2f(mt - m_new);
      l_run = fmaf(l_run, alpha, lt * beta);
      m_run = m_new;
      const float f_new = fmaxf(beta, 8.67361737988403547e-19f);   // 2^-60
      const float gamma = (alpha * f_run) * __builtin_amdgcn_rcpf(f_new);
      f_run = f_new;
      // ---- P.V
#pragma unroll
      for (int cg = 0; cg < 8; cg++) {
        v4f acc = o_run[cg];
#pragma unroll
        for (int rr = 0; rr < 4; rr++) acc[rr] = acc[rr] * gamma;
        acc = mfma_bf16x32(as_bh8(vr[0][cg]), pbv[0], acc);
        o_run[cg] = mfma_bf16x32(as_bh8(vr[1][cg]), pbv[1], acc);
      }
    }
  }

  // ---------------- epilogue: split partials (slot = share + unit, as the FP4 kernel) ----------------
  const long u = (long)b * a.hkv + kvh;
  const long slot = wave + u;
  const float l_tot = sum_x32(sum_x16(l_run));
  if (n < G) {
    const long rowi = slot * G + n;
#pragma unroll
    for (int cg = 0; cg < 8; cg++)
      *(float4 *)(a.ws_o + rowi * D + 16 * cg + 4 * q4) =
          float4{o_run[cg][0] * f_run, o_run[cg][1] * f_run, o_run[cg][2] * f_run, o_run[cg][3] * f_run};
    if (q4 == 0) *(float2 *)(a.ws_ml + rowi * 2) = float2{m_run, l_tot};
  }
  if (tb == 0 && lane == 0) {
    const long last = owner_of(uend - 1, sh.total, sh.waves);
    *(int2 *)(a.ws_meta + 2 * u) = int2{(int)slot, (int)(last - wave + 1)};
  }
  if (!next_unit(a, sh, uend)) break;
  }   // segments
}

// Append to the BF16 cache: one workgroup per (token, KV head), one thread per channel; keys
// and values rounded to bf16 (nearest even) and written in the cache layout above.
__global__ __launch_bounds__(128) void bf16_append(AppendArgs a) {
  const int tok = blockIdx.x, h = blockIdx.y, c = threadIdx.x;
  const int slot = a.slots[tok];
  if (slot < 0 || slot >= a.num_pages * a.page_size) return;
  const int page = slot / a.page_size, off = slot % a.page_size;
  const long src = ((long)tok * a.hkv + h) * 128 + c;
  const float k = load_elem(a.k_new, src, a.bf16), v = load_elem(a.v_new, src, a.bf16);
  const long ph = (long)page * a.hkv + h;
  ((uint16_t *)a.k_codes)[(ph * a.page_size + off) * 128 + c] = (uint16_t)bf16_bits(k);
  ((uint16_t *)a.v_codes)[(ph * 128 + c) * a.page_size + off] = (uint16_t)bf16_bits(v);
}

template <int G>
static hipError_t launch_bf16_g(const DecodeArgs &a, dim3 grid, hipStream_t s) {
  switch (a.page_size) {
    case 16: bf16_partials<G, 16><<<grid, 64, 0, s>>>(a); break;
    case 32: bf16_partials<G, 32><<<grid, 64, 0, s>>>(a); break;
    case 64: bf16_partials<G, 64><<<grid, 64, 0, s>>>(a); break;
    case 128: bf16_partials<G, 128><<<grid, 64, 0, s>>>(a); break;
    case 256: bf16_partials<G, 256><<<grid, 64, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_bf16_partials(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const dim3 grid((unsigned)a.n_waves);
  switch (a.group) {
    case 1: return launch_bf16_g<1>(a, grid, s);
    case 2: return launch_bf16_g<2>(a, grid, s);
    case 4: return launch_bf16_g<4>(a, grid, s);
    case 8: return launch_bf16_g<8>(a, grid, s);
    case 16: return launch_bf16_g<16>(a, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_bf16_append(const AppendArgs &a, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  bf16_append<<<dim3((unsigned)a.num_tokens, (unsigned)a.hkv), 128, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace fp4kv
