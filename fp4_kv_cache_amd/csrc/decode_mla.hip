// Paged FP4 decode attention for MLA on gfx950: all query heads share one latent head
// that serves as key and value, plus an unquantized bf16 rope part of the key.
//
// Method ("BitDecoding-FP4: Native FP4 KV Cache Decoding via Algorithm-System
// Co-Design", Article Summary: the design covers GQA and MLA models; "BitDecoding-FP4 :
// décodage natif du KV cache FP4", Analyse approfondie and Contexte): dual-residual FP4
// query, stacked query rows sharing each latent tile, attention computed on the FP4 matrix
// units without dequantizing the cache, transposed softmax with fused underflow-aware FP4
// probability quantization.
//
// Mapping onto CDNA4.  A workgroup of eight waves serves one share of the batch's 128-token
// tiles (the balanced partition of the GQA kernel, with a sequence as the unit) for four
// groups of 16 query heads: waves 0-3 ("score" waves, one per head group) keep the group's
// dual-residual query and compute Q.K^T, the transposed softmax and the FP4 probabilities;
// waves 4-7 ("value" waves) keep the group's running output and compute P.V one tile
// behind, taking the probabilities, their block exponents and the online-softmax rescale
// factor from a small LDS handoff.  Each SIMD holds one wave of each kind.  Each tile --
// latent codes (token-major), rope keys and scales -- is staged once per workgroup in LDS
// with direct global -> LDS loads, issued a whole tile ahead by the value waves.  The query is
// prepared beforehand by its own kernel (mla_qprep), once per (sequence, query head).
//
// Both contractions run on v_mfma_scale_f32_16x16x128_f8f6f4 with FP4 operands:
//  * K index -> channel: in K-step st lane group q4 (lanes 16 q4 .. + 15) holds channels
//    128 st + 32 q4 .. + 31, so a lane's A operand is 16 contiguous bytes of its token row
//    and the query is rotated and quantized directly in the B-operand layout.
//  * Token rows of the Q.K^T A operand: row 4 q + r of token group i is tile token
//    32 q + 4 i + r, so after the eight groups lane (n, q4) holds tokens 32 q4 .. + 31 of
//    head n -- the P.V B operand.
//  * MXFP4 latent (32 x 32 tiles, E8M0): one MFMA per query pass per K-step, tile and query
//    scales applied by the hardware.
//  * NVFP4 latent (16 x 16 tiles, E4M3 scale S = 2^E (1 + m/8)): the E8M0-scaled MFMA takes
//    one power of two per (row, 32-element lane group), so each K-step runs as two parity
//    passes (the query operand keeps one 16-channel half of every lane group, the other half
//    zeroed: the 16-channel block that the tile scale and the query block exponent belong to)
//    times three signed-digit passes of S (S = t0 + t1 - t2 with powers of two or zeros, each
//    the A scale of one pass, E8M0 byte 0 = 2^-127 for an absent term, whose products vanish
//    below fp32 resolution; the subtracted term's pass takes the codes with flipped signs),
//    accumulated by the MFMA: the exact products code_K * S * code_Q * 2^eQ summed in fp32.
//  * P.V: the value operand (16 channels x 32 tokens per lane) is read transposed from the
//    same token-major tile with the 4-bit transposed LDS read, so the cache holds the latent
//    once; the NVFP4 tile scale goes through the same signed-digit passes (token parities and
//    the subtracted term's sign flip on the P side).
//  * The merge kernel un-rotates and un-smooths the merged latent output:
//    out = (o H / 512) * q_smooth.
#include "decode_common.h"

namespace fp4kv {

typedef __bf16 bh8 __attribute__((ext_vector_type(8)));

constexpr int kMlaD = 512;        // latent channels
constexpr int kMlaR = 64;         // rope channels
constexpr int kMlaHeads = 16;     // query heads per wave

__device__ __forceinline__ v4f mfma_bf16(const bh8 &a, const bh8 &b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bh8 as_bh8(const uint4 &u) {
  bh8 r;
  __builtin_memcpy(&r, &u, 16);
  return r;
}

// Direct global -> LDS load of 16 bytes per lane: lane l's bytes land at lds + 16 l (lds is
// wave-uniform; inactive lanes write nothing).  Written as inline assembly because the compiler
// would make every LDS read it cannot prove disjoint from a pending LDS load wait for it, which
// defeats loading the next tile while the current one is read; the kernel waits for its own
// loads (vmcnt) before the barrier that hands a tile to the other waves.  M0 holds the LDS base
// (one wait state between writing M0 and the load).  M0 is a register the compiler reserves and
// cannot take as a clobber; no compiler-generated instruction of these kernels reads or writes it
// (their compiled code sets M0 only in these wrappers), so the wrappers disturb nothing.
__device__ __forceinline__ void lds_load16(const void *g, const void *lds) {
  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(base)), "v"(g) : "memory");
}
// The same load from a wave-uniform 64-bit base (in SGPRs) plus a 32-bit per-lane byte offset,
// so that a wave's loads from one page need no per-lane 64-bit address arithmetic.
__device__ __forceinline__ void lds_load16_so(const uint8_t *gbase, uint32_t off, const void *lds) {
  const uint32_t base = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(__builtin_amdgcn_readfirstlane(base)), "v"(off), "s"(gbase) : "memory");
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

// The three signed-digit passes of one NVFP4 Q.K^T parity pass PB, Q1 and Q2 interleaved.  The
// query operands b1 / b2 hold only the parity's 16-channel half of every lane group (the block
// that the tile scale and the query block exponent belong to), so the key operand is the full
// staged row: A scale byte d of w (the tile scale's term d), B scale byte PB of e1 / e2 (the query
// block exponents of the two halves).  The added terms t0, t1 accumulate in acc1 / acc2, the
// subtracted term t2 in acc1n / acc2n; the logit takes the difference.
template <int PB>
__device__ __forceinline__ void nv_qk_passes(const v8i &av, const v8i &b1, const v8i &b2, v4f &acc1, v4f &acc2,
                                             v4f &acc1n, v4f &acc2n, int w, int e1, int e2) {
  acc1 = mfma4<0, PB>(av, b1, acc1, w, e1);
  acc2 = mfma4<0, PB>(av, b2, acc2, w, e2);
  acc1 = mfma4<1, PB>(av, b1, acc1, w, e1);
  acc2 = mfma4<1, PB>(av, b2, acc2, w, e2);
  acc1n = mfma4<2, PB>(av, b1, acc1n, w, e1);
  acc2n = mfma4<2, PB>(av, b2, acc2n, w, e2);
}

// MLA partials.  Grid: one-dimensional; ids with equal residue mod 8 run on one XCD, and the
// head-group quads of one share take ids share % 8 + 8 (quad + quads (share / 8)), so they read
// the same latent tiles through one L2.  Any placement gives the same result.
// Iteration j of a segment: score waves on tile j, value waves on tile j - 1, direct loads of
// tile j + 1; latent tiles and scales are triple-buffered, rope double-buffered, the handoff
// double-buffered.  The page ids of up to CAP tiles of the segment sit in LDS; a longer segment
// re-stages them every CAP tiles.
template <int FMT, int P>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void mla_partials(DecodeArgs a) {
  constexpr int D = kMlaD, R = kMlaR, HG = kMlaHeads;
  constexpr bool NV = FMT == kFmtNV;
  constexpr int NPT = P >= 128 ? 1 : 128 / P;
  constexpr int CAP = kMaxSplitPages / NPT;
  constexpr int LAT = 128 * 256, ROPE = 128 * 128;
  constexpr int SCL = NV ? 8 * 32 : 4 * 16;      // scale bytes of one tile
  static_assert(P >= 32 && P % 32 == 0, "page size");
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const bool scorer = wv < 4;                 // wave-uniform role
  const int nhg = a.hq / HG, quads = (nhg + 3) / 4;
  const int rest = (int)(blockIdx.x >> 3);
  const int quad = rest % quads;
  const int share = (rest / quads) * 8 + (int)(blockIdx.x & 7);
  Share sh;
  if (!find_share(a, share, lane, sh)) return;   // the same answer in every wave
  const int hgl = wv & 3, hg = 4 * quad + hgl;
  const bool active = hg < nhg;               // wave-uniform: idle waves still load and sync
  const int h0 = (active ? hg : 0) * HG;

  __shared__ __align__(16) uint8_t lat[3 * LAT];
  __shared__ __align__(16) uint8_t rope[2 * ROPE];
  __shared__ __align__(16) uint8_t scl[3 * SCL];
  __shared__ __align__(16) uint4 hand[2][4][2][64];   // [tile & 1][group][part][lane]
  __shared__ uint32_t lut[256];
  // NVFP4: pass words of a tile's scales [tile & 1][token tile][channel block], written by the
  // value waves one iteration before their P.V reads them
  __shared__ __align__(16) uint32_t pw[NV ? 2 * 8 * 32 : 4];
  __shared__ int pgl[kMaxSplitPages];

  if constexpr (NV) {
    // E4M3 code -> its three signed-digit pass bytes (read after the first barrier)
    if (tid < 256) lut[tid] = e4m3_pass_word(tid);
  }
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  const float gk = NV ? a.gk[0] : 1.0f;
  int nzero = 0;
  const bool count_zero = a.zero_blocks != nullptr && active && scorer;

  // lane (n, q4): n = lane % 16 is the operand row / output column (head h0 + n), q4 the lane group
  for (;;) {   // one segment per sequence the share touches
  // lane indices recomputed from an opaque copy of the thread id: the compiler would otherwise
  // hoist every lane-dependent address out of the segment loop and spill inside it
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wv = tid >> 6;
  const int q4 = lane >> 4, n = lane & 15;
  const int b = sh.b, L = sh.L;
  const long uend = sh.ustart + sh.n;
  const int tb = (int)(sh.x - sh.ustart);
  const int te = (int)((sh.x1 < uend ? sh.x1 : uend) - sh.ustart);
  const int nt = te - tb;
  const int last_lp = min((L - 1) / P, a.max_pages - 1);
  const long slot = share + b;                // partial slot of (share, sequence)

  // page ids of tiles j0 .. j0 + CAP - 1 of the segment (j0 a multiple of CAP): entry
  // (j % CAP) * NPT + k is logical page (tb + j) * 128 / P + k, clamped to the sequence
  auto stage_ids = [&](int j0) {
    const int cnt = min(CAP, nt - j0) * NPT;
    for (int e = tid; e < cnt; e += 512)
      pgl[e] = phys_page(a, b, ((tb + j0 + e / NPT) * 128) / P + e % NPT, last_lp);
  };
  // stage relative tile j: 32 latent, 16 rope and the scale loads, issued by the value waves
  // (the score waves carry the longer dependency chain per tile).  Value wave vw loads tile
  // rows 32 vw .. 32 vw + 31, which lie in one page (P is a multiple of 32): one page lookup and
  // a wave-uniform base per tile.  Latent load m: lane (c, q) = (lane % 16, lane / 16) takes
  // 16-byte chunk c ^ swz_lat(r) of row r = 32 vw + 4 m + q; rope load m: lane (c, q) =
  // (lane % 8, lane / 8) takes chunk c ^ swz_rope(r) of row r = 32 vw + 8 m + q.  Since
  // swz_lat(r) = (4 ((m ^ vw) & 3) + q) and swz_rope(r) = ((q / 2) & 1) + 2 (vw & 3) there, the
  // lanes' byte offsets inside the wave's rows are fixed up to an xor of 64 ((m ^ vw) & 3).
  auto stage_tile = [&](int j) {
    if (wv < 4) return;
    const int vw = __builtin_amdgcn_readfirstlane(wv - 4);
    const int pg = __builtin_amdgcn_readfirstlane(pgl[(j % CAP) * NPT + (NPT == 1 ? 0 : (32 * vw) / P)]);
    const long row0 = (long)pg * P + ((tb + j) * 128 + 32 * vw) % P;
    const uint8_t *lg = a.k_codes + row0 * (D / 2);
    const uint8_t *rg = (const uint8_t *)a.k_rope + row0 * (2 * R);
    uint8_t *Lt = lat + (j % 3) * LAT + 8192 * vw;
    uint8_t *Rt = rope + (j & 1) * ROPE + 4096 * vw;
    const uint32_t lq = lane >> 4, rq = lane >> 3;
    const uint32_t lat_lane = 256 * lq + 16 * ((lane & 15) ^ lq);
    const uint32_t rope_lane = 128 * rq + 16 * ((lane & 7) ^ ((rq >> 1) & 1) ^ (2 * (vw & 3)));
#pragma unroll
    for (int m = 0; m < 8; m++)
      lds_load16_so(lg + 1024 * m, lat_lane ^ (64u * ((m ^ vw) & 3)), Lt + 1024 * m);
#pragma unroll
    for (int m = 0; m < 4; m++)
      lds_load16_so(rg + 1024 * m, rope_lane, Rt + 1024 * m);
    if constexpr (NV) {
      if (vw == 0 && lane < 16) {
        const int tr = lane >> 1;   // token tile (16 tokens): 32 scale bytes
        const int pg = pgl[(j % CAP) * NPT + (NPT == 1 ? 0 : 16 * tr / P)];
        const int off = (((tb + j) * 128 + 16 * tr) % P) / 16;
        lds_load16(a.k_scales + ((long)pg * (P / 16) + off) * 32 + 16 * (lane & 1), scl + (j % 3) * SCL);
      }
    } else {
      if (vw == 0 && lane < 4) {
        const int t = 32 * lane;   // token block (32 tokens): 16 scale bytes
        const int pg = pgl[(j % CAP) * NPT + (NPT == 1 ? 0 : t / P)];
        lds_load16(a.k_scales + ((long)pg * (P / 32) + (((tb + j) * 128 + t) % P) / 32) * 16, scl + (j % 3) * SCL);
      }
    }
  };
  // start of iteration j: the loads of tile j + 1 (re-staging the page ids at a window edge)
  auto next_loads = [&](int j) {
    if (j + 1 < nt) {
      if ((j + 1) % CAP == 0) {   // no wave reads the page ids now: tile j's loads were issued
        stage_ids(j + 1);
        __syncthreads();
      }
      stage_tile(j + 1);
    }
  };

  __syncthreads();   // the previous segment is done with the page ids and the tile buffers
  stage_ids(0);
  __syncthreads();
  stage_tile(0);

  if (scorer) {
    // ---------------- score waves ----------------
    // The prepared query (mla_qprep) in the B-operand layout: lane (n, q4) takes channels
    // 128 st + 32 q4 .. + 31 (st = 0..3) of head h0 + n, both passes, their block scale bytes,
    // the tensor scales and the rope query (K-step s, lane group q4: rope channels 32 s + 8 q4 ..).
    // [pass][K-step][half]: FP4 codes of the lane's 32 channels; NVFP4 keeps one 16-channel
    // half per operand (the other half zero), MXFP4 all 32 in [.][.][0]
    v8i bq[2][4][2];
    int qsb[2][4];           // their E8M0 scale bytes: NVFP4 byte p = half p, MXFP4 byte 0
    float qg[2] = {0.0f, 0.0f};
    bh8 bqr[2];
    if (active) {
      const uint8_t *rec = a.ws_q + ((long)b * a.hq + h0 + n) * kMlaQRecord;
#pragma unroll
      for (int k = 0; k < 2; k++) {
#pragma unroll
        for (int st = 0; st < 4; st++) {
          const uint4 w = *(const uint4 *)(rec + 256 * k + 4 * (16 * st + 4 * q4));
          if constexpr (NV) {
            bq[k][st][0] = v8i{(int)w.x, (int)w.y, 0, 0, 0, 0, 0, 0};
            bq[k][st][1] = v8i{0, 0, (int)w.z, (int)w.w, 0, 0, 0, 0};
            qsb[k][st] = *(const uint16_t *)(rec + 512 + 32 * k + 8 * st + 2 * q4);
          } else {
            bq[k][st][0] = bq[k][st][1] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
            qsb[k][st] = rec[512 + 32 * k + 4 * st + q4];
          }
        }
        qg[k] = *(const float *)(rec + 576 + 4 * k);
      }
#pragma unroll
      for (int st = 0; st < 2; st++) bqr[st] = as_bh8(*(const uint4 *)(rec + 640 + 2 * (32 * st + 8 * q4)));
    } else {
#pragma unroll
      for (int k = 0; k < 2; k++)
#pragma unroll
        for (int st = 0; st < 4; st++) {
          bq[k][st][0] = bq[k][st][1] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
          qsb[k][st] = 0;
        }
      bqr[0] = bqr[1] = as_bh8(uint4{0u, 0u, 0u, 0u});
    }
    // logit coefficients: s = fl32(a1 raw1) + fl32(a2 raw2) + fl32(c_r raw_rope); NVFP4 raw_k is
    // the added minus the subtracted terms' sum (each sum exact in fp32 unless the tile scales of
    // a row span more than the fp32 mantissa, so raw_k is the dot rounded once)
    const float a1 = (qg[0] * gk) * a.coef, a2 = (qg[1] * gk) * a.coef, cr = a.coef_rope;
    float m_run = -INFINITY, l_run = 0.0f, f_run = 1.0f;
    // ablation study, normalized P: the head's max and softmax denominator from a first pass
    float vM = 0.0f, vD = 1.0f;
    if (kAblation && (a.abl & kAblVanillaP) && active) {
      const float *st = a.out + ((long)b * a.hq + h0 + n) * D;
      vM = st[0];
      vD = st[1];
    }
    const float inv6gp = 1.0f / (6.0f * 0.0009765625f);   // fl32(1 / fl32(6 * 2^-10))
    const int trow = 32 * (n >> 2) + (n & 3);   // A-operand row: tile token trow + 4 i in group i
    // Byte offsets inside a tile buffer of the lane's Q.K^T operand chunks.  Row trow + 4 i has
    // latent swizzle (n & 3) + 4 ((i & 3) ^ (n / 4)) and rope swizzle ((n / 2) & 1) + 2 (n / 4),
    // so latent chunk st of group i sits at lo[st ^ (i & 3)] + 1024 i and rope chunk k at
    // ro[k] + 512 i: six per-lane bases, the rest immediate offsets.
    int lo[4], ro[2];
    {
      const int n2 = n >> 2, sr = ((n >> 1) & 1) | (n2 << 1);
#pragma unroll
      for (int v = 0; v < 4; v++) lo[v] = trow * 256 + ((4 * (v ^ n2) + (q4 ^ (n & 3))) << 4);
      ro[0] = trow * 128 + ((q4 ^ sr) << 4);
      ro[1] = trow * 128 + (((4 + q4) ^ sr) << 4);
    }

    wait_lds_loads();
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j <= nt; j++) {
      next_loads(j);
      if (active && j < nt) {
        const uint8_t *Lt = lat + (j % 3) * LAT;
        const uint8_t *Rt = rope + (j & 1) * ROPE;
        const uint8_t *St = scl + (j % 3) * SCL;
        // scales of the lane's rows.  NVFP4: pass words of (token tile 2 (n / 4) + t, channel
        // block 8 st + 2 q4 + p); MXFP4: the E8M0 bytes of 32-token block n / 4
        uint32_t lw[2][4][2];
        uint4 scc = uint4{0u, 0u, 0u, 0u};
        if constexpr (NV) {
#pragma unroll
          for (int t = 0; t < 2; t++)
#pragma unroll
            for (int st = 0; st < 4; st++) {
              const uint32_t pair = *(const uint16_t *)(St + (2 * (n >> 2) + t) * 32 + 8 * st + 2 * q4);
              lw[t][st][0] = lut[pair & 0xFFu];
              lw[t][st][1] = lut[pair >> 8];
            }
        } else {
          scc = *(const uint4 *)(St + 16 * (n >> 2));
        }
        // ---- Q.K^T: 8 token groups of 16; the operands of group i + 1 (four latent chunks,
        // two rope chunks) are read from LDS while group i computes
        float s[8][4];
        uint4 opd[2][6];
        auto read_ops = [&](int i, uint4 *o) {
#pragma unroll
          for (int st = 0; st < 4; st++) o[st] = *(const uint4 *)(Lt + lo[st ^ (i & 3)] + 1024 * i);
          o[4] = *(const uint4 *)(Rt + ro[0] + 512 * i);
          o[5] = *(const uint4 *)(Rt + ro[1] + 512 * i);
        };
        read_ops(0, opd[0]);
#pragma unroll
        for (int i = 0; i < 8; i++) {
          if (i < 7) read_ops(i + 1, opd[(i + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          const uint4 *o = opd[i & 1];
          v4f acc1 = zero, acc2 = zero, acc1n = zero, acc2n = zero, accr = zero;
#pragma unroll
          for (int st = 0; st < 4; st++) {
            if constexpr (NV) {
              const v8i av = {(int)o[st].x, (int)o[st].y, (int)o[st].z, (int)o[st].w, 0, 0, 0, 0};
              const int w0 = (int)lw[i >> 2][st][0], w1 = (int)lw[i >> 2][st][1];
              nv_qk_passes<0>(av, bq[0][st][0], bq[1][st][0], acc1, acc2, acc1n, acc2n, w0, qsb[0][st], qsb[1][st]);
              nv_qk_passes<1>(av, bq[0][st][1], bq[1][st][1], acc1, acc2, acc1n, acc2n, w1, qsb[0][st], qsb[1][st]);
            } else {
              const v8i av = {(int)o[st].x, (int)o[st].y, (int)o[st].z, (int)o[st].w, 0, 0, 0, 0};
              const int sa = (int)byte_of(scc, 4 * st + q4);
              acc1 = mfma4<0, 0>(av, bq[0][st][0], acc1, sa, qsb[0][st]);
              acc2 = mfma4<0, 0>(av, bq[1][st][0], acc2, sa, qsb[1][st]);
            }
          }
          accr = mfma_bf16(as_bh8(o[4]), bqr[0], accr);
          accr = mfma_bf16(as_bh8(o[5]), bqr[1], accr);
#pragma unroll
          for (int rr = 0; rr < 4; rr++) {
            const float raw1 = NV ? acc1[rr] - acc1n[rr] : acc1[rr];
            const float raw2 = NV ? acc2[rr] - acc2n[rr] : acc2[rr];
            const float t12 = a1 * raw1 + a2 * raw2;
            s[i][rr] = t12 + cr * accr[rr];
          }
        }
        // ---- transposed softmax (lane (n, q4) holds tokens 32 q4 .. + 31 of head n)
        const int tok0 = (tb + j) * 128;
        if (tok0 + 128 > L) {   // the last tile only: a branch, not selects on every tile
          asm volatile("" ::: "memory");
#pragma unroll
          for (int i = 0; i < 8; i++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++)
              if (tok0 + 32 * q4 + 4 * i + rr >= L) s[i][rr] = -INFINITY;
        }
        if (kAblation && (a.abl & kAblVanillaP)) {
          // ablation study only: p = 2^(s - M) / den over the whole row (M, den of the head from
          // a first pass), quantized with tensor scale 1 -- NVFP4 default E4M3 scale per 16
          // tokens (its pass word goes to the value waves), MXFP4 E8M0 per 32; no rescale, the
          // partials are summed by the merge
          float am0 = 0.0f, am1 = 0.0f;
#pragma unroll
          for (int i = 0; i < 8; i++)
#pragma unroll
            for (int rr = 0; rr < 4; rr++) {
              const float p = s[i][rr] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(s[i][rr] - vM) / vD;
              s[i][rr] = p;
              if (i < 4) am0 = fmaxf(am0, p);
              else am1 = fmaxf(am1, p);
            }
          uint32_t pk[4], w0 = 0u, w1 = 0u;
          if constexpr (NV) {
            const float am[2] = {am0, am1};
            uint32_t pwd[2];
#pragma unroll
            for (int pb = 0; pb < 2; pb++) {
              const uint32_t c = e4m3_enc_sat(am[pb] / 6.0f);
              const float S = e4m3_dec(c);
              const float r = S != 0.0f ? 1.0f / S : 0.0f;
              float t[4][4];
#pragma unroll
              for (int jj = 0; jj < 4; jj++)
#pragma unroll
                for (int rr = 0; rr < 4; rr++) t[jj][rr] = s[4 * pb + jj][rr] * r;
              pk[2 * pb] = pack8(t[0], t[1], 1.0f);
              pk[2 * pb + 1] = pack8(t[2], t[3], 1.0f);
              pwd[pb] = lut[c];
            }
            if (count_zero) {
#pragma unroll
              for (int pb = 0; pb < 2; pb++)
                if (tok0 + 32 * q4 + 16 * pb < L && ((pk[2 * pb] | pk[2 * pb + 1]) & 0x77777777u) == 0u) nzero++;
            }
            w0 = pwd[0];
            w1 = pwd[1];
          } else {
            const int pe = mx_exp(fmaxf(am0, am1));
            const float ps = ldexpf(1.0f, pe);
#pragma unroll
            for (int w = 0; w < 4; w++) pk[w] = pack8(s[2 * w], s[2 * w + 1], ps);
            if (count_zero && tok0 + 32 * q4 < L && ((pk[0] | pk[1] | pk[2] | pk[3]) & 0x77777777u) == 0u) nzero++;
            w0 = (uint32_t)(pe + 127) | ((uint32_t)(pe + 127) << 8);
          }
          m_run = 0.0f;                                  // weight 1 in the merge
          l_run = (tb == 0 && q4 == 0) ? 1.0f : 0.0f;    // the sequence's first slot carries den = 1
          hand[j & 1][hgl][0][lane] = uint4{pk[0], pk[1], pk[2], pk[3]};
          hand[j & 1][hgl][1][lane] = uint4{w0, __float_as_uint(1.0f), __float_as_uint(1.0f), w1};
        } else {
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
        // ---- fused probability quantization: NVFP4 with power-of-two block scales over 16
        // tokens and G_P = 2^-10; MXFP4 with the MX rule over the lane's 32 tokens
        uint32_t pk[4];
        int pbyte[2];
        if constexpr (NV) {
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
        } else {
          const int pe = mx_exp(__builtin_amdgcn_exp2f(fmaxf(bm0, bm1) - mt));
          pbyte[0] = pbyte[1] = pe + 127;
          const float ps = ldexpf(1.0f, pe);
#pragma unroll
          for (int w = 0; w < 4; w++) pk[w] = pack8(s[2 * w], s[2 * w + 1], ps);
          if (count_zero && tok0 + 32 * q4 < L && ((pk[0] | pk[1] | pk[2] | pk[3]) & 0x77777777u) == 0u) nzero++;
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
        }   // method P
      }
      wait_lds_loads();
      __syncthreads();
    }
    if (active) {
      const float l_tot = sum_x32(sum_x16(l_run));
      if (q4 == 0) *(float2 *)(a.ws_ml + (slot * a.hq + h0 + n) * 2) = float2{m_run, l_tot};
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
      next_loads(j);
      if constexpr (NV) {
        if (j < nt) {   // tile j's scales arrived before the last barrier
          const int e = 64 * (wv - 4) + lane;   // token tile e / 32, channel block e % 32
          pw[(j & 1) * 256 + e] = lut[scl[(j % 3) * SCL + e]];
        }
      }
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
        const uint8_t *rowa = Lt + ra * 256, *rowb = Lt + rb * 256;
        // P.V: channels 16 cg + n, tokens 32 q4 .. + 31; value operands (and NVFP4 pass words)
        // of channel groups 4 c .. 4 c + 3 are read while chunk c - 1 computes
        v2i vt[2][4][2];
        if constexpr (NV) {
          const v8i p0 = {(int)hp.x, (int)hp.y, 0, 0, 0, 0, 0, 0};
          const v8i p1 = {0, 0, (int)hp.z, (int)hp.w, 0, 0, 0, 0};
          // the subtracted term's passes take P with flipped signs
          const v8i p0n = {(int)(hp.x ^ kFp4SignBits), (int)(hp.y ^ kFp4SignBits), 0, 0, 0, 0, 0, 0};
          const v8i p1n = {0, 0, (int)(hp.z ^ kFp4SignBits), (int)(hp.w ^ kFp4SignBits), 0, 0, 0, 0};
          // pass words of the lane's token tiles 2 q4 (P parity 0) and 2 q4 + 1 (parity 1), four
          // channel groups per 16-byte read
          const uint32_t *pa = pw + (jp & 1) * 256 + (2 * q4) * 32, *pb = pa + 32;
          auto read_vals = [&](int c, v2i (*o)[2], uint4 *l) {
#pragma unroll
            for (int k = 0; k < 4; k++) {
              const int cg = 4 * c + k;
              const int off = 8 * (cg & 1);
              o[k][0] = lds_read_tr4(rowa + (((cg >> 1) ^ swa) << 4) + off);
              o[k][1] = lds_read_tr4(rowb + (((cg >> 1) ^ swb) << 4) + off);
            }
            l[0] = *(const uint4 *)(pa + 4 * c);
            l[1] = *(const uint4 *)(pb + 4 * c);
          };
          uint4 lt[2][2];
          read_vals(0, vt[0], lt[0]);
#pragma unroll
          for (int c = 0; c < 8; c++) {
            if (c < 7) read_vals(c + 1, vt[(c + 1) & 1], lt[(c + 1) & 1]);
#pragma unroll
            for (int k = 0; k < 4; k++) {
              const int cg = 4 * c + k;
              const v2i lo = vt[c & 1][k][0], hi = vt[c & 1][k][1];
              const v8i av = {lo[0], lo[1], hi[0], hi[1], 0, 0, 0, 0};
              const int l0 = (int)lt[c & 1][0][k], l1 = (int)lt[c & 1][1][k];
              if (kAblation && (a.abl & kAblVanillaP)) {   // general E4M3 P block scales
                const v4f g0 = pv_general(av, p0, p0n, o_run[cg], l0, (int)hs.x);
                o_run[cg] = pv_general(av, p1, p1n, g0, l1, (int)hs.w);
                continue;
              }
              v4f acc = mfma4<0, 0>(av, p0, o_run[cg], l0, pb0);
              acc = mfma4<1, 0>(av, p0, acc, l0, pb0);
              acc = mfma4<2, 0>(av, p0n, acc, l0, pb0);
              acc = mfma4<0, 0>(av, p1, acc, l1, pb1);
              acc = mfma4<1, 0>(av, p1, acc, l1, pb1);
              o_run[cg] = mfma4<2, 0>(av, p1n, acc, l1, pb1);
            }
          }
        } else {
          const v8i pv = {(int)hp.x, (int)hp.y, (int)hp.z, (int)hp.w, 0, 0, 0, 0};
          // E8M0 scales of the lane's token block q4: its 16 channel blocks
          const uint4 sv = *(const uint4 *)(St + 16 * q4);
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
              o_run[cg] = mfma4<0, 0>(av, pv, o_run[cg], (int)byte_of(sv, cg >> 1), pb0);
            }
          }
        }
      }
      wait_lds_loads();
      __syncthreads();
    }
    if (active) {
      // split partial (latent output, still rotated); NVFP4 applies the tensor scale here
      const float g = gk * f_run;
      float *dst = a.ws_o + (slot * a.hq + h0 + n) * D + 4 * q4;
#pragma unroll
      for (int cg = 0; cg < 32; cg++)
        *(float4 *)(dst + 16 * cg) = float4{o_run[cg][0] * g, o_run[cg][1] * g, o_run[cg][2] * g, o_run[cg][3] * g};
    }
  }
  // the share holding the sequence's first tile records where its partials are
  if (tb == 0 && quad == 0 && tid == 0) {
    const long last = owner_of(uend - 1, sh.total, sh.waves);
    *(int2 *)(a.ws_meta + 2 * b) = int2{(int)slot, (int)(last - share + 1)};
  }
  if (!next_unit(a, sh, uend)) break;
  }   // segments
  if (count_zero) {
    int z = nzero;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) z += __shfl_xor(z, o);
    if (lane == 0 && z) atomicAdd(a.zero_blocks, z);
  }
}

// Value of lane l ^ M (M = 1, 2, 4, 8): quad permutes and a row rotation by DPP, xor 4 by a
// swizzle inside each 32-lane half.
template <int M>
__device__ __forceinline__ float xlane(float x) {
  const int v = __float_as_int(x);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false));
  if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false));
  if constexpr (M == 4) return __int_as_float(__builtin_amdgcn_ds_swizzle(v, 0x101F));
  return __int_as_float(__builtin_amdgcn_update_dpp(0, v, 0x128, 0xF, 0xF, false));
}
// One Walsh-Hadamard stage across lane bit M of the values x[0..7]: the lane with the bit clear
// keeps lower + upper, the other lower - upper (fma with +-1 rounds exactly like the add or
// subtract).
template <int M>
__device__ __forceinline__ void fwht_lanes(float (&x)[8], int lane) {
  const float sg = (lane & M) ? -1.0f : 1.0f;
#pragma unroll
  for (int j = 0; j < 8; j++) {
    if constexpr (M <= 8) {
      x[j] = fmaf(sg, x[j], xlane<M>(x[j]));
    } else {
      const uint32_t u = __float_as_uint(x[j]);
      const auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                             : __builtin_amdgcn_permlane32_swap(u, u, false, false);
      x[j] = fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
    }
  }
}
// Maximum over lane bit M (M = 1 .. 32).
template <int M>
__device__ __forceinline__ float max_lanes(float x) {
  if constexpr (M <= 8) {
    return fmaxf(x, xlane<M>(x));
  } else {
    const uint32_t u = __float_as_uint(x);
    const auto r = M == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                           : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
}

// Query preparation, once per (sequence, query head) row before the partials: smoothing,
// rotation and the dual-residual FP4 query, written as a kMlaQRecord record.  One wave per row;
// lane i holds latent channels 8 i .. 8 i + 7.  Walsh-Hadamard stages h = 1, 2, 4 stay in the
// lane, h = 8 .. 256 pair lanes i ^ (h / 8) (the oracle's stage order); each butterfly keeps
// (lower + upper, lower - upper).  The quantization takes the same fp32 steps per element as
// the oracle: NVFP4 with power-of-two block scales over 16 channels and G = row max / 1536,
// MXFP4 with E8M0 scales over 32 channels; pass 2 quantizes the residual of pass 1.
template <int FMT>
__global__ __launch_bounds__(256) void mla_qprep(DecodeArgs a) {
  constexpr int D = kMlaD, R = kMlaR;
  constexpr bool NV = FMT == kFmtNV;
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long)a.batch * a.hq) return;
  uint8_t *rec = a.ws_q + row * kMlaQRecord;
  const long q0 = row * (D + R);
  float y[8];
  if (a.q_bf16) {
    const uint4 u = *(const uint4 *)((const uint16_t *)a.q + q0 + 8 * lane);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = bf16_to_f32((uint16_t)(w[j / 2] >> (16 * (j & 1))));
  } else {
    const float4 u0 = *(const float4 *)((const float *)a.q + q0 + 8 * lane);
    const float4 u1 = *(const float4 *)((const float *)a.q + q0 + 8 * lane + 4);
    y[0] = u0.x; y[1] = u0.y; y[2] = u0.z; y[3] = u0.w;
    y[4] = u1.x; y[5] = u1.y; y[6] = u1.z; y[7] = u1.w;
  }
#pragma unroll
  for (int j = 0; j < 8; j++) y[j] = y[j] * a.qs[8 * lane + j];
  if (!(kAblation && (a.abl & kAblNoRotation))) {   // (the ablation build can switch it off)
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int j = 0; j < 8; j++)
      if ((j & h) == 0) {
        const float x0 = y[j], x1 = y[j + h];
        y[j] = x0 + x1;
        y[j + h] = x0 - x1;
      }
  fwht_lanes<1>(y, lane);
  fwht_lanes<2>(y, lane);
  fwht_lanes<4>(y, lane);
  fwht_lanes<8>(y, lane);
  fwht_lanes<16>(y, lane);
  fwht_lanes<32>(y, lane);
  }
#pragma unroll
  for (int k = 0; k < 2; k++) {
    if (kAblation && k == 1 && (a.abl & kAblSingleQ)) {   // single-pass query: the second pass sees zeros
#pragma unroll
      for (int j = 0; j < 8; j++) y[j] = 0.0f;
    }
    float lmax = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; j++) lmax = fmaxf(lmax, fabsf(y[j]));
    uint32_t w = 0u;
    if constexpr (NV) {
      float rmax = max_lanes<1>(lmax);
      rmax = max_lanes<32>(max_lanes<16>(max_lanes<8>(max_lanes<4>(max_lanes<2>(rmax)))));
      const float gq = rmax / 1536.0f;
      const float sixg = 6.0f * gq;
      const float inv6g = sixg != 0.0f ? 1.0f / sixg : 0.0f;
      const float bmax = max_lanes<1>(lmax);   // 16-channel block: lanes 2 i, 2 i + 1
      const bool valid = bmax > 0.0f && gq > 0.0f;
      const int e = ceil_log2_clamp(bmax * inv6g, -9, 8);
      const float S = pow2f(e);
      const float sg = S * gq;
      const float rr = (valid && sg != 0.0f) ? 1.0f / sg : 0.0f;   // invalid: every code 0
      // codes of x * rr by the hardware conversion (nearest even, saturating at 6); the residual
      // takes dec(code) * S from the hardware decode (exact), then * G
      w = cvt_pk<0>(w, y[0] * rr, y[1] * rr, 1.0f);
      w = cvt_pk<1>(w, y[2] * rr, y[3] * rr, 1.0f);
      w = cvt_pk<2>(w, y[4] * rr, y[5] * rr, 1.0f);
      w = cvt_pk<3>(w, y[6] * rr, y[7] * rr, 1.0f);
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const v2f d = dec_pk(w, j / 2, S);
        y[j] = y[j] - d.x * gq;
        y[j + 1] = y[j + 1] - d.y * gq;
      }
      if ((lane & 1) == 0) rec[512 + 32 * k + lane / 2] = (uint8_t)(e + 127);
      if (lane == 0) *(float *)(rec + 576 + 4 * k) = gq;
    } else {
      const float bmax = max_lanes<2>(max_lanes<1>(lmax));   // 32-channel block: lanes 4 i .. 4 i + 3
      const int e = mx_exp(bmax);
      // codes of y 2^-e and the residual y - dec(code) 2^e, the conversions by the hardware
      // with scale 1 (2^e itself can be subnormal: e reaches -127)
      w = cvt_pk<0>(w, ldexpf(y[0], -e), ldexpf(y[1], -e), 1.0f);
      w = cvt_pk<1>(w, ldexpf(y[2], -e), ldexpf(y[3], -e), 1.0f);
      w = cvt_pk<2>(w, ldexpf(y[4], -e), ldexpf(y[5], -e), 1.0f);
      w = cvt_pk<3>(w, ldexpf(y[6], -e), ldexpf(y[7], -e), 1.0f);
#pragma unroll
      for (int j = 0; j < 8; j += 2) {
        const v2f d = dec_pk(w, j / 2, 1.0f);
        y[j] = y[j] - ldexpf(d.x, e);
        y[j + 1] = y[j + 1] - ldexpf(d.y, e);
      }
      if ((lane & 3) == 0) rec[512 + 32 * k + lane / 4] = (uint8_t)(e + 127);
      if (lane == 0) *(float *)(rec + 576 + 4 * k) = 1.0f;
    }
    *(uint32_t *)(rec + 256 * k + 4 * lane) = w;
  }
  // rope query as bf16 (an fp32 query rounded to nearest even)
  if (lane < R / 8) {
    uint16_t hb[8];
    if (a.q_bf16) {
#pragma unroll
      for (int j = 0; j < 8; j++) hb[j] = ((const uint16_t *)a.q)[q0 + D + 8 * lane + j];
    } else {
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const uint32_t u = __float_as_uint(((const float *)a.q)[q0 + D + 8 * lane + j]);
        hb[j] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
      }
    }
    uint4 v;
    __builtin_memcpy(&v, hb, 16);
    *(uint4 *)(rec + 640 + 16 * lane) = v;
  }
}

// Merge of one (sequence, query head) row over the sequence's partials:
// out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, then un-rotated (Walsh-Hadamard over
// the 512 channels, / 512) and un-smoothed (* q_smooth).  Lane l holds channels 8 l .. 8 l + 7.
constexpr int kMlaMergeFast = 8;   // partials per row that the merge loads all at once

__global__ __launch_bounds__(64) void mla_merge(DecodeArgs a) {
  constexpr int D = kMlaD;
  const int row = blockIdx.x, lane = threadIdx.x;
  const int b = row / a.hq, h = row % a.hq;
  float4 *dst = (float4 *)(a.out + (long)row * D + 8 * lane);
  // the sequence's slot range is read together with its length (a sequence without tiles has
  // no range: its meta words are not written and are not used)
  const int2 meta = *(const int2 *)(a.ws_meta + 2 * b);
  if (seq_tiles(a, b) == 0) {
    dst[0] = float4{0.f, 0.f, 0.f, 0.f};
    dst[1] = float4{0.f, 0.f, 0.f, 0.f};
    return;
  }
  const int nv = meta.y;
  const long r0 = (long)meta.x * a.hq + h;     // first partial row; one slot holds hq rows
  const float *ml = a.ws_ml + r0 * 2;
  const float *o = a.ws_o + r0 * D + 8 * lane;
  const long so = (long)a.hq * D, sm = 2L * a.hq;   // strides between the row's partials
  if (kAblation && (a.abl & kAblRowStats)) {
    // ablation study, first pass of normalized P: the row's max and softmax denominator
    float M = -INFINITY;
    for (int s = lane; s < nv; s += 64) M = fmaxf(M, ml[sm * s]);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k));
    float dn = 0.f;
    if (M > -INFINITY)
      for (int s = lane; s < nv; s += 64) dn = fmaf(__builtin_amdgcn_exp2f(ml[sm * s] - M), ml[sm * s + 1], dn);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) dn += __shfl_xor(dn, k);
    if (lane == 0) *(float2 *)(a.out + (long)row * D) = float2{M, dn};
    return;
  }
  float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (nv <= kMlaMergeFast) {
    // every partial of the row in flight at once; the same operations in the same order as
    // the general path below
    const float2 mlv = lane < nv ? *(const float2 *)(ml + sm * lane) : float2{-INFINITY, 0.f};
    float4 u[kMlaMergeFast][2];
#pragma unroll
    for (int s = 0; s < kMlaMergeFast; s++) {
      u[s][0] = s < nv ? *(const float4 *)(o + so * s) : float4{0.f, 0.f, 0.f, 0.f};
      u[s][1] = s < nv ? *(const float4 *)(o + so * s + 4) : float4{0.f, 0.f, 0.f, 0.f};
    }
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
    for (int s = lane; s < nv; s += 64) M = fmaxf(M, ml[sm * s]);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) M = fmaxf(M, __shfl_xor(M, k));
    for (int s = lane; s < nv; s += 64) den = fmaf(__builtin_amdgcn_exp2f(ml[sm * s] - M), ml[sm * s + 1], den);
#pragma unroll
    for (int k = 32; k >= 1; k >>= 1) den += __shfl_xor(den, k);
    for (int s = 0; s < nv; s++) {
      const float w = __builtin_amdgcn_exp2f(ml[sm * s] - M);
      const float4 u0 = *(const float4 *)(o + so * s), u1 = *(const float4 *)(o + so * s + 4);
      y[0] = fmaf(w, u0.x, y[0]); y[1] = fmaf(w, u0.y, y[1]); y[2] = fmaf(w, u0.z, y[2]); y[3] = fmaf(w, u0.w, y[3]);
      y[4] = fmaf(w, u1.x, y[4]); y[5] = fmaf(w, u1.y, y[5]); y[6] = fmaf(w, u1.z, y[6]); y[7] = fmaf(w, u1.w, y[7]);
    }
  }
  const float inv = 1.0f / den;
#pragma unroll
  for (int j = 0; j < 8; j++) y[j] *= inv;
  const float *qs = a.qs + 8 * lane;
  if (kAblation && (a.abl & kAblNoRotation)) {   // ablation study: the latent was not rotated
#pragma unroll
    for (int j = 0; j < 8; j++) y[j] = y[j] * qs[j];
  } else {
  // Walsh-Hadamard over 512 channels: stages 1, 2, 4 in the lane, 8 .. 256 across lanes
#pragma unroll
  for (int hh = 1; hh < 8; hh <<= 1)
#pragma unroll
    for (int j = 0; j < 8; j++)
      if ((j & hh) == 0) {
        const float x0 = y[j], x1 = y[j + hh];
        y[j] = x0 + x1;
        y[j + hh] = x0 - x1;
      }
  fwht_lanes<1>(y, lane);
  fwht_lanes<2>(y, lane);
  fwht_lanes<4>(y, lane);
  fwht_lanes<8>(y, lane);
  fwht_lanes<16>(y, lane);
  fwht_lanes<32>(y, lane);
#pragma unroll
  for (int j = 0; j < 8; j++) y[j] = y[j] * (1.0f / 512.0f) * qs[j];
  }
  dst[0] = float4{y[0], y[1], y[2], y[3]};
  dst[1] = float4{y[4], y[5], y[6], y[7]};
}

template <int FMT>
static hipError_t launch_mla_fmt(const DecodeArgs &a, unsigned grid, hipStream_t s) {
  switch (a.page_size) {
    case 32: mla_partials<FMT, 32><<<grid, 512, 0, s>>>(a); break;
    case 64: mla_partials<FMT, 64><<<grid, 512, 0, s>>>(a); break;
    case 128: mla_partials<FMT, 128><<<grid, 512, 0, s>>>(a); break;
    case 256: mla_partials<FMT, 256><<<grid, 512, 0, s>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// The query preparation (one wave per row), then the partials.  Grid: the planned shares rounded
// up to a multiple of 8 (one per XCD residue), times the head-group quads; shares past the
// device-side count return at once.
hipError_t launch_mla_partials(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const unsigned qgrid = (unsigned)(((long)a.batch * a.hq + 3) / 4);
  if (a.fmt == kFmtMX)
    mla_qprep<kFmtMX><<<qgrid, 256, 0, s>>>(a);
  else
    mla_qprep<kFmtNV><<<qgrid, 256, 0, s>>>(a);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  const int nhg = a.hq / kMlaHeads;
  const unsigned grid = (unsigned)(((a.n_waves + 7) / 8) * 8 * ((nhg + 3) / 4));
  return a.fmt == kFmtMX ? launch_mla_fmt<kFmtMX>(a, grid, s) : launch_mla_fmt<kFmtNV>(a, grid, s);
}

hipError_t launch_mla_merge(const DecodeArgs &a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  mla_merge<<<(unsigned)(a.batch * a.hq), 64, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace fp4kv
