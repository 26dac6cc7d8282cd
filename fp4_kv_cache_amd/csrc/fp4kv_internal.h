// Internal host-side interface between the C ABI (fp4kv_api.cpp) and the kernel
// translation units.  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp4kv.h"

namespace fp4kv {

// Page-id entries a decode workgroup holds in LDS at once: the ids of kMaxSplitPages /
// max(1, 128 / page_size) consecutive tiles of its segment, re-staged at every window edge.
constexpr int kMaxSplitPages = 512;

// Technique switches of the ablation-study build of the library (sources compiled with
// -DFP4KV_ABLATION; the product build compiles every switch out).  GQA and MLA.
constexpr int kAblSingleQ = 1;      // no dual residual: the query's second FP4 pass is zero
constexpr int kAblNoRotation = 2;   // no Hadamard rotation of keys and queries
constexpr int kAblNoSearch = 4;     // every key block keeps its default scale
constexpr int kAblVanillaP = 8;     // no underflow-aware P: P normalized over the whole row, NVFP4
                                    // with tensor scale 1 and default E4M3 block scales (MXFP4:
                                    // E8M0), from the row's max and denominator of a first pass
constexpr int kAblRowStats = 16;    // internal: that first pass's merge writes the row's (max,
                                    // denominator) into out[row][0..1] instead of the output
#ifdef FP4KV_ABLATION
constexpr bool kAblation = true;
#else
constexpr bool kAblation = false;
#endif

struct AppendArgs {
  int fmt, attn, page_size, hkv, d, rope_dim, num_pages, max_seqs, num_tokens, bf16;
  int abl;               // ablation switches (0 in the product build)
  uint8_t *k_codes, *k_scales, *v_codes, *v_scales;
  float *stage;
  uint16_t *k_rope;
  const float *gk, *gv, *ksi;
  const void *k_new, *v_new, *k_rope_new;
  const int32_t *slots, *seq_ids, *positions;
};

struct DecodeArgs {
  int fmt, page_size, hkv, group, hq, d, rope_dim, batch, max_pages, num_pages, q_bf16;
  int q_len;             // GQA: query tokens per sequence (causal), 1 for ordinary decode
  int abl;               // ablation switches (0 in the product build)
  int n_waves;           // shares of the balanced partition (an upper bound; GQA one wave each,
                         // MLA one workgroup per group of 64 query heads each)
  float softmax_scale;
  float coef;            // fl32(softmax_scale * fl32(log2(e) / head_dim))
  float coef_rope;       // fl32(softmax_scale * fl32(log2(e)))
  const uint8_t *k_codes, *k_scales, *v_codes, *v_scales;
  const uint16_t *k_rope;
  const float *gk, *gv, *qs;
  const void *q;
  const int32_t *block_table, *seq_lens;
  float *ws_o;           // partial slots [n_waves + units][rows][d]: GQA units = batch * hkv,
                         // rows = group * q_len; MLA units = batch, rows = hq
  float *ws_ml;          // same rows, [2] each
  int32_t *ws_meta;      // [units][2] = first partial slot of the unit, partial count
  uint8_t *ws_q;         // MLA: the prepared query, kMlaQRecord bytes per (sequence, head)
  float *out;            // [batch * hq][d]
  int32_t *zero_blocks;  // nullable
};

hipError_t launch_append(const AppendArgs &a, hipStream_t s);
hipError_t launch_decode_partials(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_merge(const DecodeArgs &a, hipStream_t s);
// MLA prepared query record of one (sequence, query head): the dual-residual FP4 codes of the
// rotated, smoothed latent query (pass k, channels 8 i .. 8 i + 7 in dword k * 64 + i), their
// block scale bytes (pass k at byte 512 + 32 k: NVFP4 per 16 channels, MXFP4 per 32), the two
// tensor scales (float at 576 and 580) and the rope query as bf16 (at 640).
constexpr int kMlaQRecord = 768;
hipError_t launch_mla_partials(const DecodeArgs &a, hipStream_t s);
hipError_t launch_mla_merge(const DecodeArgs &a, hipStream_t s);
hipError_t launch_bf16_partials(const DecodeArgs &a, hipStream_t s);
hipError_t launch_bf16_append(const AppendArgs &a, hipStream_t s);
hipError_t launch_cache_read(const DecodeArgs &a, uint32_t *sink, hipStream_t s);
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_pack_e2m1(const float *x, size_t n, int scale_exp, uint8_t *out, hipStream_t s);
hipError_t launch_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t s);

}  // namespace fp4kv
