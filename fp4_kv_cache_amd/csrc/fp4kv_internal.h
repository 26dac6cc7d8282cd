// Internal host-side interface between the C ABI (fp4kv_api.cpp) and the kernel
// translation units.  Not installed; not part of the ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/fp4kv.h"

namespace fp4kv {

// Page-id entries one decode workgroup stages in LDS: a split (GQA: a wave's share of one
// sequence) covers at most kMaxSplitPages / max(1, 128 / page_size) tiles of 128 tokens.
constexpr int kMaxSplitPages = 512;

struct AppendArgs {
  int fmt, attn, page_size, hkv, d, rope_dim, num_pages, max_seqs, num_tokens, bf16;
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
  int n_split, tiles_per_split;   // MLA: splits per (sequence, head group) and their tiles
  int n_waves;                    // GQA: waves of the balanced partition (an upper bound)
  float softmax_scale;
  float coef;            // fl32(softmax_scale * fl32(log2(e) / head_dim))
  float coef_rope;       // fl32(softmax_scale * fl32(log2(e)))
  const uint8_t *k_codes, *k_scales, *v_codes, *v_scales;
  const uint16_t *k_rope;
  const float *gk, *gv, *qs;
  const void *q;
  const int32_t *block_table, *seq_lens;
  float *ws_o;           // MLA: [batch * hq][n_split][d]; GQA: [n_waves + batch * hkv][group][d]
  float *ws_ml;          // same rows, [2] each
  int32_t *ws_meta;      // GQA: [batch * hkv][2] = first partial slot of the unit, partial count
  float *out;            // [batch * hq][d]
  int32_t *zero_blocks;  // nullable
};

hipError_t launch_append(const AppendArgs &a, hipStream_t s);
hipError_t launch_decode_partials(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_merge(const DecodeArgs &a, hipStream_t s);
hipError_t launch_mla_partials(const DecodeArgs &a, hipStream_t s);
hipError_t launch_mla_merge(const DecodeArgs &a, hipStream_t s);
hipError_t launch_cache_read(const DecodeArgs &a, uint32_t *sink, hipStream_t s);
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t s);
hipError_t launch_stream_copy(const void *src, void *dst, size_t bytes, hipStream_t s);

}  // namespace fp4kv
