// C ABI of libfp4kv.so (declarations and contracts in include/fp4kv.h).
// Host code only: argument validation with host scalars, split-K planning and
// kernel launches on the caller's stream.  Nothing here allocates or syncs.
#include <stddef.h>
#include <stdint.h>

#include "fp4kv_internal.h"

using namespace fp4kv;

namespace {

constexpr int kTarget = 2048;   // GQA waves: 8 single-wave groups per CU on 256 CUs
constexpr int kTargetMla = 1024;  // MLA: one wave per SIMD
constexpr int kMinTilesPerSplit = 4;   // the partial kernels' minimum share (kMinTilesPerWave)
constexpr int kTile = 128;

int block_of(int fmt) { return fmt == FP4KV_NVFP4 ? 16 : 32; }

bool pow2_page(int p) { return p == 16 || p == 32 || p == 64 || p == 128 || p == 256; }

// Scalar checks of a cache descriptor (no pointer dereference beyond `c`).
int check_shape(const fp4kv_cache *c) {
  if (!c) return FP4KV_ERR_INVALID_ARG;
  if (c->format != FP4KV_NVFP4 && c->format != FP4KV_MXFP4) return FP4KV_ERR_INVALID_ARG;
  if (c->attn != FP4KV_GQA && c->attn != FP4KV_MLA) return FP4KV_ERR_INVALID_ARG;
  if (c->num_pages <= 0 || c->num_kv_heads <= 0 || c->max_seqs <= 0) return FP4KV_ERR_INVALID_ARG;
  if (c->page_size <= 0 || c->page_size % block_of(c->format) != 0 || c->page_size > 256)
    return FP4KV_ERR_INVALID_ARG;
  if (!pow2_page(c->page_size)) return FP4KV_ERR_UNSUPPORTED;
  if ((long)c->num_pages * c->page_size > 0x7FFFFFFFL) return FP4KV_ERR_INVALID_ARG;
  if (c->attn == FP4KV_GQA) {
    if (c->rope_dim != 0) return FP4KV_ERR_INVALID_ARG;
    if (c->head_dim != 128) return c->head_dim > 0 ? FP4KV_ERR_UNSUPPORTED : FP4KV_ERR_INVALID_ARG;
  } else {
    if (c->num_kv_heads != 1) return FP4KV_ERR_INVALID_ARG;
    if (c->head_dim != 512 || c->rope_dim != 64) return FP4KV_ERR_UNSUPPORTED;
  }
  return FP4KV_OK;
}

int check_pointers(const fp4kv_cache *c) {
  if (!c->k_codes || !c->k_scales || !c->stage || !c->k_smooth_inv || !c->q_smooth)
    return FP4KV_ERR_INVALID_ARG;
  if (c->format == FP4KV_NVFP4 && !c->k_tensor_scale) return FP4KV_ERR_INVALID_ARG;
  if (c->attn == FP4KV_GQA) {
    if (!c->v_codes || !c->v_scales) return FP4KV_ERR_INVALID_ARG;
    if (c->format == FP4KV_NVFP4 && !c->v_tensor_scale) return FP4KV_ERR_INVALID_ARG;
  } else if (!c->k_rope) {
    return FP4KV_ERR_INVALID_ARG;
  }
  return FP4KV_OK;
}

struct SplitPlan {
  int n_split, tiles_per_split;
};

// units: waves per split (GQA: batch * Hkv; MLA: batch * query-head groups of 16);
// target: waves to aim for (GQA: 8 single-wave groups per CU; MLA: one wave per SIMD)
SplitPlan plan_splits(long units, int max_len, int page_size, long target) {
  int max_tiles = (max_len + kTile - 1) / kTile;
  if (max_tiles < 1) max_tiles = 1;
  if (units < 1) units = 1;
  long ns = (target + units - 1) / units;
  if (ns > max_tiles) ns = max_tiles;
  if (ns < 1) ns = 1;
  int tps = (int)((max_tiles + ns - 1) / ns);
  if (tps < kMinTilesPerSplit) tps = kMinTilesPerSplit < max_tiles ? kMinTilesPerSplit : max_tiles;
  // a split's page ids are staged in LDS by the decode kernel
  const int pages_per_tile = page_size >= kTile ? 1 : kTile / page_size;
  if (tps * pages_per_tile > kMaxSplitPages) tps = kMaxSplitPages / pages_per_tile;
  SplitPlan p;
  p.tiles_per_split = tps;
  p.n_split = (max_tiles + tps - 1) / tps;
  return p;
}

// GQA: waves of the balanced partition.  Each wave takes an equal share of all tiles of
// the batch (computed on the device from seq_lens); at most kTarget waves, but enough that
// no share exceeds the page ids a wave stages in LDS, and no more than shares of
// kMinTilesPerSplit tiles of the largest possible batch.
long plan_waves(long units, int max_len, int page_size) {
  long max_tiles = (max_len + kTile - 1) / kTile;
  if (max_tiles < 1) max_tiles = 1;
  if (units < 1) units = 1;
  const long pages_per_tile = page_size >= kTile ? 1 : kTile / page_size;
  const long max_share = kMaxSplitPages / pages_per_tile;
  const long all = units * max_tiles;
  long w = kTarget;
  const long lds_min = (all + max_share - 1) / max_share;
  if (w < lds_min) w = lds_min;
  const long useful = (all + kMinTilesPerSplit - 1) / kMinTilesPerSplit;
  if (w > useful) w = useful;
  return w < 1 ? 1 : w;
}

SplitPlan plan_for(const fp4kv_cache *c, int batch, int hq, int max_len) {
  const long b = batch > 0 ? batch : 1;
  if (c->attn == FP4KV_MLA) return plan_splits(b * (hq / 16 > 0 ? hq / 16 : 1), max_len, c->page_size, kTargetMla);
  SplitPlan p;
  const long w = plan_waves(b * c->num_kv_heads, max_len, c->page_size);
  p.n_split = w > 0x3FFFFFFFL ? -1 : (int)w;   // -1: batch too large for one launch
  p.tiles_per_split = 0;
  return p;
}

// Workspace: MLA [batch * hq][n_split] partial rows; GQA (n_waves + batch * Hkv) slots of
// `group` partial rows, then the per-unit slot ranges.  A partial row is d + 2 floats.
size_t workspace_for(const fp4kv_cache *c, int batch, int hq, int max_len, SplitPlan *out, int q_len = 1) {
  SplitPlan p = plan_for(c, batch, hq, max_len);
  if (out) *out = p;
  if (p.n_split < 0) return 0;
  if (c->attn == FP4KV_MLA) {
    size_t rows = (size_t)batch * hq * p.n_split;
    return rows * ((size_t)c->head_dim + 2) * sizeof(float);
  }
  const size_t units = (size_t)batch * c->num_kv_heads;
  const size_t rows = ((size_t)p.n_split + units) * (size_t)(hq / c->num_kv_heads) * (size_t)q_len;
  return rows * ((size_t)c->head_dim + 2) * sizeof(float) + units * 2 * sizeof(int32_t);
}

int to_status(hipError_t e) { return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP; }

int fill_decode(const fp4kv_cache *c, const void *q, int q_dtype, int batch, int hq,
                const int32_t *block_table, int max_pages, const int32_t *seq_lens,
                float softmax_scale, float *out, void *ws, size_t ws_bytes, int32_t *zero,
                bool need_q, bool need_out, DecodeArgs *a, int q_len = 1) {
  int st = check_shape(c);
  if (st) return st;
  st = check_pointers(c);
  if (st) return st;
  if (batch < 0 || hq <= 0 || max_pages <= 0) return FP4KV_ERR_INVALID_ARG;
  if (q_dtype != FP4KV_F32 && q_dtype != FP4KV_BF16) return FP4KV_ERR_INVALID_ARG;
  if (hq % c->num_kv_heads != 0) return FP4KV_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale)) return FP4KV_ERR_INVALID_ARG;
  int group = hq / c->num_kv_heads;
  if (q_len < 1) return FP4KV_ERR_INVALID_ARG;
  if (c->attn == FP4KV_GQA) {
    bool ok = group == 1 || group == 2 || group == 4 || (c->format == FP4KV_MXFP4 && group == 8);
    if (!ok) return FP4KV_ERR_UNSUPPORTED;
    // query tokens x query heads per KV head: up to two row sets of one MFMA's columns
    if (q_len > 8 || group * q_len > (c->format == FP4KV_NVFP4 ? 8 : 16)) return FP4KV_ERR_UNSUPPORTED;
    if (c->format == FP4KV_MXFP4 && c->page_size < 32) return FP4KV_ERR_UNSUPPORTED;
  } else {
    // MLA: query heads in groups of 16, pages of at least 32 tokens
    if (hq % 16 != 0 || c->page_size < 32 || q_len != 1) return FP4KV_ERR_UNSUPPORTED;
  }
  if ((long)max_pages * c->page_size > 0x7FFFFFFFL) return FP4KV_ERR_INVALID_ARG;
  if (batch > 0) {
    if (!block_table || !seq_lens || !ws) return FP4KV_ERR_INVALID_ARG;
    if (need_q && !q) return FP4KV_ERR_INVALID_ARG;
    if (need_out && !out) return FP4KV_ERR_INVALID_ARG;
  }
  // partial slots are numbered in int32 (GQA: n_waves + batch * Hkv)
  if ((long)batch * c->num_kv_heads > 0x3FFFFFFFL) return FP4KV_ERR_INVALID_ARG;
  SplitPlan p;
  size_t need = workspace_for(c, batch, hq, max_pages * c->page_size, &p, q_len);
  if (p.n_split < 0) return FP4KV_ERR_INVALID_ARG;
  if (ws_bytes < need) return FP4KV_ERR_WORKSPACE;
  DecodeArgs &d = *a;
  d.fmt = c->format;
  d.page_size = c->page_size;
  d.hkv = c->num_kv_heads;
  d.group = group;
  d.hq = hq;
  d.d = c->head_dim;
  d.rope_dim = c->rope_dim;
  d.batch = batch;
  d.max_pages = max_pages;
  d.num_pages = c->num_pages;
  d.q_bf16 = q_dtype == FP4KV_BF16;
  d.q_len = q_len;
  const bool mla = c->attn == FP4KV_MLA;
  d.n_split = mla ? p.n_split : 0;
  d.tiles_per_split = mla ? p.tiles_per_split : 0;
  d.n_waves = mla ? 0 : p.n_split;
  d.softmax_scale = softmax_scale;
  const float l2d = (float)(1.4426950408889634 / (double)c->head_dim);
  const float l2 = (float)1.4426950408889634;
  d.coef = softmax_scale * l2d;
  d.coef_rope = softmax_scale * l2;
  d.k_codes = c->k_codes;
  d.k_scales = c->k_scales;
  d.v_codes = c->v_codes;
  d.v_scales = c->v_scales;
  d.k_rope = c->k_rope;
  d.gk = c->k_tensor_scale;
  d.gv = c->v_tensor_scale;
  d.qs = c->q_smooth;
  d.q = q;
  d.block_table = block_table;
  d.seq_lens = seq_lens;
  const size_t rows = mla ? (size_t)batch * hq * p.n_split
                         : ((size_t)p.n_split + (size_t)batch * c->num_kv_heads) * (size_t)group * q_len;
  d.ws_o = (float *)ws;
  d.ws_ml = (float *)ws + rows * (size_t)c->head_dim;
  d.ws_meta = mla ? nullptr : (int32_t *)(d.ws_ml + rows * 2);
  d.out = out;
  d.zero_blocks = zero;
  return FP4KV_OK;
}

}  // namespace

extern "C" {

const char *fp4kv_status_string(int s) {
  switch (s) {
    case FP4KV_OK: return "ok";
    case FP4KV_ERR_INVALID_ARG: return "invalid argument";
    case FP4KV_ERR_UNSUPPORTED: return "unsupported configuration";
    case FP4KV_ERR_WORKSPACE: return "workspace too small";
    case FP4KV_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int fp4kv_cache_layout(const fp4kv_cache *c, size_t bytes_out[6]) {
  if (!bytes_out) return FP4KV_ERR_INVALID_ARG;
  int st = check_shape(c);
  if (st) return st;
  const size_t P = (size_t)c->page_size, d = (size_t)c->head_dim, h = (size_t)c->num_kv_heads;
  const size_t B = (size_t)block_of(c->format), np = (size_t)c->num_pages;
  bytes_out[0] = np * h * P * (d / 2);
  if (c->attn == FP4KV_GQA) {
    bytes_out[1] = np * h * P * (d / B);
    bytes_out[2] = np * h * d * (P / 2);
    bytes_out[3] = np * h * d * (P / B);
    bytes_out[5] = 0;
  } else {
    bytes_out[1] = np * (P / B) * (d / B);
    bytes_out[2] = 0;
    bytes_out[3] = 0;
    bytes_out[5] = np * P * (size_t)c->rope_dim * 2;
  }
  bytes_out[4] = (size_t)c->max_seqs * h * B * d * sizeof(float);
  return FP4KV_OK;
}

int kv_quant_append(const fp4kv_cache *c, const void *k_new, const void *v_new, int dtype,
                    int num_tokens, const int32_t *slot_mapping, const int32_t *seq_ids,
                    const int32_t *positions, const void *k_rope_new, void *stream) {
  int st = check_shape(c);
  if (st) return st;
  st = check_pointers(c);
  if (st) return st;
  if (dtype != FP4KV_F32 && dtype != FP4KV_BF16) return FP4KV_ERR_INVALID_ARG;
  if (num_tokens < 0) return FP4KV_ERR_INVALID_ARG;
  if (num_tokens == 0) return FP4KV_OK;
  if (!k_new || !slot_mapping || !seq_ids || !positions) return FP4KV_ERR_INVALID_ARG;
  if (c->attn == FP4KV_GQA && !v_new) return FP4KV_ERR_INVALID_ARG;
  if (c->attn == FP4KV_MLA && !k_rope_new) return FP4KV_ERR_INVALID_ARG;
  AppendArgs a;
  a.fmt = c->format;
  a.attn = c->attn;
  a.page_size = c->page_size;
  a.hkv = c->num_kv_heads;
  a.d = c->head_dim;
  a.rope_dim = c->rope_dim;
  a.num_pages = c->num_pages;
  a.max_seqs = c->max_seqs;
  a.num_tokens = num_tokens;
  a.bf16 = dtype == FP4KV_BF16;
  a.k_codes = c->k_codes;
  a.k_scales = c->k_scales;
  a.v_codes = c->v_codes;
  a.v_scales = c->v_scales;
  a.stage = c->stage;
  a.k_rope = c->k_rope;
  a.gk = c->k_tensor_scale;
  a.gv = c->v_tensor_scale;
  a.ksi = c->k_smooth_inv;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_rope_new = k_rope_new;
  a.slots = slot_mapping;
  a.seq_ids = seq_ids;
  a.positions = positions;
  return to_status(launch_append(a, (hipStream_t)stream));
}

size_t fp4_decode_workspace_bytes(const fp4kv_cache *c, int batch, int num_q_heads, int max_seq_len) {
  if (check_shape(c) != FP4KV_OK || batch < 0 || num_q_heads <= 0 || max_seq_len < 0) return 0;
  return workspace_for(c, batch, num_q_heads, max_seq_len, nullptr);
}

int fp4_decode_partials(const fp4kv_cache *c, const void *q, int q_dtype, int batch, int num_q_heads,
                        const int32_t *block_table, int max_pages_per_seq, const int32_t *seq_lens,
                        float softmax_scale, void *workspace, size_t workspace_bytes,
                        int32_t *zero_block_count, void *stream) {
  DecodeArgs a;
  int st = fill_decode(c, q, q_dtype, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                       softmax_scale, nullptr, workspace, workspace_bytes, zero_block_count, true,
                       false, &a);
  if (st) return st;
  if (c->attn == FP4KV_MLA) return to_status(launch_mla_partials(a, (hipStream_t)stream));
  return to_status(launch_decode_partials(a, (hipStream_t)stream));
}

int fp4_decode_merge(const fp4kv_cache *c, int batch, int num_q_heads, int max_pages_per_seq,
                     const int32_t *seq_lens, float *out, void *workspace, size_t workspace_bytes,
                     void *stream) {
  DecodeArgs a;
  int32_t dummy_bt = 0;
  int st = fill_decode(c, nullptr, FP4KV_F32, batch, num_q_heads, &dummy_bt, max_pages_per_seq,
                       seq_lens, 1.0f, out, workspace, workspace_bytes, nullptr, false, true, &a);
  if (st) return st;
  if (c->attn == FP4KV_MLA) return to_status(launch_mla_merge(a, (hipStream_t)stream));
  return to_status(launch_decode_merge(a, (hipStream_t)stream));
}

int fp4_decode_attention(const fp4kv_cache *c, const void *q, int q_dtype, int batch, int num_q_heads,
                         const int32_t *block_table, int max_pages_per_seq, const int32_t *seq_lens,
                         float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                         int32_t *zero_block_count, void *stream) {
  DecodeArgs a;
  int st = fill_decode(c, q, q_dtype, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                       softmax_scale, out, workspace, workspace_bytes, zero_block_count, true, true, &a);
  if (st) return st;
  const bool mla = c->attn == FP4KV_MLA;
  hipError_t e = mla ? launch_mla_partials(a, (hipStream_t)stream) : launch_decode_partials(a, (hipStream_t)stream);
  if (e != hipSuccess) return FP4KV_ERR_HIP;
  return to_status(mla ? launch_mla_merge(a, (hipStream_t)stream) : launch_decode_merge(a, (hipStream_t)stream));
}

size_t fp4_decode_multi_workspace_bytes(const fp4kv_cache *c, int batch, int q_len, int num_q_heads,
                                        int max_seq_len) {
  if (check_shape(c) != FP4KV_OK || batch < 0 || q_len < 1 || num_q_heads <= 0 || max_seq_len < 0) return 0;
  return workspace_for(c, batch, num_q_heads, max_seq_len, nullptr, q_len);
}

int fp4_decode_attention_multi(const fp4kv_cache *c, const void *q, int q_dtype, int batch, int q_len,
                               int num_q_heads, const int32_t *block_table, int max_pages_per_seq,
                               const int32_t *seq_lens, float softmax_scale, float *out, void *workspace,
                               size_t workspace_bytes, int32_t *zero_block_count, void *stream) {
  if (c && c->attn == FP4KV_MLA && q_len != 1) return FP4KV_ERR_UNSUPPORTED;
  DecodeArgs a;
  int st = fill_decode(c, q, q_dtype, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                       softmax_scale, out, workspace, workspace_bytes, zero_block_count, true, true, &a, q_len);
  if (st) return st;
  const bool mla = c->attn == FP4KV_MLA;
  hipError_t e = mla ? launch_mla_partials(a, (hipStream_t)stream) : launch_decode_partials(a, (hipStream_t)stream);
  if (e != hipSuccess) return FP4KV_ERR_HIP;
  return to_status(mla ? launch_mla_merge(a, (hipStream_t)stream) : launch_decode_merge(a, (hipStream_t)stream));
}

int fp4kv_cache_read(const fp4kv_cache *c, int batch, int num_q_heads, const int32_t *block_table,
                     int max_pages_per_seq, const int32_t *seq_lens, uint32_t *sink, size_t sink_words,
                     void *stream) {
  DecodeArgs a;
  int32_t dummy = 0;
  // validation as for a decode call; the workspace is not used (pass a large enough size)
  int st = fill_decode(c, &dummy, FP4KV_F32, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                       1.0f, nullptr, &dummy, ~(size_t)0, nullptr, false, false, &a);
  if (st) return st;
  if (c->attn != FP4KV_GQA) return FP4KV_ERR_UNSUPPORTED;
  if (batch > 0 && (!sink || sink_words < (size_t)a.n_waves * 64)) return FP4KV_ERR_INVALID_ARG;
  return to_status(launch_cache_read(a, sink, (hipStream_t)stream));
}

size_t fp4kv_cache_read_sink_words(const fp4kv_cache *c, int batch, int num_q_heads, int max_seq_len) {
  if (check_shape(c) != FP4KV_OK || c->attn != FP4KV_GQA || batch < 0 || num_q_heads <= 0 || max_seq_len < 0)
    return 0;
  SplitPlan p = plan_for(c, batch, num_q_heads, max_seq_len);
  return p.n_split < 0 ? 0 : (size_t)p.n_split * 64;
}

int fp4kv_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (!src || !sink || bytes == 0 || bytes % 4096 != 0) return FP4KV_ERR_INVALID_ARG;
  return to_status(launch_stream_read(src, bytes, sink, (hipStream_t)stream));
}

int fp4kv_stream_copy(const void *src, void *dst, size_t bytes, void *stream) {
  if (!src || !dst || bytes == 0 || bytes % 4096 != 0) return FP4KV_ERR_INVALID_ARG;
  return to_status(launch_stream_copy(src, dst, bytes, (hipStream_t)stream));
}

}  // extern "C"
