// C ABI of libfp4kv.so (declarations and contracts in include/fp4kv.h).
// Host code only: argument validation with host scalars, split-K planning and
// kernel launches on the caller's stream.  Nothing here allocates or syncs.
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>

#include "fp4kv_internal.h"

using namespace fp4kv;

namespace {

constexpr int kTarget = 2048;   // GQA waves: 8 single-wave groups per CU on 256 CUs
constexpr int kMlaWorkgroups = 256;   // MLA: one eight-wave workgroup per CU
constexpr int kMinTilesPerSplit = 1;   // the partial kernels' minimum share (kMinTilesPerWave)
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

// Shares of the balanced partition (GQA: one wave each; MLA: one eight-wave workgroup per
// group of 64 query heads each).  Each share takes an equal part of all 128-token tiles of the
// batch (computed on the device from seq_lens).  The most a launch uses: GQA kTarget waves,
// MLA kMlaWorkgroups workgroups.
// The environment variable FP4KV_MAX_SHARES (a positive integer) lowers that maximum, e.g. to
// leave compute units to work on other streams.
long max_shares(const fp4kv_cache *c, int hq) {
  long w = kTarget;
  if (c->attn == FP4KV_MLA) {
    const long nhg = hq / 16 > 0 ? hq / 16 : 1;
    w = kMlaWorkgroups / ((nhg + 3) / 4);
  }
  if (const char *env = getenv("FP4KV_MAX_SHARES")) {
    const long cap = strtol(env, nullptr, 10);
    if (cap > 0 && cap < w) w = cap;
  }
  return w > 0 ? w : 1;
}

// Shares a decode launch plans: the most a launch uses, but no more than shares of
// kMinTilesPerSplit tiles of the largest batch the block table can name (the device count
// follows the actual lengths and never exceeds this).  units: GQA batch * Hkv, MLA batch.
long plan_shares(const fp4kv_cache *c, long units, int hq, long max_len) {
  long max_tiles = (max_len + kTile - 1) / kTile;
  if (max_tiles < 1) max_tiles = 1;
  if (units < 1) units = 1;
  const long useful = (units * max_tiles + kMinTilesPerSplit - 1) / kMinTilesPerSplit;
  const long w = max_shares(c, hq);
  return w < useful ? w : (useful < 1 ? 1 : useful);
}

long units_of(const fp4kv_cache *c, long batch) { return c->attn == FP4KV_MLA ? batch : batch * c->num_kv_heads; }

// Workspace for `shares` shares: (shares + units) partial slots -- GQA `group * q_len` rows each,
// MLA `hq` rows each -- of d + 2 floats, then the per-unit slot ranges (two int32 per unit);
// MLA then holds the prepared query (one record per (sequence, query head)) from the next
// multiple of 256 bytes after the partials of the most shares a launch may plan.
size_t workspace_rows(const fp4kv_cache *c, long batch, int hq, long shares, int q_len) {
  const size_t units = (size_t)units_of(c, batch);
  const size_t per = c->attn == FP4KV_MLA ? (size_t)hq : (size_t)(hq / c->num_kv_heads) * (size_t)q_len;
  return ((size_t)shares + units) * per;
}
size_t partials_bytes(const fp4kv_cache *c, long batch, int hq, long shares, int q_len) {
  const size_t rows = workspace_rows(c, batch, hq, shares, q_len);
  return rows * ((size_t)c->head_dim + 2) * sizeof(float) + (size_t)units_of(c, batch) * 2 * sizeof(int32_t);
}
size_t query_offset(size_t partials) { return (partials + 255) / 256 * 256; }
size_t workspace_size(const fp4kv_cache *c, long batch, int hq, long shares, int q_len) {
  const size_t part = partials_bytes(c, batch, hq, shares, q_len);
  if (c->attn != FP4KV_MLA) return part;
  return query_offset(part) + (size_t)batch * (size_t)hq * kMlaQRecord;
}

int to_status(hipError_t e) { return e == hipSuccess ? FP4KV_OK : FP4KV_ERR_HIP; }

// Technique switches for the next calls (ablation-study build only; always 0 otherwise).
int g_ablation = 0;

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
    bool ok = group == 1 || group == 2 || group == 4 || group == 8;
    if (!ok) return FP4KV_ERR_UNSUPPORTED;
    // query tokens x query heads per KV head: up to two row sets of one MFMA's columns
    if (q_len > 8 || group * q_len > 16) return FP4KV_ERR_UNSUPPORTED;
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
  // partial slots are numbered in int32 (shares + units)
  if ((long)batch * c->num_kv_heads > 0x3FFFFFFFL) return FP4KV_ERR_INVALID_ARG;
  // the workspace must hold what the size query reports (any launch's need is at most that)
  if (ws_bytes < workspace_size(c, batch, hq, max_shares(c, hq), q_len)) return FP4KV_ERR_WORKSPACE;
  const long shares = plan_shares(c, units_of(c, batch), hq, (long)max_pages * c->page_size);
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
  d.abl = kAblation ? g_ablation : 0;
  // normalized P needs both passes of one fp4_decode_attention call, one query token
  if ((d.abl & kAblVanillaP) && (q_len != 1 || !need_q || !need_out)) return FP4KV_ERR_UNSUPPORTED;
  d.n_waves = (int)shares;
  d.softmax_scale = softmax_scale;
  // 1/head_dim of the unnormalized rotation (1 when the rotation is switched off)
  const float l2d = (float)(1.4426950408889634 / (double)((d.abl & kAblNoRotation) ? 1 : c->head_dim));
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
  const size_t rows = workspace_rows(c, batch, hq, shares, q_len);
  d.ws_o = (float *)ws;
  d.ws_ml = (float *)ws + rows * (size_t)c->head_dim;
  d.ws_meta = (int32_t *)(d.ws_ml + rows * 2);
  // the prepared query sits at a place the caller can find: the last batch * hq records of the
  // size the workspace query reports
  d.ws_q = c->attn == FP4KV_MLA
               ? (uint8_t *)ws + query_offset(partials_bytes(c, batch, hq, max_shares(c, hq), q_len))
               : nullptr;
  d.out = out;
  d.zero_blocks = zero;
  return FP4KV_OK;
}

// Scratch of fp4_decode_attention_noalloc: a file-scope device array, so every GPU the library
// runs on holds one copy (allocated with the code object, kept until the process ends).  In host
// code `scratch` names a host-side stand-in, not device memory: its device address is taken once
// per device with hipGetSymbolAddress and only that address is handed to kernels.
__device__ __align__(256) uint8_t scratch[FP4KV_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch (looked up on the first call on that device).
int scratch_of_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP4KV_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return FP4KV_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FP4KV_OK;
}

// BF16 comparison cache: scalar checks, and the GQA FP4 descriptor with the same shape
// (the two share the partition, the workspace layout and the merge).
int check_bf16(const fp4kv_bf16_cache *c) {
  if (!c) return FP4KV_ERR_INVALID_ARG;
  if (c->num_pages <= 0 || c->num_kv_heads <= 0 || c->page_size <= 0) return FP4KV_ERR_INVALID_ARG;
  if (!pow2_page(c->page_size)) return FP4KV_ERR_UNSUPPORTED;
  if ((long)c->num_pages * c->page_size > 0x7FFFFFFFL) return FP4KV_ERR_INVALID_ARG;
  if (c->head_dim != 128) return c->head_dim > 0 ? FP4KV_ERR_UNSUPPORTED : FP4KV_ERR_INVALID_ARG;
  return FP4KV_OK;
}

fp4kv_cache gqa_twin(const fp4kv_bf16_cache *c) {
  fp4kv_cache t{};
  t.format = FP4KV_MXFP4;
  t.attn = FP4KV_GQA;
  t.num_pages = c->num_pages;
  t.page_size = c->page_size;
  t.num_kv_heads = c->num_kv_heads;
  t.head_dim = 128;
  t.rope_dim = 0;
  t.max_seqs = 1;
  return t;
}

}  // namespace

extern "C" {

int bf16kv_cache_layout(const fp4kv_bf16_cache *c, size_t bytes_out[2]) {
  if (!bytes_out) return FP4KV_ERR_INVALID_ARG;
  const int st = check_bf16(c);
  if (st) return st;
  bytes_out[0] = bytes_out[1] = (size_t)c->num_pages * c->num_kv_heads * c->page_size * 128 * 2;
  return FP4KV_OK;
}

int bf16kv_append(const fp4kv_bf16_cache *c, const void *k_new, const void *v_new, int dtype, int num_tokens,
                  const int32_t *slot_mapping, void *stream) {
  int st = check_bf16(c);
  if (st) return st;
  if (dtype != FP4KV_F32 && dtype != FP4KV_BF16) return FP4KV_ERR_INVALID_ARG;
  if (num_tokens < 0) return FP4KV_ERR_INVALID_ARG;
  if (num_tokens == 0) return FP4KV_OK;
  if (!c->k || !c->v || !k_new || !v_new || !slot_mapping) return FP4KV_ERR_INVALID_ARG;
  AppendArgs a{};
  a.page_size = c->page_size;
  a.hkv = c->num_kv_heads;
  a.d = 128;
  a.num_pages = c->num_pages;
  a.num_tokens = num_tokens;
  a.bf16 = dtype == FP4KV_BF16;
  a.k_codes = (uint8_t *)c->k;
  a.v_codes = (uint8_t *)c->v;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slots = slot_mapping;
  return to_status(launch_bf16_append(a, (hipStream_t)stream));
}

size_t bf16_decode_workspace_bytes(const fp4kv_bf16_cache *c, int batch, int num_q_heads, int max_seq_len) {
  if (check_bf16(c) != FP4KV_OK || batch < 0 || num_q_heads <= 0 || max_seq_len < 0) return 0;
  const fp4kv_cache t = gqa_twin(c);
  return workspace_size(&t, batch, num_q_heads, max_shares(&t, num_q_heads), 1);
}

int bf16_decode_attention(const fp4kv_bf16_cache *c, const void *q, int q_dtype, int batch, int num_q_heads,
                          const int32_t *block_table, int max_pages_per_seq, const int32_t *seq_lens,
                          float softmax_scale, float *out, void *workspace, size_t workspace_bytes,
                          void *stream) {
  int st = check_bf16(c);
  if (st) return st;
  if (batch < 0 || num_q_heads <= 0 || max_pages_per_seq <= 0) return FP4KV_ERR_INVALID_ARG;
  if (q_dtype != FP4KV_F32 && q_dtype != FP4KV_BF16) return FP4KV_ERR_INVALID_ARG;
  if (num_q_heads % c->num_kv_heads != 0) return FP4KV_ERR_INVALID_ARG;
  if (!(softmax_scale == softmax_scale)) return FP4KV_ERR_INVALID_ARG;
  const int group = num_q_heads / c->num_kv_heads;
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16) return FP4KV_ERR_UNSUPPORTED;
  if ((long)max_pages_per_seq * c->page_size > 0x7FFFFFFFL) return FP4KV_ERR_INVALID_ARG;
  if ((long)batch * c->num_kv_heads > 0x3FFFFFFFL) return FP4KV_ERR_INVALID_ARG;
  if (batch > 0 && (!c->k || !c->v || !q || !block_table || !seq_lens || !out || !workspace))
    return FP4KV_ERR_INVALID_ARG;
  const fp4kv_cache t = gqa_twin(c);
  if (workspace_bytes < workspace_size(&t, batch, num_q_heads, max_shares(&t, num_q_heads), 1))
    return FP4KV_ERR_WORKSPACE;
  const long shares = plan_shares(&t, units_of(&t, batch), num_q_heads, (long)max_pages_per_seq * c->page_size);
  DecodeArgs d{};
  d.page_size = c->page_size;
  d.hkv = c->num_kv_heads;
  d.group = group;
  d.hq = num_q_heads;
  d.d = 128;
  d.batch = batch;
  d.max_pages = max_pages_per_seq;
  d.num_pages = c->num_pages;
  d.q_bf16 = q_dtype == FP4KV_BF16;
  d.q_len = 1;
  d.n_waves = (int)shares;
  d.softmax_scale = softmax_scale;
  d.coef = softmax_scale * (float)1.4426950408889634;
  d.k_codes = (const uint8_t *)c->k;
  d.v_codes = (const uint8_t *)c->v;
  d.q = q;
  d.block_table = block_table;
  d.seq_lens = seq_lens;
  const size_t rows = workspace_rows(&t, batch, num_q_heads, shares, 1);
  d.ws_o = (float *)workspace;
  d.ws_ml = d.ws_o + rows * 128;
  d.ws_meta = (int32_t *)(d.ws_ml + rows * 2);
  d.out = out;
  const hipError_t e = launch_bf16_partials(d, (hipStream_t)stream);
  if (e != hipSuccess) return FP4KV_ERR_HIP;
  return to_status(launch_decode_merge(d, (hipStream_t)stream));
}


#ifdef FP4KV_ABLATION
// Ablation-study build only: technique switches (kAbl* bits) for the following GQA append
// and decode calls of this process.
int fp4kv_ablation_set(int flags) {
  if (flags & ~(kAblSingleQ | kAblNoRotation | kAblNoSearch | kAblVanillaP)) return FP4KV_ERR_INVALID_ARG;
  g_ablation = flags;
  return FP4KV_OK;
}
#endif

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
  a.abl = kAblation ? g_ablation : 0;
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
  return workspace_size(c, batch, num_q_heads, max_shares(c, num_q_heads), 1);
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
  if (kAblation && (a.abl & kAblVanillaP)) {
    // ablation study, normalized P: a first pass of the method gives each row's max and
    // softmax denominator (written into out, which the second pass overwrites)
    DecodeArgs a1 = a;
    a1.abl = (a.abl & ~kAblVanillaP) | kAblRowStats;
    a1.zero_blocks = nullptr;
    if ((mla ? launch_mla_partials(a1, (hipStream_t)stream) : launch_decode_partials(a1, (hipStream_t)stream)) !=
        hipSuccess)
      return FP4KV_ERR_HIP;
    if ((mla ? launch_mla_merge(a1, (hipStream_t)stream) : launch_decode_merge(a1, (hipStream_t)stream)) != hipSuccess)
      return FP4KV_ERR_HIP;
  }
  hipError_t e = mla ? launch_mla_partials(a, (hipStream_t)stream) : launch_decode_partials(a, (hipStream_t)stream);
  if (e != hipSuccess) return FP4KV_ERR_HIP;
  return to_status(mla ? launch_mla_merge(a, (hipStream_t)stream) : launch_decode_merge(a, (hipStream_t)stream));
}

int fp4_decode_attention_noalloc(const fp4kv_cache *c, const void *q, int q_dtype, int batch, int num_q_heads,
                                 const int32_t *block_table, int max_pages_per_seq, const int32_t *seq_lens,
                                 float softmax_scale, float *out, int32_t *zero_block_count, void *stream) {
  int st = check_shape(c);
  if (st) return st;
  if (batch < 0 || num_q_heads <= 0) return FP4KV_ERR_INVALID_ARG;
  // the workspace fp4_decode_attention would need must fit the scratch array
  if (workspace_size(c, batch, num_q_heads, max_shares(c, num_q_heads), 1) > (size_t)FP4KV_NOALLOC_SCRATCH_BYTES)
    return FP4KV_ERR_WORKSPACE;
  void *ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st) return st;
  return fp4_decode_attention(c, q, q_dtype, batch, num_q_heads, block_table, max_pages_per_seq, seq_lens,
                              softmax_scale, out, ws, (size_t)FP4KV_NOALLOC_SCRATCH_BYTES, zero_block_count,
                              stream);
}

size_t fp4_decode_multi_workspace_bytes(const fp4kv_cache *c, int batch, int q_len, int num_q_heads,
                                        int max_seq_len) {
  if (check_shape(c) != FP4KV_OK || batch < 0 || q_len < 1 || num_q_heads <= 0 || max_seq_len < 0) return 0;
  return workspace_size(c, batch, num_q_heads, max_shares(c, num_q_heads), q_len);
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
  if (batch > 0 && (!sink || sink_words < (size_t)max_shares(c, num_q_heads) * 64)) return FP4KV_ERR_INVALID_ARG;
  return to_status(launch_cache_read(a, sink, (hipStream_t)stream));
}

size_t fp4kv_cache_read_sink_words(const fp4kv_cache *c, int batch, int num_q_heads, int max_seq_len) {
  if (check_shape(c) != FP4KV_OK || c->attn != FP4KV_GQA || batch < 0 || num_q_heads <= 0 || max_seq_len < 0)
    return 0;
  return (size_t)max_shares(c, num_q_heads) * 64;
}

int fp4kv_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (!src || !sink || bytes == 0 || bytes % 4096 != 0) return FP4KV_ERR_INVALID_ARG;
  return to_status(launch_stream_read(src, bytes, sink, (hipStream_t)stream));
}

int fp4kv_pack_e2m1(const float *x, size_t n, int scale_exp, uint8_t *out, void *stream) {
  if (!x || !out || n == 0 || n % 8 != 0 || scale_exp < -126 || scale_exp > 127) return FP4KV_ERR_INVALID_ARG;
  return to_status(launch_pack_e2m1(x, n, scale_exp, out, (hipStream_t)stream));
}

int fp4kv_stream_copy(const void *src, void *dst, size_t bytes, void *stream) {
  if (!src || !dst || bytes == 0 || bytes % 4096 != 0) return FP4KV_ERR_INVALID_ARG;
  return to_status(launch_stream_copy(src, dst, bytes, (hipStream_t)stream));
}

}  // extern "C"
