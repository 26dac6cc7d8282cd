/*
 * fp4kv.h -- C ABI of libfp4kv.so: a paged 4-bit microscaling KV cache and
 * decode attention over it, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes is the hot path of BitDecoding-FP4 as described in
 * "BitDecoding-FP4: Native FP4 KV Cache Decoding via Algorithm-System Co-Design"
 * (section "Article Summary", the arXiv abstract):
 *   - keys are stored after static per-channel smoothing, a Hadamard rotation
 *     over head_dim and a per-block scale search under token-wise scaling
 *     (Outlier-Aware Key Quantization);
 *   - the query is split into two FP4 tensors, the second encoding the
 *     residual of the first (Dual-Residual Query Quantization);
 *   - probabilities are quantized to FP4 inside a transposed softmax, scaled so
 *     that their E4M3 block scales do not round long-context probabilities to
 *     zero (Underflow-Aware Probability Scaling);
 *   - the query rows that share a KV head are stacked into one matrix-core
 *     operation over the paged cache ("stacked query MMA").
 * The cache formats are NVFP4 (16-element blocks, E4M3 block scale, fp32
 * tensor scale) and MXFP4 (32-element blocks, E8M0 block scale).
 *
 * Conventions for every entry point
 *   - All pointers are DEVICE pointers unless a parameter says "host".  The
 *     caller owns every buffer; the library never allocates, frees or
 *     synchronizes.  Work is enqueued on `stream` (a hipStream_t; NULL = the
 *     default stream) and runs asynchronously.
 *   - Return value: FP4KV_OK (0) or an FP4KV_ERR_* code.  Arguments are checked
 *     on the host before anything is launched; on an error nothing is enqueued.
 *     fp4kv_status_string() describes a code.
 *   - Device-side contents that break a documented precondition (page ids out
 *     of range, unsorted append batches) are not detected: the result is
 *     undefined, except that append slots and sequence ids outside their
 *     ranges are skipped.
 *
 * Cache layout (P = page_size tokens, B = 16 for NVFP4 and 32 for MXFP4, a
 * physical page holds P consecutive tokens of one sequence; sequence s's
 * logical page i is block_table[s * max_pages_per_seq + i]; a token's slot is
 * page * P + (position % P)):
 *   GQA (attn = FP4KV_GQA, head_dim d = 128):
 *     k_codes  u8 [num_pages][Hkv][P][d/2]  token-major; byte j holds channel 2j
 *                                            (low nibble) and 2j+1 (high nibble)
 *     k_scales u8 [num_pages][Hkv][P*d/B]   per (page token t, channel block q):
 *                                            NVFP4 at t*8 + q (token-major); MXFP4 at
 *                                            (((t/32)*4 + t%4)*4 + q)*8 + (t%32)/4
 *     v_codes  u8 [num_pages][Hkv][d][P/2]  channel-major; byte j holds tokens
 *                                            2j (low) and 2j+1 (high) of the page
 *     v_scales u8 [num_pages][Hkv][d*P/B]   per (channel c, page token block j) at
 *                                            ((j/J)*16 + c%16)*8*J + (c/16)*J + j%J,
 *                                            J = min(P, 32)/B
 *   (the scale orders put the scales one decode lane needs in one contiguous run)
 *     stage    f32 [max_seqs][Hkv][B][d]    unquantized values of each sequence's
 *                                            last, partly filled value block
 *   MLA (attn = FP4KV_MLA, one latent head, head_dim = 512, rope_dim = 64):
 *     k_codes  u8 [num_pages][1][P][256]    rotated latent, token-major
 *     k_scales u8 [num_pages][1][P/B][512/B] one scale per B-token x B-channel tile
 *     k_rope   bf16 [num_pages][1][P][64]   rope key, unquantized
 *     stage    f32 [max_seqs][1][B][512]    rotated latent of the partial tile
 *   (v_codes and v_scales are unused for MLA and may be NULL: the latent also serves as the
 *   value, and the decode reads its value operand from the token-major codes)
 *     v_scales unused (the tile scales serve both copies).
 *   Codes are E2M1 (bit 3 sign, magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6); NVFP4
 *   scales are E4M3 (OCP "FN"), MXFP4 scales E8M0.  A partially filled value
 *   block (or MLA tile) is stored as if its absent tokens were +0.0.
 */
#ifndef FP4KV_H
#define FP4KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum fp4kv_format { FP4KV_NVFP4 = 0, FP4KV_MXFP4 = 1 };
enum fp4kv_dtype { FP4KV_F32 = 0, FP4KV_BF16 = 1 };
enum fp4kv_attn { FP4KV_GQA = 0, FP4KV_MLA = 1 };

enum fp4kv_status {
  FP4KV_OK = 0,
  FP4KV_ERR_INVALID_ARG = 1,      /* null pointer, bad size, bad enum value         */
  FP4KV_ERR_UNSUPPORTED = 2,      /* valid but not implemented (head_dim, GQA group) */
  FP4KV_ERR_WORKSPACE = 3,        /* workspace smaller than fp4_decode_workspace_bytes */
  FP4KV_ERR_HIP = 4               /* a HIP launch failed                              */
};

/* Cache descriptor.  Plain data; the library keeps no reference to it after a
 * call returns.  Pointers are device pointers owned by the caller and sized as
 * fp4kv_cache_layout() reports.
 *   format        FP4KV_NVFP4 or FP4KV_MXFP4
 *   attn          FP4KV_GQA or FP4KV_MLA
 *   num_pages     physical pages in the pool (> 0)
 *   page_size     tokens per page; a multiple of 16 (NVFP4) or 32 (MXFP4), <= 256
 *   num_kv_heads  Hkv (GQA); must be 1 for MLA
 *   head_dim      128 (GQA) or 512 (MLA latent)
 *   rope_dim      0 (GQA) or 64 (MLA)
 *   max_seqs      rows of the stage buffer; append seq_ids are < max_seqs
 *   k_tensor_scale, v_tensor_scale  f32 [Hkv]: NVFP4 per-KV-head tensor scales G
 *                 (decoded value = code * block_scale * G); ignored for MXFP4
 *                 (may be NULL); v_tensor_scale unused for MLA
 *   k_smooth_inv  f32 [Hkv][head_dim]: static smoothing applied to keys
 *   q_smooth      f32 [Hkv][head_dim]: the matching factors applied to queries;
 *                 the caller keeps q_smooth * k_smooth_inv == 1 per channel   */
typedef struct fp4kv_cache {
  int32_t format;
  int32_t attn;
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t rope_dim;
  int32_t max_seqs;
  uint8_t *k_codes;
  uint8_t *k_scales;
  uint8_t *v_codes;
  uint8_t *v_scales;
  float *stage;
  uint16_t *k_rope;
  const float *k_tensor_scale;
  const float *v_tensor_scale;
  const float *k_smooth_inv;
  const float *q_smooth;
} fp4kv_cache;

/* Byte sizes of the six cache buffers for descriptor `c` (host pointer), in the
 * order k_codes, k_scales, v_codes, v_scales, stage, k_rope (0 for unused ones):
 * the paged 4-bit microscaling KV cache of "BitDecoding-FP4: Native FP4 KV Cache
 * Decoding via Algorithm-System Co-Design" (Article Summary) in this library's
 * layout (above).  Only the scalar fields of `c` are read.  bytes_out is a host
 * array of 6. */
int fp4kv_cache_layout(const fp4kv_cache *c, size_t bytes_out[6]);

/* Append new tokens to the cache: the KV-append quantizer (Outlier-Aware Key
 * Quantization of "BitDecoding-FP4: Native FP4 KV Cache Decoding via
 * Algorithm-System Co-Design", Article Summary, and "FP4 KV Cache Done Right",
 * section "What is actually new in BitDecoding-FP4?").
 *   k_new   [num_tokens][Hkv][head_dim] keys (MLA: the latent), dtype F32 or BF16
 *   v_new   [num_tokens][Hkv][head_dim] values (GQA); NULL for MLA
 *   k_rope_new  bf16 [num_tokens][rope_dim] (MLA), NULL for GQA
 *   slot_mapping, seq_ids, positions  i32 [num_tokens]: destination slot,
 *           sequence (stage row) and position of every new token.
 * Preconditions (not checked on the device): inside one call the tokens of a
 * sequence are contiguous in the batch, in increasing and consecutive
 * positions, and the first of them continues that sequence (its position is
 * the number of tokens the cache already holds for it); a token's slot lies in
 * the page that block_table assigns to its position.  Tokens whose slot or
 * sequence id is out of range are skipped; when that is the first token of a
 * sequence's chunk, the chunk's open value block is not staged either.  Calls
 * on one stream are applied in order.  Keys: smoothing, FWHT over head_dim, per-block scale
 * search, E2M1 packing.  Values: channel-wise scales over page-aligned blocks
 * of B tokens; the block holding the last new token of a sequence is
 * re-quantized from the stage on every call, so the bytes equal those of
 * quantizing the whole sequence at once.  num_tokens == 0 is a no-op. */
int kv_quant_append(const fp4kv_cache *c, const void *k_new, const void *v_new, int dtype,
                    int num_tokens, const int32_t *slot_mapping, const int32_t *seq_ids,
                    const int32_t *positions, const void *k_rope_new, void *stream);

/* Workspace bytes fp4_decode_attention / fp4_decode_partials need for this
 * batch shape (host function; reads only scalar fields of `c`).  The size covers
 * every block table and every set of lengths: max_seq_len is validated (>= 0)
 * but does not change it.  The decode calls refuse a smaller workspace with
 * FP4KV_ERR_WORKSPACE.  The environment variable FP4KV_MAX_SHARES (a positive
 * integer) lowers the number of shares a decode launch divides the batch's tiles
 * into -- and with it this size -- e.g. to leave compute units to other streams.
 * Returns 0 on invalid arguments. */
size_t fp4_decode_workspace_bytes(const fp4kv_cache *c, int batch, int num_q_heads,
                                  int max_seq_len);

/* Decode attention: one query token per sequence against its whole cached context
 * ("BitDecoding-FP4: Native FP4 KV Cache Decoding via Algorithm-System
 * Co-Design", Article Summary: dual-residual FP4 query, FP4 Q.K^T and P.V on the
 * matrix cores, transposed softmax with underflow-aware FP4 probabilities;
 * "BitDecoding-FP4 : décodage natif du KV cache FP4", Analyse approfondie:
 * stacked query rows sharing one cache tile), split-K over the paged blocks.
 *   q          [batch][num_q_heads][head_dim (+ rope_dim for MLA)], dtype q_dtype
 *   block_table i32 [batch][max_pages_per_seq]; seq_lens i32 [batch] (0 allowed,
 *              giving a zero output row; a length is read as clamped to
 *              [0, max_pages_per_seq * page_size]); entries past a sequence's
 *              pages are never read
 *   softmax_scale  multiplies q.k (the 1/head_dim of the unnormalized Hadamard
 *              rotation is applied internally)
 *   out        f32 [batch][num_q_heads][head_dim] (MLA: the 512-d latent
 *              output, un-rotated and un-smoothed)
 *   workspace  device scratch of at least fp4_decode_workspace_bytes(); its
 *              contents need no initialisation and are overwritten
 *   zero_block_count  nullable i32 counter; when given, the number of
 *              probability blocks that held a valid token and quantized to all
 *              zeros is ADDED to it (the caller zeroes it)
 * GQA needs num_q_heads == group * Hkv with group 1, 2, 4 or 8.
 * Launches the split-K partial kernel and the merge kernel on `stream`. */
int fp4_decode_attention(const fp4kv_cache *c, const void *q, int q_dtype, int batch,
                         int num_q_heads, const int32_t *block_table, int max_pages_per_seq,
                         const int32_t *seq_lens, float softmax_scale, float *out,
                         void *workspace, size_t workspace_bytes, int32_t *zero_block_count,
                         void *stream);

/* fp4_decode_attention without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the split-K partials go to a scratch array of FP4KV_NOALLOC_SCRATCH_BYTES that
 * the library holds on every GPU it runs on, from the first call on that GPU until the process
 * ends.  The call itself allocates and frees nothing.  It uses the scratch of the current
 * device (`stream` must belong to that device).
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (on
 * different streams, or from several host threads) race and give undefined results; calls
 * ordered on one stream are safe.  The scratch keeps the last call's contents; nothing in it
 * needs clearing between calls.  The first call on a GPU looks up the scratch's device address
 * (hipGetSymbolAddress); a caller that captures this call in a HIP graph makes one call on that
 * GPU before capturing.
 * Returns FP4KV_ERR_WORKSPACE when fp4_decode_workspace_bytes() for this shape exceeds
 * FP4KV_NOALLOC_SCRATCH_BYTES (64 MiB: GQA up to about 30,000 (sequence, KV head) units at 4
 * query heads per KV head; MLA with 128 query heads up to 92 sequences), and
 * FP4KV_ERR_HIP when the scratch address cannot be obtained; otherwise exactly as
 * fp4_decode_attention, whose kernels it runs. */
#define FP4KV_NOALLOC_SCRATCH_BYTES (64u << 20)
int fp4_decode_attention_noalloc(const fp4kv_cache *c, const void *q, int q_dtype, int batch,
                                 int num_q_heads, const int32_t *block_table, int max_pages_per_seq,
                                 const int32_t *seq_lens, float softmax_scale, float *out,
                                 int32_t *zero_block_count, void *stream);

/* Multi-token decode (speculative or multi-token-prediction verification): q_len
 * query tokens per sequence, the q_len newest tokens of each sequence (positions
 * seq_lens[b] - q_len .. seq_lens[b] - 1, already appended to the cache); query j
 * attends to tokens 0 .. seq_lens[b] - q_len + j (causal).  The rows of all q_len
 * tokens are stacked on the same key / value tiles ("BitDecoding-FP4 : décodage
 * natif du KV cache FP4", Analyse approfondie: query rows stacked into one matrix
 * operation), so the cache is read once for all of them.
 *   q    [batch][q_len][num_q_heads][head_dim], dtype q_dtype
 *   out  f32 [batch][q_len][num_q_heads][head_dim]
 * Other arguments as fp4_decode_attention; seq_lens[b] must be 0 or >= q_len.
 * GQA only (MLA: q_len 1); q_len <= 8 and group * q_len <= 16, else
 * FP4KV_ERR_UNSUPPORTED.  q_len == 1 is fp4_decode_attention. */
size_t fp4_decode_multi_workspace_bytes(const fp4kv_cache *c, int batch, int q_len, int num_q_heads,
                                        int max_seq_len);
int fp4_decode_attention_multi(const fp4kv_cache *c, const void *q, int q_dtype, int batch, int q_len,
                               int num_q_heads, const int32_t *block_table, int max_pages_per_seq,
                               const int32_t *seq_lens, float softmax_scale, float *out,
                               void *workspace, size_t workspace_bytes, int32_t *zero_block_count,
                               void *stream);

/* The two halves of fp4_decode_attention, for callers that merge split-K
 * partials themselves (e.g. across devices holding different pages of one
 * sequence) or time the stages separately.  fp4_decode_partials writes
 * partial results (o unnormalized, m the base-2 running maximum, l the
 * denominator) into the workspace; fp4_decode_merge combines the partials of
 * each query head: out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s.  Both
 * take the same arguments as fp4_decode_attention and must see the same batch
 * shape and seq_lens.
 *
 * Workspace layout (floats unless stated; W = the number of shares the library
 * plans for the batch shape, U = the units, R = rows per slot):
 *   o [W + U][R][head_dim], then (m, l) [W + U][R][2], then i32 (first slot,
 *   count) [U].  GQA: U = batch * Hkv units (sequence, KV head), in the order
 *   u = b * Hkv + kvh, R = num_q_heads / Hkv (row h % R of a slot belongs to
 *   query head h).  MLA: U = batch (a sequence is a unit), R = num_q_heads.
 *   The tiles of all units are shared out equally among the W shares; the
 *   partials of unit u are the `count` consecutive slots from `first`.  Units
 *   of empty sequences have no partials (their range is not written).  MLA
 *   also holds the prepared query, written by fp4_decode_partials before the
 *   partials, in the last batch * num_q_heads * 768 bytes of the size
 *   fp4_decode_workspace_bytes reports: per (sequence, query head), row
 *   b * num_q_heads + h, the rotated, smoothed dual-residual FP4 codes of pass k
 *   at byte 256 k (channels 2i, 2i+1 in byte i, low nibble first), their block
 *   scale bytes (E8M0 exponent + 127; NVFP4 per 16 channels, MXFP4 per 32) at
 *   512 + 32 k, the tensor scales G1, G2 (f32) at 576 and 580, and the rope
 *   query as bf16 at 640. */
int fp4_decode_partials(const fp4kv_cache *c, const void *q, int q_dtype, int batch,
                        int num_q_heads, const int32_t *block_table, int max_pages_per_seq,
                        const int32_t *seq_lens, float softmax_scale, void *workspace,
                        size_t workspace_bytes, int32_t *zero_block_count, void *stream);
int fp4_decode_merge(const fp4kv_cache *c, int batch, int num_q_heads, int max_pages_per_seq,
                     const int32_t *seq_lens, float *out, void *workspace,
                     size_t workspace_bytes, void *stream);

/* Measurement helper: reads `bytes` (a multiple of 4096) from `src` and writes
 * one word per workgroup to `sink` (>= 4096 words), to measure the achievable
 * HBM read bandwidth next to the decode kernel. */
int fp4kv_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream);

/* Diagnostic: E2M1 codes of x[i] / 2^scale_exp (n a multiple of 8, f32 in, n / 2 packed
 * bytes out, byte j = code(x[2j]) | code(x[2j+1]) << 4) computed with the hardware
 * conversion the decode kernels use to quantize the probabilities to FP4 (the fused
 * probability quantization of "BitDecoding-FP4: Native FP4 KV Cache Decoding via
 * Algorithm-System Co-Design", Article Summary), so that its rounding can be checked
 * against the format's definition.  scale_exp in [-126, 127]. */
int fp4kv_pack_e2m1(const float *x, size_t n, int scale_exp, uint8_t *out, void *stream);

/* Measurement helper: copies `bytes` (a multiple of 4096) from `src` to `dst`, the
 * known-size reference against which hardware traffic counters are scaled. */
int fp4kv_stream_copy(const void *src, void *dst, size_t bytes, void *stream);

/* Measurement helper (GQA caches): performs exactly the cache reads of
 * fp4_decode_partials for the same arguments -- same division of the batch's
 * tiles among waves, same page lookups, same loads in the same order -- without
 * any arithmetic, and folds the loaded words into `sink` (one word per lane, at
 * least fp4kv_cache_read_sink_words() words), to measure the read rate of the
 * decode kernel's own access pattern over a shuffled page table.  Arguments are
 * validated like a decode call; MLA caches return FP4KV_ERR_UNSUPPORTED. */
int fp4kv_cache_read(const fp4kv_cache *c, int batch, int num_q_heads, const int32_t *block_table,
                     int max_pages_per_seq, const int32_t *seq_lens, uint32_t *sink,
                     size_t sink_words, void *stream);
/* Sink words fp4kv_cache_read needs for this batch shape (0 on invalid arguments). */
size_t fp4kv_cache_read_sink_words(const fp4kv_cache *c, int batch, int num_q_heads,
                                   int max_seq_len);

/* ---------------------------------------------------------------------------
 * BF16 KV cache: the comparison system of the FP4 path.  The pages report the FP4
 * cache's serving gain over a BF16 KV cache ("FP4 KV Cache Done Right", section
 * "How good are the results, really?"); these entry points give the same paged
 * decode with a bfloat16 cache on the same partition and merge, so that the two
 * can be timed side by side on one GPU.  Plain softmax attention (no smoothing,
 * rotation or quantization); query and probabilities in bf16, sums in fp32.
 * Layout (head_dim 128, P = page_size tokens per page, Hkv heads):
 *   k  bf16 [num_pages][Hkv][P][128]   token-major
 *   v  bf16 [num_pages][Hkv][128][P]   channel-major
 * page_size is 16, 32, 64, 128 or 256; a token's slot is page * P + position % P. */
typedef struct fp4kv_bf16_cache {
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
  uint16_t *k;
  uint16_t *v;
} fp4kv_bf16_cache;

/* Byte sizes of k and v (host function; reads only the scalar fields). */
int bf16kv_cache_layout(const fp4kv_bf16_cache *c, size_t bytes_out[2]);

/* Append num_tokens tokens: k_new, v_new [num_tokens][Hkv][128] of dtype F32 or BF16,
 * rounded to bf16 (nearest even) into the slots slot_mapping i32 [num_tokens]; slots
 * outside the pool are skipped.  num_tokens == 0 is a no-op. */
int bf16kv_append(const fp4kv_bf16_cache *c, const void *k_new, const void *v_new, int dtype,
                  int num_tokens, const int32_t *slot_mapping, void *stream);

/* Workspace bytes of bf16_decode_attention for this batch shape (0 on invalid
 * arguments); like fp4_decode_workspace_bytes it covers every block table. */
size_t bf16_decode_workspace_bytes(const fp4kv_bf16_cache *c, int batch, int num_q_heads,
                                   int max_seq_len);

/* Decode attention over the BF16 cache, arguments and outputs as fp4_decode_attention
 * (q [batch][num_q_heads][128] of dtype q_dtype; out f32 [batch][num_q_heads][128];
 * num_q_heads / num_kv_heads in {1, 2, 4, 8, 16}).  Softmax over tiles of 64 tokens:
 * p = 2^(s - tile max), rounded to bf16 for P.V, the denominator summing the fp32 p. */
int bf16_decode_attention(const fp4kv_bf16_cache *c, const void *q, int q_dtype, int batch,
                          int num_q_heads, const int32_t *block_table, int max_pages_per_seq,
                          const int32_t *seq_lens, float softmax_scale, float *out,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code (never NULL). */
const char *fp4kv_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* FP4KV_H */
