/* Per-technique ablation study build of the library (not part of the product).
 *
 * libfp4kv_ablate.so is built from the same sources as libfp4kv.so with -DFP4KV_ABLATION.
 * It exports every entry point of fp4kv.h plus fp4kv_ablation_set, whose switches turn one
 * technique of the method off at a time, so that each technique's effect on the decode's
 * accuracy can be measured on the kernels themselves (the method's summary reports no
 * per-technique ablation: "BitDecoding-FP4 : décodage natif du KV cache FP4", Perspectives).
 * The product library libfp4kv.so contains none of the switches and does not export
 * fp4kv_ablation_set. */
#ifndef FP4KV_ABLATION_H
#define FP4KV_ABLATION_H

#include "fp4kv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* No dual-residual query: the query's second FP4 pass (the residual) is zero. */
#define FP4KV_ABL_SINGLE_Q 1
/* No Walsh-Hadamard rotation of keys (MLA: latent) and queries; for MLA the merge applies no
 * un-rotation either, and the logit coefficient takes no 1/head_dim. */
#define FP4KV_ABL_NO_ROTATION 2
/* No key scale search: every key block (MLA: latent tile) keeps its default scale. */
#define FP4KV_ABL_NO_SEARCH 4
/* No underflow-aware probability scaling: P is the softmax normalized over the whole row,
 * quantized with tensor scale 1 (NVFP4: the default E4M3 scale of each 16 probabilities;
 * MXFP4: E8M0 per 32).  fp4_decode_attention (and fp4_decode_attention_noalloc) then runs the
 * decode twice -- a first pass of the method gives each row's max and denominator -- and
 * fp4_decode_partials, fp4_decode_merge and fp4_decode_attention_multi return
 * FP4KV_ERR_UNSUPPORTED. */
#define FP4KV_ABL_NORMALIZED_P 8

/* Sets the switches (a bitwise or of FP4KV_ABL_*; 0 = the full method) for every following
 * kv_quant_append and decode call of this process (all GPUs, all host threads: set it before
 * the calls, not concurrently with them).  A cache filled under one setting must be decoded
 * under the same rotation / search switches.  Returns FP4KV_ERR_INVALID_ARG for unknown bits. */
int fp4kv_ablation_set(int flags);

#ifdef __cplusplus
}
#endif

#endif /* FP4KV_ABLATION_H */
