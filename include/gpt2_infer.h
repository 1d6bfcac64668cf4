/*
 * gpt2_infer.h -- autoregressive decoding with the kernels of the GPT-2 step
 * (C ABI): a prefill of the prompt that fills a key / value cache, then one
 * token per sequence per call, and sampling with temperature, top-k and
 * top-p (nucleus) filtering.
 *
 * What it follows: GPT From Scratch, "Architecture diagram" (GPT.generate:
 * temperature + top-k); Genesis model card, "Key Implementation Details"
 * (inference with temperature, top-k and top-p sampling) and "Roadmap" (a KV
 * cache for faster inference).  The model and its parameters are those of
 * gpt2.h (the same flat layout, tied or untied variant).
 *
 * Conventions as in gpt2.h: d_* are device pointers, work is queued on the
 * stream given at init, and the caller owns every buffer.
 */
#ifndef GPT2_INFER_H
#define GPT2_INFER_H

#include <stdint.h>

#include "gpt2.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gpt2_infer gpt2_infer;

typedef struct {
  int64_t cache_bytes;      /* key / value cache: L x max_batch x block_size x 2C
                               activations (bf16 in BF16 mode, else fp32)      */
  int64_t workspace_bytes;  /* activations of one prefill of max_batch x
                               block_size tokens                               */
} gpt2_infer_sizes;

/* Size query (d_cache == NULL: fill *sizes only) or set-up.  d_params: the
 * fp32 parameters (n_params, layout of gpt2.h); d_params_bf16: their bf16
 * copy (BF16 mode; NULL in FP32 mode).  cfg->max_batch is the number of
 * sequences decoded together.  The parameters are read, never written; they
 * must stay valid while the context is used.
 * Errors: GPT2_ERR_ARG (bad config, an FP16 config, NULL buffers, head dim
 * above 256). */
int gpt2_infer_init(const gpt2_config *cfg, const float *d_params, const void *d_params_bf16, void *d_cache,
                    void *d_workspace, void *hip_stream, gpt2_infer_sizes *sizes, gpt2_infer **out);

/* The forward pass over B prompts of T tokens (d_idx int32 (B, T)): fills
 * positions 0 .. T-1 of the cache and writes the fp32 logits of position T-1
 * of each prompt to d_logits (B, Vp).  Sets the decoded length to T.
 * Errors: GPT2_ERR_SEQ_TOO_LONG (T > block_size), GPT2_ERR_BATCH (B < 1,
 * B > max_batch, T < 1); an id outside [0, vocab_size) sets the sticky flag
 * gpt2_infer_sync_status reports (row 0 is used). */
int gpt2_infer_prefill(gpt2_infer *ctx, const int32_t *d_idx, int B, int T, float *d_logits);

/* One token per sequence (d_tokens int32 (B), B of the prefill) at position
 * len: appends its keys and values to the cache and writes the fp32 logits
 * of that position to d_logits (B, Vp); len becomes len + 1.
 * Errors: GPT2_ERR_STATE (no prefill), GPT2_ERR_SEQ_TOO_LONG (len ==
 * block_size: the context window is full). */
int gpt2_infer_decode(gpt2_infer *ctx, const int32_t *d_tokens, float *d_logits);

/* Tokens decoded so far per sequence (the next position), -1 before a prefill. */
int gpt2_infer_length(const gpt2_infer *ctx);

/* Sampling of one token per row of fp32 logits (d_logits (B, ld), columns
 * [0, vocab_size) considered; padded columns never chosen):
 *   temperature <= 0 or top_k == 1: the first largest logit (greedy);
 *   otherwise z = logits / temperature; top_k > 0 keeps the columns whose z
 *   is at least the k-th largest; p = softmax of the kept z; 0 < top_p < 1
 *   keeps the smallest set of most probable columns whose mass reaches
 *   top_p (ties at the threshold kept); the token is the first column at
 *   which the running sum of the kept p, in column order, exceeds
 *   d_uniform[b] (in [0, 1)) times their total.
 * The uniforms are inputs, so the caller's generator decides the draws.
 * Queued on hip_stream.  Errors: GPT2_ERR_ARG (vocab_size above 65,536,
 * NULL pointers, B < 1). */
int gpt2_sample(const float *d_logits, int64_t ld, int B, int vocab_size, float temperature, int top_k,
                float top_p, const float *d_uniform, int32_t *d_tokens, void *hip_stream);

/* Synchronise; GPT2_ERR_TOKEN (and clear it) if an id was out of range. */
int gpt2_infer_sync_status(gpt2_infer *ctx);

void gpt2_infer_destroy(gpt2_infer *ctx);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_INFER_H */
