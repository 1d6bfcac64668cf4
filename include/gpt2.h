/*
 * gpt2.h -- C ABI of one GPT-2 pre-training step on one AMD Instinct MI355X
 * (gfx950).  Every step of the path runs in hand-written HIP kernels; the
 * caller (e.g. PyTorch) owns every device buffer and the stream.
 *
 * What the step computes (the pages are GPT-2 pre-training write-ups):
 *   - the pre-LN decoder: token + position embedding, N blocks of
 *     [LayerNorm -> causal multi-head self-attention -> residual add;
 *      LayerNorm -> MLP C->4C (tanh GELU) -> 4C->C -> residual add],
 *     final LayerNorm, lm_head tied to the token embedding
 *     (hanzo gpt LLM.md, "GPT Model Architecture"; Genesis model card,
 *     "Architecture"; AxonLM README, "Key Features": weight tying);
 *   - mean softmax cross-entropy over every position, the softmax taken over
 *     the whole padded vocabulary (GPT From Scratch, "Key decisions":
 *     50,257 padded to 50,304);
 *   - gradient accumulation over equal micro-batches, each loss scaled by 1/k
 *     (AxonLM README, "Key Features"; GPT From Scratch, "Key decisions");
 *   - global-norm gradient clipping and AdamW with decoupled weight decay on
 *     tensors of two or more dimensions only, betas (0.9, 0.95)
 *     (AxonLM README, "Training Recipe").
 *
 * Conventions for every call:
 *   - Pointers named d_* and every pointer inside gpt2_buffers are DEVICE
 *     pointers; gpt2_config / gpt2_sizes pointers are HOST pointers.
 *   - All work is queued on the stream given to gpt2_init (a hipStream_t, or
 *     NULL for the default stream) and is asynchronous: a return of GPT2_OK
 *     means the work was queued.  Scalar results land in caller device memory.
 *   - The library never allocates device memory: activations and scratch
 *     live in the caller's workspace buffer.
 *   - One context per stream; a context is not thread-safe.
 *
 * Parameter layout: one flat fp32 vector, tensors in this order, each
 * row-major; weights are (out, in) so that y = x W^T.  Per-block tensors are
 * stored for all L blocks contiguously ([L, ...]):
 *   wte (Vp, C); wpe (block_size, C);
 *   ln1_w [L, C]; ln1_b [L, C]; qkv_w [L, 3C, C]; qkv_b [L, 3C];
 *   proj_w [L, C, C]; proj_b [L, C]; ln2_w [L, C]; ln2_b [L, C];
 *   fc_w [L, 4C, C]; fc_b [L, 4C]; fcproj_w [L, C, 4C]; fcproj_b [L, C];
 *   lnf_w (C); lnf_b (C); and lm_head (Vp, C) in the untied variant (qkv_b
 *   is absent from the layout without a QKV bias).
 * grads, adam_m and adam_v share this layout.  gpt2_tensor_info enumerates it.
 * Weight decay applies to wte, wpe, qkv_w, proj_w, fc_w, fcproj_w and lm_head.
 */
#ifndef GPT2_H
#define GPT2_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define GPT2_OK                0
#define GPT2_ERR_ARG          -1  /* bad config or argument, NULL pointer      */
#define GPT2_ERR_SEQ_TOO_LONG -2  /* T > block_size                            */
#define GPT2_ERR_BATCH        -3  /* B < 1, B > max_batch, k < 1, BF16 B*T % 8 */
#define GPT2_ERR_STATE        -4  /* backward without a matching forward       */
#define GPT2_ERR_TOKEN        -5  /* an id or target outside [0, vocab_size)   */
#define GPT2_ERR_HIP          -6  /* a HIP call or kernel launch failed        */

/* model variants (gpt2_config.variant): the untied model of the Genesis
   model card ("Model Specs": 163,009,536 parameters at vocab 50,257; the
   lm_head kept separate from the token embedding, and no bias on the QKV
   projection) is GPT2_UNTIED_HEAD | GPT2_NO_QKV_BIAS. */
#define GPT2_UNTIED_HEAD 1  /* the lm_head is its own (Vp, C) tensor "lm_head",
                               last in the layout, decayed                 */
#define GPT2_NO_QKV_BIAS 2  /* the QKV projection has no bias (no qkv_b)   */

/* precision modes */
#define GPT2_FP32 0  /* every tensor fp32                                        */
#define GPT2_BF16 1  /* bf16 GEMM/attention operands and activations, fp32
                        residual stream, statistics, loss, grads, master
                        weights and AdamW moments                              */
#define GPT2_FP16 2  /* as GPT2_BF16 with IEEE half (fp16) in place of bf16,
                        and dynamic loss scaling (gpt2_loss_scaler): the
                        Genesis model card's "Mixed Precision (AMP) -- FP16"
                        ("Training Features"), which bf16 does without (AxonLM
                        README, "Key Features": bfloat16 AMP needs no loss
                        scaling).  params_bf16 holds the fp16 copy.          */

typedef struct {
  int32_t n_layer;            /* L                                             */
  int32_t n_head;             /* NH; C % NH == 0                               */
  int32_t n_embd;             /* C; C % 8 == 0                                 */
  int32_t block_size;         /* largest T (rows of wpe)                       */
  int32_t vocab_size;         /* ids and targets lie in [0, vocab_size)        */
  int32_t padded_vocab_size;  /* Vp >= vocab_size: rows of wte, softmax width;
                                 Vp % 8 == 0 in BF16 mode                      */
  int32_t precision;          /* GPT2_FP32, GPT2_BF16 or GPT2_FP16; the 16-bit
                                 modes need C/NH == 64                         */
  int32_t max_batch;          /* largest micro-batch B the workspace holds     */
  int32_t variant;            /* 0 (GPT-2), or GPT2_UNTIED_HEAD and/or
                                 GPT2_NO_QKV_BIAS                              */
} gpt2_config;

typedef struct {
  float *params;      /* n_params fp32 master weights (caller writes them)    */
  float *grads;       /* n_params fp32                                         */
  float *adam_m;      /* n_params fp32                                         */
  float *adam_v;      /* n_params fp32                                         */
  void  *params_bf16; /* n_params bf16 copy of params (BF16 mode; else NULL)   */
  void  *workspace;   /* workspace_bytes, 256-byte aligned                     */
} gpt2_buffers;

typedef struct {
  int64_t n_params;         /* elements of params / grads / adam_m / adam_v    */
  int64_t workspace_bytes;  /* bytes of workspace for this config              */
  int64_t params_bf16_bytes;/* bytes of params_bf16 (0 in FP32 mode)           */
} gpt2_sizes;

typedef struct gpt2_ctx gpt2_ctx;  /* opaque host-side context */

/*
 * Size query and set-up.  The config is the model description of the pages'
 * GPTConfig (GPT From Scratch, "Problem": GPTConfig() is the 124M shape, the
 * toy is 4 layers, 4 heads, 128 dims, block 64; AxonLM README, "Model
 * Scales": the four GPT-2 scales).
 *   bufs == NULL: validate *cfg and fill *sizes only (no HIP call; *out is
 *   left untouched).  Otherwise bind the caller's buffers, zero grads, adam_m
 *   and adam_v on the stream, build the bf16 copy of params (BF16 mode), set
 *   the AdamW step counter to 0 and return a context in *out.
 * Errors: GPT2_ERR_ARG for an invalid config (C % NH != 0, C % 8 != 0,
 *   Vp < vocab_size, BF16 with C/NH != 64, non-positive sizes) or a NULL
 *   buffer; GPT2_ERR_HIP if a launch fails.
 */
int gpt2_init(const gpt2_config *cfg, const gpt2_buffers *bufs, void *hip_stream,
              gpt2_sizes *sizes, gpt2_ctx **out);

/*
 * Forward pass of B sequences of T tokens and the mean cross-entropy
 * (hanzo gpt LLM.md, "GPT Model Architecture" and "Transformer Blocks": token
 * + position embedding, pre-LN blocks, final LayerNorm, tied head; GPT From
 * Scratch, "Key decisions": tanh-GELU MLP with 4x expansion and the vocabulary
 * padded to 50,304; "Results": the initial loss sits near ln V).
 *   d_idx, d_targets: int32 device arrays (B, T), row-major.  The position of
 *   token (b, t) is t.  d_idx must stay valid until the matching backward.
 *   *d_loss (device fp32) = loss_scale * mean over the B*T positions of
 *   logsumexp(logits) - logit[target], the softmax over all Vp columns.
 * Saves activations in the workspace for gpt2_backward (one forward is kept;
 * a new forward replaces it).
 * Errors: GPT2_ERR_SEQ_TOO_LONG if T > block_size; GPT2_ERR_BATCH if B < 1 or
 *   B > max_batch or T < 1, or in BF16 mode if B*T is not a multiple of 8 (the
 *   weight-gradient GEMMs contract over tokens in 16-byte rows); GPT2_ERR_ARG
 *   for NULL pointers.  An id or target
 *   outside [0, vocab_size) sets a sticky device flag (row 0 / class 0 is used
 *   in its place) that gpt2_sync_status reports as GPT2_ERR_TOKEN.
 */
int gpt2_forward_loss(gpt2_ctx *ctx, const int32_t *d_idx, const int32_t *d_targets,
                      int B, int T, float loss_scale, float *d_loss);

/*
 * Backward of the last forward (the closed-form gradients of every step of
 * gpt2_forward_loss; the tied head of AxonLM README, "Key Features", makes
 * wte one tensor with one gradient): ADDS loss_scale * d(loss)/d(param) into grads
 * (the tied wte receives both its lm_head and its embedding gradient).
 * Deterministic: no floating-point atomics; fixed-order reductions.
 * Errors: GPT2_ERR_STATE if no forward is pending.
 */
int gpt2_backward(gpt2_ctx *ctx);

/*
 * Gradient accumulation over k equal micro-batches (AxonLM README, "Key
 * Features": total batch / micro-batch; GPT From Scratch, "Key decisions": it
 * matches one large batch).  One accumulation: zero grads, then for i < k
 * a forward with loss_scale 1/k on micro-batch i (d_idx + i*B*T,
 * d_targets + i*B*T) followed by its backward.  *d_mean_loss (device fp32) = sum_i loss_i / k.
 * Errors: as gpt2_forward_loss; GPT2_ERR_BATCH if k < 1.
 */
int gpt2_accumulate(gpt2_ctx *ctx, const int32_t *d_idx, const int32_t *d_targets,
                    int k, int B, int T, float *d_mean_loss);

/*
 * Global-norm clip and one AdamW step (AxonLM README, "Training Recipe":
 * clip 1.0, betas 0.9 / 0.95, weight decay 0.1 on 2-D tensors only; GPT From
 * Scratch, "Key decisions": decay only on parameters of two or more
 * dimensions; Genesis model card, "Training Features": clip_grad_norm_ at
 * 1.0) (the step counter t becomes t + 1):
 *   n = ||grads||_2 over every parameter (wte counted once);
 *   c = max_norm / (n + 1e-6); the gradients are scaled by c iff c < 1;
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2;
 *   p = p (1 - lr weight_decay) for decayed tensors, then
 *   p = p - lr (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps);
 *   and the bf16 copy of params is refreshed (BF16 mode).
 * *d_norm (device fp32) receives n; *d_clipped (device int32) 1 iff scaled.
 * grads are left unscaled.
 * FP16 mode: the gradients hold S times the true gradients (S the loss scale
 * the accumulation used); n is that of the true gradients and the update
 * uses g / S.  If n is not finite the step is skipped: params, moments, the
 * fp16 copy and t are left as they were.  Then S is updated as
 * gpt2_loss_scaler describes.  The call waits for the stream (the scale
 * update needs the step's overflow flag).
 * Errors: GPT2_ERR_ARG for NULL pointers.
 */
int gpt2_clip_adamw_step(gpt2_ctx *ctx, float lr, float beta1, float beta2, float eps,
                         float weight_decay, float max_norm, float *d_norm,
                         int32_t *d_clipped);

/*
 * Dynamic loss scaling of an FP16 context (the fp16 AMP of the Genesis model
 * card, "Training Features"; the pages give no constants, so a context starts
 * with those of PyTorch's GradScaler: scale 65536, growth factor 2, backoff
 * factor 0.5, growth interval 2000).  Every forward of the context forms the
 * gradient of loss_scale * scale * loss; gpt2_clip_adamw_step unscales, and
 * after it the scale becomes scale * backoff_factor if the step was skipped
 * (a gradient was not finite), or scale * growth_factor once growth_interval
 * consecutive steps were not skipped (good_steps counts them; a growth that
 * would overflow fp32 is not taken).
 * gpt2_loss_scaler sets the whole state (also to restore it);
 * gpt2_loss_scaler_state reads it, with skipped = 1 iff the last step was
 * skipped.  Host only.
 * Errors: GPT2_ERR_STATE unless ctx is an FP16 context; GPT2_ERR_ARG for a
 * scale that is not finite and positive, growth_factor < 1, backoff_factor
 * outside (0, 1], growth_interval < 1 or good_steps outside
 * [0, growth_interval), or NULL pointers.
 */
int gpt2_loss_scaler(gpt2_ctx *ctx, float scale, float growth_factor, float backoff_factor,
                     int32_t growth_interval, int32_t good_steps);
int gpt2_loss_scaler_state(const gpt2_ctx *ctx, float *scale, int32_t *good_steps, int32_t *skipped);

/*
 * gpt2_clip_adamw_step without a context or workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The same kernels and the same
 * arithmetic as gpt2_clip_adamw_step on the flat vectors of *bufs laid out
 * for *cfg (params, grads, adam_m, adam_v, and params_bf16 in BF16 mode;
 * workspace is ignored), with t the new AdamW step number (>= 1).  The
 * norm's partial sums and the clip factor live in a static device array of
 * the library (8,448 bytes on each GPU, held until the process ends) instead
 * of a workspace; the call allocates nothing.  Calls that overlap on one GPU
 * (two streams, or two threads) share that array and race: serialise them.
 * The device current on the calling thread must be the stream's device.
 * Errors: GPT2_ERR_ARG for an invalid config, an FP16 config (its loss
 * scaler lives in a context), NULL pointers, t < 1 or more
 * than 2^40 parameters; GPT2_ERR_HIP if the scratch address cannot be found
 * or a launch fails.
 */
int gpt2_clip_adamw_step_static(const gpt2_config *cfg, const gpt2_buffers *bufs,
                                void *hip_stream, int64_t t, float lr, float beta1,
                                float beta2, float eps, float weight_decay,
                                float max_norm, float *d_norm, int32_t *d_clipped);

/* Frees the host context (no device memory is owned). */
void gpt2_destroy(gpt2_ctx *ctx);

/* ---- helpers beyond the step itself --------------------------------------*/

/* Synchronise the stream; return GPT2_ERR_TOKEN (and clear the flag) if a
   kernel met an out-of-range id or target since the last call, GPT2_ERR_HIP on
   a HIP error, else GPT2_OK. */
int gpt2_sync_status(gpt2_ctx *ctx);

/* After the caller rewrote params on the device: rebuild the bf16 copy. */
int gpt2_sync_params(gpt2_ctx *ctx);

/* Read / set the AdamW step counter (to resume from saved p, m, v). */
int64_t gpt2_get_step(const gpt2_ctx *ctx);
int gpt2_set_step(gpt2_ctx *ctx, int64_t t);

/* Enumerate the parameter tensors in layout order: index in [0, 15..17); fills the
   name, element offset into the flat vector, element count, rank and the
   dims (at most 3).  Host only.  Returns GPT2_ERR_ARG past the last tensor. */
int gpt2_tensor_info(const gpt2_config *cfg, int index, const char **name,
                     int64_t *offset, int64_t *numel, int32_t *ndim, int64_t *dims);

/* Device address of a saved activation of the last forward (for tests):
   name in {"resid", "ln1", "ln1_mean", "ln1_rstd", "qkv", "atty", "lse",
   "ln2", "fcgd", "fcg", "lnf", "logits", "row_loss", "emb_sorted_ids",
   "emb_sorted_pos", "dresid"}; layer selects the block (for "resid", the
   index 0..2L of the residual stream).  "fcgd" is gelu'(u) and "fcg" gelu(u)
   for the MLP pre-activation u (u itself is not kept).  dtype: 0 fp32,
   1 bf16, 2 int32, 3 fp16. */
int gpt2_activation(gpt2_ctx *ctx, const char *name, int layer, void **ptr,
                    int64_t *numel, int32_t *dtype);

/* The embedding part of the backward on its own: ADDS to grads
     wte[idx[b, t]] += dx0[b, t, :]   (summed per id in position order) and
     wpe[t]        += sum_b dx0[b, t, :]
   for d_idx int32 (B, T) and d_dx0 fp32 (B, T, C) device arrays, with the
   same sort and fixed-order segment sums that gpt2_backward uses (the
   gradient of x0 = wte[idx] + wpe[t]; hanzo gpt LLM.md, "GPT Model
   Architecture": token + position embeddings).  Ids must lie in
   [0, vocab_size) (gpt2_forward_loss checks them; this call does not).
   Errors: GPT2_ERR_ARG, GPT2_ERR_SEQ_TOO_LONG, GPT2_ERR_BATCH as for
   gpt2_forward_loss. */
int gpt2_embedding_backward(gpt2_ctx *ctx, const int32_t *d_idx, const float *d_dx0,
                            int B, int T);

/* Per-launch timing with HIP events on the context's stream.  site: a leading
   run of the dot-separated parts of launch-site names (e.g. "gemm.fwd.lmhead",
   "attn.fwd", "gemm"; "gemm.fwd.fc" does not match "gemm.fwd.fcproj"), or NULL
   to stop.  Enabling clears the record.  gpt2_timing_read synchronises and
   returns the summed kernel time, the launch count and the summed
   algorithmic flops and bytes of the matched launches. */
int gpt2_timing_enable(gpt2_ctx *ctx, const char *site);
int gpt2_timing_read(gpt2_ctx *ctx, double *total_ms, int64_t *launches,
                     double *flops, double *bytes);

/* The same record split by launch site: index enumerates the distinct sites
   of the recorded launches in order of first launch (GPT2_ERR_ARG past the
   last).  Synchronises the stream.  *site is a static string; *gemm_cfg is
   the GEMM tile configuration of the site's last launch (0..22 for the bf16
   tiles, 100 for the fp32 GEMM, -2 for the grouped weight-gradient launch,
   -1 for a launch that is not a GEMM). */
int gpt2_timing_site(gpt2_ctx *ctx, int index, const char **site, double *total_ms,
                     int64_t *launches, double *flops, double *bytes, int32_t *gemm_cfg);

/* HBM stream probe: one launch of a plain fp32 stream on `stream` (NULL: the
   default stream), the reference rate that the HBM-bound kernels of the step
   are measured against; not a step of the method.  Each workgroup streams
   one contiguous range once.  mode 0 reads n floats of d_src (eight 16-byte
   loads in flight per thread) and writes one partial sum per wave to d_dst,
   which must hold at least 4 ceil(n / 8192) floats (their total is the sum
   of the n floats); mode 1
   writes 0.5 to n floats of d_dst (d_src unused, may be NULL); mode 2 copies
   n floats from d_src to d_dst.  Device pointers, 16-byte aligned, the
   caller's memory; n > 0 and a multiple of 4.  Asynchronous.
   Errors: GPT2_ERR_ARG for a bad mode, size, NULL or misaligned pointer;
   GPT2_ERR_HIP if the launch fails. */
int gpt2_stream_probe(int mode, const float *d_src, float *d_dst, int64_t n, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_H */
