/*
 * gpt2_train.h -- the training loop around the GPT-2 step of gpt2.h: the
 * learning-rate schedule, a sequential loader over token files, and
 * checkpoints of the whole training state (host-side runtime, C ABI).
 *
 * What the loop follows:
 *   - linear warmup then cosine decay of the learning rate (AxonLM README,
 *     "Key Features": cosine LR + warmup; "Training Recipe": peak 6e-4,
 *     minimum 6e-5, 715 warmup steps, 19,073 steps; GPT From Scratch,
 *     "Architecture diagram": warmup + cosine LR);
 *   - sequential batches from a token stream split over binary shard files
 *     (GPT From Scratch, "Architecture diagram": DataLoaderLite, sequential
 *     batches; AxonLM README, "Quick Start": pre-tokenized binary shards);
 *     a stream too short for one batch is an error (GPT From Scratch, "Key
 *     decisions": explicit failures);
 *   - checkpoint and resume of parameters, AdamW moments and step counter
 *     (AxonLM README, "Key Features": checkpoint resume; Genesis model card,
 *     "Training Features": auto-resume).
 * Error codes are those of gpt2.h, plus GPT2_ERR_IO.
 */
#ifndef GPT2_TRAIN_H
#define GPT2_TRAIN_H

#include <stdint.h>

#include "gpt2.h"

#ifdef __cplusplus
extern "C" {
#endif

#define GPT2_ERR_IO -7 /* a file could not be opened, read, written or parsed */

/* ---- learning-rate schedule ------------------------------------------------ */
typedef struct {
  double max_lr;         /* peak rate, reached at the end of the warmup      */
  double min_lr;         /* floor of the cosine decay                        */
  int64_t warmup_steps;  /* >= 1                                            */
  int64_t max_steps;     /* > warmup_steps: the decay ends here             */
} gpt2_lr_schedule;

/* The rate for optimizer step `step` (counted from 0):
 *   step < warmup:               max_lr (step + 1) / warmup
 *   warmup <= step <= max_steps: min_lr + (max_lr - min_lr) (1 + cos(pi r)) / 2,
 *                                r = (step - warmup) / (max_steps - warmup)
 *   step > max_steps:            min_lr
 * Host only.  Returns NaN for an invalid schedule (NULL, warmup < 1,
 * max_steps <= warmup) or step < 0. */
double gpt2_lr_at(const gpt2_lr_schedule *sched, int64_t step);

/* ---- sequential token loader ------------------------------------------------ */
/* Shards are files of little-endian token ids (dtype 0: uint16, as GPT-2's
 * 50,257-id vocabulary fits 16 bits; dtype 1: int32), read through mmap.  One
 * call of gpt2_loader_next yields one optimizer step of k micro-batches of
 * B x T tokens: the window w = s[p, p + k B T + 1) of the current shard s at
 * position p gives micro-batch i as x = w[i B T, (i + 1) B T) and
 * y = w[i B T + 1, (i + 1) B T + 1), both (B, T) row-major; then p advances
 * by k B T.  When fewer than k B T + 1 ids remain, the loader moves to the
 * next shard at position 0 (after the last shard, to the first).  Shards
 * shorter than one window are skipped. */
typedef struct gpt2_loader gpt2_loader;

/* Opens n_shards files (paths: host array of C strings).  Errors:
 * GPT2_ERR_ARG (NULL, n_shards < 1, k, B or T < 1, bad dtype), GPT2_ERR_IO
 * (a file cannot be opened or mapped, or its size is not a multiple of the
 * id size), GPT2_ERR_BATCH (no shard holds one window of k B T + 1 ids: the
 * data is too small for one batch). */
int gpt2_loader_open(const char *const *paths, int n_shards, int32_t dtype, int32_t vocab_size, int k, int B,
                     int T, gpt2_loader **out);

/* Copies the next step's ids into the device arrays d_idx and d_targets
 * (k, B, T) int32 on the HIP stream hip_stream (asynchronous; the loader
 * stages them in one of two pinned host buffers, reused once the copy that
 * read it has completed) and advances.  Errors: GPT2_ERR_ARG, GPT2_ERR_TOKEN
 * (an id of the window is outside [0, vocab_size); the loader does not
 * advance), GPT2_ERR_HIP. */
int gpt2_loader_next(gpt2_loader *ld, int32_t *d_idx, int32_t *d_targets, void *hip_stream);

/* The same window in host memory (h_idx, h_targets: k B T int32 each). */
int gpt2_loader_next_host(gpt2_loader *ld, int32_t *h_idx, int32_t *h_targets);

/* Position of the next window (shard index, id offset), e.g. for a
 * checkpoint, and a jump to a saved one.  seek returns GPT2_ERR_ARG for a
 * position at which no whole window fits. */
int gpt2_loader_state(const gpt2_loader *ld, int64_t *shard, int64_t *pos);
int gpt2_loader_seek(gpt2_loader *ld, int64_t shard, int64_t pos);

/* Waits for the loader's copies, unmaps the shards, frees the loader. */
void gpt2_loader_close(gpt2_loader *ld);

/* ---- checkpoints -------------------------------------------------------------- */
/* Writes the training state of ctx to `path`: the config, the AdamW step
 * counter, n_extra caller words (e.g. the loader position; at most 16), the
 * loss scale and its growth counter (FP16 contexts only), and the fp32
 * params, adam_m and adam_v (12 bytes per parameter).  Waits for the
 * work queued on the context's stream, then writes `path`.tmp and renames it
 * over `path`, so a crash never leaves a partial file under that name.
 * Errors: GPT2_ERR_ARG, GPT2_ERR_IO, GPT2_ERR_HIP. */
int gpt2_checkpoint_save(gpt2_ctx *ctx, const char *path, const int64_t *extra, int n_extra);

/* Restores a checkpoint written by gpt2_checkpoint_save into ctx: params,
 * adam_m, adam_v, the step counter, the loss scaler's scale and growth
 * counter (FP16), and the 16-bit copy of params (grads are
 * left as they are).  *n_extra: in, room in extra (at most 16); out, the
 * words restored.  Errors: GPT2_ERR_IO (unreadable or not a checkpoint),
 * GPT2_ERR_ARG (its model config differs from the context's: every field but
 * max_batch must match), GPT2_ERR_HIP. */
int gpt2_checkpoint_load(gpt2_ctx *ctx, const char *path, int64_t *extra, int *n_extra);

#ifdef __cplusplus
}
#endif

#endif /* GPT2_TRAIN_H */
