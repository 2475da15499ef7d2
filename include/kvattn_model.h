/* libkvattn: a random-weight decoder around the KV-cached attention path.
 *
 * The llm-perf-lab README's minimal decoder-only Transformer (its model.py
 * entry: RMSNorm, a GELU MLP, incremental decoding) at any width, driven end
 * to end on one GPU: token and position embeddings, per layer a pre-norm
 * attention block (fused QKV projection, the library's append + decode or
 * prefill kernels, output projection, residual) and a pre-norm GELU MLP
 * block, then a final RMSNorm, the LM head and a greedy argmax.  Readings
 * where the README is silent: RMSNorm x / sqrt(mean(x^2) + 1e-5) * gain, the
 * exact (erf) GELU, an MLP mlp_mult times as wide, learned absolute position
 * embeddings, no biases, an untied LM head, fused QKV rows q | k | v (head
 * major inside each).  The residual stream is fp32; weights, q/k/v and the
 * KV cache are fp16.
 *
 * Weights are one caller-owned device buffer of fp16 values packed in this
 * order (every matrix (out, in), row-major): tok_emb (vocab, d), pos_emb
 * (max_T, d); per layer: ln1 gain (d), wqkv (3d, d), wo (d, d), ln2 gain
 * (d), w_up (mlp, d), w_down (d, mlp); then ln_f gain (d), lm_head (vocab, d);
 * mlp = mlp_mult * d.
 *
 * Status codes, streams and validation as in kvattn.h: every argument is
 * checked on the host before anything is enqueued.
 */
#ifndef KVATTN_MODEL_H_
#define KVATTN_MODEL_H_

#include <stddef.h>
#include <stdint.h>

#include "kvattn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct kvattn_model kvattn_model; /* opaque, library-owned */

/* Number of fp16 values in the packed weight buffer; 0 for a non-positive
 * argument.  Pure host function. */
size_t kvattn_model_weight_elems(int layers, int d_model, int vocab, int max_T, int mlp_mult);

/* Create a decoder for `batch` sequences (1..8) of up to max_T positions over
 * the caller's packed fp16 weights (device; they must outlive the model).
 * d_model / heads must be 32, 64 or 128 and d_model a multiple of 512, at
 * most 1024 (UNSUPPORTED otherwise).  Allocates the model's KV cache
 * (kvattn_cache_alloc), activation buffers and a stream for generation. */
int kvattn_model_create(kvattn_model **out, int layers, int d_model, int heads, int vocab, int max_T,
                        int mlp_mult, int batch, const void *weights);

/* Synchronise the device and release everything the model allocated. */
int kvattn_model_free(kvattn_model *m);

/* Start over: every layer's cache lengths become 0. */
int kvattn_model_reset(kvattn_model *m, void *stream);

/* Current position (cache length) of every sequence, into host_pos[0..batch-1]. */
int kvattn_model_positions(const kvattn_model *m, int32_t *host_pos);

/* Prompt: tokens (device int32, batch x T, row-major) at positions 0..T-1.
 * Fills every layer's cache (STATE unless the caches are empty; CAPACITY if
 * T > max_T).  Writes the last position's logits (device fp32, batch x
 * vocab; may be NULL) and their argmax (device int32, batch; lowest index on
 * ties).  The projections run on the library's own matrix-core GEMM (fp16
 * inputs, fp32 accumulation), the attention as kvattn_prefill.  Token ids
 * outside [0, vocab) are clamped into it. */
int kvattn_model_prefill(kvattn_model *m, const int32_t *tokens, int T, float *logits, int32_t *next,
                         void *stream);

/* One decode step: tokens[b] (device int32) is fed at sequence b's current
 * position; every layer appends its K/V and attends its cache (the
 * library's append and decode kernels).  Logits (device fp32, batch x vocab;
 * may be NULL) and their argmax next (device int32, batch; may alias
 * tokens).  CAPACITY if a sequence is full. */
int kvattn_model_step(kvattn_model *m, const int32_t *tokens, float *logits, int32_t *next, void *stream);

/* Greedy generation of n_steps tokens per sequence: tokens (device int32,
 * batch) holds each sequence's current token and ends holding its last
 * generated one; out_tokens (device int32, n_steps x batch) receives every
 * generated token.  The steps are enqueued back to back on the model's own
 * stream (ordered after `stream` by events) with the tokens kept on the
 * device; `stream` is ordered after the last step.  CAPACITY if a sequence
 * would pass max_T. */
int kvattn_model_generate(kvattn_model *m, int n_steps, int32_t *tokens, int32_t *out_tokens, void *stream);

/* Text of the last HIP error this thread's model calls saw ("" if none). */
const char *kvattn_model_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_MODEL_H_ */
