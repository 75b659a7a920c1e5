/* C ABI of the generation stack around the decoder layer: token embedding,
 * L decoder layers (llama_layer.h), final RMSNorm, LM head, and the sampling
 * step, with a native generation loop.
 *
 * Sources, cited by page title and section:
 *   "LLM 核心机制交互讲义" (LLM mechanics lecture notes): Ch.02, the
 *     decoder-only data flow (X_0 = E[ids], L pre-norm blocks, [B,T,V]
 *     logits, generation reads the last position); Ch.04, prefill writes every
 *     layer's K/V cache, decode feeds one new token per sequence; Ch.05,
 *     sampling: temperature softmax(z / tau), greedy as an explicit argmax,
 *     the top-p nucleus (descending probability, smallest prefix reaching p,
 *     renormalised), the sign-aware repetition penalty on generated tokens,
 *     EOS as a per-row stop with max tokens as the hard bound, and the
 *     end-to-end loop.
 *   "LMDrive 大语言模型（LLM）核心推理单元": §2.1 RMSNorm (the final norm).
 *
 * Readings where the pages leave a step open: the final RMSNorm has a gain
 * and the LM head has no bias and its own weights; the repetition penalty
 * applies once per distinct generated token (not to the prompt); ties in the
 * nucleus order and in greedy go to the smaller token id; the draw inside the
 * nucleus is the inverse CDF in ascending token id with a caller-supplied
 * uniform u in [0, 1) (the library draws no random numbers).
 *
 * All pointers are device pointers unless marked "host".  Calls are
 * asynchronous on `stream` except create and generate, which synchronise it.
 * Status codes are those of llama_layer.h; llama_layer_last_error() gives the
 * detail of a failure on the calling thread. */
#ifndef LLAMA_MODEL_H
#define LLAMA_MODEL_H

#include <stdint.h>

#include "llama_layer.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  llama_layer_config layer; /* every layer's configuration (shared) */
  int32_t n_layers;         /* L >= 1 */
  int32_t vocab;            /* V >= 2 */
} llama_model_config;

/* Device pointers in the layer dtype, [out, in] row-major; copied at create. */
typedef struct {
  const void* embed;                 /* [V, d] */
  const void* final_norm;            /* [d] */
  const void* lm_head;               /* [V, d] */
  const llama_layer_weights* layers; /* host array of n_layers entries */
} llama_model_weights;

typedef struct {
  float temperature;        /* 0: greedy argmax; > 0: softmax(z / temperature) */
  float top_p;              /* nucleus mass in (0, 1]; 1: every token */
  float repetition_penalty; /* r >= 1 (1: off) */
  int32_t eos_id;           /* token that ends a row (not appended); -1: none */
} llama_sampling;

typedef struct llama_model llama_model;

/* Create the L layers (llama_layer_create each), copy the embedding and the
 * final gain, and convert the LM head to the weight-streaming GEMM's operand
 * order.  Errors: NULL, INVALID (as for the layer, or L < 1, V < 2), the
 * layer's errors, HIP, ALLOC. */
int llama_model_create(const llama_model_config* cfg, const llama_model_weights* w, void* stream,
                       llama_model** out);

/* Free the layers and every buffer the handle owns.  NULL is a no-op. */
void llama_model_destroy(llama_model* model);

/* Prefill B prompts of T tokens each at positions 0..T-1:
 *   ids        [B*T] int32 token ids (an id outside [0, V) embeds as zeros)
 *   k_caches, v_caches  host arrays of L device pointers, each [B, Hkv,
 *              max_pos, dh] in the layer dtype (as for llama_layer_prefill)
 *   logits     [B, V] fp32: the last position's logits of each prompt.
 * Errors: NULL, INVALID (B, T < 1), CAPACITY (B > 128, B*T > max_tokens or
 * T > max_pos), HIP. */
int llama_model_prefill(llama_model* model, const int32_t* ids, int32_t B, int32_t T,
                        void* const* k_caches, void* const* v_caches, float* logits, void* stream);

/* One decode step: token ids[b] at positions[b] for each of B sequences;
 * logits [B, V] fp32.  Errors as for prefill with T = 1. */
int llama_model_decode(llama_model* model, const int32_t* ids, const int32_t* positions, int32_t B,
                       void* const* k_caches, void* const* v_caches, float* logits, void* stream);

/* One token per row from logits [B, ld] (the first V entries of each row):
 * the repetition penalty over history[b, 0 .. history_len[b]) (ids outside
 * [0, V) are ignored), then greedy or a temperature softmax restricted to the
 * top-p nucleus, drawn with uniforms[b] (unused when greedy; may be NULL
 * then).  out_ids [B].  logits are not modified.  eos_id is not used here.
 * Errors: NULL, INVALID (B < 1, V < 2 or V > 2^20, ld < V, temperature < 0,
 * top_p outside (0, 1], penalty < 1, history_ld < 0), HIP. */
int llama_sample(const float* logits, int32_t B, int32_t vocab, int32_t ld, const llama_sampling* params,
                 const int32_t* history, const int32_t* history_len, int32_t history_ld,
                 const float* uniforms, int32_t* out_ids, void* stream);

/* The whole loop: prefill the B prompts (host [B*T], positions 0..T-1), then
 * repeat up to max_new times: sample every unfinished row (uniforms host
 * [max_new * B], row-major by step, NULL for greedy), end a row at eos_id
 * (not appended) or after max_new tokens, and decode the new tokens.  A
 * finished row appends nothing more.  out_ids host [B * max_new] (row b's
 * tokens at b * max_new), out_len host [B].  Synchronises the stream.
 * Errors: as for prefill and llama_sample, INVALID (max_new < 1 or
 * T + max_new > max_pos), ALLOC. */
int llama_model_generate(llama_model* model, const int32_t* prompt, int32_t B, int32_t T, int32_t max_new,
                         const llama_sampling* params, const float* uniforms, void* const* k_caches,
                         void* const* v_caches, int32_t* out_ids, int32_t* out_len, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LLAMA_MODEL_H */
