/*
 * llama_layer.h — C ABI of an MI355X (gfx950) library for one pre-norm LLaMA
 * decoder layer forward, with grouped-query attention and a KV cache.
 *
 * What one call computes (sources cited by page title and section):
 *   "LMDrive LLM core inference unit" page (LMDrive 大语言模型（LLM）核心推理单元),
 *     §2.5 LlamaDecoderLayer: pre-norm, residual + attention, residual + MLP;
 *     §2.1 LlamaRMSNorm; §2.2 LlamaRotaryEmbedding (rotate-half RoPE);
 *     §2.3 LlamaAttention (q/k/v/o projections, KV-cache append, repeat_kv GQA,
 *          softmax(q k^T / sqrt(dh) + mask) v); §2.4 LlamaMLP (SwiGLU).
 *   "LLM mechanics lecture notes" (LLM 核心机制交互讲义), Ch.02: the block
 *     equation X' = X + Attn(RMSNorm(X)), X'' = X' + SwiGLU(RMSNorm(X')),
 *     §02.1 causal mask added before the softmax; Ch.04: prefill vs decode,
 *     K/V appended to the cache, decode RoPE position = cache length.
 *
 *   xn  = RMSNorm(x; attn_norm, eps)
 *   q,k,v = xn Wq^T, xn Wk^T, xn Wv^T             (no bias)
 *   q,k  <- rotate-half RoPE at each token's position (base rope_base)
 *   K/V cache slot `pos` of the token's sequence <- k (rotated), v
 *   o   = softmax(q K^T / sqrt(dh), slots j <= pos only) V   per query head;
 *         query head h reads kv head h / (n_heads / n_kv_heads)
 *   X'  = x + o Wo^T
 *   xn2 = RMSNorm(X'; ffn_norm, eps)
 *   y   = X' + (SiLU(xn2 Wgate^T) * (xn2 Wup^T)) Wdown^T
 *
 * Layout.  Row-major everywhere.  Weights use nn.Linear's [out, in] layout.
 * Hidden states are [tokens, d_model]; token (b, t) of a prefill call is row
 * b*T + t.  Each KV cache (K and V separately) is [B, n_kv_heads, max_pos,
 * head_dim]: slot p of sequence b, kv head g starts at element
 * ((b*n_kv_heads + g)*max_pos + p)*head_dim.  Keys are stored after RoPE.
 * Positions are int32 on the device.
 *
 * Precision.  LLAMA_BF16: weights, activations, gains and caches are bf16;
 * products accumulate in fp32; RMSNorm, RoPE, softmax and the SwiGLU
 * epilogue run in fp32; the residual stream X' stays fp32 between the two
 * halves.  LLAMA_F32: everything fp32 (any shape; meant for small layers).
 *
 * Streams and ownership.  All pointers except the config/weights structs are
 * device pointers.  Calls enqueue work on `stream` (a hipStream_t; NULL is
 * the default stream) and return without waiting; a return of LLAMA_OK means
 * "enqueued".  x, y, positions and the caches stay owned by the caller;
 * y may be the same buffer as x, but must not partially overlap it.  One
 * handle owns scratch memory, so calls on the same handle must not overlap
 * (serialise them on one stream).  No call allocates device memory except
 * llama_layer_create.
 *
 * Errors.  Functions return 0 (LLAMA_OK) or a negative status; nothing is
 * launched when a call fails its argument checks.  llama_layer_last_error()
 * returns a thread-local message for the last failure on the calling thread.
 */
#ifndef LLAMA_LAYER_H
#define LLAMA_LAYER_H

#include <stdint.h>
#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  LLAMA_OK = 0,
  LLAMA_ERR_NULL = -1,         /* a required pointer is NULL */
  LLAMA_ERR_INVALID = -2,      /* inconsistent sizes (see llama_layer_create) */
  LLAMA_ERR_UNSUPPORTED = -3,  /* valid, but a shape this build has no kernel for */
  LLAMA_ERR_CAPACITY = -4,     /* B*T above max_tokens, or T above max_pos */
  LLAMA_ERR_HIP = -5,          /* a HIP runtime call failed */
  LLAMA_ERR_ALLOC = -6         /* device or host allocation failed */
};

typedef enum { LLAMA_F32 = 0, LLAMA_BF16 = 1 } llama_dtype;

typedef struct {
  int32_t d_model;     /* hidden size d */
  int32_t n_heads;     /* query heads H */
  int32_t n_kv_heads;  /* key/value heads Hkv; H % Hkv == 0 (Hkv == H: MHA) */
  int32_t head_dim;    /* dh (even); bf16 needs 128 */
  int32_t d_ff;        /* intermediate size f */
  float rms_eps;       /* RMSNorm epsilon, inside the square root (1e-6) */
  float rope_base;     /* RoPE base (10000) */
  int32_t max_pos;     /* cache capacity per sequence; every position < max_pos */
  int32_t max_tokens;  /* largest B*T a call may pass; sizes the scratch */
  int32_t dtype;       /* llama_dtype */
  int32_t bidirectional; /* 0: causal (the decoder layer).  1: the encoder-style
                            variant without the causal mask ("LARQL multimodal
                            support" page: the SigLIP encoder's attention is the
                            causal kernel without its future-column condition):
                            every new token of sequence b attends to slots
                            0 .. P_b, P_b = the largest of b's positions in the
                            call.  A decode call (T = 1) is the same either way. */
} llama_layer_config;

/* Device pointers to the caller's weights, each [out, in] row-major in the
 * layer dtype.  llama_layer_create copies them into buffers the handle owns,
 * so the caller may free them once create has returned. */
typedef struct {
  const void *attn_norm; /* [d] */
  const void *wq;        /* [H*dh, d] */
  const void *wk;        /* [Hkv*dh, d] */
  const void *wv;        /* [Hkv*dh, d] */
  const void *wo;        /* [d, H*dh] */
  const void *ffn_norm;  /* [d] */
  const void *w_gate;    /* [f, d] */
  const void *w_up;      /* [f, d] */
  const void *w_down;    /* [d, f] */
} llama_layer_weights;

typedef struct llama_layer llama_layer;

/* Validate the config, allocate the handle's weights, RoPE table (cos and sin
 * of p * base^(-2i/dh), built in fp64 on the host) and scratch, and copy the
 * weights.  Blocks until the copies on `stream` are done.  The scratch is
 * sized by max_tokens, plus, for bf16 layers with max_tokens > 128, one
 * 128 x 512 fp32 tile per compute unit (64 MiB on 256 CUs) for the partial
 * sums of projections that split their reduction over several workgroups.
 * With the environment variable LLAMA_LAYER_CHECK=1 at creation, every later
 * prefill/decode call of the handle first validates its positions on the
 * device and waits for the result (a debug aid: it synchronises the stream).
 * Errors: NULL (any pointer), INVALID (non-positive sizes, H % Hkv != 0, odd
 * dh, non-finite eps/base), UNSUPPORTED (bf16 with dh != 128, d or f not
 * multiples of 128, or d above 8192 other than 16384), HIP, ALLOC. */
int llama_layer_create(const llama_layer_config* cfg, const llama_layer_weights* w,
                       void* stream, llama_layer** out);

/* Prefill: B sequences of T new tokens each.
 * x, y       [B*T, d] (layer dtype)
 * positions  [B*T] int32: token (b, t) sits at positions[b*T + t]; within a
 *            sequence the positions are distinct and each is < max_pos.  Its
 *            rotated key and its value are written to cache slot positions[.];
 *            its query attends to slots 0 .. positions[.] of sequence b
 *            (bidirectional: 0 .. the largest position of b in the call), so
 *            slots below the sequence's new positions must already hold that
 *            sequence's earlier keys and values (a chunked prefill continues a
 *            cache; positions 0..T-1 start one).
 * k_cache, v_cache  [B, Hkv, max_pos, dh] (layer dtype), updated in place.
 * bf16 precision: the attention multiplies its softmax weights (fp16, 11
 * significant bits) with the values converted to fp16, exact for value
 * entries within +-65504 (larger magnitudes saturate there).
 * Positions are not otherwise validated: a token whose position is outside
 * [0, max_pos) writes no cache slot and gets undefined output values (every
 * access stays inside the buffers); repeated positions in a sequence give
 * undefined values for the tokens involved.
 * Errors: NULL, INVALID (B or T < 1; with LLAMA_LAYER_CHECK=1 also a
 * position outside [0, max_pos) or repeated within its sequence), CAPACITY
 * (B*T > max_tokens or T > max_pos), HIP (launch failure). */
int llama_layer_prefill(llama_layer* layer, const void* x, void* y, const int32_t* positions,
                        int32_t B, int32_t T, void* k_cache, void* v_cache, void* stream);

/* Decode: one new token for each of B sequences — the same layer with T = 1.
 * x, y [B, d]; positions [B] (normally each sequence's current cache length);
 * caches as for prefill.  Same errors as prefill with T = 1. */
int llama_layer_decode(llama_layer* layer, const void* x, void* y, const int32_t* positions,
                       int32_t B, void* k_cache, void* v_cache, void* stream);

/* ---- paged KV cache ----
 * The same prefill and decode over a paged cache, the KV-memory scheme the
 * "Llama MLP deep dive" page names (§6.4, PagedAttention) beside the "LLM
 * mechanics lecture notes" Ch.04 cache accounting: the K and V of all
 * sequences live in two caller-owned page pools, and a per-sequence block
 * table says which page holds which slots.  The results are those of the
 * contiguous calls on the cache the pages stand for (bit for bit, for the
 * same max_pos: the kernels and their order of work are the same).
 * k_pages, v_pages  [n_pages, Hkv, page_size, head_dim] (layer dtype,
 *            16-byte aligned): row r of kv head g in page i at element
 *            ((i*Hkv + g)*page_size + r)*head_dim.
 * block_table [B, blocks_per_seq] int32 (device): slot p of sequence b lives
 *            in page block_table[b*blocks_per_seq + p/page_size], row
 *            p % page_size.  Pages may be shared between sequences only for
 *            slots no call of this batch writes.
 * page_size  a positive multiple of 64 slots.
 * A sequence holds min(blocks_per_seq*page_size, max_pos) slots; positions
 * are below that.  Page ids in use must lie in [0, n_pages) (precondition;
 * an id outside writes nothing and reads in-bounds garbage, never faults;
 * LLAMA_LAYER_CHECK=1 validates them).  bf16 layers only.
 * Errors: as prefill/decode, plus NULL (block_table), INVALID (page_size not
 * a positive multiple of 64, blocks_per_seq or n_pages < 1), UNSUPPORTED (fp32
 * layer, a pool above 4 GiB), CAPACITY (T above the slots a sequence holds). */
int llama_layer_prefill_paged(llama_layer* layer, const void* x, void* y, const int32_t* positions, int32_t B,
                              int32_t T, void* k_pages, void* v_pages, const int32_t* block_table,
                              int32_t blocks_per_seq, int32_t page_size, int32_t n_pages, void* stream);
int llama_layer_decode_paged(llama_layer* layer, const void* x, void* y, const int32_t* positions, int32_t B,
                             void* k_pages, void* v_pages, const int32_t* block_table, int32_t blocks_per_seq,
                             int32_t page_size, int32_t n_pages, void* stream);

/* int8 KV cache ("LLM mechanics lecture notes" Ch.04: the cache's memory,
 * 2*B*T*Hkv*dh times the element size, is what decode streams every step,
 * and quantising it is named as a lever beside GQA/MQA; "Llama MLP deep
 * dive" page §6.4 names KV-cache quantisation).  The pages give no scheme;
 * this one: each cached row (one token's 128 dims of one kv head) is stored
 * as int8 codes and one fp32 scale, amax = max |x| over the row's bf16
 * values, scale = amax/127, code = rint(x * (127/amax)) (fp32, correctly
 * rounded divisions, round half to even; a row whose amax is below 2^-100,
 * zeros among them: scale 0, codes 0); the
 * row stands for code * scale.  Half the bytes of the bf16 cache, plus 4
 * bytes per row.
 * k_codes, v_codes  [B, Hkv, max_pos, 128] int8, 16-byte aligned.
 * k_scale, v_scale  [B, Hkv, max_pos] float, 4-byte aligned.
 * bf16 layers; contiguous caches here, page pools below. */

/* Quantize slots [0, n_slots) of B sequences of a contiguous bf16 cache
 * [B, Hkv, max_pos, 128] (e.g. after a prefill) into the int8 cache, at the
 * same slots.  Errors: NULL, INVALID (B < 1, n_slots outside [0, max_pos],
 * misaligned pointers), UNSUPPORTED (fp32 layer), HIP. */
int llama_layer_kv_quantize(llama_layer* layer, const void* k_cache, const void* v_cache, int32_t B,
                            int32_t n_slots, void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                            void* stream);

/* Prefill (a chunk of T tokens per sequence) over the int8 cache: as
 * llama_layer_prefill, with every new token's key and value rows quantized,
 * row by row, into slot positions[b*T + t] before the attention, which reads
 * every visible slot (the chunk's own rows included) as code * scale; the
 * bidirectional flag applies as for prefill.  A chunk of T tokens over an
 * empty cache is a whole prompt.  Errors: as prefill, plus NULL (a scale
 * pointer), INVALID (misaligned scales), UNSUPPORTED (fp32 layer). */
int llama_layer_prefill_int8(llama_layer* layer, const void* x, void* y, const int32_t* positions, int32_t B,
                             int32_t T, void* k_codes, void* v_codes, float* k_scale, float* v_scale,
                             void* stream);

/* Decode over the int8 cache: as llama_layer_decode, with the new token's key
 * and value quantized into slot positions[b] (codes and scale) and the
 * attention reading every visible slot as code * scale.  Errors: as decode,
 * plus NULL (a scale pointer), INVALID (misaligned scales), UNSUPPORTED (fp32
 * layer). */
int llama_layer_decode_int8(llama_layer* layer, const void* x, void* y, const int32_t* positions, int32_t B,
                            void* k_codes, void* v_codes, float* k_scale, float* v_scale, void* stream);

/* The int8 cache in page pools: as llama_layer_prefill_paged /
 * llama_layer_decode_paged (same block table, page size and capacity rules),
 * with int8 code pools k_pages, v_pages [n_pages, Hkv, page_size, 128]
 * (16-byte aligned) and fp32 scale pools k_scale_pages, v_scale_pages
 * [n_pages, Hkv, page_size] (4-byte aligned): slot p of sequence b is code
 * row p % page_size and scale p % page_size of page block_table[b][p /
 * page_size].  The rows are quantized and read as for the contiguous int8
 * cache; the output equals the contiguous int8 call's on the cache the pages
 * stand for.  Errors: as the paged calls, plus those of the int8 calls. */
int llama_layer_prefill_paged_int8(llama_layer* layer, const void* x, void* y, const int32_t* positions,
                                   int32_t B, int32_t T, void* k_pages, void* v_pages, float* k_scale_pages,
                                   float* v_scale_pages, const int32_t* block_table, int32_t blocks_per_seq,
                                   int32_t page_size, int32_t n_pages, void* stream);
int llama_layer_decode_paged_int8(llama_layer* layer, const void* x, void* y, const int32_t* positions,
                                  int32_t B, void* k_pages, void* v_pages, float* k_scale_pages,
                                  float* v_scale_pages, const int32_t* block_table, int32_t blocks_per_seq,
                                  int32_t page_size, int32_t n_pages, void* stream);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The same computation, kernels and results as
 * llama_layer_decode on a bf16 layer, but the call's scratch (normalised
 * activations, q, the attention output, the fp32 residual stream, the SwiGLU
 * product, attention split partials, the weight-streaming GEMMs' partial
 * tiles and counters) lives in a static device array of 32 MiB that the
 * library holds on each GPU it runs on until the process ends, not in the
 * handle's buffers.  The call allocates nothing and calls no allocating
 * routine; its first call on a device looks up that device's copy of the
 * array.  The counters are cleared by a small kernel at the start of every
 * call.  Every call on one GPU shares that GPU's array and leaves its
 * contents behind, so calls that overlap on one GPU (other streams, other
 * handles) race: serialise them.
 * Limits: B <= 64, and the call's scratch within 32 MiB (about 64 x (6 d +
 * 4 H dh + 2 f) bytes + split partials + 8 MiB of partial tiles: every
 * LLaMA-7B/13B/70B layer shape fits).  B is not limited by max_tokens.
 * Errors: NULL, INVALID (B < 1, misaligned pointers), UNSUPPORTED (fp32
 * layer), CAPACITY (B > 64 or the scratch would exceed 32 MiB), HIP. */
int llama_layer_decode_noalloc(llama_layer* layer, const void* x, void* y, const int32_t* positions,
                               int32_t B, void* k_cache, void* v_cache, void* stream);

/* Free everything the handle owns (waits for the device first).  NULL is a no-op. */
void llama_layer_destroy(llama_layer* layer);

/* ---- measurement aid: per-step GPU time with HIP events (bf16 layers) ----
 * A bf16 call runs seven steps, in this order (see llama_layer_step_name):
 *   0 RMSNorm of x, 1 QKV projection + RoPE + cache append, 2 attention,
 *   3 o_proj + residual, 4 RMSNorm of X', 5 gate/up projection + SwiGLU,
 *   6 down projection + residual.
 * llama_layer_profile(layer, 1) clears the totals and records a HIP event on
 * the call's stream before each step and after the last one, for every later
 * call; llama_layer_profile(layer, 2 + i) clears them and brackets step i
 * only (two events per call, so the other steps run undisturbed);
 * llama_layer_profile(layer, 0) stops recording.  No device memory is
 * allocated (events are created lazily on the first enable).  Errors: NULL,
 * INVALID (mode outside 0 .. 1 + LLAMA_LAYER_STEPS), HIP. */
#define LLAMA_LAYER_STEPS 7
int llama_layer_profile(llama_layer* layer, int enable);

/* Wait for every recorded call to finish, then write, for each step i <
 * n_steps, the total milliseconds it took over the calls recorded since the
 * last enable (step_ms[i]), and their number (*calls).  Errors: NULL, HIP. */
int llama_layer_profile_read(llama_layer* layer, double* step_ms, int n_steps, long long* calls);

/* Name of step i (0 <= i < LLAMA_LAYER_STEPS), or "" for any other i. */
const char* llama_layer_step_name(int step);

/* ---- measurement aid: ceilings of this GPU ----
 * Both launch one kernel on `stream` and return at once; the caller times
 * them there (e.g. with events) and keeps the sink (4 bytes of device memory
 * the kernels may write) alive until they finish.
 * llama_layer_ceiling_mfma: every wavefront (8 per compute unit) issues
 * n_iter rounds of 8 independent v_mfma_f32_32x32x16_bf16 on pseudo-random
 * register operands (different for consecutive MFMAs), with no memory traffic;
 * *flops (host) receives the flops issued,
 * so flops / time is the dense bf16 matrix rate the GPU sustains.
 * Errors: NULL, INVALID (n_iter < 1), HIP.
 * llama_layer_ceiling_read: reads `bytes` of device memory at `buf` (16-byte
 * aligned, bytes a positive multiple of 1024) once, the whole grid sweeping one
 * contiguous front, so bytes / time is the HBM read rate it sustains (use a
 * buffer well above the 256 MB of on-chip caches).
 * Errors: NULL, INVALID, HIP. */
int llama_layer_ceiling_mfma(int32_t n_iter, void* sink, double* flops, void* stream);
int llama_layer_ceiling_read(const void* buf, uint64_t bytes, void* sink, void* stream);

/* Static description of a status code. */
const char* llama_layer_strerror(int status);

/* Thread-local detail of the last failure on this thread ("" if none). */
const char* llama_layer_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* LLAMA_LAYER_H */
