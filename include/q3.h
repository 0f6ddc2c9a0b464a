/*
 * q3 -- C ABI of a Qwen3-0.6B-shaped decoder inference engine for AMD Instinct
 * MI355X (gfx950).
 *
 * The calls follow the pipeline of "Inside an LLM: Pure Python Inference for
 * Qwen3-0.6B on MLX" (section "The pipeline at a glance" and Step 9, the
 * generation loop): load the weights, prefill a prompt into the KV cache, then
 * run one decode step per new token and sample it.
 *
 * Conventions for every call:
 *   - Pointers marked "device" are device memory of the engine's GPU (e.g. torch
 *     tensors on that device); "host" pointers are ordinary CPU memory.
 *   - Work is enqueued on the stream given to q3_load and is asynchronous: device
 *     outputs are valid once that stream has been synchronised (q3_sync does it).
 *   - Argument, shape and capacity errors are detected on the host before anything
 *     is enqueued; the call then returns the error code and enqueues nothing.
 *   - Errors that only the device can see (a token id outside [0, vocab), a
 *     non-finite logit) set a sticky device error word that q3_sync reports.
 *   - No exception crosses the ABI. An engine must be used from one thread at a time.
 *   - q3_last_error returns a text for the last failing call on that engine.
 */
#ifndef Q3_H
#define Q3_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct q3_engine q3_engine;

typedef enum {
    Q3_OK = 0,
    Q3_ERR_ARG = -1,       /* null pointer, bad enum, out-of-range scalar */
    Q3_ERR_SHAPE = -2,     /* tensor shape/size does not match the config */
    Q3_ERR_TOKEN = -3,     /* a token id outside [0, vocab) reached the device (sticky) */
    Q3_ERR_CAPACITY = -4,  /* a sequence would exceed max_seq, or the page pool has no free page
                              ("KV cache full"); nothing was changed */
    Q3_ERR_OOM = -5,       /* device allocation failed */
    Q3_ERR_HIP = -6,       /* a HIP runtime call failed (also: no usable GPU) */
    Q3_ERR_STATE = -7,     /* call not valid in the engine's current state */
    Q3_ERR_NUMERIC = -8    /* a non-finite logit was produced (sticky) */
} q3_status;

typedef enum { Q3_F32 = 0, Q3_BF16 = 1, Q3_I8 = 2, Q3_I4 = 3 } q3_dtype;

/* Model and capacity. Only the Qwen3 block structure is supported: head_dim 128,
 * n_heads a multiple of n_kv_heads, hidden and ffn multiples of 128, a tied LM
 * head (tie_embeddings must be 1). Step 4 of the article fixes rope_theta = 1e6
 * and Step 3 rms_eps = 1e-6 for Qwen3-0.6B; both are taken from this struct. */
typedef struct {
    int32_t n_layers;      /* 28 for Qwen3-0.6B */
    int32_t hidden;        /* 1024 */
    int32_t n_heads;       /* 16 query heads */
    int32_t n_kv_heads;    /* 8 key/value heads (grouped-query attention, Step 5) */
    int32_t head_dim;      /* 128 */
    int32_t ffn;           /* 3072 (SwiGLU, Step 6) */
    int32_t vocab;         /* 151936 */
    float rms_eps;         /* 1e-6 */
    float rope_theta;      /* 1e6 */
    int32_t tie_embeddings;/* must be 1: the LM head is the embedding matrix */
    int32_t weight_dtype;  /* q3_dtype of the matrices: Q3_BF16, Q3_F32, Q3_I8 or Q3_I4 (weight-only
                              int8 / int4: the engine quantises the given bf16 / float32 matrices
                              at load with the rule of q3_quantize_i8 / q3_quantize_i4 and
                              computes with scale * code;
                              needs the Qwen3-0.6B layer shape, a bf16 cache, decode batches of at
                              most 4 rows and the persistent decode kernel) */
    int32_t kv_dtype;      /* q3_dtype of the KV cache */
    int32_t max_batch;     /* number of sequence slots (rows of a decode step) */
    int32_t max_seq;       /* KV-cache capacity per sequence, in tokens */
    int32_t kv_pages;      /* KV-cache pool, in pages of 256 token slots (each page holds those
                              slots' K and V for every layer and kv head) shared by all sequence
                              slots; 0: max_batch * ceil(max_seq / 256), enough for every slot
                              to reach max_seq. A sequence holds ceil(len / 256) pages; pages a
                              fork shares are counted once. */
} q3_config;

/* One named weight tensor in host memory, under the article's tensor names:
 * model.embed_tokens.weight [vocab, hidden]; per layer i
 * model.layers.{i}.input_layernorm.weight [hidden],
 * model.layers.{i}.self_attn.{q,k,v,o}_proj.weight ([out, in], y = x W^T),
 * model.layers.{i}.self_attn.{q,k}_norm.weight [head_dim],
 * model.layers.{i}.post_attention_layernorm.weight [hidden],
 * model.layers.{i}.mlp.{gate,up,down}_proj.weight; and model.norm.weight.
 * Matrices must have dtype == weight_dtype (Q3_BF16 or Q3_F32 when weight_dtype is Q3_I8 or Q3_I4);
 * norm weights may be Q3_F32 or Q3_BF16.
 * lm_head.weight, if given, is ignored (tied head). */
typedef struct {
    const char* name;
    const void* data;      /* host */
    int32_t dtype;         /* q3_dtype */
    int64_t numel;
} q3_tensor;

/* Create an engine on the current HIP device: copies (and repacks) every weight
 * to the device, reserves the KV-cache page pool (kv_pages pages) and the decode
 * workspace. `stream` is a hipStream_t (NULL = the null stream). The
 * caller may free the host tensors when the call returns.
 * Errors: Q3_ERR_ARG / Q3_ERR_SHAPE (config or a tensor missing / mis-sized),
 * Q3_ERR_OOM, Q3_ERR_HIP (no device). On error *out is set to NULL. */
q3_status q3_load(const q3_config* cfg, const q3_tensor* weights, int32_t n_weights,
                  void* stream, q3_engine** out);

/* Prefill (Step 9: every prompt token in one call): append the n tokens
 * `tokens` (device int32 [n]) to sequence slot `seq`, at positions
 * len(seq) .. len(seq)+n-1 where len(seq) is the slot's current cache length,
 * running every layer and writing their K/V. If `logits` is not NULL it receives
 * the logits of the last token (device float32 [vocab]); they are also kept as the
 * engine's current logits for q3_sample. Errors: Q3_ERR_ARG (seq out of range,
 * n < 1), Q3_ERR_CAPACITY (len + n > max_seq, or too few free pages). */
q3_status q3_prefill(q3_engine* e, int32_t seq, const int32_t* tokens, int32_t n,
                     float* logits);

/* One decode step (Step 9's loop body) for `batch` independent sequences: row b
 * is sequence slot b, fed the token tokens[b] (device int32 [batch]) at RoPE
 * position positions[b] (device int32 [batch]; NULL: each slot's current length, which
 * is Step 9's position rule for the newest token). The new K/V are written at slot index
 * len(b), which then grows by one. Logits of all rows go to `logits` (device
 * float32 [batch, vocab]) if not NULL, and are kept as the engine's current logits.
 * Errors: Q3_ERR_ARG (batch outside [1, max_batch]), Q3_ERR_CAPACITY. */
q3_status q3_decode_step(q3_engine* e, const int32_t* tokens, const int32_t* positions,
                         int32_t batch, float* logits);

/* Sampling (Step 8): for each of `batch` rows of `logits` (device float32
 * [batch, vocab]; NULL: the engine's current logits), write one token id to
 * tokens_out (device int32 [batch]). temperature == 0: argmax, lowest id on ties.
 * Otherwise logits / temperature -> softmax -> order by (logit desc, id asc) ->
 * keep the first #{k : cum_k < top_p} + 1 tokens (at most vocab) -> renormalise ->
 * return the first kept token whose cumulative probability exceeds uniforms[b]
 * (device float32 [batch], each in [0, 1)). Masses are float64, accumulated as
 * 2^-s fixed point so the result does not depend on summation order.
 * Errors: Q3_ERR_ARG (batch, temperature < 0, missing uniforms). */
q3_status q3_sample(q3_engine* e, const float* logits, int32_t batch, float temperature,
                    float top_p, const float* uniforms, int32_t* tokens_out);

/* Weight-only int8 codes of a [rows, cols] matrix (host memory, dtype Q3_BF16 or Q3_F32),
 * one scale per row ("What the script leaves out": production weights in 8 bits; the
 * article gives no scheme, so the plainest symmetric one): s = fl32(max_k |w_k| / 127),
 * q_k = round-half-even(fl32(w_k / s)) clamped to [-127, 127], q = 0 for an all-zero row;
 * the quantised weight is s * q. q: host int8 [rows, cols]; scale: host float [rows].
 * Host code only (no GPU). This is the rule q3_load applies for Q3_I8. Errors: Q3_ERR_ARG. */
q3_status q3_quantize_i8(const void* w, int32_t dtype, int64_t rows, int64_t cols, int8_t* q, float* scale);

/* Weight-only int4 codes, the same rule with 7 in place of 127 (the article's 4-bit
 * production weights; one scale per row, no group size being given): s = fl32(max_k |w_k| / 7),
 * q_k = round-half-even(fl32(w_k / s)) clamped to [-7, 7]. q: host int8 [rows, cols], one code
 * per byte (the engine packs two per byte on the device); scale: host float [rows].
 * Host code only (no GPU). This is the rule q3_load applies for Q3_I4. Errors: Q3_ERR_ARG. */
q3_status q3_quantize_i4(const void* w, int32_t dtype, int64_t rows, int64_t cols, int8_t* q, float* scale);

/* Empty sequence slot `seq` (its cache length becomes 0) and return its cache pages to the
 * pool (a page shared with another slot by q3_kv_fork stays with that slot). A slot can be
 * emptied and refilled (q3_prefill) between two decode steps of the others: continuous
 * batching. */
q3_status q3_reset(q3_engine* e, int32_t seq);

/* Fill slots 0 .. len-1 of one (sequence, layer) of the KV cache from k and v
 * (host or device, kv_dtype, layout [n_kv_heads][len][head_dim]) -- a cache that
 * was computed elsewhere. Sets the sequence's length to len once it is
 * called for every layer with the same len (the length is set on each call); pages beyond
 * len are returned to the pool. Waits for the engine's stream before returning.
 * Errors: Q3_ERR_ARG, Q3_ERR_CAPACITY (len > max_seq, or no free page). */
q3_status q3_kv_import(q3_engine* e, int32_t seq, int32_t layer, const void* k,
                       const void* v, int32_t len);

/* Prefix reuse: sequence slot dst gets the first len cached tokens of slot src (every
 * layer's K and V; len <= src's length) and its length becomes len, so a prompt prefix
 * shared by several sequences is prefilled once and each continues with its own tokens
 * (q3_prefill / q3_decode_step append after slot len-1). No data moves: dst's page table
 * points at src's first ceil(len / 256) pages. A shared page is copied (copy on write) by
 * the first sequence that appends into it, so each keeps its own tokens after the prefix.
 * Whatever dst held is released; src is unchanged. The result equals prefilling the prefix
 * into dst itself (Step 5's cache holds only the prefix's K/V, which depend on nothing
 * after it). fork(a, b, len(a)) followed by q3_reset(a) moves a sequence to another slot.
 * Errors: Q3_ERR_ARG (bad slots, src == dst, len above src's length). */
q3_status q3_kv_fork(q3_engine* e, int32_t src, int32_t dst, int32_t len);

/* Copy slots 0 .. len-1 of one (sequence, layer) of the KV cache out to k and v (host or
 * device, kv_dtype, layout [n_kv_heads][len][head_dim]; caller-owned), the inverse of
 * q3_kv_import: the keys as stored (after QK-norm and RoPE, Step 5) and the values.
 * Waits for the engine's stream before returning. Errors: Q3_ERR_ARG (bad slot, layer or
 * pointer, or len above the sequence's current length). */
q3_status q3_kv_export(q3_engine* e, int32_t seq, int32_t layer, void* k, void* v, int32_t len);

/* Current cache length of a sequence slot, as tracked by the host (-1 on error). */
int32_t q3_seq_len(const q3_engine* e, int32_t seq);

/* Pages of the KV-cache pool not held by any sequence slot (-1 on error). */
int32_t q3_kv_free_pages(const q3_engine* e);

/* Wait for the engine's stream; report (and clear) the sticky device error word:
 * Q3_ERR_TOKEN or Q3_ERR_NUMERIC, else Q3_OK (or Q3_ERR_HIP on a runtime error).
 * Q3_ERR_HIP with the text "a cross-workgroup wait timed out" means a persistent decode
 * launch gave up waiting (its workgroups were not all resident, e.g. under an ordinary
 * launch on a shared GPU): the layers after the wait did not run, yet the lengths of the
 * rows of that step advanced, so the KV cache of every sequence decoded since the
 * previous successful q3_sync is undefined and must be q3_reset before reuse. The
 * engine itself (its hand-over words) is restored and stays usable. */
q3_status q3_sync(q3_engine* e);

/* Text describing the last error on this engine (never NULL). */
const char* q3_last_error(const q3_engine* e);

/* Event timing of one kernel family (section "Tracing" of the engine's design):
 * between q3_profile_begin and q3_profile_end, every launch of that family on the
 * engine's stream is bracketed by a pair of hipEvents. q3_profile_end synchronises and
 * returns the summed kernel time in milliseconds, the number of launches, and the
 * algorithmic bytes and flops of those launches (weights, K/V and activations each
 * counted once; decode-step bytes count the tied embedding once, as the LM head).
 * Any output pointer may be NULL. */
typedef enum {
    Q3_PROF_OFF = -1,
    Q3_PROF_DECODE_STEP = 0,   /* one whole decode step (all layers, LM head) */
    Q3_PROF_GEMV = 1,          /* decode projections (QKV, o, gate/up, down) */
    Q3_PROF_LMHEAD = 2,        /* decode LM head + argmax */
    Q3_PROF_ATTN_DECODE = 3,   /* decode attention (split-K + combine) */
    Q3_PROF_GEMM = 4,          /* prefill projections on the matrix cores */
    Q3_PROF_ATTN_PREFILL = 5   /* prefill flash attention */
} q3_prof_kind;
q3_status q3_profile_begin(q3_engine* e, int32_t kind);
q3_status q3_profile_end(q3_engine* e, double* total_ms, int64_t* launches, double* bytes,
                         double* flops);

/* How decode rows run ("The pipeline at a glance": one forward pass per new token).
 * 0 (default): one cooperative launch per decode step (every layer, the LM head and the
 * argmax in a single persistent kernel whose 256 workgroups hand values to each other
 * through device-memory words that hold a "not written" sentinel until their producer
 * stores them, and through fixed-point sums whose top bits count the arrived
 * contributions; a small tail kernel after every launch restores those words) when the model has the Qwen3-0.6B layer shape
 * (hidden 1024, 16/8 heads of 128, FFN 3072) with bf16 weights and cache, the GPU has
 * 256 compute units and the step has at most 4 rows; else one launch per operation.
 * 1: always one launch per operation. 2: always the persistent kernel (Q3_ERR_STATE if
 * the model or GPU does not allow it). 3: as 0, but the persistent kernel is dispatched as
 * an ordinary launch (for tools that cannot trace cooperative launches): it then relies
 * on all 256 workgroups being resident together, which holds when no other work shares
 * the GPU; otherwise its bounded waits expire and q3_sync reports Q3_ERR_HIP. */
q3_status q3_set_decode_path(q3_engine* e, int32_t path);

/* Phase timestamps of the persistent decode kernel: while enabled (n > 0), every launch
 * writes the GPU's 100 MHz real-time clock at its phase boundaries (kernel start, then
 * per layer at each hand-over between workgroups, then the end) as seen by the first and
 * the last workgroup into dev_out (device uint64 [2][n]; row 0 first workgroup, row 1 last;
 * slots past n are dropped). n = 0 turns it off. */
q3_status q3_profile_trace(q3_engine* e, unsigned long long* dev_out, int32_t n);

/* Release all device memory of the engine. NULL is allowed. */
void q3_free(q3_engine* e);

#ifdef __cplusplus
}
#endif

#endif /* Q3_H */
