/*
 * q3 op-level C ABI: each call runs one step of the forward pass on caller-owned
 * device buffers, with the same kernels the engine uses. They exist so that every
 * step can be checked on its own against a CPU reference. Conventions as in q3.h:
 * device pointers, asynchronous on `stream` (a hipStream_t, NULL = null stream),
 * host-side argument checks return an error before anything is enqueued. Calls that
 * need scratch memory allocate it and synchronise the stream before returning.
 * bf16 tensors are passed as their 16-bit patterns.
 */
#ifndef Q3_OPS_H
#define Q3_OPS_H

#include <stdint.h>

#include "q3.h"

#ifdef __cplusplus
extern "C" {
#endif

/* dtype code of the single operations for "bf16 pair rows": a float32 value a is carried as
 * hi = bf16(a), lo = bf16(a - hi) (~16 significant bits); a row of width n holds the n hi
 * parts, then the n lo parts (2n bf16). */
#define Q3_OP_PAIR 2

/* RMSNorm ("Inside an LLM ...", Step 3) of `rows` rows of width d:
 * out = x * (1 / sqrt(mean(x^2) + eps)) * w.  x: float32 [rows][d]; w: float32 [d];
 * out: float32 (out_dtype Q3_F32) or bf16 (Q3_BF16) [rows][d], or bf16 pair rows
 * (Q3_OP_PAIR) [rows][2d]. */
q3_status q3_op_rmsnorm(const float* x, const float* w, void* out, int32_t out_dtype, int32_t rows,
                        int32_t d, float eps, void* stream);

/* Decode projection (Steps 5/6): y[b][n] = sum_k W[n][k] x[b][k], for b < B.
 * W: [N][K] of w_dtype (row-major, K % 8 == 0, N even); x: float32 [B][K].
 * epilogue 0: y float32 [B][N] stored; 1: y float32 [B][N] += result (residual);
 * 2: SwiGLU -- W holds 2F rows packed in blocks of 16 gate rows followed by the 16
 * matching up rows, y float32 [B][F] = silu(gate) * up, F = N / 2. */
q3_status q3_op_gemv(const void* W, int32_t w_dtype, const float* x, float* y, int32_t N, int32_t K,
                     int32_t B, int32_t epilogue, void* stream);

/* Prefill projection on the matrix cores: C = A W^T, W bf16 [N][K] (N % 128 == 0,
 * K % 64 == 0), float32 accumulation. A [M][K] is bf16 (a_dtype Q3_BF16), or float32
 * (Q3_F32): then each element enters as a bf16 hi + lo pair, hi = bf16(a),
 * lo = bf16(a - hi), two matrix-core products per tile (~2^-17 relative error), or
 * already such pairs (Q3_OP_PAIR, A bf16 [M][2K]).
 * epilogue 0: C float32 [M][N]; 1: C float32 [M][N] += result; 2: SwiGLU (W packed as
 * for q3_op_gemv), C float32 [M][N/2]; 3: C bf16 [M][N]; 4: SwiGLU to bf16 pair rows,
 * C bf16 [M][N] (N/2 hi parts, then N/2 lo parts); 5: split-K partials, C float32
 * [splits][M][N], partial z = the product over k-tiles [z n / splits, (z+1) n / splits) of
 * the n = K / 64 tiles (1 <= splits <= K / 64; splits must be 1 for the other epilogues).
 * colscale (NULL or float32 [N]): output column n is multiplied by colscale[n] before the
 * epilogue (for SwiGLU, gate and up columns each by their own) -- the per-row scales of
 * int8 or int4 weights whose codes W holds as bf16. */
q3_status q3_op_gemm(const void* A, int32_t a_dtype, const uint16_t* W, void* C, int32_t M, int32_t N,
                     int32_t K, int32_t epilogue, int32_t splits, const float* colscale, void* stream);

/* Per-head QK-norm and RoPE of one decode row per sequence, plus the KV append
 * (Steps 4 and 5). qkv: float32 [B][(n_heads + 2 n_kv_heads) * 128] (q heads, k heads,
 * v heads); q_norm, k_norm: float32 [128]; positions: int32 [B]; slots: int32 [B]
 * (slot index written in each row's cache). q_out: float32 [B][n_heads][128] (rotated);
 * k_cache, v_cache: kv_dtype [B][n_kv_heads][t_cap][128], row b's slot slots[b] is
 * overwritten with the rotated key / raw value. */
q3_status q3_op_qk_norm_rope(const float* qkv, const float* q_norm, const float* k_norm,
                             const int32_t* positions, const int32_t* slots, int32_t B, int32_t n_heads,
                             int32_t n_kv_heads, float eps, float rope_theta, float* q_out,
                             void* k_cache, void* v_cache, int32_t kv_dtype, int32_t t_cap, void* stream);

/* Decode attention (Step 5, one query row per sequence, no mask): q: float32
 * [B][n_heads][128] (rotated); k_cache, v_cache: kv_dtype [B][n_kv_heads][t_cap][128];
 * lens: int32 [B] -- row b sees slots 0 .. lens[b]-1 (1 <= lens[b] <= max_len <= t_cap);
 * o: float32 [B][n_heads * 128]. Query head h reads kv head h / 2 (n_heads = 2 n_kv_heads). */
q3_status q3_op_attn_decode(const float* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                            int32_t t_cap, const int32_t* lens, int32_t B, int32_t n_heads,
                            int32_t n_kv_heads, int32_t max_len, float* o, void* stream);

/* Causal prefill attention (Step 5) of M new rows at slots t0 .. t0+M-1 of one sequence:
 * q: float32 [n_heads][M][128] (rotated); k_cache, v_cache: bf16 [n_kv_heads][t_cap][128]
 * with slots 0 .. t0+M-1 filled; row i sees slots j <= t0 + i. o: float32 [M][n_heads * 128]
 * (o_dtype Q3_F32) or bf16 pair rows [M][2 * n_heads * 128] (Q3_OP_PAIR).
 * q and the softmax weights enter the matrix-core products as bf16 hi + lo pairs. */
q3_status q3_op_attn_prefill(const float* q, const uint16_t* k_cache, const uint16_t* v_cache,
                             int32_t t_cap, int32_t M, int32_t t0, int32_t n_heads, int32_t n_kv_heads,
                             void* o, int32_t o_dtype, void* stream);

/* Sampling of B rows of float32 logits [B][V] (Step 8), same rule as q3_sample. */
q3_status q3_op_sample(const float* logits, int32_t B, int32_t V, float temperature, float top_p,
                       const float* uniforms, int32_t* tokens_out, void* stream);

/* The same sampling with no memory allocation, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): no hipMalloc, hipFree or allocating library call is made. The scratch
 * memory lives in a fixed device array of the library (about 10.5 MB, held on each GPU
 * the library runs on until the process ends), so B <= Q3_SAMPLE_NOALLOC_MAX_ROWS and
 * V <= Q3_SAMPLE_NOALLOC_MAX_VOCAB; larger calls return Q3_ERR_SHAPE before anything is
 * enqueued. Every call on one GPU uses that GPU's one array: calls that overlap on a GPU
 * (other streams, other threads) race and must be serialised by the caller. */
#define Q3_SAMPLE_NOALLOC_MAX_ROWS 4
#define Q3_SAMPLE_NOALLOC_MAX_VOCAB 262144
q3_status q3_op_sample_noalloc(const float* logits, int32_t B, int32_t V, float temperature, float top_p,
                               const float* uniforms, int32_t* tokens_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q3_OPS_H */
