// Launchers of the q3 HIP kernels (all enqueue on the given stream, never sync).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "decode_mega.h"
#include "kv_layout.h"

namespace q3 {

enum WDtype { DT_F32 = 0, DT_BF16 = 1 };

// (the cache layout, KvLayout, is in kv_layout.h; the persistent decode kernel's
// parameters in decode_mega.h)

// ---- elementwise.hip
// x[r, :] = E[tok[r], :] widened to float32 (times rowscale[tok[r]] when given: int8 codes held
// as bf16). Out-of-range ids set Q3_DEVERR_TOKEN and give a zero row.
hipError_t launch_embed(const int32_t* tok, const void* E, int wdt, float* x, int rows, int d,
                        int vocab, unsigned* err, hipStream_t s, const float* rowscale = nullptr);
// out[r, :] = rmsnorm(x[r, :]) * w; out_mode 0 float32, 1 bf16, 2 bf16 pair rows [rows][2d]
// (d hi parts, then d lo parts). With nparts > 0, first x[r, :] += parts[0][r, :] + ... +
// parts[nparts-1][r, :] (in that order; parts [nparts][rows][d] float32) and x is written back.
hipError_t launch_rmsnorm(float* x, const float* w, void* out, int out_mode, int rows, int d,
                          float eps, hipStream_t s, const float* parts = nullptr, int nparts = 0);
// Decode rows: per-head RMSNorm of q and k, RoPE at the row's position, K/V append at
// slot lens[seq]. qkv: [B][(Hq + 2 Hkv) * 128] float32. q_out: [B][Hq][128] float32.
// kc/vc: the layer's cache base, slots addressed through lay (t_cap bounds the slot).
// positions may be NULL (= slot).
// With nparts > 1, qkv holds nparts split-K partials [nparts][B][...], summed in order.
hipError_t launch_qk_rope_decode(const float* qkv, const int32_t* positions, const int32_t* lens,
                                 int seq_base, int B, const float* q_norm, const float* k_norm,
                                 const float* inv_freq, float eps, float* q_out, void* kc, void* vc,
                                 int kv_bf16, int t_cap, const KvLayout& lay, int Hq, int Hkv, hipStream_t s,
                                 int nparts = 1);
// SwiGLU of the summed split-K partials [nparts][B][2F] of the packed gate/up projection,
// to bf16 pair rows [B][2F].
hipError_t launch_swiglu_parts(const float* parts, int nparts, int B, int F, void* out_pair, hipStream_t s);
// Prefill rows of sequence seq at slots/positions t0 .. t0+M-1. q_out: [Hq][M][128] float32.
// kc/vc: the layer's cache base, bf16, addressed through lay.
hipError_t launch_qk_rope_prefill(const float* qkv, int M, int t0, const float* q_norm,
                                  const float* k_norm, const float* inv_freq, float eps,
                                  float* q_out, uint16_t* kc, uint16_t* vc, const KvLayout& lay, int seq, int Hq,
                                  int Hkv, hipStream_t s);
// lens[seq_base + b] += by for b < B.
hipError_t launch_len_advance(int32_t* lens, int seq_base, int B, int by, hipStream_t s);
// Slots 0 .. n-1 of page src_page into page dst_page, for every layer and kv head of the K and
// V page pools ([n_layers][pages][Hkv][kKvPage][128], kv_bytes per element; page_elems and
// layer_elems are the strides of a page and of a layer).
hipError_t launch_kv_page_copy(void* kc, void* vc, size_t page_elems, size_t layer_elems, int n_layers, int Hkv,
                               int kv_bytes, int src_page, int dst_page, int n, hipStream_t s);
// Slots 0 .. len-1 of one (sequence, layer) between the paged cache and a dense buffer
// [Hkv][len][128] (device memory): to_cache = true writes the cache (an import), false reads it.
hipError_t launch_kv_dense(void* kc_layer, void* vc_layer, const KvLayout& lay, int seq, int Hkv, int kv_bytes,
                           void* dk, void* dv, int len, bool to_cache, hipStream_t s);
// pt[seq * max_pages + first + i] = pages[i] for i < n (n <= 64); lens[seq] = len when len >= 0.
hipError_t launch_set_pages(int32_t* pt, int max_pages, int seq, int first, const int32_t* pages, int n,
                            int32_t* lens, int len, hipStream_t s);
// dst[i] = v for i < n (64-bit words); graph-safe replacement for a memset.
hipError_t launch_fill_u64(unsigned long long* dst, unsigned long long v, int n, hipStream_t s);

// ---- gemv.hip (decode projections: float32 activations, bf16 / float32 weights)
enum GemvEpi { GEMV_STORE = 0, GEMV_RESID = 1, GEMV_SWIGLU = 2 };
// y[b, n] (=, +=) sum_k W[n, k] x[b, k]. SWIGLU: W holds 2F rows in blocks of 16 gate rows
// followed by the 16 matching up rows; y[b, j] = silu(gate_j) * up_j, j < F = N / 2.
hipError_t launch_gemv(const void* W, int wdt, const float* x, float* y, int N, int K, int B,
                       int epi, hipStream_t s);
// LM head: logits[b, v] = sum_k E[v, k] h[b, k]; amax[b] = max over v of pack(logit, v).
hipError_t launch_lmhead(const void* E, int wdt, const float* h, float* logits,
                         unsigned long long* amax, int V, int K, int B, unsigned* err, hipStream_t s);

// ---- attn_decode.hip (split-K GQA over the cache, one query row per sequence)
// Visible keys of row b: slots 0 .. lens[seq_base + b] + len_extra - 1.
size_t attn_decode_workspace_bytes(int B, int Hkv, int max_T);
// o: float32 [B][Hq*128], or (o_pair) bf16 pair rows [B][2*Hq*128].
hipError_t launch_attn_decode(const float* q, const void* kc, const void* vc, int kv_bf16,
                              int t_cap, const KvLayout& lay, const int32_t* lens, int len_extra, int seq_base,
                              int B, int Hq, int Hkv, int max_T, float* ws, void* o, int o_pair, hipStream_t s);

// ---- gemm.hip (prefill projections on MFMA: A [M,K] x bf16 W [N,K]^T, fp32 accumulate)
// a_mode: A bf16 [M][K]; float32 [M][K] split into bf16 hi + lo while staging; or a bf16
// pair [M][2K] (per row the K hi parts, then the K lo parts). Split / pair: two MFMAs per tile.
enum GemmAMode { GEMM_A_BF16 = 0, GEMM_A_F32 = 1, GEMM_A_PAIR = 2 };
// Epilogues; SWIGLU_PAIR writes C as bf16 pair rows [M][N] (N/2 hi, then N/2 lo);
// PARTIAL_F32 (with splits > 1 blocks along K) writes C[split][M][N] float32 partials.
enum GemmEpi { GEMM_F32 = 0, GEMM_RESID_F32 = 1, GEMM_SWIGLU_F32 = 2, GEMM_BF16 = 3, GEMM_SWIGLU_PAIR = 4,
               GEMM_PARTIAL_F32 = 5 };
// colscale (int8 weights: W holds the codes in bf16): output column n is multiplied by
// colscale[n] before the epilogue (for SwiGLU, the gate and up columns by their own scales).
hipError_t launch_gemm(const void* A, int a_mode, const uint16_t* W, void* C, int M, int N, int K, int epi,
                       hipStream_t s, int splits = 1, const float* colscale = nullptr);

// ---- attn_prefill.hip (causal GQA flash attention on MFMA)
// q: [Hq][M][128] float32 rows at slots t0..t0+M-1 of sequence seq; kc/vc: the layer's
// cache base (bf16) addressed through lay; o: [M][Hq*128] float32, or (o_pair) bf16 pair
// rows [M][2*Hq*128] (hi parts, then lo parts).
hipError_t launch_attn_prefill(const float* q, const uint16_t* kc, const uint16_t* vc, const KvLayout& lay,
                               int seq, int M, int t0, int Hq, int Hkv, void* o, int o_pair, hipStream_t s);

// ---- sample.hip
hipError_t launch_argmax_rows(const float* logits, unsigned long long* amax, int V, int B,
                              unsigned* err, hipStream_t s);
hipError_t launch_greedy(const unsigned long long* amax, int32_t* out, int B, hipStream_t s);
size_t sample_workspace_bytes(int V, int B);
// ws: sample_workspace_bytes; the select kernel leaves it zeroed, so a workspace that was
// zeroed once and is only used here may pass ws_zeroed = true.
hipError_t launch_sample(const float* logits, const unsigned long long* amax, int V, int B,
                         float temperature, float top_p, const float* u, int32_t* out, void* ws,
                         bool ws_zeroed, hipStream_t s);

}  // namespace q3
