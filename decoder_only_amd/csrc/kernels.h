// Launchers of the q3 HIP kernels (all enqueue on the given stream, never sync).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace q3 {

enum WDtype { DT_F32 = 0, DT_BF16 = 1 };

// Where the K (or V) cache keeps slot `slot` of kv head g of sequence `seq`, as an element
// offset from the cache's base for the layer in question.
//   paged (pt != NULL): a page holds kKvPage consecutive slots of one sequence, for every
//     layer and kv head ([layer][head][kKvPage][128]); pt[seq][slot / kKvPage] is the page
//     id; page_stride = elements per page, head_stride = kKvPage * 128 (the layer's base
//     already points at its part of page 0);
//   contiguous (pt == NULL): [seq][head][t_cap][128] from the layer's base; page_stride =
//     elements per sequence, head_stride = t_cap * 128.
// Within one page (or one contiguous run) consecutive slots of a head are 128 elements
// apart, so a range that does not cross a page boundary is one strided run.
constexpr int kKvPage = 256;
struct KvLayout {
    const int32_t* pt;
    int max_pages;          // page-table entries per sequence
    size_t page_stride, head_stride;
#ifdef __HIPCC__
    __host__ __device__ __forceinline__ size_t off(int seq, int g, int slot) const {
        if (pt)
            return (size_t)pt[(size_t)seq * max_pages + (slot >> 8)] * page_stride + (size_t)g * head_stride +
                   (size_t)(slot & (kKvPage - 1)) * 128;
        return (size_t)seq * page_stride + (size_t)g * head_stride + (size_t)slot * 128;
    }
#endif
};
static_assert(kKvPage == 256, "KvLayout::off divides by shifting");
inline KvLayout kv_contiguous(int Hkv, int t_cap) {
    return KvLayout{nullptr, 0, (size_t)Hkv * t_cap * 128, (size_t)t_cap * 128};
}

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
// kc/vc: layer base of the cache [S][Hkv][t_cap][128]. positions may be NULL (= slot).
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
// V page pools (pages of [n_layers][Hkv][kKvPage][128], kv_bytes per element).
hipError_t launch_kv_page_copy(void* kc, void* vc, size_t page_elems, int n_layers, int Hkv, int kv_bytes,
                               int src_page, int dst_page, int n, hipStream_t s);
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

// ---- decode_mega.hip (whole decode step in one cooperative launch; fixed Qwen3-0.6B layer
// shape: hidden 1024, 16/8 heads of 128, FFN 3072; bf16 weights and KV; 1..4 rows)
// Matrices of one layer: bf16 weights, or (int8 weights) one buffer per matrix holding the
// int8 codes [rows][cols] followed by the rows' float32 scales [rows].
struct MegaLayer {
    const uint16_t *wqkv, *wo, *wgu, *wd;
    const float *in_norm, *post_norm, *q_norm, *k_norm;
};
struct MegaParams {
    int n_layers, vocab, B, seq_base, t_cap;
    int slots[4];                   // cache slot (= current length) of each row
    int causal;                     // 0: row b is sequence seq_base + b; 1: every row is sequence
                                    // seq_base at consecutive slots, and row b also attends the
                                    // rows before it in this launch (a short prompt)
    int head_first;                 // rows b >= head_first get the LM head: logits row b - head_first
                                    // and argmax candidates; B: no LM head at all
    float eps;
    const MegaLayer* layers;        // device array [n_layers]
    const uint16_t* embed;          // bf16 [vocab][hidden], or int8 codes followed by the row scales
    const float *final_norm, *inv_freq;
    uint16_t *kc, *vc;              // cache bases (layer l at + l * kv_layer_elems)
    size_t kv_layer_elems;
    KvLayout kv;                    // slot addressing from a layer's base
    const int32_t* tokens;
    const int32_t* positions;       // may be NULL (position = slot)
    float* ex;                      // exchange words (sentinel = not written), (n_layers + 1) * ex_layer
    size_t ex_layer;
    float* logits;
    unsigned long long* cand;       // [4][256] per-workgroup argmax candidates
    unsigned* err;
    unsigned long long* trace;      // optional phase timestamps [2][trace_n] (NULL: off)
    int trace_n;
    int w8;                         // 1: every matrix (and the embedding) is int8 codes + row scales
};
hipError_t decode_mega_prepare();
// cooperative: hipLaunchCooperativeKernel (co-residency guaranteed); else an ordinary launch.
hipError_t launch_decode_mega(const MegaParams& p, bool cooperative, hipStream_t s);
// Attention chunks whose partials a launch over rows of visible lengths T[0..B) writes per
// row (the largest count over the rows; 0 without split-K attention).
int decode_mega_chunks(const int* T, int B);
// After each launch: argmax over the per-workgroup candidates of the nout rows that had the
// LM head, the lengths advanced (lens[seq_base + b] += 1 per row; causal: lens[seq_base] += B),
// the initial state back into the exchange words used (pt_chunks from decode_mega_chunks),
// and the greedy token of each output row into greedy_out when it is not NULL.
hipError_t launch_mega_tail(const unsigned long long* cand, unsigned long long* amax, int* lens, int seq_base,
                            int B, float* ex, size_t ex_layer, int n_layers, int pt_chunks, int32_t* greedy_out,
                            hipStream_t s, int nout, int causal);
// Sentinel into all `words` exchange words (at load).
hipError_t launch_mega_fill(float* ex, size_t words, hipStream_t s);
size_t decode_mega_exchange_words_per_layer();
constexpr int kMegaMaxRows = 4;
// cache page ids a persistent-kernel workgroup holds per row (its attention range of at most
// 32 chunks' share, plus one when the range does not start on a page), and the longest
// context that bounds: ceil(T / 32) rounded to 64 keys spans at most 33 whole pages
constexpr int kMegaPageIds = 34;
constexpr int kMegaMaxSlots = 32 * (kMegaPageIds - 1) * kKvPage;
constexpr int kMegaShortSlots = 240;   // launches whose rows see at most this many slots run the
                                       // short-context instance (the only one that takes causal rows)
constexpr int kMegaMaxLayers = 64;
constexpr int kMegaWorkgroups = 256;

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
