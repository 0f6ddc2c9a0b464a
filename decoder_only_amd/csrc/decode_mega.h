// Parameters and launchers of the persistent decode kernel (decode_mega.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kv_layout.h"

namespace q3 {

// ---- decode_mega.hip (whole decode step in one cooperative launch; fixed Qwen3-0.6B layer
// shape: hidden 1024, 16/8 heads of 128, FFN 3072; bf16 or int8 weights, bf16 KV; 1..4 rows)
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
    int wq;                         // 0: bf16 matrices; 1 (2): every matrix (and the embedding) is int8
                                    // (int4) codes + row scales
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

}  // namespace q3
