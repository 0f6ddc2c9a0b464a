// Embedding gather, RMSNorm, and the fused QK-norm + RoPE + KV-cache append.
//
// Sources ("Inside an LLM: Pure Python Inference for Qwen3-0.6B on MLX"):
//   Step 2  -- the embedding is a row lookup in the [vocab, hidden] matrix;
//   Step 3  -- RMSNorm: x / sqrt(mean(x^2) + eps) times a per-feature weight;
//   Step 4  -- RoPE on split halves: pair (i, i + 64) of a 128-wide head turns by
//              position * theta^(-i/64) (angles built in float32);
//   Step 5  -- QK-norm (RMSNorm over each 128-wide q and k head, before RoPE) and
//              the KV cache, which stores rotated keys and raw values.
#include "common.h"
#include "kernels.h"

namespace q3 {

template <typename WT>
__global__ void k_embed(const int32_t* __restrict__ tok, const WT* __restrict__ E,
                        float* __restrict__ x, int d, int vocab, unsigned* err, const float* __restrict__ rowscale) {
    const int r = blockIdx.x;
    int t = tok[r];
    const bool ok = (t >= 0) && (t < vocab);
    if (!ok && threadIdx.x == 0) atomicOr(err, Q3_DEVERR_TOKEN);
    const WT* src = E + (size_t)(ok ? t : 0) * d;
    float* dst = x + (size_t)r * d;
    const float sc = rowscale && ok ? rowscale[t] : 1.f;   // int8 codes: the row's scale
    for (int i = threadIdx.x; i < d; i += blockDim.x) dst[i] = ok ? (rowscale ? ldw(src, i) * sc : ldw(src, i)) : 0.f;
}

hipError_t launch_embed(const int32_t* tok, const void* E, int wdt, float* x, int rows, int d,
                        int vocab, unsigned* err, hipStream_t s, const float* rowscale) {
    if (rows <= 0) return hipSuccess;
    if (wdt == DT_BF16)
        hipLaunchKernelGGL(k_embed<bf16>, dim3(rows), dim3(256), 0, s, tok, (const bf16*)E, x, d, vocab, err,
                           rowscale);
    else
        hipLaunchKernelGGL(k_embed<float>, dim3(rows), dim3(256), 0, s, tok, (const float*)E, x, d, vocab, err,
                           rowscale);
    return hipGetLastError();
}

// MODE 0: float32 out [rows][d]; 1: bf16 [rows][d]; 2: bf16 pair rows [rows][2d]
// (hi = bf16(v) in the first d, lo = bf16(v - hi) in the second d).
template <int MODE>
__global__ void k_rmsnorm(float* __restrict__ x, const float* __restrict__ w, void* __restrict__ out, int d,
                          float eps, const float* __restrict__ parts, int nparts, int rows) {
    __shared__ float red[16];
    const int r = blockIdx.x;
    float* xr = x + (size_t)r * d;
    float ss = 0.f;
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        float v = xr[i];
        if (nparts > 0) {
            // partials in batches of 8 loads in flight, added in order p = 0, 1, ...
            const float* pp = parts + (size_t)r * d + i;
            const size_t stride = (size_t)rows * d;
            int p = 0;
            for (; p + 8 <= nparts; p += 8) {
                float t[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) t[u] = pp[(size_t)(p + u) * stride];
#pragma unroll
                for (int u = 0; u < 8; ++u) v += t[u];
            }
            for (; p < nparts; ++p) v += pp[(size_t)p * stride];
            xr[i] = v;
        }
        ss += v * v;
    }
    ss = block_sum(ss, red);    // (its barriers also order the x write-back before the reads below)
    const float rs = 1.0f / sqrtf(ss / (float)d + eps);
    for (int i = threadIdx.x; i < d; i += blockDim.x) {
        const float v = (xr[i] * rs) * w[i];
        if constexpr (MODE == 0) {
            static_cast<float*>(out)[(size_t)r * d + i] = v;
        } else if constexpr (MODE == 1) {
            static_cast<bf16*>(out)[(size_t)r * d + i] = f2bf(v);
        } else {
            bf16* o = static_cast<bf16*>(out) + (size_t)r * 2 * d;
            const bf16 h = f2bf(v);
            o[i] = h;
            o[d + i] = f2bf(v - bf2f(h));
        }
    }
}

hipError_t launch_rmsnorm(float* x, const float* w, void* out, int out_mode, int rows, int d,
                          float eps, hipStream_t s, const float* parts, int nparts) {
    if (rows <= 0) return hipSuccess;
    if (nparts < 0 || (nparts > 0 && !parts)) return hipErrorInvalidValue;
    // many partials per element (batched decode): a thread per element keeps more loads in flight
    const dim3 blk(nparts > 8 && d >= 1024 ? 1024 : 256);
    if (out_mode == 0) hipLaunchKernelGGL(k_rmsnorm<0>, dim3(rows), blk, 0, s, x, w, out, d, eps, parts, nparts, rows);
    else if (out_mode == 1) hipLaunchKernelGGL(k_rmsnorm<1>, dim3(rows), blk, 0, s, x, w, out, d, eps, parts, nparts, rows);
    else if (out_mode == 2) hipLaunchKernelGGL(k_rmsnorm<2>, dim3(rows), blk, 0, s, x, w, out, d, eps, parts, nparts, rows);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

// One wave per (row, head). Lane i owns the RoPE pair (i, i + 64) of the 128-wide head.
// Returns the normalised and rotated pair; RMSNorm as (x * r) * w with r = 1/sqrt(mean + eps).
__device__ __forceinline__ void norm_rope_pair(float& x1, float& x2, const float* w, int i,
                                               float eps, int pos, const float* inv_freq) {
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
    x1 = (x1 * r) * w[i];
    x2 = (x2 * r) * w[i + 64];
    // angle = fl32(fl32(pos) * f_i): one float32 multiply; cos/sin evaluated in double.
    const float ang = __fmul_rn((float)pos, inv_freq[i]);
    double sd, cd;
    sincos((double)ang, &sd, &cd);
    const float c = (float)cd, sn = (float)sd;
    const float y1 = __fsub_rn(__fmul_rn(x1, c), __fmul_rn(x2, sn));
    const float y2 = __fadd_rn(__fmul_rn(x1, sn), __fmul_rn(x2, c));
    x1 = y1;
    x2 = y2;
}

template <typename KT>
__global__ void k_qk_rope_decode(const float* __restrict__ qkv, const int32_t* __restrict__ positions,
                                 const int32_t* __restrict__ lens, int seq_base,
                                 const float* __restrict__ qn, const float* __restrict__ kn,
                                 const float* __restrict__ inv_freq, float eps,
                                 float* __restrict__ q_out, KT* __restrict__ kc, KT* __restrict__ vc,
                                 int t_cap, KvLayout lay, int Hq, int Hkv, int nparts) {
    const int b = blockIdx.x, hd = blockIdx.y, i = threadIdx.x;
    const int width = (Hq + 2 * Hkv) * 128;
    const float* row = qkv + (size_t)b * width + hd * 128;
    const int seq = seq_base + b;
    const int slot = lens[seq];
    if ((unsigned)slot >= (unsigned)t_cap) return;   // capacity is checked on the host
    const int pos = positions ? positions[b] : slot;
    float x1 = row[i], x2 = row[i + 64];
    for (int p = 1; p < nparts; ++p) {               // split-K partials, added in order
        const float* rp = row + (size_t)p * gridDim.x * width;
        x1 += rp[i];
        x2 += rp[i + 64];
    }
    if (hd >= Hq + Hkv) {  // value head: stored as is
        const int g = hd - Hq - Hkv;
        const size_t base = lay.off(seq, g, slot);
        stkv(vc, base + i, x1);
        stkv(vc, base + i + 64, x2);
        return;
    }
    norm_rope_pair(x1, x2, hd < Hq ? qn : kn, i, eps, pos, inv_freq);
    if (hd < Hq) {
        float* qo = q_out + ((size_t)b * Hq + hd) * 128;
        qo[i] = x1;
        qo[i + 64] = x2;
    } else {
        const int g = hd - Hq;
        const size_t base = lay.off(seq, g, slot);
        stkv(kc, base + i, x1);
        stkv(kc, base + i + 64, x2);
    }
}

hipError_t launch_qk_rope_decode(const float* qkv, const int32_t* positions, const int32_t* lens,
                                 int seq_base, int B, const float* q_norm, const float* k_norm,
                                 const float* inv_freq, float eps, float* q_out, void* kc, void* vc,
                                 int kv_bf16, int t_cap, const KvLayout& lay, int Hq, int Hkv, hipStream_t s,
                                 int nparts) {
    if (B <= 0) return hipSuccess;
    if (nparts < 1) return hipErrorInvalidValue;
    dim3 grid(B, Hq + 2 * Hkv);
    if (kv_bf16)
        hipLaunchKernelGGL(k_qk_rope_decode<bf16>, grid, dim3(64), 0, s, qkv, positions, lens, seq_base,
                           q_norm, k_norm, inv_freq, eps, q_out, (bf16*)kc, (bf16*)vc, t_cap, lay, Hq, Hkv, nparts);
    else
        hipLaunchKernelGGL(k_qk_rope_decode<float>, grid, dim3(64), 0, s, qkv, positions, lens, seq_base,
                           q_norm, k_norm, inv_freq, eps, q_out, (float*)kc, (float*)vc, t_cap, lay, Hq, Hkv,
                           nparts);
    return hipGetLastError();
}

// a[b][j] = silu(g) * u with g, u the sums of nparts split-K partials of the packed
// gate/up projection (blocks of 16 gate rows then the 16 matching up rows), written as
// bf16 pair rows [B][2F] (F hi parts, then F lo parts).
__global__ void k_swiglu_parts(const float* __restrict__ parts, int nparts, int B, int F,
                               bf16* __restrict__ out) {
    const int b = blockIdx.y, j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= F) return;
    const int n = 32 * (j >> 4) + (j & 15);
    const size_t stride = (size_t)B * 2 * F;
    const float* pg = parts + (size_t)b * 2 * F + n;
    float g = pg[0], u = pg[16];
    for (int p = 1; p < nparts; ++p) {
        g += pg[p * stride];
        u += pg[p * stride + 16];
    }
    const float a = g / (1.0f + expf(-g)) * u;
    const bf16 h = f2bf(a);
    out[(size_t)b * 2 * F + j] = h;
    out[(size_t)b * 2 * F + F + j] = f2bf(a - bf2f(h));
}

hipError_t launch_swiglu_parts(const float* parts, int nparts, int B, int F, void* out_pair, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    if (nparts < 1 || F % 16) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_swiglu_parts, dim3((F + 255) / 256, B), dim3(256), 0, s, parts, nparts, B, F,
                       (bf16*)out_pair);
    return hipGetLastError();
}

// One block (four waves) per row: lane i evaluates the RoPE factors of its pair once (the
// angle depends on the position and i only) and wave w takes heads w, w + 4, ... with the
// same operations as norm_rope_pair.
__global__ __launch_bounds__(256) void k_qk_rope_prefill(const float* __restrict__ qkv, int M, int t0,
                                                         const float* __restrict__ qn, const float* __restrict__ kn,
                                                         const float* __restrict__ inv_freq, float eps,
                                                         float* __restrict__ q_out, bf16* __restrict__ kc,
                                                         bf16* __restrict__ vc, KvLayout lay, int seq, int Hq,
                                                         int Hkv) {
    const int r = blockIdx.x, i = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int nh = Hq + 2 * Hkv, width = nh * 128;
    const int slot = t0 + r;
    const float ang = __fmul_rn((float)slot, inv_freq[i]);
    double sd, cd;
    sincos((double)ang, &sd, &cd);
    const float c = (float)cd, sn = (float)sd;
    for (int hd = wid; hd < nh; hd += 4) {
        const float* row = qkv + (size_t)r * width + hd * 128;
        float x1 = row[i], x2 = row[i + 64];
        if (hd >= Hq + Hkv) {
            const size_t base = lay.off(seq, hd - Hq - Hkv, slot);
            vc[base + i] = f2bf(x1);
            vc[base + i + 64] = f2bf(x2);
            continue;
        }
        const float* w = hd < Hq ? qn : kn;
        const float ss = wave_sum(x1 * x1 + x2 * x2);
        const float rr = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
        x1 = (x1 * rr) * w[i];
        x2 = (x2 * rr) * w[i + 64];
        const float y1 = __fsub_rn(__fmul_rn(x1, c), __fmul_rn(x2, sn));
        const float y2 = __fadd_rn(__fmul_rn(x1, sn), __fmul_rn(x2, c));
        if (hd < Hq) {
            float* qo = q_out + ((size_t)hd * M + r) * 128;
            qo[i] = y1;
            qo[i + 64] = y2;
        } else {
            const size_t base = lay.off(seq, hd - Hq, slot);
            kc[base + i] = f2bf(y1);
            kc[base + i + 64] = f2bf(y2);
        }
    }
}

hipError_t launch_qk_rope_prefill(const float* qkv, int M, int t0, const float* q_norm,
                                  const float* k_norm, const float* inv_freq, float eps,
                                  float* q_out, uint16_t* kc, uint16_t* vc, const KvLayout& lay, int seq, int Hq,
                                  int Hkv, hipStream_t s) {
    if (M <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_qk_rope_prefill, dim3(M), dim3(256), 0, s, qkv, M, t0, q_norm, k_norm, inv_freq, eps,
                       q_out, kc, vc, lay, seq, Hq, Hkv);
    return hipGetLastError();
}

__global__ void k_len_advance(int32_t* lens, int seq_base, int B, int by) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) lens[seq_base + b] += by;
}

hipError_t launch_len_advance(int32_t* lens, int seq_base, int B, int by, hipStream_t s) {
    hipLaunchKernelGGL(k_len_advance, dim3((B + 255) / 256), dim3(256), 0, s, lens, seq_base, B, by);
    return hipGetLastError();
}

// Page copy (prefix reuse): slots 0 .. n-1 of page src into page dst, for every (layer,
// kv head) run of the page ([layer][page][head][kKvPage][128]) in the K and V pools;
// blockIdx.y = (layer * Hkv + head) * 2 + (0: K, 1: V), one 16-byte unit per thread.
__global__ void k_kv_page_copy(uint4* __restrict__ kc, uint4* __restrict__ vc, size_t page_u, size_t layer_u, int Hkv,
                               int src, int dst, size_t run_u, size_t n_u) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint4* base = ((int)blockIdx.y & 1) ? vc : kc;
    const int r = (int)blockIdx.y >> 1, layer = r / Hkv, head = r % Hkv;
    const size_t off = (size_t)layer * layer_u + (size_t)head * run_u + i;
    if (i < n_u) base[(size_t)dst * page_u + off] = base[(size_t)src * page_u + off];
}

hipError_t launch_kv_page_copy(void* kc, void* vc, size_t page_elems, size_t layer_elems, int n_layers, int Hkv,
                               int kv_bytes, int src_page, int dst_page, int n, hipStream_t s) {
    if (n_layers <= 0 || n <= 0) return hipSuccess;
    if (n > kKvPage || (128 * kv_bytes) % 16) return hipErrorInvalidValue;
    const size_t u = 16 / kv_bytes;     // elements per 16-byte unit
    const size_t n_u = (size_t)n * 128 / u;
    const dim3 grid((unsigned)((n_u + 255) / 256), (unsigned)(n_layers * Hkv * 2));
    hipLaunchKernelGGL(k_kv_page_copy, grid, dim3(256), 0, s, (uint4*)kc, (uint4*)vc, page_elems / u, layer_elems / u,
                       Hkv, src_page, dst_page, (size_t)kKvPage * 128 / u, n_u);
    return hipGetLastError();
}

// Dense [Hkv][len][128] buffer <-> the cache slots 0 .. len-1 of one (sequence, layer):
// thread = one 16-byte unit of one row; blockIdx.y = head * 2 + (0: K, 1: V).
__global__ void k_kv_dense(uint4* __restrict__ kc, uint4* __restrict__ vc, KvLayout lay, int seq, uint4* dk,
                           uint4* dv, int len, int units_per_row, int to_cache) {
    const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int g = (int)blockIdx.y >> 1;
    const bool isv = blockIdx.y & 1;
    if (i >= (size_t)len * units_per_row) return;
    const int slot = (int)(i / units_per_row), u = (int)(i % units_per_row);
    // the layout's element offsets become unit offsets (a row of 128 elements is units_per_row units)
    const size_t c = lay.off(seq, g, slot) / (128 / units_per_row) + u;
    const size_t d = ((size_t)g * len + slot) * units_per_row + u;
    uint4* cache = isv ? vc : kc;
    uint4* dense = isv ? dv : dk;
    if (to_cache) cache[c] = dense[d];
    else dense[d] = cache[c];
}

hipError_t launch_kv_dense(void* kc_layer, void* vc_layer, const KvLayout& lay, int seq, int Hkv, int kv_bytes,
                           void* dk, void* dv, int len, bool to_cache, hipStream_t s) {
    if (len <= 0) return hipSuccess;
    if ((128 * kv_bytes) % 16) return hipErrorInvalidValue;
    const int upr = 128 * kv_bytes / 16;
    const size_t n = (size_t)len * upr;
    const dim3 grid((unsigned)((n + 255) / 256), (unsigned)(Hkv * 2));
    hipLaunchKernelGGL(k_kv_dense, grid, dim3(256), 0, s, (uint4*)kc_layer, (uint4*)vc_layer, lay, seq, (uint4*)dk,
                       (uint4*)dv, len, upr, to_cache ? 1 : 0);
    return hipGetLastError();
}

// Page-table entries and a length set on the stream (a kernel, so the update is ordered
// with the launches around it and safe under graph capture).
struct PageSet {
    int32_t p[64];
};
__global__ void k_set_pages(int32_t* pt, int max_pages, int seq, int first, PageSet v, int n, int32_t* lens,
                            int len) {
    const int i = threadIdx.x;
    if (i < n) pt[(size_t)seq * max_pages + first + i] = v.p[i];
    if (i == 0 && len >= 0) lens[seq] = len;
}

hipError_t launch_set_pages(int32_t* pt, int max_pages, int seq, int first, const int32_t* pages, int n,
                            int32_t* lens, int len, hipStream_t s) {
    if (n < 0 || n > 64) return hipErrorInvalidValue;
    PageSet v{};
    for (int i = 0; i < n; ++i) v.p[i] = pages[i];
    hipLaunchKernelGGL(k_set_pages, dim3(1), dim3(64), 0, s, pt, max_pages, seq, first, v, n, lens, len);
    return hipGetLastError();
}

__global__ void k_fill_u64(unsigned long long* dst, unsigned long long v, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) dst[i] = v;
}

hipError_t launch_fill_u64(unsigned long long* dst, unsigned long long v, int n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_fill_u64, dim3((n + 255) / 256), dim3(256), 0, s, dst, v, n);
    return hipGetLastError();
}

}  // namespace q3
