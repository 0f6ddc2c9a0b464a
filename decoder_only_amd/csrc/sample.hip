// Sampling ("Inside an LLM ...", Step 8): greedy argmax at temperature 0, otherwise
// temperature -> softmax -> top-p nucleus (smallest prefix, in descending-probability
// order, whose mass reaches top_p) -> renormalise -> draw with a supplied uniform
// (inverse CDF; the article's categorical draw with the random number passed in).
//
// Order: logit descending, then token id ascending. Masses m_j = exp(l_j/T - l_max/T)
// are evaluated in float64 and held as unsigned 2^-s fixed point (s = 63 - ceil(log2 V),
// so no sum can overflow); integer sums make every cumulative mass independent of the
// summation order, hence deterministic. Both decisions reduce to "the first token, in
// order, whose cumulative mass C reaches an integer threshold":
//   nucleus mass N = C at the first token with C >= max(1, ceil(top_p * S))
//   (N = S when no token qualifies, i.e. the whole vocabulary is kept);
//   the drawn token is the first with C >= floor(u * N) + 1, i.e. C > u * N.
// The search is a radix select on the order-preserving 32-bit key of the logit:
// a 65536-bucket histogram of masses over the key's upper 16 bits (many blocks,
// integer atomics), then two 8-bit levels inside the crossing bucket, then the tie
// group (equal logits, equal masses) resolved by token id.
#include "common.h"
#include "kernels.h"

namespace q3 {

namespace {

constexpr int NB1 = 65536;
typedef unsigned long long u64;

struct RowWs {           // per-row workspace layout (in u64 words)
    static constexpr size_t hist = 0;          // [NB1]
    static constexpr size_t words = NB1;
};

__global__ void k_argmax_rows(const float* __restrict__ logits, u64* __restrict__ amax, int V,
                              unsigned* err) {
    __shared__ u64 red[16];
    const int b = blockIdx.y;
    const float* l = logits + (size_t)b * V;
    u64 best = 0ull;
    bool bad = false;
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < V; j += gridDim.x * blockDim.x) {
        const float v = l[j];
        bad |= !isfinite(v);
        const u64 k = pack_argmax(v, (uint32_t)j);
        best = k > best ? k : best;
    }
    if (bad) atomicOr(err, Q3_DEVERR_NONFINITE);
    for (int o = 32; o >= 1; o >>= 1) {
        const u64 other = __shfl_xor(best, o, 64);
        best = other > best ? other : best;
    }
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < (int)(blockDim.x >> 6); ++w) best = red[w] > best ? red[w] : best;
        atomicMax(amax + b, best);
    }
}

__global__ void k_greedy(const u64* __restrict__ amax, int32_t* __restrict__ out, int B) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) out[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)(amax[b] & 0xFFFFFFFFull));
}

// Fixed-point mass of one logit; every pass evaluates it with these exact operations.
// z = l / T and z_max = l_max / T are float64 divisions of the float32 logits.
__device__ __forceinline__ u64 mass_of(float v, double T, double zmax, double scale) {
    return __double2ull_rn(__dmul_rn(exp(__dsub_rn(__ddiv_rn((double)v, T), zmax)), scale));
}

__device__ __forceinline__ double row_zmax(const u64* amax, int b, double T) {
    return __ddiv_rn((double)key_to_float((uint32_t)(amax[b] >> 32)), T);
}

// Fixed-point masses into the row's 65536-bucket histogram (keyed by the upper 16 bits).
__global__ __launch_bounds__(256) void k_sample_hist(const float* __restrict__ logits,
                                                     const u64* __restrict__ amax, int V, double Td,
                                                     double scale, u64* __restrict__ ws) {
    const int b = blockIdx.y;
    const float* l = logits + (size_t)b * V;
    u64* hist = ws + (size_t)b * RowWs::words + RowWs::hist;
    const double zmax = row_zmax(amax, b, Td);
    for (int j = blockIdx.x * blockDim.x + threadIdx.x; j < V; j += gridDim.x * blockDim.x) {
        const float v = l[j];
        const u64 m = mass_of(v, Td, zmax, scale);
        if (m) atomicAdd(hist + (ordered_key(v) >> 16), m);
    }
}

// Exclusive prefix sum of one u64 per thread over a 1024-thread block; returns the total.
__device__ u64 block_scan_excl(u64 v, u64* lds /*>= 16*/, u64& excl) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    u64 inc = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const u64 t = __shfl_up(inc, o, 64);
        if (lane >= o) inc += t;
    }
    __syncthreads();
    if (lane == 63) lds[wid] = inc;
    __syncthreads();
    u64 base = 0, total = 0;
    for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
        if (w < wid) base += lds[w];
        total += lds[w];
    }
    excl = base + inc - v;
    return total;
}

struct SelState {
    u64 above;      // mass of every token ordered before the candidate set
    uint32_t prefix;
    int found;
    u64 cum;        // C at the selected token
    int32_t id;
};

// First token in order with C >= thr (1 <= thr <= total mass). Block of 1024 threads.
__device__ void select_first(const float* __restrict__ l, const u64* __restrict__ hist, int V,
                             double Td, double zmax, double scale, u64 thr, u64* scan_lds,
                             u64* h2, SelState* st) {
    const int tid = threadIdx.x;
    if (tid == 0) { st->found = 0; st->prefix = 0; st->above = 0; }
    // level 1: thread tid owns buckets 65535 - 64*tid - k, k = 0..63 (descending order)
    u64 s = 0;
    for (int k = 0; k < 64; ++k) s += hist[NB1 - 1 - (64 * tid + k)];
    u64 excl;
    block_scan_excl(s, scan_lds, excl);   // synchronises
    if (excl < thr && excl + s >= thr) {
        u64 r = excl;
        for (int k = 0; k < 64; ++k) {
            const int bk = NB1 - 1 - (64 * tid + k);
            const u64 r2 = r + hist[bk];
            if (r2 >= thr) { st->prefix = (uint32_t)bk; st->above = r; break; }
            r = r2;
        }
    }
    __syncthreads();
    // levels 2 and 3: 8 key bits each, inside the chosen bucket
    for (int lev = 0; lev < 2; ++lev) {
        const int shift = lev == 0 ? 8 : 0;
        const uint32_t want = st->prefix;
        if (tid < 256) h2[tid] = 0ull;
        __syncthreads();
        for (int j = tid; j < V; j += blockDim.x) {
            const float v = l[j];
            const uint32_t key = ordered_key(v);
            if ((key >> (shift + 8)) == want) atomicAdd(h2 + ((key >> shift) & 255u), mass_of(v, Td, zmax, scale));
        }
        __syncthreads();
        if (tid == 0) {
            u64 r = st->above;
            uint32_t pick = 0;            // lowest sub-bucket if rounding left no crossing
            u64 above = r;
            for (int k = 255; k >= 0; --k) {
                const u64 r2 = r + h2[k];
                if (h2[k]) { pick = (uint32_t)k; above = r; }
                if (r2 >= thr) { pick = (uint32_t)k; above = r; break; }
                r = r2;
            }
            st->prefix = (want << 8) | pick;
            st->above = above;
        }
        __syncthreads();
    }
    // the exact key: its members (equal logits, hence equal masses) are ordered by id
    const uint32_t kstar = st->prefix;
    const u64 mstar = mass_of(key_to_float(kstar), Td, zmax, scale);
    const int per = (V + (int)blockDim.x - 1) / (int)blockDim.x;
    const int j0 = tid * per, j1 = min(V, j0 + per);
    u64 cnt = 0;
    for (int j = j0; j < j1; ++j) cnt += ordered_key(l[j]) == kstar;
    u64 cexcl;
    const u64 ntie = block_scan_excl(cnt, scan_lds, cexcl);
    const u64 need = thr > st->above ? thr - st->above : 1ull;
    u64 kidx = mstar ? (need + mstar - 1) / mstar - 1 : 0;
    if (ntie && kidx >= ntie) kidx = ntie - 1;
    if (cnt && cexcl <= kidx && kidx < cexcl + cnt) {
        u64 c = cexcl;
        for (int j = j0; j < j1; ++j) {
            if (ordered_key(l[j]) == kstar) {
                if (c == kidx) { st->id = j; st->cum = st->above + (kidx + 1) * mstar; st->found = 1; break; }
                ++c;
            }
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(1024) void k_sample_select(const float* __restrict__ logits,
                                                        const u64* __restrict__ amax, int V,
                                                        double Td, double scale, float top_p,
                                                        const float* __restrict__ u,
                                                        u64* __restrict__ ws,
                                                        int32_t* __restrict__ out) {
    __shared__ u64 scan_lds[16];
    __shared__ u64 h2[256];
    __shared__ SelState st;
    if (threadIdx.x == 0) st.id = 0;
    const int b = blockIdx.x;
    const float* l = logits + (size_t)b * V;
    const u64* hist = ws + (size_t)b * RowWs::words + RowWs::hist;
    const double zmax = row_zmax(amax, b, Td);
    // total mass S (bucket t*64 .. t*64+63 per thread)
    u64 s = 0;
    for (int k = 0; k < 64; ++k) s += hist[64 * threadIdx.x + k];
    u64 dummy;
    const u64 S = block_scan_excl(s, scan_lds, dummy);
    // nucleus mass N (the whole vocabulary when top_p >= 1)
    u64 N = S;
    if (top_p < 1.0f) {
        const double tA = ceil((double)top_p * (double)S);
        const u64 thrA = tA < 1.0 ? 1ull : (tA >= (double)S ? S : (u64)tA);
        select_first(l, hist, V, Td, zmax, scale, thrA, scan_lds, h2, &st);
        if (st.found) N = st.cum;
        __syncthreads();                  // every thread has N before the state is reused
    }
    // draw: first token with C >= floor(u N) + 1
    double tB = floor((double)u[b] * (double)N) + 1.0;
    u64 thrB = tB >= (double)N ? N : (u64)tB;
    if (thrB < 1) thrB = 1;
    select_first(l, hist, V, Td, zmax, scale, thrB, scan_lds, h2, &st);
    if (threadIdx.x == 0) out[b] = st.found ? st.id : (int32_t)(0xFFFFFFFFu - (uint32_t)(amax[b] & 0xFFFFFFFFull));
    // leave the row's histogram zeroed for the next call
    __syncthreads();
    u64* hw = ws + (size_t)b * RowWs::words + RowWs::hist;
    for (int k = 0; k < 64; ++k) hw[64 * threadIdx.x + k] = 0ull;
}

}  // namespace

hipError_t launch_argmax_rows(const float* logits, unsigned long long* amax, int V, int B,
                              unsigned* err, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    hipError_t e = launch_fill_u64(amax, 0ull, B, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_argmax_rows, dim3(64, B), dim3(256), 0, s, logits, amax, V, err);
    return hipGetLastError();
}

hipError_t launch_greedy(const unsigned long long* amax, int32_t* out, int B, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_greedy, dim3((B + 255) / 256), dim3(256), 0, s, amax, out, B);
    return hipGetLastError();
}

size_t sample_workspace_bytes(int V, int B) {
    (void)V;
    return (size_t)B * RowWs::words * sizeof(u64);
}

hipError_t launch_sample(const float* logits, const unsigned long long* amax, int V, int B,
                         float temperature, float top_p, const float* u, int32_t* out, void* ws,
                         bool ws_zeroed, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    if (temperature == 0.f) return launch_greedy(amax, out, B, s);
    int lg = 0;
    while ((1ll << lg) < (long long)V) ++lg;
    const double scale = ldexp(1.0, 63 - lg);
    const double Td = (double)temperature;
    u64* w = (u64*)ws;
    hipError_t e = hipSuccess;
    if (!ws_zeroed && (e = launch_fill_u64(w, 0ull, (int)(B * RowWs::words), s)) != hipSuccess) return e;
    const int nblk = (V + 255) / 256 < 512 ? (V + 255) / 256 : 512;
    hipLaunchKernelGGL(k_sample_hist, dim3(nblk, B), dim3(256), 0, s, logits, amax, V, Td, scale, w);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_sample_select, dim3(B), dim3(1024), 0, s, logits, amax, V, Td, scale, top_p,
                       u, w, out);
    return hipGetLastError();
}

}  // namespace q3
