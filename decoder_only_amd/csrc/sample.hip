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
// a 65536-bucket histogram of masses over the key's upper 16 bits and the sums of its
// 256-bucket groups (many blocks, integer atomics); many blocks each find the bucket where
// the cumulative mass crosses the threshold (the same result in every block, from the
// group sums and one group's buckets) and gather that bucket's members as packed (key,
// ~id) words; one block sorts them (key descending, id ascending -- independent of the
// gather order) and walks their masses to the crossing token. A bucket with more members
// than the sort holds falls back to two 8-bit refinement levels and an id-ordered tie pass
// over the whole row. Five launches per draw with a nucleus (histogram; nucleus gather;
// nucleus walk; draw gather; draw walk, which also leaves the workspace zeroed), three
// without.
#include "common.h"
#include "kernels.h"

namespace q3 {

namespace {

constexpr int NB1 = 65536;
typedef unsigned long long u64;
typedef __attribute__((ext_vector_type(2))) unsigned long long u64x2;

constexpr int SORT_CAP = 4096;   // bucket members sorted in shared memory

struct RowWs {           // per-row workspace layout (in u64 words)
    static constexpr size_t hist = 0;          // [NB1] masses by upper key half (left zeroed)
    static constexpr size_t gsum = NB1;        // [256] sums of 256-bucket groups
    static constexpr size_t state = NB1 + 256; // [8] selection state (SelWord)
    static constexpr size_t list = NB1 + 264;  // [V] members of the crossing bucket
    static size_t words(int V) { return NB1 + 264 + (size_t)V; }
};
// state words of a row (SW_COUNT is zero whenever a gather starts: the walk that reads it
// clears it)
enum SelWord { SW_ABOVE = 0, SW_THR = 1, SW_N = 2, SW_BUCKET = 3, SW_COUNT = 4, SW_S = 5 };

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

// Fixed-point masses into the row's 65536-bucket histogram (keyed by the upper 16 bits)
// and its 256 group sums. Each block first sums its tokens' masses per bucket in shared
// memory (a direct-mapped table of HIST_SLOTS buckets, slot = bucket mod HIST_SLOTS; a
// bucket whose slot another bucket holds goes straight to memory), then adds its
// non-empty slots to the row's histogram: the memory-side atomics drop from one per token
// to about one per bucket and block. Integer sums: the histogram does not depend on the
// order of the additions.
constexpr int HIST_SLOTS = 8192, HIST_THREADS = 1024, HIST_BLOCKS = 32;
constexpr unsigned HIST_EMPTY = 0xFFFFFFFFu;
__global__ __launch_bounds__(HIST_THREADS) void k_sample_hist(const float* __restrict__ logits,
                                                              const u64* __restrict__ amax, int V, double Td,
                                                              double scale, u64* __restrict__ ws, size_t row_words) {
    __shared__ unsigned lkey[HIST_SLOTS];
    __shared__ u64 lmass[HIST_SLOTS];
    __shared__ u64 lgroup[256];          // this block's masses per 256-bucket group
    const int b = blockIdx.y;
    const float* l = logits + (size_t)b * V;
    u64* hist = ws + (size_t)b * row_words + RowWs::hist;
    u64* gsum = ws + (size_t)b * row_words + RowWs::gsum;
    for (int i = threadIdx.x; i < HIST_SLOTS; i += HIST_THREADS) {
        lkey[i] = HIST_EMPTY;
        lmass[i] = 0ull;
    }
    if (threadIdx.x < 256) lgroup[threadIdx.x] = 0ull;
    __syncthreads();
    const double zmax = row_zmax(amax, b, Td);
    for (int j = blockIdx.x * HIST_THREADS + threadIdx.x; j < V; j += gridDim.x * HIST_THREADS) {
        const float v = l[j];
        const u64 m = mass_of(v, Td, zmax, scale);
        if (!m) continue;
        const unsigned k = ordered_key(v) >> 16, slot = k % HIST_SLOTS;
        const unsigned old = atomicCAS(&lkey[slot], HIST_EMPTY, k);
        if (old == HIST_EMPTY || old == k) {
            atomicAdd(&lmass[slot], m);
        } else {
            atomicAdd(hist + k, m);
            atomicAdd(&lgroup[k >> 8], m);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < HIST_SLOTS; i += HIST_THREADS)
        if (lkey[i] != HIST_EMPTY) {
            atomicAdd(hist + lkey[i], lmass[i]);
            atomicAdd(&lgroup[lkey[i] >> 8], lmass[i]);
        }
    // the group sums: one memory-side atomic per block and non-empty group (a row's masses
    // fall in a few groups; per-bucket atomics on those words would queue up)
    __syncthreads();
    if (threadIdx.x < 256 && lgroup[threadIdx.x]) atomicAdd(gsum + threadIdx.x, lgroup[threadIdx.x]);
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

// Level 1 of the search: the bucket (upper 16 key bits) where the cumulative mass in
// order reaches thr = thr_of(S), S being the sum of all masses, and the mass of all buckets
// before it: first over the 256 group sums (descending), then over the 256 buckets of the
// crossing group. Threads 0..255 of the block scan; every thread returns thr after the
// result is in *st, and S in S_out.
template <typename ThrFn>
__device__ u64 select_bucket(const u64* __restrict__ hist, const u64* __restrict__ gsum, ThrFn thr_of,
                             u64* scan_lds, SelState* st, u64& S_out) {
    const int tid = threadIdx.x;
    __shared__ u64 lv[2];                  // crossing group, mass before it
    if (tid == 0) { st->found = 0; st->prefix = 0; st->above = 0; lv[0] = 0; lv[1] = 0; }
    const u64 g = tid < 256 ? gsum[255 - tid] : 0ull;
    u64 excl;
    const u64 S = block_scan_excl(g, scan_lds, excl);   // synchronises
    const u64 thr = thr_of(S);
    if (tid < 256 && excl < thr && excl + g >= thr) { lv[0] = 255 - tid; lv[1] = excl; }
    __syncthreads();
    const uint32_t G = (uint32_t)lv[0];
    const u64 above0 = lv[1];
    const u64 h = tid < 256 ? hist[256 * G + 255 - tid] : 0ull;
    u64 ex2;
    block_scan_excl(h, scan_lds, ex2);
    if (tid < 256 && above0 + ex2 < thr && above0 + ex2 + h >= thr) {
        st->prefix = 256 * G + 255 - tid;
        st->above = above0 + ex2;
    }
    __syncthreads();
    S_out = S;
    return thr;
}

// The rest of the search over the whole row, from st->prefix (bucket) and st->above.
__device__ void select_refine(const float* __restrict__ l, int V, double Td, double zmax, double scale, u64 thr,
                              u64* scan_lds, u64* h2, SelState* st) {
    const int tid = threadIdx.x;
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

// Stage of a selection: NUC finds the nucleus mass N (top_p < 1), DRAW the drawn token.
enum { SEL_NUC = 0, SEL_DRAW = 1 };

// Many blocks: the threshold of this stage, its crossing bucket (every block finds the
// same; block 0 records it for the walk), and the bucket's members into the row's list as
// (key << 32) | (~id).
template <int STAGE>
__global__ __launch_bounds__(256) void k_sel_gather(const float* __restrict__ logits, u64* __restrict__ ws,
                                                    size_t row_words, int V, float top_p,
                                                    const float* __restrict__ u) {
    __shared__ u64 scan_lds[16];
    __shared__ SelState st;
    const int b = blockIdx.y;
    const float* l = logits + (size_t)b * V;
    u64* w = ws + (size_t)b * row_words;
    const u64* hist = w + RowWs::hist;
    const u64* gs = w + RowWs::gsum;
    u64* sw = w + RowWs::state;
    // this thread's first two logits and the nucleus mass, requested together with the sums
    const int j0 = blockIdx.x * blockDim.x + threadIdx.x, js = gridDim.x * blockDim.x;
    const float v0 = j0 < V ? l[j0] : 0.f;
    const float v1 = j0 + js < V ? l[j0 + js] : 0.f;
    const u64 Nw = (STAGE == SEL_DRAW && top_p < 1.0f) ? sw[SW_N] : 0ull;
    const float ub = STAGE == SEL_DRAW ? u[b] : 0.f;
    u64 S;
    const u64 thr = select_bucket(hist, gs, [&](u64 s) {
        if (STAGE == SEL_NUC) {
            const double tA = ceil((double)top_p * (double)s);
            return tA < 1.0 ? 1ull : (tA >= (double)s ? s : (u64)tA);
        }
        const u64 N = top_p < 1.0f ? Nw : s;
        const double tB = floor((double)ub * (double)N) + 1.0;
        const u64 t = tB >= (double)N ? N : (u64)tB;
        return t < 1 ? 1ull : t;
    }, scan_lds, &st, S);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        sw[SW_ABOVE] = st.above;
        sw[SW_THR] = thr;
        sw[SW_BUCKET] = st.prefix;
        if (STAGE == SEL_NUC) sw[SW_S] = S;
    }
    const uint32_t want = st.prefix;
    unsigned* count = reinterpret_cast<unsigned*>(sw + SW_COUNT);
    u64* list = w + RowWs::list;
    auto visit = [&](float v, int j) {
        const uint32_t key = ordered_key(v);
        if ((key >> 16) == want) {
            const unsigned i = atomicAdd(count, 1u);
            if (i < (unsigned)V) list[i] = ((u64)key << 32) | (u64)(0xFFFFFFFFu - (uint32_t)j);
        }
    };
    if (j0 < V) visit(v0, j0);
    if (j0 + js < V) visit(v1, j0 + js);
    for (int j = j0 + 2 * js; j < V; j += js) visit(l[j], j);
}

// One block per row: sort the bucket's members (descending packed word = key descending,
// id ascending), walk their masses from SW_ABOVE to the first cumulative mass >= SW_THR.
// NUC stores that mass as N; DRAW writes the token and zeroes the row's histogram.
// Runs with 1024 threads (the walk takes 4 members per thread).
template <int STAGE>
__global__ __launch_bounds__(1024) void k_sel_final(const float* __restrict__ logits, const u64* __restrict__ amax,
                                                    int V, double Td, double scale, u64* __restrict__ ws,
                                                    size_t row_words, int32_t* __restrict__ out) {
    __shared__ __align__(16) u64 e[SORT_CAP];
    __shared__ u64 scan_lds[16];
    __shared__ u64 h2[256];
    __shared__ SelState st;
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const float* l = logits + (size_t)b * V;
    u64* w = ws + (size_t)b * row_words;
    u64* sw = w + RowWs::state;
    // one round of reads: the state words, the first blockDim members of the list (read
    // whether or not they were written this call; only the first n are used), the maximum
    // and, for the draw, the group sums that tell which histogram groups to clear
    const u64 above = sw[SW_ABOVE], thr = sw[SW_THR], cw = sw[SW_COUNT], bucket = sw[SW_BUCKET];
    const u64 first = tid < V ? w[RowWs::list + tid] : 0ull;
    const u64 gsv = STAGE == SEL_DRAW ? w[RowWs::gsum + (tid >> 2)] : 0ull;
    const double zmax = row_zmax(amax, b, Td);
    const int n = (int)min((u64)V, cw & 0xFFFFFFFFull);
    if (tid == 0) { st.found = 0; st.id = 0; st.cum = 0; st.above = above; st.prefix = (uint32_t)bucket; }
    if (n <= SORT_CAP) {
        if (n <= (int)blockDim.x && 2 * n <= SORT_CAP) {
            // one member per thread: its place in the descending order is the number of
            // larger words (all distinct: the ids differ), so it is written straight there
            // (past the unsorted copy, which every thread reads meanwhile); the count reads
            // 16 members per round of eight 16-byte shared-memory reads
            const u64 mine = first;
            if (tid < n) e[tid] = mine;
            __syncthreads();
            int rank = 0;
            if (tid < n) {
                const u64x2* e2 = reinterpret_cast<const u64x2*>(e);
                int j = 0;
                for (; j + 16 <= n; j += 16) {
                    u64x2 a[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) a[k] = e2[(j >> 1) + k];
#pragma unroll
                    for (int k = 0; k < 8; ++k) rank += (int)(a[k][0] > mine) + (int)(a[k][1] > mine);
                }
                for (; j < n; ++j) rank += e[j] > mine;
            }
            __syncthreads();
            if (tid < n) e[SORT_CAP / 2 + rank] = mine;
            __syncthreads();
            if (tid < n) e[tid] = e[SORT_CAP / 2 + tid];
            __syncthreads();
        } else {
            int P = 64;
            while (P < n) P <<= 1;
            for (int i = tid; i < P; i += blockDim.x) e[i] = i < n ? (i == tid ? first : w[RowWs::list + i]) : 0ull;
            __syncthreads();
            for (int k = 2; k <= P; k <<= 1)          // bitonic sort, descending
                for (int j = k >> 1; j > 0; j >>= 1) {
                    for (int i = tid; i < P; i += blockDim.x) {
                        const int pr = i ^ j;
                        if (pr > i) {
                            const u64 a = e[i], c = e[pr];
                            const bool desc = (i & k) == 0;
                            if (desc ? a < c : a > c) { e[i] = c; e[pr] = a; }
                        }
                    }
                    __syncthreads();
                }
        }
        // masses in order: thread t takes entries 4t .. 4t+3
        u64 m[4], sum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int i = 4 * tid + q;
            m[q] = i < n ? mass_of(key_to_float((uint32_t)(e[i] >> 32)), Td, zmax, scale) : 0ull;
            sum += m[q];
        }
        u64 excl;
        block_scan_excl(sum, scan_lds, excl);
        u64 c = above + excl;
        if (c < thr) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = 4 * tid + q;
                if (i < n && c + m[q] >= thr) {
                    st.id = (int32_t)(0xFFFFFFFFu - (uint32_t)(e[i] & 0xFFFFFFFFull));
                    st.cum = c + m[q];
                    st.found = 1;
                    break;
                }
                c += m[q];
            }
        }
        __syncthreads();
    } else {
        __syncthreads();
        select_refine(l, V, Td, zmax, scale, thr, scan_lds, h2, &st);
    }
    if (STAGE == SEL_NUC) {
        if (tid == 0) sw[SW_N] = st.found ? st.cum : sw[SW_S];
    } else {
        if (tid == 0) out[b] = st.found ? st.id : (int32_t)(0xFFFFFFFFu - (uint32_t)(amax[b] & 0xFFFFFFFFull));
        // leave the histogram zeroed for the next call: the groups that received mass
        // (a group sum is zero only if all of its buckets are), then the group sums
        u64* hist = w + RowWs::hist;
        const int g = tid >> 2, quarter = tid & 3;
        if (gsv != 0ull)
            for (int i = 0; i < 64; ++i) hist[256 * g + 64 * quarter + i] = 0ull;
        __syncthreads();
        if (tid < 256) w[RowWs::gsum + tid] = 0ull;
    }
    if (tid == 0) sw[SW_COUNT] = 0ull;   // the next gather starts from zero
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
    return (size_t)B * RowWs::words(V) * sizeof(u64);
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
    const size_t rw = RowWs::words(V);
    if (!ws_zeroed && (e = launch_fill_u64(w, 0ull, (int)(B * rw), s)) != hipSuccess) return e;
    const int nblk = (V + 255) / 256 < 512 ? (V + 255) / 256 : 512;
    hipLaunchKernelGGL(k_sample_hist, dim3(HIST_BLOCKS, B), dim3(HIST_THREADS), 0, s, logits, amax, V, Td, scale, w, rw);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (top_p < 1.0f) {
        hipLaunchKernelGGL(k_sel_gather<SEL_NUC>, dim3(nblk, B), dim3(256), 0, s, logits, w, rw, V, top_p, u);
        hipLaunchKernelGGL(k_sel_final<SEL_NUC>, dim3(B), dim3(1024), 0, s, logits, amax, V, Td, scale, w, rw, out);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(k_sel_gather<SEL_DRAW>, dim3(nblk, B), dim3(256), 0, s, logits, w, rw, V, top_p, u);
    hipLaunchKernelGGL(k_sel_final<SEL_DRAW>, dim3(B), dim3(1024), 0, s, logits, amax, V, Td, scale, w, rw, out);
    return hipGetLastError();
}

}  // namespace q3
