// Decode attention: one new query row per sequence against its KV cache
// ("Inside an LLM ...", Step 5: scaled dot-product scores q.k * 128^-0.5, softmax,
// weighted sum of V; grouped-query attention where query heads 2g and 2g+1 both read
// kv head g; a decode row sees every cached slot, so no mask).
//
// Split-K: the visible slots are cut into chunks of CHUNK keys; a block owns one
// (sequence, kv head, chunk) and streams that chunk's K and V once for both query
// heads of the group, producing (max, sum, weighted V) per head. A combine kernel merges
// the chunks' partial results with the usual max-rescaling. bf16 caches use the
// matrix-core kernel below; float32 caches (the toy model) a vector-unit kernel.
#include "common.h"
#include "kernels.h"

namespace q3 {

namespace {

constexpr int CHUNK = 256;     // keys per block (64 per wave): one page of a paged cache
static_assert(CHUNK == kKvPage, "a decode chunk is one cache page");
constexpr int G = 2;           // query heads per kv head
constexpr int PART = 2 + 128;  // (max, sum, acc[128]) per (chunk, head)

__device__ __forceinline__ void ld8(const bf16* p, float* w) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[2 * i] = __uint_as_float(u[i] << 16);
        w[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
}
__device__ __forceinline__ void ld8(const float* p, float* w) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// Merge running state (m2, l2, a2) into (m, l, a).
__device__ __forceinline__ void merge(float& m, float& l, float* a, float m2, float l2, const float* a2) {
    if (l2 == 0.f) return;
    if (l == 0.f) {
        m = m2; l = l2;
#pragma unroll
        for (int i = 0; i < 8; ++i) a[i] = a2[i];
        return;
    }
    const float mn = fmaxf(m, m2);
    const float c1 = expf(m - mn), c2 = expf(m2 - mn);
    l = l * c1 + l2 * c2;
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = a[i] * c1 + a2[i] * c2;
    m = mn;
}

template <typename KT>
__global__ __launch_bounds__(256) void k_attn_decode_part(
    const float* __restrict__ q, const KT* __restrict__ kc, const KT* __restrict__ vc, int t_cap, KvLayout lay,
    const int32_t* __restrict__ lens, int len_extra, int seq_base, int Hq, int Hkv, int nchunk,
    float* __restrict__ part) {
    __shared__ float sm[4][G][PART];
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int grp = lane >> 4, sub = lane & 15;
    const int seq = seq_base + b;
    const int T = min(lens[seq] + len_extra, t_cap);
    const float scale = 0.088388346f;  // fl32(128^-0.5)

    float qv[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const float* qp = q + ((size_t)b * Hq + g * G + h) * 128 + sub * 8;
#pragma unroll
        for (int i = 0; i < 8; ++i) qv[h][i] = qp[i];
    }
    float m[G], l[G], acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        m[h] = -INFINITY; l[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
    }
    const int kbeg = c * CHUNK + wid * 64;
    const int kend = min(kbeg + 64, T);
    // the chunk is one page (CHUNK == kKvPage): its keys are one strided run. The page is
    // looked up whatever the length (c < the table's width: c * CHUNK < max_T <= t_cap), so
    // that lookup and the length load go out together; it is used only for keys < T.
    const size_t chunk_base = lay.off(seq, g, c * CHUNK);
    for (int kk = kbeg + grp; kk < kend; kk += 4) {
        float kv[8], vv[8];
        ld8(kc + chunk_base + (size_t)(kk - c * CHUNK) * 128 + sub * 8, kv);
        ld8(vc + chunk_base + (size_t)(kk - c * CHUNK) * 128 + sub * 8, vv);
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float d = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) d += qv[h][i] * kv[i];
            const float s = sum16(d) * scale;
            const float mn = fmaxf(m[h], s);
            const float corr = expf(m[h] - mn);
            const float p = expf(s - mn);
            l[h] = l[h] * corr + p;
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[h][i] = acc[h][i] * corr + p * vv[i];
            m[h] = mn;
        }
    }
    // merge the four 16-lane groups of the wave (lanes sub, sub+16, sub+32, sub+48)
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float a2[8];
            const float m2 = __shfl_xor(m[h], off, 64), l2 = __shfl_xor(l[h], off, 64);
#pragma unroll
            for (int i = 0; i < 8; ++i) a2[i] = __shfl_xor(acc[h][i], off, 64);
            merge(m[h], l[h], acc[h], m2, l2, a2);
        }
    }
    if (grp == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            if (sub == 0) { sm[wid][h][0] = m[h]; sm[wid][h][1] = l[h]; }
#pragma unroll
            for (int i = 0; i < 8; ++i) sm[wid][h][2 + sub * 8 + i] = acc[h][i];
        }
    }
    __syncthreads();
    // merge the four waves: thread t < G*128 owns (head t / 128, dim t % 128)
    if (threadIdx.x < G * 128) {
        const int h = threadIdx.x >> 7, d = threadIdx.x & 127;
        float M = -INFINITY;
        for (int w = 0; w < 4; ++w)
            if (sm[w][h][1] > 0.f) M = fmaxf(M, sm[w][h][0]);
        float L = 0.f, A = 0.f;
        for (int w = 0; w < 4; ++w) {
            if (sm[w][h][1] > 0.f) {
                const float cf = expf(sm[w][h][0] - M);
                L += sm[w][h][1] * cf;
                A += sm[w][h][2 + d] * cf;
            }
        }
        float* pp = part + ((((size_t)b * Hkv + g) * nchunk + c) * G + h) * PART;
        if (d == 0) { pp[0] = M; pp[1] = L; }
        pp[2 + d] = A;
    }
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

// bf16 cache: the same (sequence, kv head, chunk) partial state, computed in two passes.
// Scores S^T = K q^T on the matrix cores (a wave takes 64 keys as four 16-key tiles whose K
// rows are loaded straight into A-operand registers; q, split into bf16 hi + lo, is the B
// operand with the two query heads as columns 0 and 1), then the chunk's max and sum per
// head through shared memory, then P.V on the vector units (16 lane groups, 8 dims per
// lane, V rows loaded before the scores are computed) with no per-key rescaling.
__global__ __launch_bounds__(256, 2) void k_attn_decode_mfma(
    const float* __restrict__ q, const bf16* __restrict__ kc, const bf16* __restrict__ vc, int t_cap, KvLayout lay,
    const int32_t* __restrict__ lens, int len_extra, int seq_base, int Hq, int Hkv, int nchunk,
    float* __restrict__ part) {
    __shared__ float sp[G][CHUNK];     // scores, then probabilities
    __shared__ float hs[G][4];         // per-head wave maxima [0..1] and sums [2..3]
    // each wave's 64 K rows (16-byte chunk c of row r at c ^ (r & 15)); after the scores the
    // same memory holds the P.V partials of the 16 lane groups
    __shared__ u32x4 sK[4][64 * 16];
    float (*wm)[G][128] = reinterpret_cast<float (*)[G][128]>(&sK[0][0]);
    static_assert(sizeof(float) * 16 * G * 128 <= sizeof(u32x4) * 4 * 64 * 16, "P.V partials fit the K rows");
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, quad = lane >> 4, col = lane & 15;
    const int seq = seq_base + b;
    const int T = min(lens[seq] + len_extra, t_cap);
    const int k0 = c * CHUNK + wid * 64;             // this wave's first key
    // the chunk is one page (CHUNK == kKvPage): keys key, offset head_base + key * 128. The
    // page is looked up whatever the length (c < the table's width: c * CHUNK < max_T <=
    // t_cap), so that lookup and the length load go out together; it is used for keys < T.
    const size_t head_base = lay.off(seq, g, c * CHUNK) - (size_t)c * CHUNK * 128;
    const float scale = 0.088388346f;                // fl32(128^-0.5)

    // V rows for P.V: lane group (wid, quad) takes keys k0 + quad + 4 i, lane col dims 8 col ..
    // (16 lanes read a whole 256-byte row, once: non-temporal loads)
    u32x4 vr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int key = k0 + quad + 4 * i;
        vr[i] = key < T ? __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(vc + head_base + (size_t)key * 128 + 8 * col))
                        : u32x4{0u, 0u, 0u, 0u};
    }
    // q^T (B operand): lane holds q[head col][32 ks + 8 quad + e] for col < 2, else zeros
    bf16x8 qh[4], ql[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        f32x8 x = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (col < G) {
            const f32x4* qp = reinterpret_cast<const f32x4*>(q + ((size_t)b * Hq + g * G + col) * 128 + 32 * ks + 8 * quad);
            const f32x4 u0 = qp[0], u1 = qp[1];
            x = f32x8{u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
        }
        qh[ks] = __builtin_convertvector(x, bf16x8);
        ql[ks] = __builtin_convertvector(x - __builtin_convertvector(qh[ks], f32x8), bf16x8);
    }
    // K rows, whole: instruction i brings keys k0 + 4 i + quad, lane col their chunk col (16
    // lanes read a 256-byte row once: non-temporal loads). Through this wave's LDS rows into
    // the A-operand layout (tile t row col = key k0 + 16 t + col, dims 32 ks + 8 quad ..);
    // the wave reads only what it wrote, so no barrier.
    u32x4 kraw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int key = k0 + 4 * i + quad;
        kraw[i] = key < T ? __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(kc + head_base + (size_t)key * 128 + 8 * col))
                          : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int r = 4 * i + quad;
        sK[wid][r * 16 + (col ^ (r & 15))] = kraw[i];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
        bf16x8 ka[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int r = 16 * t + col;
            ka[ks] = __builtin_bit_cast(bf16x8, sK[wid][r * 16 + ((4 * ks + quad) ^ (r & 15))]);
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8 a = ka[ks];
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[ks], sc, 0, 0, 0);
            sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[ks], sc, 0, 0, 0);
        }
        if (col < G) {                               // D[key 4 quad + r][head col]
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int kl = wid * 64 + 16 * t + 4 * quad + r;
                sp[col][kl] = c * CHUNK + kl < T ? sc[r] * scale : -INFINITY;
            }
        }
    }
    __syncthreads();
    // chunk max and sum per head: head h = tid / 128 over keys i and i + 128
    float M, L;
    {
        const int h = tid >> 7, i = tid & 127;
        const float x0 = sp[h][i], x1 = sp[h][i + 128];
        const float wmx = wave_max(fmaxf(x0, x1));
        if (lane == 0) hs[h][wid & 1] = wmx;
        __syncthreads();
        M = fmaxf(hs[h][0], hs[h][1]);
        const float p0 = x0 == -INFINITY ? 0.f : __expf(x0 - M);
        const float p1 = x1 == -INFINITY ? 0.f : __expf(x1 - M);
        sp[h][i] = p0;
        sp[h][i + 128] = p1;
        const float ws = wave_sum(p0 + p1);
        if (lane == 0) hs[h][2 + (wid & 1)] = ws;
        __syncthreads();
        L = hs[h][2] + hs[h][3];
    }
    // P.V
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int kl = wid * 64 + quad + 4 * i;
        const float p0 = sp[0][kl], p1 = sp[1][kl];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v0 = __uint_as_float(vr[i][e] << 16), v1 = __uint_as_float(vr[i][e] & 0xFFFF0000u);
            acc[0][2 * e] += p0 * v0;
            acc[0][2 * e + 1] += p0 * v1;
            acc[1][2 * e] += p1 * v0;
            acc[1][2 * e + 1] += p1 * v1;
        }
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) wm[wid * 4 + quad][h][8 * col + e] = acc[h][e];
    __syncthreads();
    {
        const int h = tid >> 7, d = tid & 127;
        float a[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) a[j] = wm[j][h][d];
#pragma unroll
        for (int hh = 1; hh < 16; hh <<= 1)
#pragma unroll
            for (int j = 0; j + hh < 16; j += 2 * hh) a[j] += a[j + hh];
        float* pp = part + ((((size_t)b * Hkv + g) * nchunk + c) * G + h) * PART;
        if (d == 0) { pp[0] = M; pp[1] = L; }     // L == 0 (M = -inf) when the chunk is empty
        pp[2 + d] = a[0];
    }
}

// o_pair: o is bf16 pair rows [B][2 * Hq * 128] (hi parts, then lo parts), else float32.
template <bool PAIR>
__global__ __launch_bounds__(128) void k_attn_decode_combine(
    const float* __restrict__ part, const int32_t* __restrict__ lens, int len_extra, int seq_base,
    int Hq, int Hkv, int nchunk, void* __restrict__ o) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    const int g = h / G, hh = h % G;
    const int T = lens[seq_base + b] + len_extra;
    const int nc = min(nchunk, (T + CHUNK - 1) / CHUNK);
    const float* base = part + (((size_t)b * Hkv + g) * nchunk) * G * PART;
    // one pass over the chunk states in batches of 16 (loads in flight together), the
    // running state rescaled to each batch's maximum; empty chunks (sum 0) weigh 0
    float M = -INFINITY, L = 0.f, A = 0.f;
    for (int c0 = 0; c0 < nc; c0 += 16) {
        float mv[16], lv[16], av[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float* pp = base + ((size_t)(c0 + u) * G + hh) * PART;
            const bool in = c0 + u < nc;
            mv[u] = in ? pp[0] : 0.f;
            lv[u] = in ? pp[1] : 0.f;
            av[u] = in ? pp[2 + d] : 0.f;
        }
        float bm = M;
#pragma unroll
        for (int u = 0; u < 16; ++u) bm = fmaxf(bm, lv[u] > 0.f ? mv[u] : -INFINITY);
        if (bm == -INFINITY) continue;             // no keys yet
        const float cs = L > 0.f ? expf(M - bm) : 0.f;
        L *= cs;
        A *= cs;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const float cf = lv[u] > 0.f ? expf(mv[u] - bm) : 0.f;
            L += lv[u] * cf;
            A += av[u] * cf;
        }
        M = bm;
    }
    const float v = L > 0.f ? A / L : 0.f;
    if constexpr (PAIR) {
        bf16* row = static_cast<bf16*>(o) + (size_t)b * 2 * Hq * 128;
        const bf16 hi = f2bf(v);
        row[h * 128 + d] = hi;
        row[(size_t)Hq * 128 + h * 128 + d] = f2bf(v - bf2f(hi));
    } else {
        static_cast<float*>(o)[((size_t)b * Hq + h) * 128 + d] = v;
    }
}

}  // namespace

size_t attn_decode_workspace_bytes(int B, int Hkv, int max_T) {
    const int nchunk = (max_T + CHUNK - 1) / CHUNK;
    return (size_t)B * Hkv * nchunk * G * PART * sizeof(float);
}

hipError_t launch_attn_decode(const float* q, const void* kc, const void* vc, int kv_bf16,
                              int t_cap, const KvLayout& lay, const int32_t* lens, int len_extra, int seq_base,
                              int B, int Hq, int Hkv, int max_T, float* ws, void* o, int o_pair, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    if (Hq != G * Hkv || max_T > t_cap) return hipErrorInvalidValue;   // (chunks index the page table)
    const int nchunk = (max_T + CHUNK - 1) / CHUNK;
    dim3 grid(nchunk, Hkv, B);
    if (kv_bf16)
        hipLaunchKernelGGL(k_attn_decode_mfma, grid, dim3(256), 0, s, q, (const bf16*)kc,
                           (const bf16*)vc, t_cap, lay, lens, len_extra, seq_base, Hq, Hkv, nchunk, ws);
    else
        hipLaunchKernelGGL(k_attn_decode_part<float>, grid, dim3(256), 0, s, q, (const float*)kc,
                           (const float*)vc, t_cap, lay, lens, len_extra, seq_base, Hq, Hkv, nchunk, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (o_pair)
        hipLaunchKernelGGL(k_attn_decode_combine<true>, dim3(Hq, B), dim3(128), 0, s, ws, lens, len_extra,
                           seq_base, Hq, Hkv, nchunk, (void*)o);
    else
        hipLaunchKernelGGL(k_attn_decode_combine<false>, dim3(Hq, B), dim3(128), 0, s, ws, lens, len_extra,
                           seq_base, Hq, Hkv, nchunk, (void*)o);
    return hipGetLastError();
}

}  // namespace q3
