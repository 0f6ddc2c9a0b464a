// Persistent decode step: the whole forward pass of one decode step -- embedding, every
// layer, final RMSNorm, tied LM head with fused argmax -- in ONE cooperative launch of
// 256 workgroups (one per CU). ("Inside an LLM: Pure Python Inference for Qwen3-0.6B on
// MLX", Steps 2-8; Step 9's decode loop runs one launch per generated token.)
//
// Why: a decode step streams 1.19 GB of bf16 weights (150 us at 8 TB/s) through ~170
// small dependent operations; as separate kernels each costs ~4-8 us of launch and ramp.
//
// Synchronisation is dataflow, not barriers: every value one workgroup hands to another
// is a float32 word in an exchange buffer that holds a sentinel NaN pattern until it is
// written, with one coherent (agent-scope) store; the consumer polls exactly the words it
// needs, 16 bytes per load with the coherent-load bit, until none holds the sentinel.
// One memory round trip thus carries both the data and the "it is ready" signal. Each
// layer has its own buffers, so a word is written once per launch; the small tail kernel
// that follows every launch puts the sentinel back into every word the launch used (also
// after a launch that gave up waiting). The two reductions among hand-overs, x' = x + the
// O-projection partials of the 8 kv groups and x'' = x' + the down-projection partials of
// 8 column blocks, are summed in memory instead: 64-bit fixed-point words with
// device-scope atomic adds, whose top bits count the arrivals. On MI355X one all-to-all
// hand-over among 256 workgroups takes ~2 us this way (~1 us within a group of 32), so the
// layout below is built around four per layer, two of them group-local. Workgroup w is
// (g, j) = (w % 8, w / 8): the dispatcher places workgroup w on XCD w % 8, so each kv
// group's 32 workgroups share one XCD and its L2, and the group-local words are stored
// with workgroup scope (they stay in that L2) instead of being written through to memory.
//
// Per layer, for each row b (hand-overs marked ->):
//   A  poll the x sums (1024) -> RMSNorm -> 16 of the 512 rows of [Wq;Wk;Wv] that kv
//      group g needs                                                  -> QKV words
//   B  workgroup (g, j), kv group g = query heads 2g, 2g+1, j < 32: poll the group's
//      q/k/v (512) -> QK-norm + RoPE -> KV append (j == 0) -> attention of both heads,
//      recomputed by the 32 workgroups of the group (K/V staged through LDS) -> rows
//      32j..32j+31 of Wo[:, 256g:256g+256] . o, plus x for g = 0   -> added to x' sums
//      (long context: split-K partials per (group, chunk), merged again by every
//       workgroup of the group, then the same O-projection partial)
//   C  poll the x' sums (1024, complete when all 8 groups added) -> RMSNorm -> gate/up
//      rows of 12 SwiGLU columns in group g's block 384g .. 384g+383   -> A words
//   D  workgroup (g, j): poll a[384g .. 384g+383] (written by the 32 workgroups of group
//      g in C) -> rows 32j..32j+31 of Wd[:, 384g:384g+384] . a, plus x' for g = 0
//                                                                     -> added to x'' sums
// then poll x, RMSNorm, 594 rows of the tied LM head per workgroup; each workgroup
// writes its packed (logit, id) maximum per row, reduced by a small tail kernel. Each
// workgroup issues the loads of its next weight slice right after finishing a phase, so
// HBM streaming overlaps the waiting.
// Fixed shape: hidden 1024, 16 query / 8 kv heads of 128, FFN 3072, bf16 weights and KV
// cache, 1..4 rows.
#include "common.h"
#include "decode_mega.h"

namespace q3 {

namespace {

constexpr int D = 1024, HQ = 16, HKV = 8, DH = 128, F = 3072, NQKV = 4096;
constexpr int NWG = 256, NT = 256;
constexpr int BMAX = 4;
constexpr int PART = 2 + DH;     // (max, sum, acc[128]) per (chunk, head)
constexpr int MAXCH = 32;        // attention chunks per kv group (long context)
constexpr int SHORT_T = kMegaShortSlots;   // visible slots up to which every group workgroup attends itself
typedef unsigned long long u64;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;

// words per (layer, row) in each exchange buffer
constexpr size_t W_X = (size_t)2 * D, W_QKV = NQKV, W_P = (size_t)2 * D, W_A = F;   // W_X, W_P: D 64-bit sums
constexpr int DCOLS = F / HKV;    // columns of a per down-projection block (phase D)
static_assert(DCOLS == 6 * 8 * 8, "phase D: 8 lanes per row, 6 chunks of 8 columns each");
constexpr size_t W_PT = (size_t)MAXCH * HKV * 2 * PART;   // [chunk][group][head][PART]
constexpr int PT_CHUNK = HKV * 2 * PART;                     // words per chunk index

constexpr unsigned SENT = 0x7FC0DEADu;   // "not written yet" (a NaN no computation yields)
constexpr int SC1 = 16;                  // cache-policy bit of an agent-coherent access

// A poll reads the same address again and again with nothing the compiler sees writing it:
// every read takes its offset through an empty asm statement, which the compiler must treat
// as producing a new value, so it can neither hoist the read out of the loop nor merge two
// reads (it still tracks each read for its wait counters).
__device__ __forceinline__ int fresh(int v) {
    asm volatile("" : "+v"(v));
    return v;
}

// A hand-over word whose consumers all run on the producer's XCD (workgroups w with the
// same w % 8 share one XCD and its L2): a workgroup-scope store stays in that L2, where the
// consumers' agent-coherent loads find it; it is invisible to other XCDs. Measured on
// MI355X: a round trip between two workgroups of one XCD takes ~0.93 us this way against
// ~1.32 us with agent-scope stores, which write through to memory. Issued as a plain vector
// store: the compiler's own store would make it wait for the store to complete before the
// data register is reused (a memory round trip per hand-over); the hardware reads a dword
// store's data at issue.
__device__ __forceinline__ void put_xcd(float* p, float v) {
    unsigned u = __float_as_uint(v);
    if (u == SENT) u = 0x7FC00000u;      // keep real NaNs distinguishable from "not written"
    asm volatile("global_store_dword %0, %1, off sc0" ::"v"(p), "v"(u) : "memory");
}

// 8 bf16 (one 16-byte chunk) dotted with 8 floats.
__device__ __forceinline__ float dot8(const u32x4 w, const float* x) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        s += __uint_as_float(w[i] << 16) * x[2 * i];
        s += __uint_as_float(w[i] & 0xFFFF0000u) * x[2 * i + 1];
    }
    return s;
}

// sum over i < N of dot8(w[i], x[(first + step i) * 8 ...]): every shared-memory read is
// issued before the first multiply, and each chunk has its own accumulator.
template <int N>
__device__ __forceinline__ float dot_chunks(const u32x4* w, const float* x, int first, int step) {
    f32x4 a[2 * N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const f32x4* src = reinterpret_cast<const f32x4*>(x + (first + step * i) * 8);
        a[2 * i] = src[0];
        a[2 * i + 1] = src[1];
    }
    // (left to itself the scheduler pairs the reads with their products, one round trip per
    // pair)
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * N, 0);
    float part[N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float t = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x4& v = a[2 * i + (e >> 1)];
            t += __uint_as_float(w[i][e] << 16) * v[(e & 1) * 2];
            t += __uint_as_float(w[i][e] & 0xFFFF0000u) * v[(e & 1) * 2 + 1];
        }
        part[i] = t;
    }
#pragma unroll
    for (int h = 1; h < N; h <<= 1)
#pragma unroll
        for (int i = 0; i + h < N; i += 2 * h) part[i] += part[i + h];
    return part[0];
}

// Loads through global-address-space pointers: the weight pointers come from a table in
// memory, so the compiler cannot infer their address space and would emit flat loads,
// which also count against the LDS wait counter -- every LDS access or lane shuffle would
// then wait for all weight prefetches in flight.
#define GLOBAL_AS __attribute__((address_space(1)))
// Weight chunks: every weight byte of a step is read by exactly one workgroup, once, so
// they are loaded non-temporally (streaming reads reach ~7 TB/s this way on MI355X against
// ~6 TB/s with the default cache policy).
__device__ __forceinline__ u32x4 ldw16(const bf16* p) { return __builtin_nontemporal_load((const GLOBAL_AS u32x4*)(p)); }
// Lanes 2m and 2m + 1 each hold 4 consecutive elements (lo: elements 8m .. 8m + 3 in lane
// 2m, hi: 8m + 4 .. 8m + 7 in lane 2m + 1); after pair8 both hold all 8, as (lo, hi).
__device__ __forceinline__ void pair8(const f32x4 mine, f32x4& lo, f32x4& hi) {
    f32x4 other;
#pragma unroll
    for (int e = 0; e < 4; ++e) other[e] = dpp_mov<kDppQuadXor1>(mine[e]);
    const bool odd = threadIdx.x & 1;
    lo = odd ? other : mine;
    hi = odd ? mine : other;
}
// 8 bf16 (one 16-byte chunk) dotted with (lo, hi)
__device__ __forceinline__ float dot8v(const u32x4 w, const f32x4 lo, const f32x4 hi) {
    return ((__uint_as_float(w[0] << 16) * lo[0] + __uint_as_float(w[0] & 0xFFFF0000u) * lo[1]) +
            (__uint_as_float(w[1] << 16) * lo[2] + __uint_as_float(w[1] & 0xFFFF0000u) * lo[3])) +
           ((__uint_as_float(w[2] << 16) * hi[0] + __uint_as_float(w[2] & 0xFFFF0000u) * hi[1]) +
            (__uint_as_float(w[3] << 16) * hi[2] + __uint_as_float(w[3] & 0xFFFF0000u) * hi[3]));
}
// Weight-only int8: codes q in [-127, 127], one byte each; a code becomes a float exactly
// (sign-extending bit extract, then int to float) and multiplies x without cancellation
// (an offset-binary code u = q + 128 would save the extract but sum terms ~3x the size of
// the result: measured 2e-3 relative L2 on the 28-layer logits against ~5e-4). The row's
// scale multiplies the finished row sum. A chunk is 8 codes (8 bytes), at the same columns
// as a bf16 chunk of 16 bytes.
// Weight-only int4: codes q in [-7, 7], two per byte (code k of a row in byte k / 2, the
// low nibble for even k), so a chunk of 8 codes is one 32-bit word, code i in bits
// 4i .. 4i + 3; each code is sign-extended exactly as the int8 ones, with the row scale
// applied the same way.
// WQ: 0 bf16 weights, 1 int8 codes, 2 int4 codes.
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
template <int WQ> struct WChunk { typedef u32x4 T; };
template <> struct WChunk<1> { typedef u32x2 T; };
template <> struct WChunk<2> { typedef unsigned T; };
__device__ __forceinline__ u32x2 ldw8(const uint8_t* p) { return __builtin_nontemporal_load((const GLOBAL_AS u32x2*)(p)); }
__device__ __forceinline__ unsigned ldw4(const uint8_t* p) { return __builtin_nontemporal_load((const GLOBAL_AS unsigned*)(p)); }
// the chunk of the 8 weights at element e (a multiple of 8) of the matrix
template <int WQ>
__device__ __forceinline__ typename WChunk<WQ>::T ldwc(const void* base, size_t e) {
    if constexpr (WQ == 1) return ldw8(static_cast<const uint8_t*>(base) + e);
    else if constexpr (WQ == 2) return ldw4(static_cast<const uint8_t*>(base) + e / 2);
    else return ldw16(static_cast<const bf16*>(base) + e);
}
// quantised matrix buffer: the codes of its n_codes weights (n_codes bytes for int8,
// n_codes / 2 for int4), then the rows' float32 scales
template <int WQ>
__device__ __forceinline__ const float* row_scales(const void* m, size_t n_codes) {
    return reinterpret_cast<const float*>(static_cast<const uint8_t*>(m) + (WQ == 2 ? n_codes / 2 : n_codes));
}
__device__ __forceinline__ float sb(unsigned w, int k) { return (float)((int)(w << (24 - 8 * k)) >> 24); }
// 8 codes dotted with (lo, hi)
__device__ __forceinline__ float dot8v(const u32x2 w, const f32x4 lo, const f32x4 hi) {
    return ((sb(w[0], 0) * lo[0] + sb(w[0], 1) * lo[1]) + (sb(w[0], 2) * lo[2] + sb(w[0], 3) * lo[3])) +
           ((sb(w[1], 0) * hi[0] + sb(w[1], 1) * hi[1]) + (sb(w[1], 2) * hi[2] + sb(w[1], 3) * hi[3]));
}
// sum over i < N of chunk i of codes dotted with x[(first + step i) * 8 ...], as the bf16
// dot_chunks: every shared-memory read first, one accumulator per chunk
template <int N>
__device__ __forceinline__ float dot_chunks(const u32x2* w, const float* x, int first, int step) {
    f32x4 a[2 * N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const f32x4* src = reinterpret_cast<const f32x4*>(x + (first + step * i) * 8);
        a[2 * i] = src[0];
        a[2 * i + 1] = src[1];
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * N, 0);
    float part[N];
#pragma unroll
    for (int i = 0; i < N; ++i) part[i] = dot8v(w[i], a[2 * i], a[2 * i + 1]);
#pragma unroll
    for (int h = 1; h < N; h <<= 1)
#pragma unroll
        for (int i = 0; i + h < N; i += 2 * h) part[i] += part[i + h];
    return part[0];
}

__device__ __forceinline__ float sn(unsigned w, int k) { return (float)((int)(w << (28 - 4 * k)) >> 28); }
// 8 int4 codes dotted with (lo, hi)
__device__ __forceinline__ float dot8v(const unsigned w, const f32x4 lo, const f32x4 hi) {
    return ((sn(w, 0) * lo[0] + sn(w, 1) * lo[1]) + (sn(w, 2) * lo[2] + sn(w, 3) * lo[3])) +
           ((sn(w, 4) * hi[0] + sn(w, 5) * hi[1]) + (sn(w, 6) * hi[2] + sn(w, 7) * hi[3]));
}
template <int N>
__device__ __forceinline__ float dot_chunks(const unsigned* w, const float* x, int first, int step) {
    f32x4 a[2 * N];
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const f32x4* src = reinterpret_cast<const f32x4*>(x + (first + step * i) * 8);
        a[2 * i] = src[0];
        a[2 * i + 1] = src[1];
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * N, 0);
    float part[N];
#pragma unroll
    for (int i = 0; i < N; ++i) part[i] = dot8v(w[i], a[2 * i], a[2 * i + 1]);
#pragma unroll
    for (int h = 1; h < N; h <<= 1)
#pragma unroll
        for (int i = 0; i + h < N; i += 2 * h) part[i] += part[i + h];
    return part[0];
}

__device__ __forceinline__ f32x4 ldf4(const float* p) { return *(const GLOBAL_AS f32x4*)(p); }
__device__ __forceinline__ float ldf(const float* p) { return *(const GLOBAL_AS float*)(p); }
// A pointer every lane holds alike, moved into scalar registers here (the empty asm keeps
// the read at this point of the program).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
    const unsigned long long v = (unsigned long long)p;
    unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v), hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
    asm volatile("" : "+s"(lo), "+s"(hi));
    return (T*)((unsigned long long)hi << 32 | lo);
}

// Poll the 16-byte chunks cidx(i), i < nch (nch <= K * 256; cidx = word offset of the
// chunk's first word from `base`, a multiple of 4), into dst[4 i .. 4 i + 3] until none of
// their words holds the sentinel. Thread t owns chunks t + 256 k and re-reads only those
// it still misses; a wave leaves the loop as soon as all its lanes are done, then one
// barrier joins the workgroup. `words` bounds the buffer (reads past it return zero
// instead of touching other memory). Returns false after ~0.1 s without completion (the
// caller then leaves the kernel, and so, through their own waits, do all others).
struct NoSentinel {   // a chunk is complete when none of its words holds the sentinel
    __device__ __forceinline__ bool operator()(const u32x4 v) const {
        return v[0] != SENT && v[1] != SENT && v[2] != SENT && v[3] != SENT;
    }
};

template <int K, typename CIDX, typename READY = NoSentinel>
__device__ __forceinline__ bool poll(const float* base, size_t words, CIDX cidx, int nch, float* dst, unsigned* err,
                                     READY ready = READY{}) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(words * 4), 0x00020000);
    unsigned todo = 0;
#pragma unroll
    for (int k = 0; k < K; ++k)
        if ((int)threadIdx.x + NT * k < nch) todo |= 1u << k;
    int spins = 0;
    bool ok = true;
    for (;;) {
        u32x4 v[K];
#pragma unroll
        for (int k = 0; k < K; ++k)
            if (todo & (1u << k))
                v[k] = __builtin_amdgcn_raw_buffer_load_b128(rs, fresh((int)(cidx(threadIdx.x + NT * k) * 4)), 0, SC1);
#pragma unroll
        for (int k = 0; k < K; ++k) {
            if ((todo & (1u << k)) && ready(v[k])) {
                *reinterpret_cast<u32x4*>(dst + 4 * (threadIdx.x + NT * k)) = v[k];
                todo &= ~(1u << k);
            }
        }
        if (!__any(todo != 0)) break;
        if (++spins > (1 << 16)) {
            atomicOr(err, Q3_DEVERR_SYNC);
            ok = false;
            break;
        }
    }
    return __syncthreads_and(ok);
}

// The O-projection partials of the 8 kv groups (and the down-projection partials of the 8
// column blocks) are summed in memory: each group adds its
// value to a 64-bit word with a device-scope atomic add, as an integer, so the sum does not
// depend on the order of arrival. A contribution is 2^60 (bits 60..63 count the arrived
// groups) + round(v * 2^30) + 2^52 (bias: every contribution's value field is positive and
// below 2^53, so 8 of them stay below 2^56). A value that is not finite or has |v| >= 2^22
// adds 2^56 instead (bits 56..59 then make the sum read as NaN). The words start at zero;
// a sum is complete when its count field reads 8.
constexpr int FX_SHIFT = 30;
constexpr float FX_LIMIT = 4194304.0f;   // 2^22
__device__ __forceinline__ void fx_add(u64* p, float v) {
    u64 c = 1ull << 60;
    if (fabsf(v) < FX_LIMIT) c += (u64)(__float2ll_rn(v * (float)(1 << FX_SHIFT)) + (1ll << 52));
    else c += 1ull << 56;
    __hip_atomic_fetch_add(p, c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float fx_value(u64 s) {
    if ((s >> 56) & 0xFull) return __uint_as_float(0x7FC00000u);
    const long long q = (long long)(s & ((1ull << 56) - 1)) - (long long)HKV * (1ll << 52);
    return (float)((double)q * (1.0 / (double)(1ll << FX_SHIFT)));
}
struct FxComplete {   // both 64-bit sums of the chunk have all HKV contributions
    __device__ __forceinline__ bool operator()(const u32x4 v) const {
        return (v[1] >> 28) == (unsigned)HKV && (v[3] >> 28) == (unsigned)HKV;
    }
};
// the four sums of a thread's two polled chunks (FxPair) as floats
__device__ __forceinline__ f32x4 fx_vec4(const u32x4 (&c)[2]) {
    return f32x4{fx_value((u64)c[0][1] << 32 | c[0][0]), fx_value((u64)c[0][3] << 32 | c[0][2]),
                 fx_value((u64)c[1][1] << 32 | c[1][0]), fx_value((u64)c[1][3] << 32 | c[1][2])};
}

// Like `poll`, but without the closing barrier, and the chunks stay in the polling
// thread's registers: out[k] = chunk cidx(threadIdx.x + NT k). Returns this thread's
// success; the caller joins the workgroup with __syncthreads_and of it.
template <int K, typename CIDX, typename READY = NoSentinel>
__device__ __forceinline__ bool poll_own(const float* base, size_t words, CIDX cidx, u32x4 (&out)[K], unsigned* err,
                                         READY ready = READY{}) {
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)(words * 4), 0x00020000);
    // Two rounds in flight: round n + 1 is issued right before round n is checked (every
    // round re-reads all K chunks; a chunk found complete is kept from its round). Measured
    // on the bs1 step: faster than one round in flight; spreading the two rounds half a
    // round trip apart, or a third round, was slower.
    unsigned todo = (1u << K) - 1;
    auto load = [&](int k) {
        return __builtin_amdgcn_raw_buffer_load_b128(rs, fresh((int)(cidx(threadIdx.x + NT * k) * 4)), 0, SC1);
    };
    u32x4 va[K];
#pragma unroll
    for (int k = 0; k < K; ++k) va[k] = load(k);
    for (int spins = 0; spins < (1 << 15); ++spins) {
        u32x4 vb[K];
#pragma unroll
        for (int k = 0; k < K; ++k) vb[k] = load(k);
        asm volatile("" ::: "memory");   // keeps the issue of this round before the check
#pragma unroll
        for (int k = 0; k < K; ++k)
            if ((todo & (1u << k)) && ready(va[k])) {
                out[k] = va[k];
                todo &= ~(1u << k);
            }
        if (!__any(todo != 0)) return true;
#pragma unroll
        for (int k = 0; k < K; ++k) va[k] = load(k);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < K; ++k)
            if ((todo & (1u << k)) && ready(vb[k])) {
                out[k] = vb[k];
                todo &= ~(1u << k);
            }
        if (!__any(todo != 0)) return true;
    }
    atomicOr(err, Q3_DEVERR_SYNC);
    return false;
}

struct FxPair {   // thread t's chunks k = 0, 1: the sums 4t .. 4t+3 (chunk i = t + NT k)
    __device__ __forceinline__ size_t operator()(int i) const { return (size_t)8 * (i % NT) + 4 * (i / NT); }
};

constexpr int TRACE_MAX = 400;   // phase timestamps kept per traced workgroup
constexpr int PGMAX = kMegaPageIds;   // cache page ids per row held in shared memory
constexpr int STAGE = 256;       // K/V rows of the staging area
constexpr int SHOT = 240;        // cached rows staged per shot (the new key follows them)
constexpr int SHOTD = 120;       // the same with two staging halves of 128 rows (long variant)
constexpr int LONG_T = 8192;     // contexts above this take the long variant of the kernel

struct Smem {
    union {
        struct {
            float act[BMAX][D];            // normed x of the LM head; phase D: the polled slice of a
            float part[MAXCH * 2 * PART];  // polled chunk partials (long context combine)
            float wm[16][2][PART];         // attention state per (wave, 16-lane key group)
        } s;
        struct {
            float rd[BMAX][24][NT / 2];    // partial dot products of phases A, C, D per lane pair
        } r;
        struct {                           // attention: staged cache rows of one kv head
            bf16 k[STAGE][DH];
            bf16 v[STAGE][DH];
        } kv;
    } u;
    float xg[BMAX][32];            // layer input x at rows 32j..32j+31 (phase-B row block)
    float xr[BMAX][32];            // x' at rows 32j..32j+31 (residual of the phase-D row block)
    float red[BMAX][16];           // block reductions
    float in[BMAX][4 * DH];        // polled group inputs: q (2 x 128), k (128), v (128)
    __attribute__((aligned(16))) bf16 qb[2][2][DH];   // rotated queries of the group: bf16 hi, lo parts
    float kn[DH], vn[DH];          // new key / value (bf16-rounded values)
    float o[BMAX][2 * DH];         // attention output of the group, per row
    float att[2][PART];            // merged attention state (max, sum, acc) per head
    __attribute__((aligned(16))) float sp[STAGE][2];   // scores, then probabilities (key, head)
    __attribute__((aligned(16))) float hs[2][4];   // per-wave softmax maximum of each head
    __attribute__((aligned(16))) float wl[2][4];   // per-wave softmax sum of each head
    float gu[24][BMAX];            // gate/up results
    float rc[BMAX][64], rs[BMAX][64];   // cos / sin of the row's position times frequency i
    MegaLayer layers[kMegaMaxLayers];
    unsigned long long tr[TRACE_MAX];   // phase timestamps (trace only)
    int pg[BMAX][PGMAX];           // cache page ids of this workgroup's attention range, per row
    int pg0[BMAX];                 // (the range's first page)
    __attribute__((aligned(16))) bf16 knc[BMAX][DH];   // causal rows: every row's new key / value
    __attribute__((aligned(16))) bf16 vnc[BMAX][DH];   // (bf16: the values are bf16-rounded already)
};
constexpr size_t kStaticShared = 4 * BMAX * sizeof(unsigned long long);   // wbest of the LM head
static_assert(sizeof(Smem) + kStaticShared <= 160 * 1024, "shared memory of one CU");

// Per-thread values loaded together with a phase's weight slice: the RMSNorm weights of
// its 4 elements, and for phase B the QK-norm weights of its RoPE pair.
struct Pre {
    f32x4 nw;
    float qk1, qk2;
    float sa, so, sg, sd;   // int8 weights: scale of the row this thread finishes in phase A, B, C, D
};


__device__ __forceinline__ int clamp_tok(const MegaParams& p, int b) {
    const int t = p.tokens[b];
    return (t >= 0 && t < p.vocab) ? t : 0;
}

// RMSNorm split in two: thread t owns elements 4t..4t+3 of each row. norm_own replaces
// them by x * w and hands their sum of squares to the row's per-wave slots (red[b][wave]);
// after the caller's next barrier, norm_scale gives rsqrt(mean(x^2) + eps), by which the
// consumers multiply their dot products (so that barrier is the only one of the norm).
__device__ __forceinline__ void norm_own(Smem& sm, int b, const f32x4 v, const f32x4 wv) {
    const int k = threadIdx.x * 4;
    float ss = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
#pragma unroll
    for (int e = 0; e < 4; ++e) sm.u.s.act[b][k + e] = v[e] * wv[e];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) sm.red[b][threadIdx.x >> 6] = ss;
}
// The same for a thread that keeps its normed elements in registers: returns x * w.
__device__ __forceinline__ f32x4 norm_part(Smem& sm, int b, const f32x4 v, const f32x4 wv) {
    float ss = v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3];
    ss = wave_sum(ss);
    if ((threadIdx.x & 63) == 0) sm.red[b][threadIdx.x >> 6] = ss;
    return f32x4{v[0] * wv[0], v[1] * wv[1], v[2] * wv[2], v[3] * wv[3]};
}
__device__ __forceinline__ float norm_scale(const MegaParams& p, const Smem& sm, int b) {
    const float ss = (sm.red[b][0] + sm.red[b][1]) + (sm.red[b][2] + sm.red[b][3]);
    return 1.0f / sqrtf(ss * (1.0f / D) + p.eps);
}

// QK-norm + RoPE of one 128-wide head held by a wave: lane i owns the pair (i, i + 64).
__device__ __forceinline__ void norm_rope(float& x1, float& x2, const Pre& pre, float eps, float c, float sn) {
    const float ss = wave_sum(x1 * x1 + x2 * x2);
    const float r = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
    x1 = (x1 * r) * pre.qk1;
    x2 = (x2 * r) * pre.qk2;
    const float y1 = __fsub_rn(__fmul_rn(x1, c), __fmul_rn(x2, sn));
    const float y2 = __fadd_rn(__fmul_rn(x1, sn), __fmul_rn(x2, c));
    x1 = y1;
    x2 = y2;
}

// Sequence slot of row b.
template <bool CAUSAL>
__device__ __forceinline__ int row_seq(const MegaParams& p, int b) { return p.seq_base + (CAUSAL ? 0 : b); }

// One kv head of one row in one layer: the head's base within every cache page, and the row
// whose page ids (sm.pg) locate the slots.
struct KvHead {
    size_t lb;
    int b;
};
__device__ __forceinline__ KvHead kv_head(const MegaParams& p, int layer, int b, int g) {
    return KvHead{(size_t)layer * p.kv_layer_elems + (size_t)g * p.kv.head_stride, b};
}
// element offset of a slot (in the row's prefetched page range) of a kv head
__device__ __forceinline__ size_t kv_page_base(const MegaParams& p, const Smem& sm, const KvHead& kh, int page) {
    return kh.lb + (size_t)sm.pg[kh.b][page - sm.pg0[kh.b]] * p.kv.page_stride;
}
__device__ __forceinline__ size_t kv_slot(const MegaParams& p, const Smem& sm, const KvHead& kh, int slot) {
    return kv_page_base(p, sm, kh, slot >> 8) + (size_t)(slot & (kKvPage - 1)) * DH;
}


// Polled q/k/v of group g (sm.in[b]) -> rotated q, bf16-rounded new k, v in shared memory;
// `append` writes k, v into the cache at `slot`.
template <bool CAUSAL>
__device__ __forceinline__ void group_prep(const MegaParams& p, Smem& sm, const Pre& pre, int layer, int b, int g,
                           int slot, bool append) {
    const int wid = threadIdx.x >> 6, i = threadIdx.x & 63;
    const float* in = sm.in[b];                     // [q0 128 | q1 128 | k 128 | v 128]
    float x1 = in[wid * DH + i], x2 = in[wid * DH + i + 64];
    if (wid < 3) norm_rope(x1, x2, pre, p.eps, sm.rc[b][i], sm.rs[b][i]);
    if (wid < 2) {                                  // q = hi + lo + O(2^-17 q), the MFMA operands
        // (packed conversions; the halves are taken apart with integer operations)
        const unsigned hb = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{x1, x2}, bf16x2));
        const float r1 = x1 - __uint_as_float(hb << 16), r2 = x2 - __uint_as_float(hb & 0xFFFF0000u);
        const unsigned lb = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{r1, r2}, bf16x2));
        sm.qb[wid][0][i] = (bf16)(hb & 0xFFFFu);
        sm.qb[wid][0][i + 64] = (bf16)(hb >> 16);
        sm.qb[wid][1][i] = (bf16)(lb & 0xFFFFu);
        sm.qb[wid][1][i + 64] = (bf16)(lb >> 16);
    } else {
        const bf16 h1 = f2bf(x1), h2 = f2bf(x2);
        // (causal rows keep every row's new key / value for the rows after it; otherwise one
        // buffer serves each row in turn)
        if constexpr (CAUSAL) {
            bf16* dc = wid == 2 ? sm.knc[b] : sm.vnc[b];
            dc[i] = h1;
            dc[i + 64] = h2;
        } else {
            float* dst = wid == 2 ? sm.kn : sm.vn;
            dst[i] = bf2f(h1);
            dst[i + 64] = bf2f(h2);
        }
        if (append) {
            // (a wave-uniform choice: a per-lane one reads the pointer with a vector load and
            // then waits for every outstanding load, the weight prefetch included)
            bf16* cache = (__builtin_amdgcn_readfirstlane(wid) == 2 ? p.kc : p.vc) +
                          kv_slot(p, sm, kv_head(p, layer, b, g), slot);
            cache[i] = h1;
            cache[i + 64] = h2;
        }
    }
    __syncthreads();
}

// Optional trace: thread 0 of workgroups 0 and NWG-1 records the 100 MHz real-time clock
// at phase boundaries, in shared memory (a global store here would hold up the next wait
// on the memory counter); the kernel's end copies the marks to p.trace[{0,1}][slot].
__device__ __forceinline__ void trace_at(const MegaParams& p, Smem& sm, int slot) {
    if (p.trace && threadIdx.x == 0 && (blockIdx.x == 0 || blockIdx.x == NWG - 1) && slot < TRACE_MAX)
        sm.tr[slot] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void trace_flush(const MegaParams& p, const Smem& sm, int n) {
    if (p.trace && threadIdx.x == 0 && (blockIdx.x == 0 || blockIdx.x == NWG - 1))
        for (int i = 0; i < n && i < p.trace_n && i < TRACE_MAX; ++i)
            p.trace[(blockIdx.x == 0 ? 0 : p.trace_n) + i] = sm.tr[i];
}

#define LDS_AS __attribute__((address_space(3)))

// Issue asynchronous copies of cache rows base .. base+n-1 (n <= STAGE) of one kv head into
// sm.u.kv (row i <- slot base + i), global -> LDS without registers: one instruction moves
// 4 rows (64 lanes x 16 bytes, lane l to byte 16 l). Complete after s_waitcnt + barrier.
// K rows are stored swizzled: 16-byte chunk c of row r sits in slot c ^ (r & 15) (lane l
// loads the chunk that belongs in its slot), so the 16 rows of a matrix-core fragment read
// at one column hit 16 different bank groups.
__device__ __forceinline__ int kslot(int r, int c) { return c ^ (r & 15); }

// Stage cached rows [base, base + n) of one kv head into shared memory: wave w loads the
// 16-row tiles t = w, w + 4, ... (the tiles it attends), four rows per instruction.
// (A shot of at most 240 rows spans at most two cache pages: their bases are read once.)
__device__ __forceinline__ void kv_stage(const MegaParams& p, Smem& sm, const KvHead& kh, int base, int n) {
    if (n <= 0) return;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int pa = base >> 8;
    const size_t offa = kv_page_base(p, sm, kh, pa);
    const size_t offb = ((base + n - 1) >> 8) != pa ? kv_page_base(p, sm, kh, pa + 1) : offa;
    for (int t = wid; 16 * t < n; t += 4) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int r0 = 16 * t + 4 * q4;
            const int r = r0 + (lane >> 4), sl = lane & 15;
            if (r < n) {
                const int slot = base + r;
                const size_t row = ((slot >> 8) == pa ? offa : offb) + (size_t)(slot & (kKvPage - 1)) * DH;
                __builtin_amdgcn_global_load_lds((const GLOBAL_AS void*)(p.kc + row + 8 * kslot(r, sl)),
                                                 (LDS_AS void*)&sm.u.kv.k[r0][0], 16, 0, 0);
                __builtin_amdgcn_global_load_lds((const GLOBAL_AS void*)(p.vc + row + 8 * sl),
                                                 (LDS_AS void*)&sm.u.kv.v[r0][0], 16, 0, 0);
            }
        }
    }
}

// Long variant: the staging area is two halves of 128 rows; shot s uses half s % 2, so
// the next shot's rows load while the current one is computed. Wave w stages tile slots
// w and w + 4 of the half (rows past n repeat row n - 1: every wave issues exactly
// KV_DB_LOADS loads per shot, so a fixed wait count separates the two shots).
constexpr int KV_DB_LOADS = 16;
__device__ __forceinline__ void kv_stage_db(const MegaParams& p, Smem& sm, const KvHead& kh, int base, int n,
                                            int half) {
    if (n <= 0) return;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int pa = base >> 8;
    const size_t offa = kv_page_base(p, sm, kh, pa);
    const size_t offb = ((base + n - 1) >> 8) != pa ? kv_page_base(p, sm, kh, pa + 1) : offa;
#pragma unroll
    for (int st = 0; st < 2; ++st) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const int r0 = 16 * (wid + 4 * st) + 4 * q4;
            const int r = min(r0 + (lane >> 4), n - 1), sl = lane & 15;
            const int slot = base + r;
            const size_t row = ((slot >> 8) == pa ? offa : offb) + (size_t)(slot & (kKvPage - 1)) * DH;
            __builtin_amdgcn_global_load_lds((const GLOBAL_AS void*)(p.kc + row + 8 * kslot(r0 + (lane >> 4), sl)),
                                             (LDS_AS void*)&sm.u.kv.k[128 * half + r0][0], 16, 0, 2);
            __builtin_amdgcn_global_load_lds((const GLOBAL_AS void*)(p.vc + row + 8 * sl),
                                             (LDS_AS void*)&sm.u.kv.v[128 * half + r0][0], 16, 0, 2);
        }
    }
}

// cached rows of [k0, k1) in the first shot (slot T-1 is the new key, kept in shared memory)
__device__ __forceinline__ int first_shot(int k0, int k1, int T, int shot = SHOT) {
    return max(0, min(min(k1, T - 1), k0 + shot) - k0);
}

__device__ __forceinline__ void unpack8(const u32x4 w, float* f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[2 * e] = __uint_as_float(w[e] << 16);
        f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
}

// Attention of both heads of the group for row b over slots [k0, k1) of T visible ones,
// the last nnew of which are new in this launch (rows b - nnew + 1 .. b, kept in shared
// memory). The caller issued the first shot (kv_stage of the cached rows in range, up to
// SHOT of them, at k0), waited for it and passed a barrier; longer ranges are staged here
// shot by shot (SHOT rows; the new keys are appended as the rows after the cached ones of
// the last shot). Wave w owns the 16-key tiles t = w, w + 4, ... of every shot: it stages
// them, computes their scores S^T = K q^T on the matrix cores (columns 0 and 1 the two
// heads; K rows are exact bf16 operands, q is split into bf16 hi + lo), keeps its own
// running softmax state per head (max, sum, unnormalised P.V with 16 lanes x 8 dims per
// key group), so no barrier is needed until the four wave states are merged (Step 6's
// softmax over all keys, assembled from partial maxima and sums; exponentials in base 2
// on scores scaled by log2(e)). Writes the normalised output of both heads to o_out, or,
// when o_out is null, leaves the merged per-head state (base-2 max, sum, unnormalised
// acc[128]) in sm.att.
template <bool DB, bool CAUSAL, bool SHORT = false>
__device__ __forceinline__ void attend(const MegaParams& p, Smem& sm, const KvHead& hb, int k0, int k1, int T, float* o_out,
                                       int b, int nnew_rt) {
    const int nnew = CAUSAL ? nnew_rt : 1;
    constexpr int SH = DB ? SHOTD : SHOT;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6, quad = lane >> 4, col = lane & 15;
    // scores are kept in the base-2 domain: s * log2(e), with s = q.k / sqrt(128)
    const float scale = 0.088388346f * 1.44269504f;
    bf16x8 qh[4], ql[4];                // B operand: lane holds q[head col][32 ks + 8 quad + i]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        if (col < 2) {
            qh[ks] = *reinterpret_cast<const bf16x8*>(&sm.qb[col][0][32 * ks + 8 * quad]);
            ql[ks] = *reinterpret_cast<const bf16x8*>(&sm.qb[col][1][32 * ks + 8 * quad]);
        } else {
            qh[ks] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
            ql[ks] = qh[ks];
        }
    }
    float Mw[2] = {-INFINITY, -INFINITY}, Lw[2] = {0.f, 0.f}, acc[2][8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    const int ce = min(k1, T - nnew);              // end of the cached rows in range
    for (int base = k0, shot = 0;; base += SH, ++shot) {
        const int n = max(0, min(ce, base + SH) - base);
        const bool last = base + SH >= ce;
        const int ro = DB ? 128 * (shot & 1) : 0;  // first staging row of this shot
        if constexpr (DB) {
            // the next shot into the other half (read two shots ago), then wait for this one:
            // all but this wave's KV_DB_LOADS newest loads
            const int nn = last ? 0 : max(0, min(ce, base + 2 * SH) - (base + SH));
            kv_stage_db(p, sm, hb, base + SH, nn, (shot + 1) & 1);
            static_assert(KV_DB_LOADS == 16, "the wait below encodes vmcnt(16)");
            if (nn > 0) __builtin_amdgcn_s_waitcnt(0x4F70);   // vmcnt(16)
            else __builtin_amdgcn_s_waitcnt(0x0F70);          // vmcnt(0)
        } else if (base != k0) {                   // this wave's tiles of the next shot
            __builtin_amdgcn_s_waitcnt(0);         // (its reads of the previous shot are done)
            kv_stage(p, sm, hb, base, n);
            __builtin_amdgcn_s_waitcnt(0);
        }
        const bool with_new = last && k1 == T;
        const int nk = n + (with_new ? nnew : 0);
        if constexpr (CAUSAL) {
            if (with_new && lane < 32) {           // the new keys / values as rows n .. n + nnew - 1
                for (int i = 0; i < nnew; ++i) {
                    const int r = n + i;
                    if (wid != ((r >> 4) & 3)) continue;   // the wave that owns the row's tile writes it
                    const int c = lane & 15;
                    const u32x4 u = *reinterpret_cast<const u32x4*>(
                        (lane < 16 ? sm.knc[b - nnew + 1 + i] : sm.vnc[b - nnew + 1 + i]) + 8 * c);
                    *reinterpret_cast<u32x4*>(lane < 16 ? &sm.u.kv.k[ro + r][8 * kslot(r, c)] : &sm.u.kv.v[ro + r][8 * c]) = u;
                }
            }
        } else if (with_new && wid == ((n >> 4) & 3) && lane < 32) {   // the new key / value as row n
            const int c = lane & 15;
            const float* src = (lane < 16 ? sm.kn : sm.vn) + 8 * c;
            u32x4 u;                               // exact: already bf16 values
#pragma unroll
            for (int e = 0; e < 4; ++e)
                u[e] = __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{src[2 * e], src[2 * e + 1]}, bf16x2));
            *reinterpret_cast<u32x4*>(lane < 16 ? &sm.u.kv.k[ro + n][8 * kslot(n, c)] : &sm.u.kv.v[ro + n][8 * c]) = u;
        }
        const int ntile = (nk + 15) >> 4;
        for (int t = wid; t < ntile; t += 4) {
            f32x4 sh = {0.f, 0.f, 0.f, 0.f}, sl = sh;   // hi and lo products: two chains
            bf16x8 a[4];                           // all fragment reads of the tile first
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                a[ks] = *reinterpret_cast<const bf16x8*>(&sm.u.kv.k[ro + 16 * t + col][8 * kslot(col, 4 * ks + quad)]);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                sh = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], qh[ks], sh, 0, 0, 0);
                sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], ql[ks], sl, 0, 0, 0);
            }
            // keep the four fragment reads ahead of the products (one LDS wait per tile)
            __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
            if (col < 2) {                         // D[key 4 quad + r][head col]
#pragma unroll
                for (int r = 0; r < 4; ++r) sm.sp[16 * t + 4 * quad + r][col] = (sh[r] + sl[r]) * scale;
            }
        }
        if constexpr (SHORT) {
            // Whole range in this one shot (nk <= 256 keys): the softmax of head h over all
            // nk scores by wave h alone (lane: keys lane + 64 i; keys past nk get probability
            // 0), so P.V needs no running maxima and the four waves' partial products are a
            // plain sum.
            __syncthreads();                       // every wave's scores are in sm.sp
            if (wid < 2) {
                float x[4], mx = -INFINITY;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int key = lane + 64 * i;
                    x[i] = key < nk ? sm.sp[key][wid] : -INFINITY;
                    mx = fmaxf(mx, x[i]);
                }
                mx = wave_max(mx);
                float sum = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pr = lane + 64 * i < nk ? __builtin_amdgcn_exp2f(x[i] - mx) : 0.f;
                    sm.sp[lane + 64 * i][wid] = pr;
                    sum += pr;
                }
                sum = wave_sum(sum);
                if (lane == 0) sm.wl[wid][0] = sum;
            }
            // value rows past the last key of its tile: zero (their probabilities are zero, and
            // a stale row could hold anything); the wave that owns the tile writes and reads them
            if (wid == ((ntile - 1) & 3)) {
                for (int r = nk + (lane >> 4); r < 16 * ntile; r += 4)
                    *reinterpret_cast<u32x4*>(&sm.u.kv.v[ro + r][8 * col]) = u32x4{0u, 0u, 0u, 0u};
            }
            __syncthreads();                       // probabilities visible to every wave
            // P.V of this wave's tiles: lane group quad takes keys 16 t + 4 i + quad, lane col
            // dims 8 col .. 8 col + 7
            for (int t = wid; t < ntile; t += 4) {
                u32x4 vv[4];
                f32x2 pp[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 16 * t + 4 * i + quad;
                    vv[i] = *reinterpret_cast<const u32x4*>(&sm.u.kv.v[ro + r][8 * col]);
                    pp[i] = *reinterpret_cast<const f32x2*>(&sm.sp[r][0]);
                }
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // all reads of the tile first
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float v[8];
                    unpack8(vv[i], v);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        acc[0][e] += pp[i][0] * v[e];
                        acc[1][e] += pp[i][1] * v[e];
                    }
                }
            }
            // sum over the four lane groups (the keys of a tile): lanes col, col + 16, +32, +48
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float x = acc[h][e];
                    auto a32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
                    x = __uint_as_float(a32[0]) + __uint_as_float(a32[1]);
                    auto a16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
                    acc[h][e] = __uint_as_float(a16[0]) + __uint_as_float(a16[1]);
                }
            // the waves' partial products go into the K staging rows (not read after the first
            // barrier above): [wave][head][128]
            float* part = reinterpret_cast<float*>(&sm.u.kv.k[0][0]);
            if (quad == 0) {
#pragma unroll
                for (int h = 0; h < 2; ++h)
#pragma unroll
                    for (int e = 0; e < 8; ++e) part[(wid * 2 + h) * DH + 8 * col + e] = acc[h][e];
            }
            __syncthreads();
            {
                const int h = tid >> 7, dd = tid & 127;
                const float tot = (part[(0 * 2 + h) * DH + dd] + part[(1 * 2 + h) * DH + dd]) +
                                  (part[(2 * 2 + h) * DH + dd] + part[(3 * 2 + h) * DH + dd]);
                o_out[h * DH + dd] = tot / sm.wl[h][0];
            }
            __syncthreads();                       // o complete; shared memory free again
            return;
        }
        // this wave's softmax statistics over the shot: lane (tile slot quad, key col)
        for (int t0 = wid; t0 < ntile; t0 += 16) {
            const int key = 16 * (t0 + 4 * quad) + col;
            const bool valid = key < nk;
            float x[2], mn[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                x[h] = valid ? sm.sp[key][h] : -INFINITY;
                mn[h] = fmaxf(Mw[h], wave_max(x[h]));
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float pr = valid ? __builtin_amdgcn_exp2f(x[h] - mn[h]) : 0.f;
                sm.sp[key][h] = pr;                // 0 past the last key
                const float corr = Lw[h] > 0.f ? __builtin_amdgcn_exp2f(Mw[h] - mn[h]) : 0.f;
                Lw[h] = Lw[h] * corr + wave_sum(pr);
                Mw[h] = mn[h];
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= corr;
            }
        }
        // rows past the last key in its tile: zero values (their probabilities are zero too),
        // so P.V can run over whole tiles
        if (wid == ((ntile - 1) & 3)) {
            for (int r = nk + (lane >> 4); r < 16 * ntile; r += 4)
                *reinterpret_cast<u32x4*>(&sm.u.kv.v[ro + r][8 * col]) = u32x4{0u, 0u, 0u, 0u};
        }
        // P.V of this wave's keys: lane group quad takes keys 16 t + 4 i + quad, lane col
        // dims 8 col .. 8 col + 7
        for (int t = wid; t < ntile; t += 4) {
            u32x4 vv[4];
            f32x2 pp[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 16 * t + 4 * i + quad;
                vv[i] = *reinterpret_cast<const u32x4*>(&sm.u.kv.v[ro + r][8 * col]);
                pp[i] = *reinterpret_cast<const f32x2*>(&sm.sp[r][0]);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);   // all reads of the tile first
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v[8];
                unpack8(vv[i], v);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    acc[0][e] += pp[i][0] * v[e];
                    acc[1][e] += pp[i][1] * v[e];
                }
            }
        }
        if (last) break;
    }
    __syncthreads();                               // the staged rows share memory with wm
    const int slot = wid * 4 + quad;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sm.u.s.wm[slot][h][8 * col + e] = acc[h][e];
        if (lane == 0) {
            sm.hs[h][wid] = Mw[h];
            sm.wl[h][wid] = Lw[h];
        }
    }
    __syncthreads();
    {
        const int h = tid >> 7, dd = tid & 127;
        // the four waves' states read at once (read one by one under their conditions, they
        // were a chain of dependent shared-memory round trips)
        const f32x4 hv = *reinterpret_cast<const f32x4*>(sm.hs[h]);
        const f32x4 lv = *reinterpret_cast<const f32x4*>(sm.wl[h]);
        float M = -INFINITY;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) M = fmaxf(M, lv[w2] > 0.f ? hv[w2] : -INFINITY);
        float cw[4], L = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const float e = __builtin_amdgcn_exp2f(hv[w2] - M);   // 0 for a wave without keys
            cw[w2] = lv[w2] > 0.f ? e : 0.f;
            L += lv[w2] * cw[w2];
        }
        float av[16];
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) av[s2] = sm.u.s.wm[s2][h][dd] * cw[s2 >> 2];
#pragma unroll
        for (int hh = 1; hh < 16; hh <<= 1)
#pragma unroll
            for (int s2 = 0; s2 + hh < 16; s2 += 2 * hh) av[s2] += av[s2 + hh];
        if (o_out) {
            o_out[h * DH + dd] = L > 0.f ? av[0] / L : 0.f;
        } else {
            if (dd == 0) { sm.att[h][0] = M; sm.att[h][1] = L; }
            sm.att[h][2 + dd] = av[0];
        }
    }
    __syncthreads();
}

// x'[b][32j + r] += Wo[32j + r, 256g:256g+256] . o[b] (fixed-point sum over the groups);
// thread t: row r = t >> 3, 16-byte chunks sub + 8i (i < 4) of the 32 in the row segment.
// Group 0's contribution also carries the residual x.
template <typename WT>
__device__ __forceinline__ void oproj_partial(Smem& sm, const WT* pf, float* P, int g, int j, int B, float sc) {
    const int r = threadIdx.x >> 3, sub = threadIdx.x & 7;
    for (int b = 0; b < B; ++b) {
        float s = dot_chunks<4>(pf, sm.o[b], sub, 8);
        s = sum8(s);
        if constexpr (sizeof(WT) < 16) s *= sc;   // quantised weights: row scale
        if (g == 0) s = sm.xg[b][r] + s;
        if (sub == 0) fx_add(reinterpret_cast<u64*>(P + (size_t)b * W_P) + 32 * j + r, s);
    }
}

// x''[b][32j + r] += Wd[32j + r, DCOLS g : DCOLS (g + 1)] . a[b] (fixed-point sum over the
// column blocks; block 0's contribution also carries the residual x'); thread t: row
// r = t >> 3, 16-byte chunks sub + 8 i (i < 6) of the 48 in the row segment.
template <typename WT>
__device__ __forceinline__ void down_partial(Smem& sm, const WT* pf, float* Xn, int g, int j, int B, float sc) {
    const int r = threadIdx.x >> 3, sub = threadIdx.x & 7;
    for (int b = 0; b < B; ++b) {
        float s = dot_chunks<6>(pf, sm.u.s.act[b], sub, 8);
        s = sum8(s);
        if constexpr (sizeof(WT) < 16) s *= sc;   // quantised weights: row scale
        if (g == 0) s = sm.xr[b][r] + s;
        if (sub == 0) fx_add(reinterpret_cast<u64*>(Xn + (size_t)b * W_X) + 32 * j + r, s);
    }
}

template <int WQ>
__device__ __forceinline__ void pf_oproj(const MegaLayer& L, typename WChunk<WQ>::T* pf, Pre& pre, int g, int j) {
    const int r = threadIdx.x >> 3, sub = threadIdx.x & 7;
    const size_t base = (size_t)(32 * j + r) * (HQ * DH) + 256 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) pf[i] = ldwc<WQ>(L.wo, base + (sub + 8 * i) * 8);
    if constexpr (WQ) pre.so = ldf(row_scales<WQ>(L.wo, (size_t)D * HQ * DH) + 32 * j + r);
}

// Rows of phase C: rr < 12 the gate rows of the workgroup's 12 SwiGLU columns, then their
// 12 up rows.
__device__ __forceinline__ int gu_col0(int w) { return DCOLS * (w & 7) + 12 * (w >> 3); }
__device__ __forceinline__ int gu_row(int w, int rr) {
    const int col = gu_col0(w) + (rr < 12 ? rr : rr - 12);
    return 32 * (col >> 4) + (col & 15) + (rr < 12 ? 0 : 16);
}

// First of the 16 rows of [Wq;Wk;Wv] that workgroup w projects in phase A: rows 16j ..
// 16j + 15 of its kv group g's 512 (query heads 2g, 2g + 1, key head g, value head g), so
// the q/k/v hand-over stays among the 32 workgroups of the group, on one XCD.
__device__ __forceinline__ int qkv_row0(int w) {
    const int g = w & 7, r = 16 * (w >> 3);
    return r < 2 * DH ? 2 * DH * g + r : (r < 3 * DH ? HQ * DH + DH * g + (r - 2 * DH) : (HQ + HKV) * DH + DH * g + (r - 3 * DH));
}

// Phases A, C, D: thread t polls 4 consecutive columns; with its pair lane t ^ 1 it holds
// the 8 columns 8 (t >> 1) .. + 7 (pair8), and it owns half of the phase's rows
// (by t & 1) at those columns: one 16-byte chunk per row.
template <int WQ>
__device__ __forceinline__ void pf_qkv(const MegaParams& p, const MegaLayer& L, typename WChunk<WQ>::T* pf, Pre& pre,
                                       int w) {
    const size_t base = (size_t)(qkv_row0(w) + 8 * (threadIdx.x & 1)) * D + 8 * (threadIdx.x >> 1);
#pragma unroll
    for (int i = 0; i < 8; ++i)
        pf[i] = ldwc<WQ>(L.wqkv, base + (size_t)i * D);
    if constexpr (WQ) pre.sa = ldf(row_scales<WQ>(L.wqkv, (size_t)NQKV * D) + qkv_row0(w) + (threadIdx.x >> 4));
    pre.nw = ldf4(L.in_norm + 4 * threadIdx.x);
    const int i = threadIdx.x & 63;
    const float* qk = (threadIdx.x >> 6) < 2 ? L.q_norm : L.k_norm;
    pre.qk1 = ldf(qk + i);
    pre.qk2 = ldf(qk + i + 64);
}
// gate/up rows i < 12 of the thread into pf[4 + i], in two parts: rows i0 <= i < i1
// (int8: the second part also loads the scale of the row this thread finishes in phase C)
template <int WQ, int I0, int I1>
__device__ __forceinline__ void pf_gu(const void* wgu, typename WChunk<WQ>::T* pf, Pre& pre, int w) {
    const size_t base = 8 * (threadIdx.x >> 1);
    const int r0 = 12 * (threadIdx.x & 1);
#pragma unroll
    for (int i = I0; i < I1; ++i) pf[4 + i] = ldwc<WQ>(wgu, base + (size_t)gu_row(w, r0 + i) * D);
    if constexpr (WQ && I1 == 12) {
        if (threadIdx.x < 192) pre.sg = ldf(row_scales<WQ>(wgu, (size_t)2 * F * D) + gu_row(w, threadIdx.x >> 3));
    }
}
// pf[i] = row 32j + (t >> 3) of Wd at columns DCOLS g + 8 ((t & 7) + 8 i) .. + 7 (i < 6)
template <int WQ>
__device__ __forceinline__ void pf_down(const MegaLayer& L, typename WChunk<WQ>::T* pf, Pre& pre, int g, int j) {
    const size_t base = (size_t)(32 * j + (threadIdx.x >> 3)) * F + DCOLS * g + 8 * (threadIdx.x & 7);
#pragma unroll
    for (int i = 0; i < 6; ++i) pf[i] = ldwc<WQ>(L.wd, base + 64 * i);
    if constexpr (WQ) pre.sd = ldf(row_scales<WQ>(L.wd, (size_t)D * F) + 32 * j + (threadIdx.x >> 3));
}

static_assert(MAXCH == 32, "kMegaMaxSlots assumes 32 chunks");
// long-context attention split: number of chunks (<= 32) and keys per chunk (multiple of 64)
__host__ __device__ __forceinline__ void chunking(int T, int& nch, int& ch) {
    nch = min(MAXCH, (T + 63) / 64);
    ch = ((T + nch - 1) / nch + 63) & ~63;
    nch = (T + ch - 1) / ch;
}

// word offset of chunk i (4 words) of group gg's inputs within a row's QKV words:
// q heads 2gg, 2gg+1 (64 chunks) | k head gg (32) | v head gg (32)
__device__ __forceinline__ size_t group_chunk(int gg, int i) {
    return i < 64 ? (size_t)256 * gg + 4 * i
                  : (i < 96 ? (size_t)HQ * DH + DH * gg + 4 * (i - 64) : (size_t)(HQ + HKV) * DH + DH * gg + 4 * (i - 96));
}

// MODE 0: every row has at most SHORT_T visible slots (each workgroup of a kv group attends
// the whole range); 1: split-K attention over chunks; 2: the same with the chunk rows staged
// in double-buffered halves (contexts above LONG_T). Separate instances, so the code and
// registers of one path do not touch the others.
template <int MODE, bool CAUSAL, int WQ>
__global__ __launch_bounds__(NT, 1) void k_decode_mega(MegaParams p) {
    constexpr bool LONG = MODE == 2;
    static_assert(!CAUSAL || MODE == 0, "causal rows run in the short-context instance only");
    extern __shared__ __align__(16) unsigned char smem_raw[];
    Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
    const int w = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int B = p.B;
    typedef typename WChunk<WQ>::T WT;   // one weight chunk: 8 bf16, 8 int8 codes or 8 int4 codes
    WT pf[16];
    Pre pre;
    // kv group and row block: the 32 workgroups of group g are those with w % 8 == g, which
    // the dispatcher places on XCD g (workgroup w runs on XCD w % 8)
    const int g = w & 7, j = w >> 3;

    // layer table into shared memory (scalar loads would hold up every later LDS wait)
    {
        const int words = p.n_layers * (int)(sizeof(MegaLayer) / 4);
        const unsigned* src = reinterpret_cast<const unsigned*>(p.layers);
        unsigned* dst = reinterpret_cast<unsigned*>(sm.layers);
        for (int i = tid; i < words; i += NT) dst[i] = *(const GLOBAL_AS unsigned*)(src + i);
    }
    if (w == 0 && tid < B) {
        const int t = p.tokens[tid];
        if (t < 0 || t >= p.vocab) atomicOr(p.err, Q3_DEVERR_TOKEN);
    }
    // cache page ids of the slots this workgroup stages or appends, per row: MODE 0 the
    // row's whole range [0, T); the split-K instances the workgroup's chunk of it
    if (tid < B * PGMAX) {
        const int b = tid / PGMAX, i = tid % PGMAX;
        const int T = p.slots[b] + 1;
        int k0 = 0, k1 = T;
        if constexpr (MODE != 0) {
            int nch, ch;
            chunking(T, nch, ch);
            const int c = w >> 3;
            k0 = c < nch ? c * ch : 0;
            k1 = c < nch ? min(T, k0 + ch) : 0;
        }
        const int first = k0 >> 8, last = k1 > k0 ? (k1 - 1) >> 8 : first - 1;
        if (i == 0) sm.pg0[b] = first;
        if (first + i <= last)
            sm.pg[b][i] = p.kv.pt[(size_t)row_seq<CAUSAL>(p, b) * p.kv.max_pages + first + i];
    }
    // RoPE factors of this step (the same for every layer): cos / sin of fl32(pos * f_i),
    // evaluated in double precision and rounded to float
    if (tid < 64 * B) {
        const int b = tid >> 6, i = tid & 63;
        const int pos = p.positions ? p.positions[b] : p.slots[b];
        const float ang = __fmul_rn((float)pos, ldf(p.inv_freq + i));
        double sd, cd;
        sincos((double)ang, &sd, &cd);
        sm.rc[b][i] = (float)cd;
        sm.rs[b][i] = (float)sd;
    }
    __syncthreads();
    pf_qkv<WQ>(p, sm.layers[0], pf, pre, w);
    int tslot = 0;
    trace_at(p, sm, tslot++);

    for (int layer = 0; layer < p.n_layers; ++layer) {
        const MegaLayer& L = sm.layers[layer];
        float* X = p.ex + (size_t)layer * p.ex_layer;        // layer input x
        float* QKV = X + (size_t)BMAX * W_X;
        float* P = QKV + (size_t)BMAX * W_QKV;                // O-projection partials per kv group
        float* A = P + (size_t)BMAX * W_P;
        float* PT = A + (size_t)BMAX * W_A;                   // chunk partials (long context)
        float* Xn = X + p.ex_layer;                           // next layer's input

        // ---------------- A: x -> RMSNorm -> QKV rows 16w .. 16w+15
        // Thread t polls x[4t .. 4t+3] and dots them (normed) with the 16 rows' weights at
        // those columns as soon as they arrive; one barrier, then the 256 partial sums of
        // each row are added (the same scheme in C and D).
        bool ok = true;
        for (int b = 0; b < B; ++b) {
            f32x4 v;                      // this thread's elements 4 tid .. 4 tid + 3 of x
            if (layer == 0) {
                const int t = clamp_tok(p, b);
                if constexpr (WQ == 1) {     // row t of the embedding: codes times the row's scale
                    const uint8_t* e8p = reinterpret_cast<const uint8_t*>(p.embed);
                    const unsigned e8 = *(const GLOBAL_AS unsigned*)(e8p + (size_t)t * D + 4 * tid);
                    const float es = ldf(row_scales<WQ>(p.embed, (size_t)p.vocab * D) + t);
                    v = f32x4{sb(e8, 0) * es, sb(e8, 1) * es, sb(e8, 2) * es, sb(e8, 3) * es};
                } else if constexpr (WQ == 2) {   // (int4: the 4 codes in 2 bytes)
                    const uint8_t* e4p = reinterpret_cast<const uint8_t*>(p.embed);
                    const unsigned e4 = *(const GLOBAL_AS unsigned short*)(e4p + ((size_t)t * D + 4 * tid) / 2);
                    const float es = ldf(row_scales<WQ>(p.embed, (size_t)p.vocab * D) + t);
                    v = f32x4{sn(e4, 0) * es, sn(e4, 1) * es, sn(e4, 2) * es, sn(e4, 3) * es};
                } else {
                    const unsigned* e = reinterpret_cast<const unsigned*>(p.embed + (size_t)t * D + 4 * tid);
                    const unsigned e0 = *(const GLOBAL_AS unsigned*)e, e1 = *(const GLOBAL_AS unsigned*)(e + 1);
                    v = f32x4{__uint_as_float(e0 << 16), __uint_as_float(e0 & 0xFFFF0000u), __uint_as_float(e1 << 16),
                              __uint_as_float(e1 & 0xFFFF0000u)};
                }
            } else {
                u32x4 c[2];
                ok = poll_own<2>(X + (size_t)b * W_X, W_X, FxPair{}, c, p.err, FxComplete{}) && ok;
                v = fx_vec4(c);
            }
            if ((tid >> 3) == j) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.xg[b][4 * (tid & 7) + e] = v[e];
            }
            f32x4 lo, hi;
            pair8(norm_part(sm, b, v, pre.nw), lo, hi);
#pragma unroll
            for (int i = 0; i < 8; ++i) sm.u.r.rd[b][8 * (tid & 1) + i][tid >> 1] = dot8v(pf[i], lo, hi);
        }
        trace_at(p, sm, tslot++);
        if (!__syncthreads_and(ok)) return;
        trace_at(p, sm, tslot++);
        {
            const int r = tid >> 4, sub = tid & 15;
            for (int b = 0; b < B; ++b) {
                const f32x4* src = reinterpret_cast<const f32x4*>(sm.u.r.rd[b][r]);
                const f32x4 q0 = src[sub], q1 = src[sub + 16];
                float s = ((q0[0] + q0[1]) + (q0[2] + q0[3])) + ((q1[0] + q1[1]) + (q1[2] + q1[3]));
                s = sum16(s) * norm_scale(p, sm, b);
                if constexpr (WQ) s *= pre.sa;
                if (sub == 0) put_xcd(QKV + (size_t)b * W_QKV + qkv_row0(w) + r, s);
            }
        }
        pf_oproj<WQ>(L, pf, pre, g, j);
        trace_at(p, sm, tslot++);

        // ---------------- B: attention of kv group g and its O-projection partial
        __syncthreads();                  // act (read above) shares memory with the K/V staging
        if constexpr (MODE == 0) {
            for (int b = 0; b < B; ++b) {
                const int slot = p.slots[b], T = slot + 1;
                // new keys of this launch that row b sees (held in shared memory, not read back
                // from the cache, which other workgroups of this launch are still writing)
                const int nnew = CAUSAL ? b + 1 : 1;
                const KvHead hb = kv_head(p, layer, b, g);
                kv_stage(p, sm, hb, 0, first_shot(0, T, T - nnew + 1));   // in flight while q/k/v arrive
                if (!poll<1>(QKV + (size_t)b * W_QKV, W_QKV, [&](int i) { return group_chunk(g, i); }, DH, sm.in[b], p.err))
                    return;
                __builtin_amdgcn_s_waitcnt(0);                  // staged rows landed (barrier below)
                if (b == 0) pf_gu<WQ, 0, 4>(L.wgu, pf, pre, w);
                if (b == 0) trace_at(p, sm, tslot++);
                group_prep<CAUSAL>(p, sm, pre, layer, b, g, slot, j == 0);
                if (b == 0) trace_at(p, sm, tslot++);
                attend<false, CAUSAL, true>(p, sm, hb, 0, T, T, sm.o[b], b, nnew);
            }
        } else {
            // B1: unit w = (group w % 8, chunk w / 8) attends its chunk, per row
            const int gg = w & 7, c = w >> 3;
            for (int b = 0; b < B; ++b) {
                const int slot = p.slots[b], T = slot + 1;
                int nch, ch;
                chunking(T, nch, ch);
                if (c < nch) {
                    const int k0 = c * ch, k1 = min(T, k0 + ch);
                    const KvHead hb = kv_head(p, layer, b, gg);
                    if (LONG) kv_stage_db(p, sm, hb, k0, first_shot(k0, k1, T, SHOTD), 0);
                    else kv_stage(p, sm, hb, k0, first_shot(k0, k1, T));
                    if (!poll<1>(QKV + (size_t)b * W_QKV, W_QKV, [&](int i) { return group_chunk(gg, i); }, DH, sm.in[b],
                                 p.err))
                        return;
                    __builtin_amdgcn_s_waitcnt(0);
                    if (b == 0) pf_gu<WQ, 0, 4>(L.wgu, pf, pre, w);
                    if (b == 0) trace_at(p, sm, tslot++);
                    group_prep<false>(p, sm, pre, layer, b, gg, slot, k1 == T);
                    if (b == 0) trace_at(p, sm, tslot++);
                    attend<LONG, false>(p, sm, hb, k0, k1, T, nullptr, b, 1);
                    float* pt = PT + (size_t)b * W_PT + (size_t)c * PT_CHUNK + (size_t)gg * 2 * PART;
                    for (int e = tid; e < 2 * PART; e += NT) put_xcd(pt + e, sm.att[e / PART][e % PART]);
                    __syncthreads();
                } else if (b == 0) {
                    pf_gu<WQ, 0, 4>(L.wgu, pf, pre, w);
                    trace_at(p, sm, tslot++);
                    trace_at(p, sm, tslot++);
                }
            }
            // combine: every workgroup of group g merges the group's chunks itself (one
            // hand-over instead of a combine workgroup followed by a broadcast)
            for (int b = 0; b < B; ++b) {
                const int T = p.slots[b] + 1;
                int nch, ch;
                chunking(T, nch, ch);
                // chunk i: partial c = i / 65, 16-byte piece i % 65 of group g's 260 words
                auto pidx = [&](int i) -> size_t {
                    return (size_t)(i / 65) * PT_CHUNK + (size_t)g * 2 * PART + 4 * (i % 65);
                };
                if (!poll<9>(PT + (size_t)b * W_PT, W_PT, pidx, nch * 65, sm.u.s.part, p.err)) return;
                // chunks in batches of 8 whose reads are all issued before their use (a
                // chunk past nch repeats the last one with zero weight); sums in chunk order
                const int h = tid >> 7, dd = tid & 127;
                float M = -INFINITY;
                for (int c0 = 0; c0 < nch; c0 += 8) {
                    float mv[8], lv[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float* pp = sm.u.s.part + ((size_t)min(c0 + u, nch - 1) * 2 + h) * PART;
                        mv[u] = pp[0];
                        lv[u] = pp[1];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) M = fmaxf(M, lv[u] > 0.f ? mv[u] : -INFINITY);
                }
                float Ls = 0.f, Acc = 0.f;
                for (int c0 = 0; c0 < nch; c0 += 8) {
                    float mv[8], lv[8], av[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float* pp = sm.u.s.part + ((size_t)min(c0 + u, nch - 1) * 2 + h) * PART;
                        mv[u] = pp[0];
                        lv[u] = c0 + u < nch ? pp[1] : 0.f;
                        av[u] = pp[2 + dd];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float cf = lv[u] > 0.f ? __builtin_amdgcn_exp2f(mv[u] - M) : 0.f;
                        Ls += lv[u] * cf;
                        Acc += av[u] * cf;
                    }
                }
                sm.o[b][h * DH + dd] = Ls > 0.f ? Acc / Ls : 0.f;
                __syncthreads();
            }
        }
        trace_at(p, sm, tslot++);
        {
            // phase C's weight pointers are taken from the layer table before the atomics of
            // the O projection: read after them, the compiler waits for every outstanding
            // memory operation (the atomics' round trip included) before the table read
            const bf16* wgu = uniform_ptr(L.wgu);
            const float* pnorm = uniform_ptr(L.post_norm);
            oproj_partial(sm, pf, P, g, j, B, pre.so);
            pf_gu<WQ, 4, 12>(wgu, pf, pre, w);
            pre.nw = ldf4(pnorm + 4 * tid);
        }
        trace_at(p, sm, tslot++);

        // ---------------- C: x' (summed in memory) -> RMSNorm -> gate/up of 12 columns -> SwiGLU
        bool okc = true;
        for (int b = 0; b < B; ++b) {
            u32x4 c[2];                   // thread t: the sums 4t .. 4t+3
            okc = poll_own<2>(P + (size_t)b * W_P, 2 * D, FxPair{}, c, p.err, FxComplete{}) && okc;
            if (b == 0) trace_at(p, sm, tslot++);
            const f32x4 xv = fx_vec4(c);
            if ((tid >> 3) == j) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sm.xr[b][4 * (tid & 7) + e] = xv[e];
            }
            f32x4 lo, hi;
            pair8(norm_part(sm, b, xv, pre.nw), lo, hi);
#pragma unroll
            for (int i = 0; i < 12; ++i) sm.u.r.rd[b][12 * (tid & 1) + i][tid >> 1] = dot8v(pf[4 + i], lo, hi);
        }
        trace_at(p, sm, tslot++);
        if (!__syncthreads_and(okc)) return;
        trace_at(p, sm, tslot++);
        {
            if (tid < 192) {              // row rr = t >> 3: 8 threads, then 8 lanes
                const int rr = tid >> 3, sub = tid & 7;
                for (int b = 0; b < B; ++b) {
                    const f32x4* src = reinterpret_cast<const f32x4*>(sm.u.r.rd[b][rr]);
                    f32x4 q[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) q[i] = src[sub + 8 * i];
                    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);   // all four reads first
                    float s = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) s += (q[i][0] + q[i][1]) + (q[i][2] + q[i][3]);
                    s = sum8(s);
                    if (sub == 0) sm.gu[rr][b] = s * norm_scale(p, sm, b) * (WQ ? pre.sg : 1.0f);
                }
            }
            __syncthreads();
            if (tid < 12 * B) {
                const int c = tid % 12, b = tid / 12;
                const float gt = sm.gu[c][b], up = sm.gu[12 + c][b];
                put_xcd(A + (size_t)b * W_A + gu_col0(w) + c, gt / (1.0f + expf(-gt)) * up);
            }
        }
        pf_down<WQ>(L, pf, pre, g, j);
        trace_at(p, sm, tslot++);

        // ---------------- D: rows 32j..32j+31 of Wd[:, DCOLS g : DCOLS (g + 1)] . a (plus x' for
        // g = 0) -> added to the sums of x''; only the group's own slice of a is polled
        if constexpr (MODE == 0) {
            // two reads in flight per chunk; threads past the 96 chunks poll duplicates
            // (measured faster here, slower in the split-K instances)
            bool okd = true;
            for (int b = 0; b < B; ++b) {
                u32x4 c[1];
                okd = poll_own<1>(A + (size_t)b * W_A, W_A,
                                  [&](int i) { return (size_t)DCOLS * g + 4 * (i % (DCOLS / 4)); }, c, p.err) && okd;
                if (tid < DCOLS / 4) *reinterpret_cast<u32x4*>(&sm.u.s.act[b][4 * tid]) = c[0];
            }
            if (!__syncthreads_and(okd)) return;
        } else {
            for (int b = 0; b < B; ++b) {
                if (!poll<1>(A + (size_t)b * W_A, W_A, [&](int i) { return (size_t)DCOLS * g + 4 * i; }, DCOLS / 4,
                             sm.u.s.act[b], p.err))
                    return;
            }
        }
        trace_at(p, sm, tslot++);
        down_partial(sm, pf, Xn, g, j, B, pre.sd);
        if (layer + 1 < p.n_layers) pf_qkv<WQ>(p, sm.layers[layer + 1], pf, pre, w);
        else pre.nw = ldf4(p.final_norm + 4 * tid);
        trace_at(p, sm, tslot++);
        __syncthreads();
    }

    // ---------------- final RMSNorm + LM head rows [r0, r1) + per-workgroup argmax, for the
    // rows b >= head_first (a chunk of a prompt whose logits nobody reads has none)
    const int hf = CAUSAL ? p.head_first : 0;
    if (CAUSAL && hf >= B) {
        trace_flush(p, sm, tslot);
        return;
    }
    const int r0 = (int)((long long)p.vocab * w / NWG), r1 = (int)((long long)p.vocab * (w + 1) / NWG);
    const int rsub = tid >> 4, sub = tid & 15;   // 16 rows per pass, 16 lanes per row
    WT b0[8], b1[8], b2[8];                        // three passes: two loads in flight
    float s0 = 1.f, s1 = 1.f, s2 = 1.f;            // int8: the rows' scales
    auto load_rows = [&](int base, WT* dst, float& sc) {
        const int row = base + rsub;
        if (row < r1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) dst[i] = ldwc<WQ>(p.embed, (size_t)row * D + (sub + 16 * i) * 8);
            if constexpr (WQ) sc = ldf(row_scales<WQ>(p.embed, (size_t)p.vocab * D) + row);
        }
    };
    load_rows(r0, b0, s0);                         // in flight while the last layer finishes
    load_rows(r0 + 16, b1, s1);
    {
        const float* Xl = p.ex + (size_t)p.n_layers * p.ex_layer;
        bool okl = true;
        for (int b = hf; b < B; ++b) {
            u32x4 c[2];
            okl = poll_own<2>(Xl + (size_t)b * W_X, W_X, FxPair{}, c, p.err, FxComplete{}) && okl;
            norm_own(sm, b, fx_vec4(c), pre.nw);
        }
        if (!__syncthreads_and(okl)) return;
        trace_at(p, sm, tslot++);
    }
    float rn[BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) rn[b] = b >= hf && b < B ? norm_scale(p, sm, b) : 0.f;
    u64 best[BMAX] = {0ull, 0ull, 0ull, 0ull};
    bool bad = false;
    {
        auto rows_dot = [&](int base, const WT* wv, float sc) {
            const int row = base + rsub;
#pragma unroll
            for (int b = 0; b < BMAX; ++b) {
                if (b >= B) break;
                if (b < hf) continue;
                float s = 0.f;
                if (row < r1) s = dot_chunks<8>(wv, sm.u.s.act[b], sub, 16);
                s = sum16(s) * rn[b];
                if constexpr (WQ) s *= sc;
                if (row < r1 && sub == 0) {
                    p.logits[(size_t)(b - hf) * p.vocab + row] = s;
                    bad |= !isfinite(s);
                    const u64 key = pack_argmax(s, (uint32_t)row);
                    best[b] = key > best[b] ? key : best[b];
                }
            }
        };
        for (int base = r0; base < r1; base += 48) {
            load_rows(base + 32, b2, s2);
            rows_dot(base, b0, s0);
            load_rows(base + 48, b0, s0);
            rows_dot(base + 16, b1, s1);
            load_rows(base + 64, b1, s1);
            rows_dot(base + 32, b2, s2);
        }
    }
    if (bad) atomicOr(p.err, Q3_DEVERR_NONFINITE);
    __shared__ u64 wbest[4][BMAX];
#pragma unroll
    for (int b = 0; b < BMAX; ++b) {
        if (b >= B) break;
        if (b < hf) continue;
        u64 v = best[b];
        for (int o = 32; o >= 1; o >>= 1) {
            const u64 t = __shfl_xor(v, o, 64);
            v = t > v ? t : v;
        }
        if (lane == 0) wbest[tid >> 6][b] = v;
    }
    __syncthreads();
    if (tid >= hf && tid < B) {
        u64 v = wbest[0][tid];
        for (int wv = 1; wv < 4; ++wv) v = wbest[wv][tid] > v ? wbest[wv][tid] : v;
        p.cand[(size_t)(tid - hf) * NWG + w] = v;
    }
    trace_at(p, sm, tslot++);
    trace_flush(p, sm, tslot);
}

}  // namespace

size_t decode_mega_exchange_words_per_layer() {
    return (size_t)BMAX * (W_X + W_QKV + W_P + W_A + W_PT);
}

// Tail of a persistent decode step, run after every launch (also one that gave up):
// lengths advanced (lens[seq_base + b] += 1 per row, or lens[seq_base] += B for causal
// rows of one sequence); blocks b < nout (the rows that had the LM head): amax[b] = max
// over the 256 workgroup candidates of output row b (packed logit key | ~id) and, when
// greedy_out is given, the greedy token (Step 8's argmax, lowest id on ties); all blocks:
// the initial state back into every exchange word the launch may have written -- per
// layer, rows < B of the x and x' sums (zero), q/k/v and a, and pt_words words of chunk
// partials per row -- with coherent stores.
__global__ void k_mega_tail(const u64* __restrict__ cand, u64* __restrict__ amax, int* __restrict__ lens,
                            int seq_base, int B, float* ex, size_t ex_layer, int n_layers, int pt_words,
                            int32_t* __restrict__ greedy_out, int nout, int causal) {
    if (threadIdx.x == 0) {
        if (causal) {
            if (blockIdx.x == 0) lens[seq_base] += B;
        } else if ((int)blockIdx.x < B) {
            lens[seq_base + blockIdx.x] += 1;
        }
    }
    if ((int)blockIdx.x < nout) {
        const int b = blockIdx.x;
        u64 v = cand[(size_t)b * NWG + threadIdx.x];
        for (int o = 32; o >= 1; o >>= 1) {
            const u64 t = __shfl_xor(v, o, 64);
            v = t > v ? t : v;
        }
        __shared__ u64 r[4];
        if ((threadIdx.x & 63) == 0) r[threadIdx.x >> 6] = v;
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int i = 0; i < 4; ++i) v = r[i] > v ? r[i] : v;
            amax[b] = v;
            if (greedy_out) greedy_out[b] = (int32_t)(0xFFFFFFFFu - (uint32_t)(v & 0xFFFFFFFFull));
        }
    }
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)ex, (short)0, (int)((size_t)(n_layers + 1) * ex_layer * 4), 0x00020000);
    const u32x4 sv = {SENT, SENT, SENT, SENT}, zv = {0u, 0u, 0u, 0u};
    const int nseg = (n_layers + 1) * 5 * B;
    for (int seg = blockIdx.x; seg < nseg; seg += gridDim.x) {
        const int l = seg / (5 * B), kind = (seg % (5 * B)) / B, b = seg % B;
        if (l == n_layers && kind != 0) continue;       // past the last layer only x exists
        size_t off = (size_t)l * ex_layer;
        int cnt;
        if (kind == 0) { off += (size_t)b * W_X; cnt = (int)W_X; }
        else if (kind == 1) { off += BMAX * W_X + (size_t)b * W_QKV; cnt = (int)W_QKV; }
        else if (kind == 2) { off += BMAX * (W_X + W_QKV) + (size_t)b * W_P; cnt = 2 * D; }
        else if (kind == 3) { off += BMAX * (W_X + W_QKV + W_P) + (size_t)b * W_A; cnt = (int)W_A; }
        else { off += BMAX * (W_X + W_QKV + W_P + W_A) + (size_t)b * W_PT; cnt = pt_words; }
        for (int i = 4 * threadIdx.x; i < cnt; i += 4 * blockDim.x)
            __builtin_amdgcn_raw_buffer_store_b128(kind == 0 || kind == 2 ? zv : sv, rs, (int)((off + i) * 4), 0, SC1);
    }
}

// Initial state of the exchange words: the sentinel, and zero in the x and x' sums.
__global__ void k_mega_fill(float* ex, size_t words, size_t ex_layer) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)ex, (short)0, (int)(words * 4), 0x00020000);
    const u32x4 sv = {SENT, SENT, SENT, SENT}, zv = {0u, 0u, 0u, 0u};
    constexpr size_t p0 = BMAX * (W_X + W_QKV), p1 = p0 + BMAX * W_P;
    for (size_t i = 4 * ((size_t)blockIdx.x * blockDim.x + threadIdx.x); i < words; i += 4 * (size_t)gridDim.x * blockDim.x) {
        const size_t o = i % ex_layer;
        __builtin_amdgcn_raw_buffer_store_b128(o < BMAX * W_X || (o >= p0 && o < p1) ? zv : sv, rs, (int)(i * 4), 0, SC1);
    }
}

int decode_mega_chunks(const int* T, int B) {
    int Tmax = 0;
    for (int b = 0; b < B; ++b) Tmax = std::max(Tmax, T[b]);
    if (Tmax <= SHORT_T) return 0;                 // no split-K attention in this launch
    int m = 0;                                     // (a shorter row can have more chunks)
    for (int b = 0; b < B; ++b) {
        int nch, ch;
        chunking(T[b], nch, ch);
        m = std::max(m, nch);
    }
    return m;
}

hipError_t launch_mega_tail(const unsigned long long* cand, unsigned long long* amax, int* lens, int seq_base,
                            int B, float* ex, size_t ex_layer, int n_layers, int pt_chunks, int32_t* greedy_out,
                            hipStream_t s, int nout, int causal) {
    if (B < 1 || B > BMAX || n_layers < 1 || ex_layer != decode_mega_exchange_words_per_layer() || pt_chunks < 0 ||
        pt_chunks > MAXCH || nout < 0 || nout > B)
        return hipErrorInvalidValue;
    const int pt_words = pt_chunks * PT_CHUNK;
    hipLaunchKernelGGL(k_mega_tail, dim3(NWG), dim3(NT), 0, s, cand, amax, lens, seq_base, B, ex, ex_layer, n_layers,
                       pt_words, greedy_out, nout, causal);
    return hipGetLastError();
}

hipError_t launch_mega_fill(float* ex, size_t words, hipStream_t s) {
    const size_t ex_layer = decode_mega_exchange_words_per_layer();
    if (words % 4 || words % ex_layer || words * 4 > 0x7FFFFFF0ull) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_mega_fill, dim3(1024), dim3(256), 0, s, ex, words, ex_layer);
    return hipGetLastError();
}

// [bf16 / int8 / int4 weights][short, split-K, split-K double-buffered, short with causal rows]
static const void* const kInstances[3][4] = {
    {(const void*)k_decode_mega<0, false, 0>, (const void*)k_decode_mega<1, false, 0>,
     (const void*)k_decode_mega<2, false, 0>, (const void*)k_decode_mega<0, true, 0>},
    {(const void*)k_decode_mega<0, false, 1>, (const void*)k_decode_mega<1, false, 1>,
     (const void*)k_decode_mega<2, false, 1>, (const void*)k_decode_mega<0, true, 1>},
    {(const void*)k_decode_mega<0, false, 2>, (const void*)k_decode_mega<1, false, 2>,
     (const void*)k_decode_mega<2, false, 2>, (const void*)k_decode_mega<0, true, 2>}};

hipError_t launch_decode_mega(const MegaParams& p, bool cooperative, hipStream_t s) {
    if (p.B < 1 || p.B > BMAX || p.n_layers < 1 || p.n_layers > kMegaMaxLayers || p.head_first < 0 ||
        p.head_first > p.B || p.wq < 0 || p.wq > 2)
        return hipErrorInvalidValue;
    int Tmax = 0;
    for (int b = 0; b < p.B; ++b) Tmax = std::max(Tmax, p.slots[b] + 1);
    if (p.causal) {                  // consecutive slots of one sequence, short instance only
        for (int b = 1; b < p.B; ++b)
            if (p.slots[b] != p.slots[0] + b) return hipErrorInvalidValue;
        if (Tmax > SHORT_T) return hipErrorInvalidValue;
    }
    if (!p.causal && p.head_first != 0) return hipErrorInvalidValue;
    const int mode = p.causal ? 3 : Tmax <= SHORT_T ? 0 : Tmax <= LONG_T ? 1 : 2;
    const void* fn = kInstances[p.wq][mode];
    if (cooperative) {
        void* args[] = {(void*)&p};
        return hipLaunchCooperativeKernel(fn, dim3(NWG), dim3(NT), args, sizeof(Smem), s);
    }
    void* args[] = {(void*)&p};
    return hipLaunchKernel(fn, dim3(NWG), dim3(NT), args, sizeof(Smem), s);
}

hipError_t decode_mega_prepare() {
    for (int wq = 0; wq < 3; ++wq) {
        for (const void* fn : kInstances[wq]) {
            const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Smem));
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

}  // namespace q3
