// Prefill attention: causal grouped-query attention of M new rows of one sequence
// ("Inside an LLM ...", Step 5: scores q.k * 128^-0.5, causal mask so a row never sees
// a later slot, softmax, weighted sum of V; query heads 2g, 2g+1 read kv head g).
//
// Flash-style, on the matrix cores. Work item: 64 query rows (a query tile) of one query
// head, one wave per 16 rows; the waves walk the key tiles (64 keys) up to the causal limit
// of their rows, keeping a running max / sum per row (float32, base-2 exponentials) -- the
// n x n score matrix is never stored. A block takes two query tiles, the heaviest and the
// lightest left (nqt-1-b and b), so every block walks nqt + 1 key tiles. HB = 2: the block
// holds both query heads of one kv head (eight waves), so each staged K/V tile feeds both;
// HB = 1 (four waves, one head) when that would leave compute units idle.
//
// Per key tile the waves compute S^T = K Q^T (A = K tile from LDS, B = the wave's Q rows
// held in registers). In that accumulator layout a lane holds 4 consecutive keys of one
// query row for each 16-key tile, which is exactly what the B operand of O^T = V^T P^T
// needs once both operands agree on the order of the contraction (key) index; so the
// probabilities go from accumulators to bf16 operands without touching LDS. V is stored
// transposed in LDS ([dim][key], keys in the operand's order) for the A operand.
//
// Pipeline: K/V tiles pass through a two-stage LDS ring (one barrier per tile); the global
// loads run two tiles ahead, and the scores of tile kt + 1 are issued before the softmax of
// tile kt, so the exponentials and operand splits overlap the matrix-core work.
//
// Precision: K and V are bf16 (the cache's own format, exact as operands). q (float32) and
// the probabilities (float32) are each split into bf16 hi + lo parts and take two MFMAs,
// so both products keep ~16 significant bits; the output is float32.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace q3 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr int BQ = 64;    // query rows per block (per head)
constexpr int BKV = 64;   // keys per tile

// K tile: 64 rows (keys) x 16 chunks of 16 B; chunk c of row r at c ^ (r & 15).
__device__ __forceinline__ int kidx(int key, int ck) { return key * 16 + (ck ^ (key & 15)); }

// V^T tile: 128 rows (dims) x 8 chunks of 16 B. Chunk c = 4 * kb + lg of a row holds the
// keys that lane group lg feeds to the P.V product of key block kb (32 keys): keys
// 32kb + 4lg + {0..3}, then 32kb + 16 + 4lg + {0..3}, so each operand is one 16-byte read.
// Chunk c of row d sits at c ^ ((d ^ (d >> 3)) & 7), spreading both the fragment reads
// (16 consecutive dims) and the staging writes (dims 8 apart) over the banks.
__device__ __forceinline__ int vt_chunk(int d, int c) { return d * 8 + (c ^ ((d ^ (d >> 3)) & 7)); }
__device__ __forceinline__ int vt_off(int d, int key) {  // offset in bf16 elements
    const int w = key & 31;
    return vt_chunk(d, (key >> 5) * 4 + ((w >> 2) & 3)) * 8 + (w >> 4) * 4 + (w & 3);
}

typedef __attribute__((ext_vector_type(8))) float f32x8;

// 8 float32 -> bf16 hi parts and bf16 lo parts, as two 8-element operands (hardware
// round-to-nearest-even conversions, two values per instruction).
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
    const f32x8 x = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
    hi = __builtin_convertvector(x, bf16x8);
    const f32x8 hf = __builtin_convertvector(hi, f32x8);
    lo = __builtin_convertvector(x - hf, bf16x8);
}

// Combine a per-lane value over the four lanes of a query row (lanes l, l^16, l^32, l^48)
// with the lane-swap instructions (no LDS round trip).
__device__ __forceinline__ float row_max4(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row_sum4(float x) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <bool PAIR, int HB, bool PAGED>
__global__ __launch_bounds__(256 * HB, 1) void k_attn_prefill(const float* __restrict__ q,
                                                                   const bf16* __restrict__ kc,
                                                                   const bf16* __restrict__ vc, KvLayout lay,
                                                                   int seq, int M, int t0, int Hq, int Hkv,
                                                                   void* __restrict__ o) {
    constexpr int NT = 256 * HB;       // threads
    constexpr int NP = 2 / HB;         // key pairs each thread stages per tile
    __shared__ u32x4 sK[2][BKV * 16];
    __shared__ u32x4 sV[2][128 * 8];
    const int nqt = (M + BQ - 1) / BQ;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int h = HB == 1 ? (int)blockIdx.y : (int)blockIdx.y * 2 + (wid >> 2);
    const int g = HB == 1 ? (int)blockIdx.y >> 1 : (int)blockIdx.y;
    const int l16 = lane & 15, lg = lane >> 4;
    const float scale_log2 = 0.088388346f * 1.4426950408889634f;
    const int ck = tid & 15;           // staging: 16-byte chunk of each key row
    // cache addressing: a 64-key tile lies within one page (paged) or one contiguous run
    const int32_t* __restrict__ ptab = PAGED ? lay.pt + (size_t)seq * lay.max_pages : nullptr;
    const size_t hbase = PAGED ? (size_t)g * lay.head_stride : (size_t)seq * lay.page_stride + (size_t)g * lay.head_stride;

    for (int pass = 0; pass < 2; ++pass) {
        // heaviest (latest) query tiles first
        const int qt = pass == 0 ? nqt - 1 - (int)blockIdx.x : (int)blockIdx.x;
        if (pass == 1 && qt >= nqt - 1 - (int)blockIdx.x) break;   // the middle tile of an odd count
        if (pass == 1) __syncthreads();                             // the ring is about to be refilled
        const int qbase = qt * BQ + (wid & 3) * 16;                 // first row of this wave

        // Q^T as B operand (hi and lo parts): lane holds q row (l16), dims ks*32 + 8*lg .. +8.
        bf16x8 qh[4], ql[4];
        {
            const int row = qbase + l16;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
                if (row < M) {
                    const f32x4* p = reinterpret_cast<const f32x4*>(q + ((size_t)h * M + row) * 128 + ks * 32 + lg * 8);
                    const f32x4 a = p[0], b = p[1];
                    v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
                    v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
                }
                split8(v, qh[ks], ql[ks]);
            }
        }
        f32x4 oacc[8];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float mrow = -INFINITY;   // running max of the row, in log2 units (scores x scale_log2)
        float lpart = 0.f;        // this lane's share of the running sum (its 4 keys per 16)

        const int first_slot = t0 + qt * BQ;                        // slot of the block's first row
        const int last_slot = t0 + min(M, (qt + 1) * BQ) - 1;
        const int ntiles = last_slot / BKV + 1;
        const int kdiag = (first_slot + 1) / BKV;    // tiles from here on may hold keys after some row
        const int qslot = t0 + qbase + l16;

        // Tile addresses. Tiles past the last are clamped to it and keys past last_slot to
        // last_slot, so every load reads written cache entries: such keys only meet rows that
        // mask them (probability 0 times a finite value) or padding rows past M.
        auto page_of = [&](int tile) __attribute__((always_inline)) -> int {
            return PAGED ? ptab[min(tile, ntiles - 1) >> 2] : 0;
        };
        auto tile_base = [&](int pid, int tile) __attribute__((always_inline)) -> size_t {
            tile = min(tile, ntiles - 1);
            return PAGED ? (size_t)pid * lay.page_stride + hbase + (size_t)((tile & 3) * BKV) * 128
                         : hbase + (size_t)tile * BKV * 128;
        };
        // global -> registers: thread t takes chunk ck of key pairs t / 16 + (NT / 16) * j
        u32x4 kreg[NP][2], vreg[NP][2];
        auto gload = [&](u32x4 (&r)[NP][2], const bf16* base, int pid, int tile) __attribute__((always_inline)) {
            const size_t tb = tile_base(pid, tile);
            const int kmax = last_slot - min(tile, ntiles - 1) * BKV;
#pragma unroll
            for (int j = 0; j < NP; ++j)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int key = min(2 * ((tid >> 4) + (NT / 16) * j) + u, kmax);
                    r[j][u] = *reinterpret_cast<const u32x4*>(base + tb + (size_t)key * 128 + ck * 8);
                }
        };
        auto put_k = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const int key0 = 2 * ((tid >> 4) + (NT / 16) * j);
                sK[buf][kidx(key0, ck)] = kreg[j][0];
                sK[buf][kidx(key0 + 1, ck)] = kreg[j][1];
            }
        };
        auto put_v = [&](int buf) __attribute__((always_inline)) {
            bf16* vt = reinterpret_cast<bf16*>(sV[buf]);
#pragma unroll
            for (int j = 0; j < NP; ++j) {
                const int key0 = 2 * ((tid >> 4) + (NT / 16) * j);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned a = (vreg[j][0][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    const unsigned b = (vreg[j][1][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    *reinterpret_cast<unsigned*>(&vt[vt_off(ck * 8 + e, key0)]) = a | (b << 16);
                }
            }
        };
        // S^T[key][row] of one key tile: 4 key tiles of 16, the hi and lo parts of q
        auto scores = [&](int buf, f32x4 (&sc)[4]) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 4; ++j) sc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                bf16x8 a[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) a[j] = __builtin_bit_cast(bf16x8, sK[buf][kidx(j * 16 + l16, ks * 4 + lg)]);
#pragma unroll
                for (int j = 0; j < 4; ++j) sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], qh[ks], sc[j], 0, 0, 0);
#pragma unroll
                for (int j = 0; j < 4; ++j) sc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j], ql[ks], sc[j], 0, 0, 0);
            }
        };
        // One tile of the pipeline. On entry (after the barrier) the ring holds K_{kt+1} and
        // V_kt, the registers hold K_{kt+2} and V_{kt+1}, cur holds the scores of tile kt,
        // pk / pv are the page ids of tiles kt+3 / kt+2. Past the last tile the products,
        // stores and loads still run (on stages and addresses no longer read), so the body has
        // no branch between the matrix-core work and the softmax.
        int pk = 0, pv = 0;
        auto step = [&](int kt, f32x4 (&cur)[4], f32x4 (&nxt)[4], auto mask) __attribute__((always_inline)) {
            __syncthreads();   // the previous tile's reads of the stages refilled below are done
            scores((kt + 1) & 1, nxt);
            // causal mask (the last one or two tiles), online softmax of tile kt
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = cur[j][r];
                    if constexpr (decltype(mask)::value)
                        if (kt * BKV + j * 16 + lg * 4 + r > qslot) v = -INFINITY;
                    cur[j][r] = v;
                    mx = fmaxf(mx, v);
                }
            // the scale is positive, so the max of the scaled scores is the scaled max. The
            // row's reference moves only when its max outgrows it by more than 8 (base 2):
            // the probabilities stay below 2^8 (exact as hi + lo operands, summed in float32)
            // and the accumulators are rescaled only on those rare tiles; the softmax does not
            // depend on the reference chosen.
            const float mcand = fmaxf(mrow, row_max4(mx) * scale_log2);
            const float mnew = mcand > mrow + 8.0f ? mcand : mrow;
            const float corr = __builtin_amdgcn_exp2f(mrow - mnew);   // 1 if kept; 0 on the first tile
            mrow = mnew;
            float ps = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pr = __builtin_amdgcn_exp2f(__builtin_fmaf(cur[j][r], scale_log2, -mnew));
                    cur[j][r] = pr;
                    ps += pr;
                }
            lpart = lpart * corr + ps;
            bf16x8 ph[2], pl[2];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const float p8[8] = {cur[2 * kb][0], cur[2 * kb][1], cur[2 * kb][2], cur[2 * kb][3],
                                     cur[2 * kb + 1][0], cur[2 * kb + 1][1], cur[2 * kb + 1][2], cur[2 * kb + 1][3]};
                split8(p8, ph[kb], pl[kb]);
            }
            if (__ballot(corr != 1.0f)) {   // rescale only when some row's max moved
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) oacc[dt] *= corr;
            }
            // O += P V
            const int vb = kt & 1;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                bf16x8 a[8];
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    a[dt] = __builtin_bit_cast(bf16x8, sV[vb][vt_chunk(dt * 16 + l16, kb * 4 + lg)]);
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[dt], ph[kb], oacc[dt], 0, 0, 0);
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[dt], pl[kb], oacc[dt], 0, 0, 0);
            }
            // refill: K_{kt+2} -> stage kt&1, V_{kt+1} -> stage (kt+1)&1; request K_{kt+3}, V_{kt+2}
            put_k(kt & 1);
            put_v((kt + 1) & 1);
            gload(kreg, kc, pk, kt + 3);
            gload(vreg, vc, pv, kt + 2);
            pv = pk;
            pk = page_of(kt + 4);
        };

        // prologue: K_0, V_0 and K_1 staged; S_0; K_2 and V_1 requested
        {
            const int p0 = page_of(0), p1 = page_of(1), p2 = page_of(2);
            gload(kreg, kc, p0, 0);
            gload(vreg, vc, p0, 0);
            put_k(0);
            put_v(0);
            gload(kreg, kc, p1, 1);
            put_k(1);
            gload(kreg, kc, p2, 2);
            gload(vreg, vc, p1, 1);
            pk = page_of(3);
            pv = p2;
        }
        __syncthreads();
        f32x4 sa[4], sb[4];
        scores(0, sa);
        using Plain = std::integral_constant<bool, false>;
        using Masked = std::integral_constant<bool, true>;
        // Pairs of unmasked tiles in a loop without branches (one register assignment for
        // the two score buffers, no moves between differently compiled copies of a step),
        // then the rest: at most one unmasked tile (even) and the masked ones.
        const int nplain = min(kdiag, ntiles);
        int kt = 0;
        for (; kt + 2 <= nplain; kt += 2) {
            step(kt, sa, sb, Plain{});
            step(kt + 1, sb, sa, Plain{});
        }
        if (kt < nplain) {
            step(kt, sa, sb, Plain{});
            ++kt;
        }
        for (; kt < ntiles; ++kt) {
            if (kt & 1) step(kt, sb, sa, Masked{});
            else step(kt, sa, sb, Masked{});
        }

        // O^T accumulator: lane holds query row (l16), dims dt*16 + 4*lg + r.
        const float lrow = row_sum4(lpart);
        const int row = qbase + l16;
        if (row < M) {
            const float inv = 1.0f / lrow;
            if constexpr (PAIR) {
                // bf16 pair row: Hq*128 hi parts, then Hq*128 lo parts
                const size_t HD = (size_t)Hq * 128;
                bf16* orow = static_cast<bf16*>(o) + (size_t)row * 2 * HD + h * 128;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) {
                    unsigned hw[2], lw[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const float a0 = oacc[dt][2 * e] * inv, a1 = oacc[dt][2 * e + 1] * inv;
                        const bf16 h0 = f2bf(a0), h1 = f2bf(a1);
                        hw[e] = (unsigned)h0 | ((unsigned)h1 << 16);
                        lw[e] = (unsigned)f2bf(a0 - bf2f(h0)) | ((unsigned)f2bf(a1 - bf2f(h1)) << 16);
                    }
                    *reinterpret_cast<u32x2*>(orow + dt * 16 + lg * 4) = u32x2{hw[0], hw[1]};
                    *reinterpret_cast<u32x2*>(orow + HD + dt * 16 + lg * 4) = u32x2{lw[0], lw[1]};
                }
            } else {
                float* orow = static_cast<float*>(o) + (size_t)row * Hq * 128 + h * 128;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
                    *reinterpret_cast<f32x4*>(orow + dt * 16 + lg * 4) =
                        f32x4{oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv, oacc[dt][3] * inv};
            }
        }
    }   // pass
}

}  // namespace

hipError_t launch_attn_prefill(const float* q, const uint16_t* kc, const uint16_t* vc, const KvLayout& lay,
                               int seq, int M, int t0, int Hq, int Hkv, void* o, int o_pair, hipStream_t s) {
    static_assert(kKvPage % BKV == 0, "a key tile lies within one cache page");
    if (M <= 0) return hipSuccess;
    if (Hq != 2 * Hkv) return hipErrorInvalidValue;
    const int nqt = (M + BQ - 1) / BQ;
    // one head per block (four waves, one wave per SIMD, the full register file) while that
    // grid fits the compute units at one block each; past that both heads of a kv head per
    // block (eight waves), each staged K/V tile feeding both
    const bool both = (size_t)((nqt + 1) / 2) * Hq > 256;
    const dim3 grid((nqt + 1) / 2, both ? Hkv : Hq);
    const bool paged = lay.pt != nullptr;
#define Q3_ATTN_LAUNCH(P, H, G)                                                                               \
    hipLaunchKernelGGL((k_attn_prefill<P, H, G>), grid, dim3(256 * H), 0, s, q, kc, vc, lay, seq, M, t0, Hq, Hkv, o)
    if (both) {
        if (paged) { if (o_pair) Q3_ATTN_LAUNCH(true, 2, true); else Q3_ATTN_LAUNCH(false, 2, true); }
        else { if (o_pair) Q3_ATTN_LAUNCH(true, 2, false); else Q3_ATTN_LAUNCH(false, 2, false); }
    } else {
        if (paged) { if (o_pair) Q3_ATTN_LAUNCH(true, 1, true); else Q3_ATTN_LAUNCH(false, 1, true); }
        else { if (o_pair) Q3_ATTN_LAUNCH(true, 1, false); else Q3_ATTN_LAUNCH(false, 1, false); }
    }
#undef Q3_ATTN_LAUNCH
    return hipGetLastError();
}

}  // namespace q3
