// Prefill attention: causal grouped-query attention of M new rows of one sequence
// ("Inside an LLM ...", Step 5: scores q.k * 128^-0.5, causal mask so a row never sees
// a later slot, softmax, weighted sum of V; query heads 2g, 2g+1 read kv head g).
//
// Flash-style, on the matrix cores. A block owns 64 query rows of both query heads of
// one kv head (four waves: head x 32-row half) and walks the key tiles (64 keys) up to
// the causal limit of its last row, keeping a running max / sum per row (float32, base-2
// exponentials) -- the n x n score matrix is never stored.
//
// Per key tile the waves compute S^T = K Q^T (A = K tile from LDS, B = the wave's Q rows
// held in registers). In that accumulator layout a lane holds 4 consecutive keys of one
// query row for each 16-key tile, which is exactly what the B operand of O^T = V^T P^T
// needs once both operands agree on the order of the contraction (key) index; so the
// probabilities go from accumulators to bf16 operands without touching LDS. V is stored
// transposed in LDS ([dim][key]) for the A operand.
//
// Precision: K and V are bf16 (the cache's own format, exact as operands). q (float32) and
// the probabilities (float32) are each split into bf16 hi + lo parts and take two MFMAs,
// so both products keep ~16 significant bits; the output is float32.
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
// V^T tile: 128 rows (dims) x 8 chunks of 16 B (64 keys); chunk c of row d at
// c ^ ((d ^ (d >> 3)) & 7): the fragment reads (16 consecutive dims) and the staging writes
// (dims 8 apart) both spread over the banks.
__device__ __forceinline__ int vt_off(int d, int key) {  // offset in bf16 elements
    const int ck = key >> 3;
    return d * 64 + ((ck ^ ((d ^ (d >> 3)) & 7)) << 3) + (key & 7);
}

__device__ __forceinline__ unsigned int pack2(bf16 a, bf16 b) { return (unsigned)a | ((unsigned)b << 16); }

typedef __attribute__((ext_vector_type(8))) float f32x8;

// 8 float32 -> bf16 hi parts and bf16 lo parts, as two 8-element operands (hardware
// round-to-nearest-even conversions, two values per instruction).
__device__ __forceinline__ void split8(const float* v, bf16x8& hi, bf16x8& lo) {
    const f32x8 x = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
    hi = __builtin_convertvector(x, bf16x8);
    const f32x8 hf = __builtin_convertvector(hi, f32x8);
    lo = __builtin_convertvector(x - hf, bf16x8);
}

// BAL = true (the launched form): block (b, query head h) takes query tiles nqt-1-b and
// then b, each wave 16 rows (RT = 1), so every block walks nqt + 1 key tiles (tile i needs
// i + 1), and the register footprint allows two blocks per compute unit, whose
// score / softmax / P.V chains then interleave on the matrix cores. BAL = false: block
// (query tile, kv head g) covers both query heads of g, each wave 32 rows (RT = 2); it
// halves the K/V staging per product but runs one block per compute unit, and measured
// 1.1x (2048 rows) to 1.8x (8192 rows) slower.
template <bool PAIR, bool BAL>
__global__ __launch_bounds__(256, BAL ? 2 : 1) void k_attn_prefill(const float* __restrict__ q, const bf16* __restrict__ kc,
                                                      const bf16* __restrict__ vc, KvLayout lay, int seq, int M,
                                                      int t0, int Hq, int Hkv, void* __restrict__ o) {
    constexpr int RT = BAL ? 1 : 2;
    __shared__ u32x4 sK[BKV * 16];
    __shared__ bf16 sVT[128 * BKV];
    const int nqt = (M + BQ - 1) / BQ;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int h = BAL ? (int)blockIdx.y : (int)blockIdx.y * 2 + (wid >> 1);
    const int g = BAL ? (int)blockIdx.y >> 1 : (int)blockIdx.y;
    const int l16 = lane & 15, lg = lane >> 4;
    const float scale_log2 = 0.088388346f * 1.4426950408889634f;

    for (int pass = 0; pass < (BAL ? 2 : 1); ++pass) {
    // heaviest (latest) query tiles first
    const int qt = pass == 0 ? nqt - 1 - (int)blockIdx.x : (int)blockIdx.x;
    if (pass == 1 && qt >= nqt - 1 - (int)blockIdx.x) break;   // the middle tile of an odd count
    const int qbase = qt * BQ + (BAL ? wid * 16 : (wid & 1) * 32);   // first row of this wave

    // Q^T as B operand (hi and lo parts): lane holds q row (l16) of q-tile c, dims
    // ks*32 + 8*lg .. +8.
    bf16x8 qh[RT][4], ql[RT][4];
#pragma unroll
    for (int c = 0; c < RT; ++c) {
        const int row = qbase + c * 16 + l16;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            if (row < M) {
                const f32x4* p = reinterpret_cast<const f32x4*>(q + ((size_t)h * M + row) * 128 + ks * 32 + lg * 8);
                const f32x4 a = p[0], b = p[1];
                v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
                v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
            }
            split8(v, qh[c][ks], ql[c][ks]);
        }
    }
    f32x4 oacc[8][RT];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int c = 0; c < RT; ++c) oacc[dt][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrow[RT], lrow[RT];
#pragma unroll
    for (int c = 0; c < RT; ++c) {
        mrow[c] = -INFINITY;
        lrow[c] = 0.f;
    }

    const int block_last_row = min(M, (qt + 1) * BQ) - 1;
    const int last_slot = t0 + block_last_row;
    const int ntiles = last_slot / BKV + 1;

    // K/V of tile kt + 1 are loaded into registers while tile kt is in use. Thread t takes
    // 16-byte chunk ck = t % 16 of the key pairs t / 16 and t / 16 + 16.
    const int ck = tid & 15;
    u32x4 kreg[2][2], vreg[2][2];
    auto kv_load = [&](int kt) {
        // a 64-key tile lies within one page: one strided run from the tile's first slot
        const size_t tb = lay.off(seq, g, kt * BKV);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int key = 2 * ((tid >> 4) + 16 * j) + u;
                const int slot = kt * BKV + key;
                kreg[j][u] = u32x4{0u, 0u, 0u, 0u};
                vreg[j][u] = u32x4{0u, 0u, 0u, 0u};
                if (slot <= last_slot) {
                    kreg[j][u] = *reinterpret_cast<const u32x4*>(kc + tb + (size_t)key * 128 + ck * 8);
                    vreg[j][u] = *reinterpret_cast<const u32x4*>(vc + tb + (size_t)key * 128 + ck * 8);
                }
            }
    };
    kv_load(0);
    for (int kt = 0; kt < ntiles; ++kt) {
        __syncthreads();
        // stage K (row-major, swizzled) and V^T (two keys per 32-bit store); slots beyond
        // last_slot are zero-filled
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int key0 = 2 * ((tid >> 4) + 16 * j);
            sK[kidx(key0, ck)] = kreg[j][0];
            sK[kidx(key0 + 1, ck)] = kreg[j][1];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const unsigned a = (vreg[j][0][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                const unsigned b = (vreg[j][1][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                *reinterpret_cast<unsigned*>(&sVT[vt_off(ck * 8 + e, key0)]) = a | (b << 16);
            }
        }
        __syncthreads();
        if (kt + 1 < ntiles) kv_load(kt + 1);

        // S^T[key][row] for 4 key tiles x RT row tiles
        f32x4 s[4][RT];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int c = 0; c < RT; ++c) s[j][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, sK[kidx(j * 16 + l16, ks * 4 + lg)]);
#pragma unroll
                for (int c = 0; c < RT; ++c) s[j][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qh[c][ks], s[j][c], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < RT; ++c) s[j][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ql[c][ks], s[j][c], 0, 0, 0);
            }
        }
        // scale, causal mask, online softmax (per query row = l16 of tile c)
        const bool diag = (kt + 1) * BKV - 1 > t0 + qbase;   // some key may be after some row
#pragma unroll
        for (int c = 0; c < RT; ++c) {
            const int qslot = t0 + qbase + c * 16 + l16;
            float mx = -INFINITY;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    float v = s[j][c][r] * scale_log2;
                    if (diag) {
                        const int kslot = kt * BKV + j * 16 + lg * 4 + r;
                        if (kslot > qslot) v = -INFINITY;
                    }
                    s[j][c][r] = v;
                    mx = fmaxf(mx, v);
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float mnew = fmaxf(mrow[c], mx);
            const float corr = __builtin_amdgcn_exp2f(mrow[c] - mnew);   // 0 on the first tile (mrow = -inf)
            float sum = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = __builtin_amdgcn_exp2f(s[j][c][r] - mnew);
                    s[j][c][r] = p;
                    sum += p;
                }
            sum += __shfl_xor(sum, 16, 64);
            sum += __shfl_xor(sum, 32, 64);
            lrow[c] = lrow[c] * corr + sum;
            mrow[c] = mnew;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) oacc[dt][c] *= corr;
        }
        // P^T operands: for key block kb (32 keys = tiles 2kb, 2kb+1) lane group lg holds
        // keys {32kb + 4lg + i, 32kb + 16 + 4lg + i : i < 4}; V^T uses the same order.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            bf16x8 ph[RT], pl[RT];
#pragma unroll
            for (int c = 0; c < RT; ++c) {
                const float pv[8] = {s[2 * kb][c][0], s[2 * kb][c][1], s[2 * kb][c][2], s[2 * kb][c][3],
                                     s[2 * kb + 1][c][0], s[2 * kb + 1][c][1], s[2 * kb + 1][c][2], s[2 * kb + 1][c][3]};
                split8(pv, ph[c], pl[c]);
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const int d = dt * 16 + l16;
                const u32x2 lo = *reinterpret_cast<const u32x2*>(&sVT[vt_off(d, kb * 32 + lg * 4)]);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(&sVT[vt_off(d, kb * 32 + 16 + lg * 4)]);
                const u32x4 av = {lo.x, lo.y, hi.x, hi.y};
                const bf16x8 a = __builtin_bit_cast(bf16x8, av);
#pragma unroll
                for (int c = 0; c < RT; ++c) oacc[dt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, ph[c], oacc[dt][c], 0, 0, 0);
#pragma unroll
                for (int c = 0; c < RT; ++c) oacc[dt][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pl[c], oacc[dt][c], 0, 0, 0);
            }
        }
    }
    // O^T accumulator: lane holds query row (l16) of tile c, dims dt*16 + 4*lg + r.
#pragma unroll
    for (int c = 0; c < RT; ++c) {
        const int row = qbase + c * 16 + l16;
        if (row >= M) continue;
        const float inv = 1.0f / lrow[c];
        if constexpr (PAIR) {
            // bf16 pair row: Hq*128 hi parts, then Hq*128 lo parts
            const size_t HD = (size_t)Hq * 128;
            bf16* orow = static_cast<bf16*>(o) + (size_t)row * 2 * HD + h * 128;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                unsigned hw[2], lw[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const float a0 = oacc[dt][c][2 * e] * inv, a1 = oacc[dt][c][2 * e + 1] * inv;
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
                    f32x4{oacc[dt][c][0] * inv, oacc[dt][c][1] * inv, oacc[dt][c][2] * inv, oacc[dt][c][3] * inv};
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
    const dim3 grid((nqt + 1) / 2, Hq);
    if (o_pair)
        hipLaunchKernelGGL((k_attn_prefill<true, true>), grid, dim3(256), 0, s, q, kc, vc, lay, seq, M, t0, Hq, Hkv, o);
    else
        hipLaunchKernelGGL((k_attn_prefill<false, true>), grid, dim3(256), 0, s, q, kc, vc, lay, seq, M, t0, Hq, Hkv, o);
    return hipGetLastError();
}

}  // namespace q3
