// Prefill projections on the matrix cores: C = A W^T with A [M, K] activations and
// W [N, K] bf16 weights in the [out, in] layout of the article's projections
// ("Inside an LLM ...", Step 5 q/k/v/o, Step 6 gate/up/down), float32 accumulation.
//
// Block tile BM x 128 x 64 (BM = 64 at every shape in use; the template also takes 128),
// four waves in a 2 x 2 grid, each wave a BM/2 x 64 sub-tile of
// v_mfma_f32_16x16x32_bf16 tiles. Global -> registers (the next k-tile, in flight during
// the current one's products) -> LDS. LDS rows are 8 chunks of 16 bytes, chunk c of row r stored at
// c ^ (r & 7) so the 16-lane fragment reads of one chunk column hit distinct banks.
//
// A is bf16 (one MFMA per tile), or carries ~16 significant bits as a bf16 pair
// a = hi + lo (two MFMAs per tile, hi W + lo W; the weights are exact bf16, so the product
// keeps relative error ~2^-17 instead of 2^-9 -- what the float32 reference needs at 28
// layers). The pair either comes ready-made from the producing kernel (rows of 2K bf16:
// the K hi parts, then the K lo parts) or is split here from float32 A while staging.
//
// Epilogues: float32 store, float32 residual add (x += A W^T), SwiGLU (W packs 16 gate rows
// then the 16 matching up rows; a lane holds both) to float32 or to bf16 pair rows, bf16,
// and split-K partials (gridDim.z blocks along K, each writing its float32 partial product,
// summed by the consumer in a fixed order).
// Requires N % 128 == 0 and K % 64 == 0; rows >= M are masked.
#include "common.h"
#include "kernels.h"

namespace q3 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int BN = 128, BK = 64;

__device__ __forceinline__ int swz(int row, int ck) { return row * 8 + (ck ^ (row & 7)); }

__device__ __forceinline__ unsigned int pack2(bf16 a, bf16 b) { return (unsigned)a | ((unsigned)b << 16); }

// 8 float32 -> 8 bf16 hi parts and 8 bf16 lo parts (a = hi + lo + O(2^-17 a)).
__device__ __forceinline__ void split8(const f32x4& x0, const f32x4& x1, u32x4& hi, u32x4& lo) {
    const float v[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
    bf16 h[8], l[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        h[i] = f2bf(v[i]);
        l[i] = f2bf(v[i] - bf2f(h[i]));
    }
    hi = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
    lo = u32x4{pack2(l[0], l[1]), pack2(l[2], l[3]), pack2(l[4], l[5]), pack2(l[6], l[7])};
}

// NB = LDS buffers: 2 (the next k-tile is stored while the current one is read; one block
// per compute unit at BM = 128) or 1 (two barriers per k-tile, two blocks per compute unit).
template <int AM, int EPI, int BM, int NB>
__global__ __launch_bounds__(256, 3 - NB) void k_gemm(const void* __restrict__ Av, const bf16* __restrict__ W,
                                                      void* __restrict__ C, int M, int N, int K,
                                                      const float* __restrict__ cs) {
    constexpr bool SPLIT = AM != GEMM_A_BF16;
    constexpr int FM = BM / 32;          // 16-row fragments per wave along M
    constexpr int AJ = BM * 8 / 256;     // 16-byte A chunks per thread and k-tile
    __shared__ u32x4 sA[NB][BM * 8];
    __shared__ u32x4 sL[SPLIT ? NB : 1][SPLIT ? BM * 8 : 1];
    __shared__ u32x4 sB[NB][BN * 8];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    // Tile of this block. Workgroup b (in launch order) runs on XCD b % 8, and the XCD's
    // blocks in flight together are consecutive in b / 8. So XCD c takes a contiguous range
    // of the tiles, ordered in column groups of 4 row tiles: the blocks an XCD runs at once
    // then cover a compact patch of C, and their A and W rows are shared in its L2.
    int bx = blockIdx.x, by = blockIdx.y, bz = blockIdx.z;
    {
        const int nx = gridDim.x, ny = gridDim.y;
        const int total = nx * ny * gridDim.z;
        if (total % 8 == 0 && ny > 1) {            // (one row tile: no A to share)
            const int b = blockIdx.x + nx * (blockIdx.y + ny * blockIdx.z);
            const int t = (b % 8) * (total / 8) + b / 8;
            bz = t / (nx * ny);
            const int r = t % (nx * ny), g = r / (4 * nx), rows = min(4, ny - 4 * g), i = r % (4 * nx);
            by = 4 * g + i % rows;
            bx = i / rows;
        }
    }
    const int m0 = by * BM, n0 = bx * BN;
    const size_t lda = AM == GEMM_A_PAIR ? 2 * (size_t)K : (size_t)K;

    u32x4 ra[AJ], rl[AJ], rb[4];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto gload = [&](int kt) {
#pragma unroll
        for (int j = 0; j < AJ; ++j) {
            const int q = tid + 256 * j, row = q >> 3, ck = q & 7;
            const int gm = m0 + row;
            if constexpr (AM == GEMM_A_F32) {
                f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
                if (gm < M) {
                    const f32x4* p = reinterpret_cast<const f32x4*>(static_cast<const float*>(Av) + gm * lda + kt * BK + ck * 8);
                    x0 = p[0];
                    x1 = p[1];
                }
                split8(x0, x1, ra[j], rl[j]);
            } else {
                const bf16* A = static_cast<const bf16*>(Av) + gm * lda + kt * BK + ck * 8;
                ra[j] = gm < M ? *reinterpret_cast<const u32x4*>(A) : zero;
                if constexpr (AM == GEMM_A_PAIR) rl[j] = gm < M ? *reinterpret_cast<const u32x4*>(A + K) : zero;
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = tid + 256 * j, row = q >> 3, ck = q & 7;
            rb[j] = *reinterpret_cast<const u32x4*>(W + (size_t)(n0 + row) * K + kt * BK + ck * 8);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < AJ; ++j) {
            const int q = tid + 256 * j, row = q >> 3, ck = q & 7;
            sA[buf][swz(row, ck)] = ra[j];
            if constexpr (SPLIT) sL[buf][swz(row, ck)] = rl[j];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = tid + 256 * j, row = q >> 3, ck = q & 7;
            sB[buf][swz(row, ck)] = rb[j];
        }
    };

    f32x4 acc[FM][4];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // split-K: block z of gridDim.z takes k-tiles [z nk / S, (z + 1) nk / S)
    const int nkt = K / BK, S = gridDim.z, z = bz;
    const int kt0 = (int)((long long)nkt * z / S), nk = (int)((long long)nkt * (z + 1) / S);
    gload(kt0);
    sstore(0);
    __syncthreads();
    for (int kt = kt0; kt < nk; ++kt) {
        const int cur = NB == 2 ? ((kt - kt0) & 1) : 0;
        if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 a[FM], b[4];
            const int ck = ks * 4 + (lane >> 4);
#pragma unroll
            for (int i = 0; i < FM; ++i)
                a[i] = __builtin_bit_cast(bf16x8, sA[cur][swz(wm * (BM / 2) + i * 16 + (lane & 15), ck)]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                b[j] = __builtin_bit_cast(bf16x8, sB[cur][swz(wn * 64 + j * 16 + (lane & 15), ck)]);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            if constexpr (SPLIT) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    a[i] = __builtin_bit_cast(bf16x8, sL[cur][swz(wm * (BM / 2) + i * 16 + (lane & 15), ck)]);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }
        if constexpr (NB == 2) {
            if (kt + 1 < nk) sstore(cur ^ 1);
            __syncthreads();
        } else {
            __syncthreads();
            if (kt + 1 < nk) {
                sstore(0);
                __syncthreads();
            }
        }
    }

    // D layout of 16x16 MFMA: lane holds column (lane & 15), rows 4 * (lane >> 4) + r.
    const int col_l = lane & 15, row_l = 4 * (lane >> 4);
    if (cs) {                          // int8 weights: each output column times its row scale
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float c = cs[n0 + wn * 64 + j * 16 + col_l];
#pragma unroll
            for (int i = 0; i < FM; ++i) acc[i][j] *= c;
        }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + wm * (BM / 2) + i * 16 + row_l + r;
            if (row >= M) continue;
            if (EPI == GEMM_SWIGLU_F32 || EPI == GEMM_SWIGLU_PAIR) {
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const float g = acc[i][2 * p][r], u = acc[i][2 * p + 1][r];
                    const int col = (n0 + wn * 64 + 32 * p) / 2 + col_l;
                    const float a = g / (1.0f + expf(-g)) * u;
                    if (EPI == GEMM_SWIGLU_F32) {
                        reinterpret_cast<float*>(C)[(size_t)row * (N / 2) + col] = a;
                    } else {                     // pair row of N bf16: N/2 hi, then N/2 lo
                        bf16* out = reinterpret_cast<bf16*>(C) + (size_t)row * N;
                        const bf16 h = f2bf(a);
                        out[col] = h;
                        out[N / 2 + col] = f2bf(a - bf2f(h));
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = n0 + wn * 64 + j * 16 + col_l;
                    const float v = acc[i][j][r];
                    if (EPI == GEMM_F32) reinterpret_cast<float*>(C)[(size_t)row * N + col] = v;
                    else if (EPI == GEMM_PARTIAL_F32)
                        reinterpret_cast<float*>(C)[((size_t)z * M + row) * N + col] = v;
                    else if (EPI == GEMM_RESID_F32) reinterpret_cast<float*>(C)[(size_t)row * N + col] += v;
                    else reinterpret_cast<bf16*>(C)[(size_t)row * N + col] = f2bf(v);
                }
            }
        }
    }
}

}  // namespace

template <int AM, int BM, int NB>
static hipError_t launch_t(const void* A, const uint16_t* W, void* C, int M, int N, int K, int epi, int splits,
                           hipStream_t s, const float* cs) {
    dim3 grid(N / BN, (M + BM - 1) / BM, splits);
    switch (epi) {
        case GEMM_F32: hipLaunchKernelGGL((k_gemm<AM, GEMM_F32, BM, NB>), grid, dim3(256), 0, s, A, W, C, M, N, K, cs); break;
        case GEMM_RESID_F32: hipLaunchKernelGGL((k_gemm<AM, GEMM_RESID_F32, BM, NB>), grid, dim3(256), 0, s, A, W, C, M, N, K, cs); break;
        case GEMM_SWIGLU_F32: hipLaunchKernelGGL((k_gemm<AM, GEMM_SWIGLU_F32, BM, NB>), grid, dim3(256), 0, s, A, W, C, M, N, K, cs); break;
        case GEMM_BF16: hipLaunchKernelGGL((k_gemm<AM, GEMM_BF16, BM, NB>), grid, dim3(256), 0, s, A, W, C, M, N, K, cs); break;
        case GEMM_SWIGLU_PAIR: hipLaunchKernelGGL((k_gemm<AM, GEMM_SWIGLU_PAIR, BM, NB>), grid, dim3(256), 0, s, A, W, C, M, N, K, cs); break;
        case GEMM_PARTIAL_F32: hipLaunchKernelGGL((k_gemm<AM, GEMM_PARTIAL_F32, BM, NB>), grid, dim3(256), 0, s, A, W, C, M, N, K, cs); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int AM>
static hipError_t launch_bm(const void* A, const uint16_t* W, void* C, int M, int N, int K, int epi, int splits,
                            hipStream_t s, const float* cs) {
    // 64-row tiles: with one LDS buffer (two barriers per k-tile) several blocks share a
    // compute unit and hide each other's loads; with fewer than two blocks per compute unit
    // the double-buffered variant is faster. (Measured on MI355X at the prefill shapes,
    // M = 2047 and 32767: 128-row tiles were 5-25% slower everywhere.)
    const long long blocks64 = (long long)(N / BN) * ((M + 63) / 64) * splits;
    if (blocks64 < 512) return launch_t<AM, 64, 2>(A, W, C, M, N, K, epi, splits, s, cs);
    return launch_t<AM, 64, 1>(A, W, C, M, N, K, epi, splits, s, cs);
}

hipError_t launch_gemm(const void* A, int a_mode, const uint16_t* W, void* C, int M, int N, int K, int epi,
                       hipStream_t s, int splits, const float* cs) {
    if (M <= 0) return hipSuccess;
    if (N % BN != 0 || K % BK != 0 || splits < 1 || splits > K / BK || (splits > 1 && epi != GEMM_PARTIAL_F32))
        return hipErrorInvalidValue;
    switch (a_mode) {
        case GEMM_A_BF16: return launch_bm<GEMM_A_BF16>(A, W, C, M, N, K, epi, splits, s, cs);
        case GEMM_A_F32: return launch_bm<GEMM_A_F32>(A, W, C, M, N, K, epi, splits, s, cs);
        case GEMM_A_PAIR: return launch_bm<GEMM_A_PAIR>(A, W, C, M, N, K, epi, splits, s, cs);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace q3
