// Prefill projections on the matrix cores: C = A W^T with A [M, K] bf16 activations and
// W [N, K] bf16 weights in the [out, in] layout of the article's projections
// ("Inside an LLM ...", Step 5 q/k/v/o, Step 6 gate/up/down), float32 accumulation.
//
// Block tile 128 x 128 x 64, four waves in a 2 x 2 grid, each wave a 64 x 64 sub-tile of
// 4 x 4 v_mfma_f32_16x16x32_bf16 tiles. Global -> registers -> LDS with two LDS buffers
// (one barrier per k-tile). LDS rows are 8 chunks of 16 bytes, chunk c of row r stored at
// c ^ (r & 7) so the 16-lane fragment reads of one chunk column hit distinct banks.
//
// A may be bf16, or float32: then each element is split while staging into
// hi = bf16(a) and lo = bf16(a - hi) and every tile takes two MFMAs (hi W + lo W). The
// weights are exactly bf16, so the product keeps ~16 significant bits of the activations
// (relative error ~2^-17) instead of 8 -- what the float32 reference needs at 28 layers.
//
// Epilogues: float32 store, float32 residual add (x += A W^T), SwiGLU to float32 (W packs
// 16 gate rows then the 16 matching up rows; a lane holds both), bf16 store.
// Requires N % 128 == 0 and K % 64 == 0; rows >= M are masked.
#include "common.h"
#include "kernels.h"

namespace q3 {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int BM = 128, BN = 128, BK = 64;

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

template <typename AT, int EPI>
__global__ __launch_bounds__(256, 1) void k_gemm(const AT* __restrict__ A, const bf16* __restrict__ W,
                                                 void* __restrict__ C, int M, int N, int K) {
    constexpr bool SPLIT = sizeof(AT) == 4;
    __shared__ u32x4 sA[2][BM * 8];
    __shared__ u32x4 sL[SPLIT ? 2 : 1][SPLIT ? BM * 8 : 1];
    __shared__ u32x4 sB[2][BN * 8];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;

    u32x4 ra[4], rl[4], rb[4];
    const u32x4 zero = {0u, 0u, 0u, 0u};
    auto gload = [&](int kt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = tid + 256 * j, row = q >> 3, ck = q & 7;
            const int gm = m0 + row;
            if constexpr (SPLIT) {
                f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
                if (gm < M) {
                    const f32x4* p = reinterpret_cast<const f32x4*>(A + (size_t)gm * K + kt * BK + ck * 8);
                    x0 = p[0];
                    x1 = p[1];
                }
                split8(x0, x1, ra[j], rl[j]);
            } else {
                ra[j] = gm < M ? *reinterpret_cast<const u32x4*>(A + (size_t)gm * K + kt * BK + ck * 8) : zero;
            }
            rb[j] = *reinterpret_cast<const u32x4*>(W + (size_t)(n0 + row) * K + kt * BK + ck * 8);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = tid + 256 * j, row = q >> 3, ck = q & 7;
            sA[buf][swz(row, ck)] = ra[j];
            if constexpr (SPLIT) sL[buf][swz(row, ck)] = rl[j];
            sB[buf][swz(row, ck)] = rb[j];
        }
    };

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 a[4], b[4];
            const int ck = ks * 4 + (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = __builtin_bit_cast(bf16x8, sA[cur][swz(wm * 64 + i * 16 + (lane & 15), ck)]);
                b[i] = __builtin_bit_cast(bf16x8, sB[cur][swz(wn * 64 + i * 16 + (lane & 15), ck)]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            if constexpr (SPLIT) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[i] = __builtin_bit_cast(bf16x8, sL[cur][swz(wm * 64 + i * 16 + (lane & 15), ck)]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // D layout of 16x16 MFMA: lane holds column (lane & 15), rows 4 * (lane >> 4) + r.
    const int col_l = lane & 15, row_l = 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = m0 + wm * 64 + i * 16 + row_l + r;
            if (row >= M) continue;
            if (EPI == GEMM_SWIGLU_F32) {
                float* out = reinterpret_cast<float*>(C) + (size_t)row * (N / 2);
#pragma unroll
                for (int p = 0; p < 2; ++p) {
                    const float g = acc[i][2 * p][r], u = acc[i][2 * p + 1][r];
                    const int col = (n0 + wn * 64 + 32 * p) / 2 + col_l;
                    out[col] = g / (1.0f + expf(-g)) * u;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int col = n0 + wn * 64 + j * 16 + col_l;
                    const float v = acc[i][j][r];
                    if (EPI == GEMM_F32) reinterpret_cast<float*>(C)[(size_t)row * N + col] = v;
                    else if (EPI == GEMM_RESID_F32) reinterpret_cast<float*>(C)[(size_t)row * N + col] += v;
                    else reinterpret_cast<bf16*>(C)[(size_t)row * N + col] = f2bf(v);
                }
            }
        }
    }
}

}  // namespace

template <typename AT>
static hipError_t launch_t(const AT* A, const uint16_t* W, void* C, int M, int N, int K, int epi, hipStream_t s) {
    dim3 grid(N / BN, (M + BM - 1) / BM);
    switch (epi) {
        case GEMM_F32: hipLaunchKernelGGL((k_gemm<AT, GEMM_F32>), grid, dim3(256), 0, s, A, W, C, M, N, K); break;
        case GEMM_RESID_F32: hipLaunchKernelGGL((k_gemm<AT, GEMM_RESID_F32>), grid, dim3(256), 0, s, A, W, C, M, N, K); break;
        case GEMM_SWIGLU_F32: hipLaunchKernelGGL((k_gemm<AT, GEMM_SWIGLU_F32>), grid, dim3(256), 0, s, A, W, C, M, N, K); break;
        case GEMM_BF16: hipLaunchKernelGGL((k_gemm<AT, GEMM_BF16>), grid, dim3(256), 0, s, A, W, C, M, N, K); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_gemm(const void* A, int a_f32, const uint16_t* W, void* C, int M, int N, int K, int epi,
                       hipStream_t s) {
    if (M <= 0) return hipSuccess;
    if (N % BN != 0 || K % BK != 0) return hipErrorInvalidValue;
    if (a_f32) return launch_t<float>((const float*)A, W, C, M, N, K, epi, s);
    return launch_t<bf16>((const bf16*)A, W, C, M, N, K, epi, s);
}

}  // namespace q3
