// Decode-time projections: y = x W^T with float32 activations and bf16 (or float32)
// weights stored [out, in] row-major ("Inside an LLM ...", Step 5: q/k/v/o
// projections; Step 6: gate/up/down; Step 8: LM head tied to the embedding).
//
// Memory-bound: every weight byte is read once per call. One wave owns two weight rows;
// lanes stride the row in 16-byte bf16 chunks (8 elements), so each wave instruction
// reads 1 KiB of contiguous row data. Activations (at most 8 rows per block) are read
// from L2 and shared by the two rows.
#include "common.h"
#include "kernels.h"

namespace q3 {

namespace {

enum { EPI_LMHEAD = 3 };

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ void load8(const bf16* p, float* w) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[2 * i] = __uint_as_float(u[i] << 16);
        w[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ void load8(const float* p, float* w) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
    w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
}

// Weight chunks: read once per call, non-temporally (streaming reads reach ~7 TB/s this
// way on MI355X against ~6 TB/s with the default cache policy).
__device__ __forceinline__ void loadw8(const bf16* p, float* w) {
    const u32x4 v = __builtin_nontemporal_load((const __attribute__((address_space(1))) u32x4*)(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        w[2 * i] = __uint_as_float(v[i] << 16);
        w[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
}

__device__ __forceinline__ void loadw8(const float* p, float* w) {
    typedef __attribute__((ext_vector_type(4))) float f4;
    const f4 a = __builtin_nontemporal_load((const __attribute__((address_space(1))) f4*)(p));
    const f4 b = __builtin_nontemporal_load((const __attribute__((address_space(1))) f4*)(p + 4));
    w[0] = a[0]; w[1] = a[1]; w[2] = a[2]; w[3] = a[3];
    w[4] = b[0]; w[5] = b[1]; w[6] = b[2]; w[7] = b[3];
}

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

template <typename WT, int BB, int EPI>
__global__ __launch_bounds__(256) void k_gemv(const WT* __restrict__ W, const float* __restrict__ x,
                                              float* __restrict__ y, int N, int K, int B,
                                              unsigned long long* __restrict__ amax,
                                              unsigned* __restrict__ err) {
    __shared__ unsigned long long red[4][BB];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int b0 = blockIdx.y * BB;
    const int nb = min(BB, B - b0);
    const int unit = blockIdx.x * 4 + wid;           // output pair / SwiGLU column
    const int units = N / 2;
    const bool active = unit < units;
    int r0, r1;
    if (EPI == GEMV_SWIGLU) {
        r0 = (unit >> 4) * 32 + (unit & 15);       // gate row; its up row is 16 further
        r1 = r0 + 16;
    } else {
        r0 = 2 * unit;
        r1 = r0 + 1;
    }
    float acc0[BB], acc1[BB];
#pragma unroll
    for (int b = 0; b < BB; ++b) { acc0[b] = 0.f; acc1[b] = 0.f; }
    if (active) {
        const WT* w0p = W + (size_t)r0 * K;
        const WT* w1p = W + (size_t)r1 * K;
        for (int k = lane * 8; k < K; k += 512) {
            float w0[8], w1[8];
            loadw8(w0p + k, w0);
            loadw8(w1p + k, w1);
#pragma unroll
            for (int b = 0; b < BB; ++b) {
                if (b < nb) {
                    float xv[8];
                    load8(x + (size_t)(b0 + b) * K + k, xv);
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        acc0[b] += w0[i] * xv[i];
                        acc1[b] += w1[i] * xv[i];
                    }
                }
            }
        }
    }
#pragma unroll
    for (int b = 0; b < BB; ++b) {
        acc0[b] = wave_sum(acc0[b]);
        acc1[b] = wave_sum(acc1[b]);
    }
    if (EPI == EPI_LMHEAD) {
        if (lane == 0) {
#pragma unroll
            for (int b = 0; b < BB; ++b) {
                unsigned long long best = 0ull;
                if (active && b < nb) {
                    float* yr = y + (size_t)(b0 + b) * N;
                    yr[r0] = acc0[b];
                    yr[r1] = acc1[b];
                    if (!isfinite(acc0[b]) || !isfinite(acc1[b])) atomicOr(err, Q3_DEVERR_NONFINITE);
                    const unsigned long long k0 = pack_argmax(acc0[b], r0), k1 = pack_argmax(acc1[b], r1);
                    best = k0 > k1 ? k0 : k1;
                }
                red[wid][b] = best;
            }
        }
        __syncthreads();
        if (threadIdx.x < nb) {
            const int b = threadIdx.x;
            unsigned long long m = red[0][b];
            for (int w = 1; w < 4; ++w) m = red[w][b] > m ? red[w][b] : m;
            atomicMax(amax + b0 + b, m);
        }
        return;
    }
    if (!active || lane != 0) return;
#pragma unroll
    for (int b = 0; b < BB; ++b) {
        if (b >= nb) break;
        float* yr = y + (size_t)(b0 + b) * (EPI == GEMV_SWIGLU ? units : N);
        if (EPI == GEMV_STORE) {
            yr[r0] = acc0[b];
            yr[r1] = acc1[b];
        } else if (EPI == GEMV_RESID) {
            yr[r0] += acc0[b];
            yr[r1] += acc1[b];
        } else {
            yr[unit] = silu_mul(acc0[b], acc1[b]);
        }
    }
}

template <typename WT, int EPI>
hipError_t launch_t(const WT* W, const float* x, float* y, int N, int K, int B,
                    unsigned long long* amax, unsigned* err, hipStream_t s) {
    constexpr int BB = 8;
    const int units = N / 2;
    dim3 grid((units + 3) / 4, (B + BB - 1) / BB);
    hipLaunchKernelGGL((k_gemv<WT, BB, EPI>), grid, dim3(256), 0, s, W, x, y, N, K, B, amax, err);
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_any(const void* W, int wdt, const float* x, float* y, int N, int K, int B,
                      unsigned long long* amax, unsigned* err, hipStream_t s) {
    if (wdt == DT_BF16) return launch_t<bf16, EPI>((const bf16*)W, x, y, N, K, B, amax, err, s);
    return launch_t<float, EPI>((const float*)W, x, y, N, K, B, amax, err, s);
}

}  // namespace

hipError_t launch_gemv(const void* W, int wdt, const float* x, float* y, int N, int K, int B,
                       int epi, hipStream_t s) {
    if (B <= 0 || N <= 0) return hipSuccess;
    switch (epi) {
        case GEMV_STORE: return launch_any<GEMV_STORE>(W, wdt, x, y, N, K, B, nullptr, nullptr, s);
        case GEMV_RESID: return launch_any<GEMV_RESID>(W, wdt, x, y, N, K, B, nullptr, nullptr, s);
        case GEMV_SWIGLU: return launch_any<GEMV_SWIGLU>(W, wdt, x, y, N, K, B, nullptr, nullptr, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_lmhead(const void* E, int wdt, const float* h, float* logits,
                         unsigned long long* amax, int V, int K, int B, unsigned* err, hipStream_t s) {
    if (B <= 0) return hipSuccess;
    return launch_any<EPI_LMHEAD>(E, wdt, h, logits, V, K, B, amax, err, s);
}

}  // namespace q3
