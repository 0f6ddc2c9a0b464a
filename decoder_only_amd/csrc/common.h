// Shared device helpers of the q3 engine (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define Q3_WAVE 64

// Sticky device error bits (reported by q3_sync).
#define Q3_DEVERR_TOKEN 1u
#define Q3_DEVERR_NONFINITE 2u
#define Q3_DEVERR_SYNC 4u       // a cross-workgroup wait of the persistent decode kernel timed out

namespace q3 {

typedef uint16_t bf16;  // raw bf16 bit pattern

__device__ __forceinline__ float bf2f(bf16 b) { return __uint_as_float(((uint32_t)b) << 16); }

// float32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ bf16 f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16)(u >> 16);
}

// Load one weight element as float (bf16 or float32 storage).
__device__ __forceinline__ float ldw(const bf16* p, size_t i) { return bf2f(p[i]); }
__device__ __forceinline__ float ldw(const float* p, size_t i) { return p[i]; }

__device__ __forceinline__ void stkv(bf16* p, size_t i, float v) { p[i] = f2bf(v); }
__device__ __forceinline__ void stkv(float* p, size_t i, float v) { p[i] = v; }

// Cross-lane reductions with DPP moves inside rows of 16 lanes (no LDS round trip) and
// v_readlane across rows. DPP controls: quad_perm [1,0,3,2] and [2,3,0,1] swap neighbours
// at distance 1 and 2; row_half_mirror / row_mirror reverse 8- and 16-lane groups, which
// pair each half with the other one.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140;

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Sum over aligned groups of 8 / 16 lanes; every lane of the group gets the sum. The lanes
// of a group must be active together.
__device__ __forceinline__ float sum8(float v) {
    v += dpp_mov<kDppQuadXor1>(v);
    v += dpp_mov<kDppQuadXor2>(v);
    v += dpp_mov<kDppRowHalfMirror>(v);
    return v;
}
__device__ __forceinline__ float sum16(float v) {
    v = sum8(v);
    v += dpp_mov<kDppRowMirror>(v);
    return v;
}
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, dpp_mov<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_mov<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_mov<kDppRowHalfMirror>(v));
    v = fmaxf(v, dpp_mov<kDppRowMirror>(v));
    return v;
}

// Whole-wave sum / max (all 64 lanes active); the result is wave-uniform.
__device__ __forceinline__ float wave_sum(float v) {
    v = sum16(v);
    return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

__device__ __forceinline__ float wave_max(float v) {
    v = max16(v);
    return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}

// Order-preserving map float32 -> uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t ordered_key(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// Packed (logit, id) so that a 64-bit max picks the largest logit, then the lowest id.
__device__ __forceinline__ unsigned long long pack_argmax(float v, uint32_t id) {
    return ((unsigned long long)ordered_key(v) << 32) | (unsigned long long)(0xFFFFFFFFu - id);
}

// Block-wide sum for blockDim.x a multiple of 64 (<= 1024). `red` has >= 16 floats.
__device__ __forceinline__ float block_sum(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if (lane == 0) red[wid] = v;
    __syncthreads();
    float t = 0.f;
    for (int i = 0; i < nw; ++i) t += red[i];
    return t;
}

}  // namespace q3
