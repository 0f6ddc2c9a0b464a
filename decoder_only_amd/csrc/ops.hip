// Op-level C ABI (include/q3_ops.h): one kernel family per call, on caller buffers.
#include <cmath>
#include <mutex>
#include <vector>

#include "common.h"
#include "kernels.h"
#include "q3_ops.h"

using namespace q3;

namespace {

// Scratch for ops that need it: allocated per call, released after the stream drains.
struct Scratch {
    void* p = nullptr;
    hipStream_t s;
    explicit Scratch(hipStream_t st) : s(st) {}
    bool get(size_t bytes) { return hipMalloc(&p, bytes < 256 ? 256 : bytes) == hipSuccess; }
    ~Scratch() {
        if (p) {
            hipStreamSynchronize(s);
            hipFree(p);
        }
    }
};

q3_status st(hipError_t e) { return e == hipSuccess ? Q3_OK : Q3_ERR_HIP; }

}  // namespace

extern "C" q3_status q3_op_rmsnorm(const float* x, const float* w, void* out, int32_t out_dtype, int32_t rows,
                                   int32_t d, float eps, void* stream) {
    if (!x || !w || !out || rows < 0 || d <= 0 || (out_dtype != Q3_F32 && out_dtype != Q3_BF16 && out_dtype != Q3_OP_PAIR))
        return Q3_ERR_ARG;
    return st(launch_rmsnorm(const_cast<float*>(x), w, out, out_dtype == Q3_F32 ? 0 : (out_dtype == Q3_BF16 ? 1 : 2), rows, d, eps,
                             (hipStream_t)stream));
}

extern "C" q3_status q3_op_gemv(const void* W, int32_t w_dtype, const float* x, float* y, int32_t N, int32_t K,
                                int32_t B, int32_t epilogue, void* stream) {
    if (!W || !x || !y || N <= 0 || K <= 0 || B < 0 || (w_dtype != Q3_F32 && w_dtype != Q3_BF16)) return Q3_ERR_ARG;
    if (K % 8 || N % 2 || epilogue < 0 || epilogue > 2) return Q3_ERR_SHAPE;
    if (epilogue == GEMV_SWIGLU && N % 32) return Q3_ERR_SHAPE;
    return st(launch_gemv(W, w_dtype == Q3_BF16 ? DT_BF16 : DT_F32, x, y, N, K, B, epilogue, (hipStream_t)stream));
}

extern "C" q3_status q3_op_gemm(const void* A, int32_t a_dtype, const uint16_t* W, void* C, int32_t M, int32_t N,
                                int32_t K, int32_t epilogue, int32_t splits, const float* colscale,
                                void* stream) {
    if (!A || !W || !C || M < 0 || N <= 0 || K <= 0 || epilogue < 0 || epilogue > 5 ||
        (a_dtype != Q3_F32 && a_dtype != Q3_BF16 && a_dtype != Q3_OP_PAIR))
        return Q3_ERR_ARG;
    if (N % 128 || K % 64) return Q3_ERR_SHAPE;
    if (splits < 1 || splits > K / 64 || (splits > 1 && epilogue != GEMM_PARTIAL_F32)) return Q3_ERR_ARG;
    const int mode = a_dtype == Q3_F32 ? GEMM_A_F32 : (a_dtype == Q3_BF16 ? GEMM_A_BF16 : GEMM_A_PAIR);
    return st(launch_gemm(A, mode, W, C, M, N, K, epilogue, (hipStream_t)stream, splits, colscale));
}

extern "C" q3_status q3_op_qk_norm_rope(const float* qkv, const float* q_norm, const float* k_norm,
                                        const int32_t* positions, const int32_t* slots, int32_t B, int32_t n_heads,
                                        int32_t n_kv_heads, float eps, float rope_theta, float* q_out,
                                        void* k_cache, void* v_cache, int32_t kv_dtype, int32_t t_cap,
                                        void* stream) {
    if (!qkv || !q_norm || !k_norm || !positions || !slots || !q_out || !k_cache || !v_cache || B < 0 ||
        n_heads <= 0 || n_kv_heads <= 0 || t_cap <= 0 || (kv_dtype != Q3_F32 && kv_dtype != Q3_BF16))
        return Q3_ERR_ARG;
    hipStream_t s = (hipStream_t)stream;
    std::vector<float> f(64);
    for (int i = 0; i < 64; ++i) f[i] = (float)std::pow((double)rope_theta, -(double)i / 64);
    Scratch sc(s);
    if (!sc.get(64 * sizeof(float))) return Q3_ERR_OOM;
    if (hipMemcpyAsync(sc.p, f.data(), 64 * sizeof(float), hipMemcpyHostToDevice, s) != hipSuccess) return Q3_ERR_HIP;
    return st(launch_qk_rope_decode(qkv, positions, slots, 0, B, q_norm, k_norm, (const float*)sc.p, eps, q_out,
                                    k_cache, v_cache, kv_dtype == Q3_BF16, t_cap, kv_contiguous(n_kv_heads, t_cap), n_heads,
                                    n_kv_heads, s));
}

extern "C" q3_status q3_op_attn_decode(const float* q, const void* k_cache, const void* v_cache, int32_t kv_dtype,
                                       int32_t t_cap, const int32_t* lens, int32_t B, int32_t n_heads,
                                       int32_t n_kv_heads, int32_t max_len, float* o, void* stream) {
    if (!q || !k_cache || !v_cache || !lens || !o || B < 0 || t_cap <= 0 || max_len < 1 || max_len > t_cap ||
        (kv_dtype != Q3_F32 && kv_dtype != Q3_BF16))
        return Q3_ERR_ARG;
    if (n_heads != 2 * n_kv_heads) return Q3_ERR_SHAPE;
    hipStream_t s = (hipStream_t)stream;
    Scratch sc(s);
    if (!sc.get(attn_decode_workspace_bytes(B, n_kv_heads, max_len))) return Q3_ERR_OOM;
    return st(launch_attn_decode(q, k_cache, v_cache, kv_dtype == Q3_BF16, t_cap, kv_contiguous(n_kv_heads, t_cap), lens,
                                 0, 0, B, n_heads,
                                 n_kv_heads, max_len, (float*)sc.p, o, 0, s));
}

extern "C" q3_status q3_op_attn_prefill(const float* q, const uint16_t* k_cache, const uint16_t* v_cache,
                                        int32_t t_cap, int32_t M, int32_t t0, int32_t n_heads, int32_t n_kv_heads,
                                        void* o, int32_t o_dtype, void* stream) {
    if (!q || !k_cache || !v_cache || !o || M < 0 || t0 < 0 || t_cap <= 0 || (int64_t)t0 + M > t_cap ||
        (o_dtype != Q3_F32 && o_dtype != Q3_OP_PAIR))
        return Q3_ERR_ARG;
    if (n_heads != 2 * n_kv_heads) return Q3_ERR_SHAPE;
    return st(launch_attn_prefill(q, k_cache, v_cache, kv_contiguous(n_kv_heads, t_cap), 0, M, t0, n_heads, n_kv_heads, o,
                                  o_dtype == Q3_OP_PAIR,
                                  (hipStream_t)stream));
}

extern "C" q3_status q3_op_sample(const float* logits, int32_t B, int32_t V, float temperature, float top_p,
                                  const float* uniforms, int32_t* tokens_out, void* stream) {
    if (!logits || !tokens_out || B < 0 || V <= 0 || !(temperature >= 0.f)) return Q3_ERR_ARG;
    if (temperature > 0.f && !uniforms) return Q3_ERR_ARG;
    if (B == 0) return Q3_OK;
    hipStream_t s = (hipStream_t)stream;
    Scratch sc(s);
    const size_t amax_bytes = (size_t)B * 8;
    if (!sc.get(amax_bytes + sample_workspace_bytes(V, B) + 256)) return Q3_ERR_OOM;
    unsigned long long* amax = (unsigned long long*)sc.p;
    unsigned* err = (unsigned*)((char*)sc.p + amax_bytes);
    void* ws = (char*)sc.p + amax_bytes + 256;
    hipError_t e = hipMemsetAsync(err, 0, 4, s);
    if (e == hipSuccess) e = launch_argmax_rows(logits, amax, V, B, err, s);
    if (e == hipSuccess) e = launch_sample(logits, amax, V, B, temperature, top_p, uniforms, tokens_out, ws, false, s);
    return st(e);
}

// ---------------------------------------------------------------------------------
// Sampling without allocation: the same kernels as q3_op_sample, with their scratch
// (per-row argmax words, an error word, the per-row selection workspace) in a file-scope
// device array instead of memory allocated per call. Each GPU the library runs on holds
// its own copy of the array, at its own address, until the process ends.
// ---------------------------------------------------------------------------------
namespace {

constexpr int kNoAllocRows = Q3_SAMPLE_NOALLOC_MAX_ROWS;
constexpr int kNoAllocVocab = Q3_SAMPLE_NOALLOC_MAX_VOCAB;
constexpr size_t kNoAllocHeader = 256;   // [0, 32): argmax word per row; [32, 40): error word
// Selection workspace per row: a 65,536-bucket histogram, 264 words of group sums and state,
// and one word per vocabulary entry (the sampler's layout; checked against
// sample_workspace_bytes at every call).
constexpr size_t kNoAllocWsBytes = (size_t)kNoAllocRows * (65536 + 264 + (size_t)kNoAllocVocab) * 8;
constexpr size_t kNoAllocBytes = kNoAllocHeader + kNoAllocWsBytes;
static_assert(kNoAllocRows * 8 <= 32, "argmax words fit the header");

static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};   // device address of `scratch` on each device

// Device address of this device's copy of `scratch`; looked up once per device, with that
// device current (in host code the array's name is only a stand-in, never an address).
q3_status scratch_address(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return Q3_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return Q3_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return Q3_OK;
}

}  // namespace

extern "C" q3_status q3_op_sample_noalloc(const float* logits, int32_t B, int32_t V, float temperature, float top_p,
                                          const float* uniforms, int32_t* tokens_out, void* stream) {
    if (!logits || !tokens_out || B < 0 || V <= 0 || !(temperature >= 0.f)) return Q3_ERR_ARG;
    if (temperature > 0.f && !uniforms) return Q3_ERR_ARG;
    if (B > kNoAllocRows || V > kNoAllocVocab || sample_workspace_bytes(V, B) > kNoAllocWsBytes)
        return Q3_ERR_SHAPE;
    if (B == 0) return Q3_OK;
    void* base = nullptr;
    if (q3_status s0 = scratch_address(&base); s0 != Q3_OK) return s0;
    hipStream_t s = (hipStream_t)stream;
    unsigned long long* amax = (unsigned long long*)base;
    unsigned long long* err = (unsigned long long*)((char*)base + 32);
    void* ws = (char*)base + kNoAllocHeader;
    // the error word starts at zero (a fill kernel, not a memset: safe under graph capture);
    // the selection workspace is cleared by launch_sample itself (ws_zeroed = false), and
    // launch_argmax_rows clears the argmax words
    hipError_t e = launch_fill_u64(err, 0ull, 1, s);
    if (e == hipSuccess) e = launch_argmax_rows(logits, amax, V, B, (unsigned*)err, s);
    if (e == hipSuccess) e = launch_sample(logits, amax, V, B, temperature, top_p, uniforms, tokens_out, ws, false, s);
    return st(e);
}
