// q3 engine: device weight store, KV cache, workspaces and the launch plans of prefill
// and decode, behind the C ABI of include/q3.h.
//
// Pipeline ("Inside an LLM: Pure Python Inference for Qwen3-0.6B on MLX", "The
// pipeline at a glance" and Steps 2-9): embed -> n_layers x [RMSNorm -> Q/K/V ->
// QK-norm -> RoPE -> KV append -> GQA attention -> o_proj + residual -> RMSNorm ->
// SwiGLU FFN + residual] -> final RMSNorm -> tied LM head -> sampling.
//
// Precision plan: decode rows keep float32 activations (bf16 or float32 weights, float32
// accumulation). Prefill of a long prompt runs its rows through the matrix-core path:
// float32 activations enter every MFMA product as a bf16 hi + lo pair (two MFMAs; the
// bf16 weights and the bf16 K/V cache are exact operands), so the path keeps ~16
// significant bits where a single bf16 rounding would cost ~5e-3 relative error in the
// logits. The last row's last layer after its K/V append, and its LM head, run on the
// single-row float32 kernels (with int8 or int4 weights the last row takes the decode path).
#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <unordered_map>
#include <vector>

#include "common.h"
#include "kernels.h"
#include "q3.h"

using namespace q3;

namespace {
constexpr int kPrefillMfmaMin = 16;   // prompts shorter than this run row by row
constexpr int kPrefillSplitRows = 8192;   // prefill below this many rows: split-K O / down projections
constexpr int kPrefillSplits = 4;         // at most this many K splits there
}

struct q3_engine {
    q3_config cfg{};
    hipStream_t stream = nullptr;
    int device = 0;
    std::string err = "ok";
    std::vector<void*> allocs;

    struct Layer {
        void *wqkv, *wo, *wgu, *wd;       // bf16 (or float32) matrices; int8 / int4 engines: the codes as bf16
        float *in_norm, *post_norm, *q_norm, *k_norm;
        uint8_t *wqkv8 = nullptr, *wo8 = nullptr, *wgu8 = nullptr, *wd8 = nullptr;   // int8 / int4: the codes (+ row scales)
        float *sqkv = nullptr, *so = nullptr, *sgu = nullptr, *sd = nullptr;          // int8 / int4: row scales
    };
    void* embed = nullptr;
    uint8_t* embed8 = nullptr;     // int8 / int4: embedding codes and row scales
    float* escale = nullptr;
    std::vector<Layer> layers;
    float* final_norm = nullptr;
    float* inv_freq = nullptr;

    // KV cache: a pool of pages, page = kKvPage token slots of every layer and kv head,
    // stored layer-major, [layer][page][kv head][slot][head_dim] in each of kc, vc (one
    // layer's cache is one region, as the kernels of a layer stream it). A sequence's page
    // table row lists its pages in slot order; a page held by several sequences
    // (q3_kv_fork) is copied by the first one that writes into it.
    void* kc = nullptr;
    void* vc = nullptr;
    size_t kv_layer_elems = 0;     // one layer's region (every page)
    size_t page_elems = 0;         // one page within a layer
    int n_pages = 0, max_pages = 0;                // pool size; table entries per sequence
    int32_t* d_pt = nullptr;                       // page table [max_batch][max_pages]
    std::vector<int32_t> h_pt;                     // its host copy
    std::vector<int32_t> h_npages;                 // pages each sequence holds
    std::vector<int32_t> refs;                     // sequences holding each page
    std::vector<int32_t> free_pages;
    void* kv_dense = nullptr;                      // staging for q3_kv_import / q3_kv_export
    size_t kv_dense_bytes = 0;
    KvLayout layout() const { return KvLayout{d_pt, max_pages, page_elems, (size_t)kKvPage * 128}; }
    int32_t* d_len = nullptr;
    std::vector<int32_t> h_len;
    unsigned* d_err = nullptr;

    // decode workspace (max_batch rows)
    float *x = nullptr, *h = nullptr, *qkv = nullptr, *q = nullptr, *o = nullptr, *a = nullptr;
    float* logits = nullptr;
    unsigned long long* amax = nullptr;
    float* attn_ws = nullptr;
    float* parts = nullptr;        // split-K partial products of the batched decode projections
    static constexpr int kMaxSplits = 32;
    int attn_ws_T = 0;
    void* sample_ws = nullptr;
    const float* cur_logits = nullptr;
    int cur_rows = 0;

    // event timing of one kernel family (q3_profile_begin / q3_profile_end)
    struct Prof {
        int kind = -1;
        std::vector<hipEvent_t> ev;   // pairs (start, stop)
        size_t used = 0;
        double bytes = 0, flops = 0;
        int64_t launches = 0;
    } prof;

    // persistent decode kernel state (decode_mega.hip)
    bool mega_ok = false;          // shape supported and co-residency possible
    int decode_path = 0;           // 0 auto, 1 per-kernel launches, 2 persistent kernel, 3 auto with ordinary launch
    MegaLayer* d_layers = nullptr;
    float* m_ex = nullptr;                   // exchange words, (n_layers + 1) layers
    size_t m_ex_layer = 0;
    unsigned long long* m_cand = nullptr;    // per-workgroup argmax candidates
    // The tail of the last persistent launch is deferred to the next call, so that a greedy
    // q3_sample right after it is the same launch.
    bool tail_pending = false;
    int tail_B = 0, tail_seq_base = 0, tail_chunks = 0;
    int tail_nout = 0, tail_causal = 0;      // rows with the LM head; rows of one sequence
    unsigned long long* m_trace = nullptr;   // caller's device buffer for phase timestamps
    int m_trace_n = 0;

    // prefill workspace (grown on demand)
    int pf_cap = 0;
    float* pf_parts = nullptr;     // split-K partials of the prefill O / down projections (short prompts)
    float *pf_x = nullptr, *pf_qkv = nullptr, *pf_h = nullptr, *pf_q = nullptr, *pf_o = nullptr,
          *pf_a = nullptr;

    bool i8() const { return cfg.weight_dtype == Q3_I8; }
    bool i4() const { return cfg.weight_dtype == Q3_I4; }
    bool quant() const { return i8() || i4(); }   // weight-only int8 or int4
    // bytes per weight a decode step streams (int8 / int4: the codes; their row scales are
    // counted apart)
    double wbytes() const {
        return cfg.weight_dtype == Q3_F32 ? 4.0 : cfg.weight_dtype == Q3_BF16 ? 2.0 : cfg.weight_dtype == Q3_I8 ? 1.0 : 0.5;
    }
    size_t kvbytes() const { return cfg.kv_dtype == Q3_BF16 ? 2 : 4; }
    int qkv_rows() const { return (cfg.n_heads + 2 * cfg.n_kv_heads) * cfg.head_dim; }

    q3_status fail(q3_status st, const std::string& msg) {
        err = msg;
        return st;
    }
    bool hip_ok(hipError_t e, const char* what) {
        if (e == hipSuccess) return true;
        err = std::string(what) + ": " + hipGetErrorString(e);
        return false;
    }
    void* alloc(size_t bytes) {
        void* p = nullptr;
        if (hipMalloc(&p, bytes < 256 ? 256 : bytes) != hipSuccess) return nullptr;
        allocs.push_back(p);
        return p;
    }
    void release(void* p) {
        for (auto& q : allocs)
            if (q == p) { hipFree(q); q = nullptr; }
    }
};

// Record an event pair around one launch of the profiled kernel family.
static void prof_mark(q3_engine* e, int kind, bool start, double bytes = 0, double flops = 0) {
    auto& p = e->prof;
    if (p.kind != kind) return;
    if (start) {
        while (p.ev.size() < p.used + 2) {
            hipEvent_t ev;
            if (hipEventCreate(&ev) != hipSuccess) return;
            p.ev.push_back(ev);
        }
        hipEventRecord(p.ev[p.used], e->stream);
        p.bytes += bytes;
        p.flops += flops;
        p.launches += 1;
    } else {
        hipEventRecord(p.ev[p.used + 1], e->stream);
        p.used += 2;
    }
}

#define HIPCHK(e, call)                                              \
    do {                                                             \
        if (!(e)->hip_ok((call), #call)) return Q3_ERR_HIP;          \
    } while (0)

// ---------------------------------------------------------------------------------
// load
// ---------------------------------------------------------------------------------

namespace {

bool is_norm(const std::string& leaf) {
    return leaf == "input_layernorm" || leaf == "post_attention_layernorm" || leaf == "q_norm" ||
           leaf == "k_norm" || leaf == "norm";
}

std::vector<float> to_f32(const q3_tensor& t) {
    std::vector<float> out((size_t)t.numel);
    if (t.dtype == Q3_F32) {
        memcpy(out.data(), t.data, (size_t)t.numel * 4);
    } else {
        const uint16_t* s = (const uint16_t*)t.data;
        for (int64_t i = 0; i < t.numel; ++i) {
            uint32_t u = (uint32_t)s[i] << 16;
            memcpy(&out[i], &u, 4);
        }
    }
    return out;
}

}  // namespace

// Weight-only rule of one row (q3_quantize_i8, Q = 127; q3_quantize_i4, Q = 7):
// s = fl32(max |w| / Q), q = round half to even of fl32(w / s), clamped to [-Q, Q]; an
// all-zero row gives s = 0, q = 0. Every step is one IEEE float32 operation (no
// contraction), so any implementation agrees.
static void quantize_row(const float* w, int64_t n, int qmax, int8_t* q, float* s) {
    float amax = 0.f;
    for (int64_t k = 0; k < n; ++k) amax = std::max(amax, std::fabs(w[k]));
    const float fq = (float)qmax;
    const float sc = amax / fq;
    *s = sc;
    for (int64_t k = 0; k < n; ++k) {
        float r = sc > 0.f ? std::nearbyint(w[k] / sc) : 0.f;
        r = std::min(fq, std::max(-fq, r));
        q[k] = (int8_t)r;
    }
}

static q3_status quantize_matrix(const void* w, int32_t dtype, int64_t rows, int64_t cols, int qmax, int8_t* q,
                                 float* scale) {
    if (!w || !q || !scale || rows < 0 || cols <= 0 || (dtype != Q3_F32 && dtype != Q3_BF16)) return Q3_ERR_ARG;
    std::vector<float> row((size_t)cols);
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t k = 0; k < cols; ++k) {
            if (dtype == Q3_F32) {
                row[k] = ((const float*)w)[r * cols + k];
            } else {
                const uint32_t bits = (uint32_t)((const uint16_t*)w)[r * cols + k] << 16;
                memcpy(&row[k], &bits, 4);
            }
        }
        quantize_row(row.data(), cols, qmax, q + r * cols, scale + r);
    }
    return Q3_OK;
}

extern "C" q3_status q3_quantize_i8(const void* w, int32_t dtype, int64_t rows, int64_t cols, int8_t* q,
                                    float* scale) {
    return quantize_matrix(w, dtype, rows, cols, 127, q, scale);
}

extern "C" q3_status q3_quantize_i4(const void* w, int32_t dtype, int64_t rows, int64_t cols, int8_t* q,
                                    float* scale) {
    return quantize_matrix(w, dtype, rows, cols, 7, q, scale);
}

static_assert(kMegaMaxSlots == 270336, "the int8 / int4 limit quoted below");
static q3_status validate_config(const q3_config* c, std::string& why) {
    if (!c) { why = "config is NULL"; return Q3_ERR_ARG; }
    if (c->n_layers < 0 || c->hidden <= 0 || c->n_heads <= 0 || c->n_kv_heads <= 0 || c->ffn <= 0 ||
        c->vocab <= 0 || c->max_batch <= 0 || c->max_seq <= 0) { why = "non-positive size in config"; return Q3_ERR_ARG; }
    if (c->head_dim != 128) { why = "head_dim must be 128"; return Q3_ERR_ARG; }
    if (c->n_heads != 2 * c->n_kv_heads) { why = "n_heads must be 2 * n_kv_heads"; return Q3_ERR_ARG; }
    if (c->hidden % 128 || c->ffn % 128 || (c->n_heads * 128) % 128) { why = "hidden and ffn must be multiples of 128"; return Q3_ERR_ARG; }
    if (c->vocab % 2) { why = "vocab must be even"; return Q3_ERR_ARG; }
    if (c->tie_embeddings != 1) { why = "only a tied LM head is supported"; return Q3_ERR_ARG; }
    if ((c->weight_dtype != Q3_F32 && c->weight_dtype != Q3_BF16 && c->weight_dtype != Q3_I8 &&
         c->weight_dtype != Q3_I4) ||
        (c->kv_dtype != Q3_F32 && c->kv_dtype != Q3_BF16)) { why = "bad dtype"; return Q3_ERR_ARG; }
    if ((c->weight_dtype == Q3_I8 || c->weight_dtype == Q3_I4) && (c->kv_dtype != Q3_BF16 || c->hidden != 1024 || c->n_heads != 16 ||
                                     c->n_kv_heads != 8 || c->ffn != 3072 || c->n_layers < 1 ||
                                     c->n_layers > kMegaMaxLayers || c->max_batch > kMegaMaxRows ||
                                     c->max_seq > kMegaMaxSlots)) {
        why = "int8 and int4 weights need the Qwen3-0.6B layer shape, a bf16 cache, at most 4 sequence slots "
              "and max_seq <= 270336";
        return Q3_ERR_ARG;
    }
    if (c->kv_pages < 0) { why = "kv_pages must be >= 0"; return Q3_ERR_ARG; }
    if ((int64_t)c->max_batch * ((c->max_seq + kKvPage - 1) / kKvPage) > INT32_MAX) {
        why = "max_batch * max_seq too large";
        return Q3_ERR_ARG;
    }
    if (!(c->rms_eps > 0.f) || !(c->rope_theta > 1.f)) { why = "bad rms_eps or rope_theta"; return Q3_ERR_ARG; }
    return Q3_OK;
}

extern "C" q3_status q3_load(const q3_config* cfg, const q3_tensor* weights, int32_t n_weights,
                             void* stream, q3_engine** out) {
    if (!out) return Q3_ERR_ARG;
    *out = nullptr;
    std::string why;
    q3_status st = validate_config(cfg, why);
    if (st != Q3_OK) return st;
    if (!weights || n_weights <= 0) return Q3_ERR_ARG;
    const q3_config& c = *cfg;
    std::unordered_map<std::string, const q3_tensor*> byname;
    for (int i = 0; i < n_weights; ++i) {
        if (!weights[i].name || !weights[i].data) return Q3_ERR_ARG;
        byname[weights[i].name] = &weights[i];
    }
    const int d = c.hidden, dh = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads, F = c.ffn, V = c.vocab;
    const bool i8 = c.weight_dtype == Q3_I8 || c.weight_dtype == Q3_I4;   // quantised weights
    const bool i4 = c.weight_dtype == Q3_I4;
    const size_t wb = c.weight_dtype == Q3_F32 ? 4 : 2;   // bytes per element of L.wqkv etc.

    auto need = [&](const std::string& name, int64_t numel, bool norm, const q3_tensor** t) -> q3_status {
        auto it = byname.find(name);
        if (it == byname.end()) return Q3_ERR_SHAPE;
        if (it->second->numel != numel) return Q3_ERR_SHAPE;
        if (!norm && !i8 && it->second->dtype != c.weight_dtype) return Q3_ERR_SHAPE;
        if (!norm && i8 && it->second->dtype != Q3_F32 && it->second->dtype != Q3_BF16) return Q3_ERR_SHAPE;
        if (norm && it->second->dtype != Q3_F32 && it->second->dtype != Q3_BF16) return Q3_ERR_SHAPE;
        *t = it->second;
        return Q3_OK;
    };
    // check every tensor before touching the device
    const q3_tensor* t;
    if ((st = need("model.embed_tokens.weight", (int64_t)V * d, false, &t)) != Q3_OK) return st;
    if ((st = need("model.norm.weight", d, true, &t)) != Q3_OK) return st;
    for (int l = 0; l < c.n_layers; ++l) {
        const std::string p = "model.layers." + std::to_string(l) + ".";
        if ((st = need(p + "input_layernorm.weight", d, true, &t)) != Q3_OK) return st;
        if ((st = need(p + "post_attention_layernorm.weight", d, true, &t)) != Q3_OK) return st;
        if ((st = need(p + "self_attn.q_norm.weight", dh, true, &t)) != Q3_OK) return st;
        if ((st = need(p + "self_attn.k_norm.weight", dh, true, &t)) != Q3_OK) return st;
        if ((st = need(p + "self_attn.q_proj.weight", (int64_t)Hq * dh * d, false, &t)) != Q3_OK) return st;
        if ((st = need(p + "self_attn.k_proj.weight", (int64_t)Hkv * dh * d, false, &t)) != Q3_OK) return st;
        if ((st = need(p + "self_attn.v_proj.weight", (int64_t)Hkv * dh * d, false, &t)) != Q3_OK) return st;
        if ((st = need(p + "self_attn.o_proj.weight", (int64_t)d * Hq * dh, false, &t)) != Q3_OK) return st;
        if ((st = need(p + "mlp.gate_proj.weight", (int64_t)F * d, false, &t)) != Q3_OK) return st;
        if ((st = need(p + "mlp.up_proj.weight", (int64_t)F * d, false, &t)) != Q3_OK) return st;
        if ((st = need(p + "mlp.down_proj.weight", (int64_t)d * F, false, &t)) != Q3_OK) return st;
    }

    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return Q3_ERR_HIP;

    q3_engine* e = new q3_engine();
    e->cfg = c;
    e->stream = (hipStream_t)stream;
    hipGetDevice(&e->device);
    auto oom = [&]() { q3_free(e); return Q3_ERR_OOM; };

    auto upload = [&](const void* src, size_t bytes) -> void* {
        void* p = e->alloc(bytes);
        if (p && hipMemcpy(p, src, bytes, hipMemcpyHostToDevice) != hipSuccess) return nullptr;
        return p;
    };
    auto upload_norm = [&](const std::string& name) -> float* {
        std::vector<float> f = to_f32(*byname[name]);
        return (float*)upload(f.data(), f.size() * 4);
    };

    // int8 / int4 weights: each matrix, its rows in the engine's packed order, quantised row
    // by row; uploaded as the codes (the persistent decode kernel: one byte each, or two
    // int4 codes per byte, code k in byte k / 2, the low nibble for even k), as the codes in
    // bf16 (exact: |q| <= 127; the prefill GEMMs, which apply the scale per output column)
    // and the scales
    auto quant_upload = [&](const std::vector<std::pair<const q3_tensor*, int64_t>>& rows, int cols, void** bf16q,
                            uint8_t** u8, float** sc) -> bool {
        const size_t R = rows.size();
        const size_t cbytes = i4 ? R * cols / 2 : R * cols;   // (cols is even)
        std::vector<uint16_t> hq(R * cols);
        std::vector<uint8_t> hu(cbytes, 0);
        std::vector<float> hs(R), rowf(cols);
        std::vector<int8_t> qrow(cols);
        for (size_t r = 0; r < R; ++r) {
            const q3_tensor* t = rows[r].first;
            const int64_t src = rows[r].second * cols;
            for (int k = 0; k < cols; ++k) {
                if (t->dtype == Q3_F32) {
                    rowf[k] = ((const float*)t->data)[src + k];
                } else {
                    const uint32_t bits = (uint32_t)((const uint16_t*)t->data)[src + k] << 16;
                    memcpy(&rowf[k], &bits, 4);
                }
            }
            quantize_row(rowf.data(), cols, i4 ? 7 : 127, qrow.data(), &hs[r]);
            for (int k = 0; k < cols; ++k) {
                const float f = (float)qrow[k];
                uint32_t b;
                memcpy(&b, &f, 4);
                hq[r * cols + k] = (uint16_t)(b >> 16);
                if (i4) {
                    const size_t at = r * cols + k;
                    hu[at / 2] |= (uint8_t)(((unsigned)qrow[k] & 0xFu) << (4 * (at & 1)));
                } else {
                    hu[r * cols + k] = (uint8_t)qrow[k];
                }
            }
        }
        // the persistent kernel's buffer: the codes, then the scales (it finds them at a fixed offset)
        hu.resize(cbytes + 4 * R);
        memcpy(hu.data() + cbytes, hs.data(), 4 * R);
        if (!(*bf16q = upload(hq.data(), hq.size() * 2)) || !(*u8 = (uint8_t*)upload(hu.data(), hu.size())))
            return false;
        *sc = (float*)(*u8 + cbytes);
        return true;
    };
    auto rows_of = [&](std::vector<std::pair<const q3_tensor*, int64_t>>& v, const std::string& name, int64_t r0,
                       int64_t n) {
        const q3_tensor* t = byname[name];
        for (int64_t r = r0; r < r0 + n; ++r) v.emplace_back(t, r);
    };
    if (i8) {
        std::vector<std::pair<const q3_tensor*, int64_t>> rows;
        rows_of(rows, "model.embed_tokens.weight", 0, V);
        if (!quant_upload(rows, d, &e->embed, &e->embed8, &e->escale)) return oom();
    } else {
        e->embed = upload(byname["model.embed_tokens.weight"]->data, (size_t)V * d * wb);
        if (!e->embed) return oom();
    }
    if (!(e->final_norm = upload_norm("model.norm.weight"))) return oom();
    e->layers.resize(c.n_layers);
    std::vector<uint8_t> buf;
    for (int l = 0; l < c.n_layers; ++l) {
        const std::string p = "model.layers." + std::to_string(l) + ".";
        auto& L = e->layers[l];
        if (i8) {
            std::vector<std::pair<const q3_tensor*, int64_t>> r;
            rows_of(r, p + "self_attn.q_proj.weight", 0, (int64_t)Hq * dh);
            rows_of(r, p + "self_attn.k_proj.weight", 0, (int64_t)Hkv * dh);
            rows_of(r, p + "self_attn.v_proj.weight", 0, (int64_t)Hkv * dh);
            if (!quant_upload(r, d, &L.wqkv, &L.wqkv8, &L.sqkv)) return oom();
            r.clear();
            rows_of(r, p + "self_attn.o_proj.weight", 0, d);
            if (!quant_upload(r, Hq * dh, &L.wo, &L.wo8, &L.so)) return oom();
            r.clear();
            for (int j = 0; j < F / 16; ++j) {          // gate/up packed as for bf16 weights
                rows_of(r, p + "mlp.gate_proj.weight", 16 * j, 16);
                rows_of(r, p + "mlp.up_proj.weight", 16 * j, 16);
            }
            if (!quant_upload(r, d, &L.wgu, &L.wgu8, &L.sgu)) return oom();
            r.clear();
            rows_of(r, p + "mlp.down_proj.weight", 0, d);
            if (!quant_upload(r, F, &L.wd, &L.wd8, &L.sd)) return oom();
            if (!(L.in_norm = upload_norm(p + "input_layernorm.weight"))) return oom();
            if (!(L.post_norm = upload_norm(p + "post_attention_layernorm.weight"))) return oom();
            if (!(L.q_norm = upload_norm(p + "self_attn.q_norm.weight"))) return oom();
            if (!(L.k_norm = upload_norm(p + "self_attn.k_norm.weight"))) return oom();
            continue;
        }
        // QKV packed as [q rows; k rows; v rows]
        const size_t qb = (size_t)Hq * dh * d * wb, kb = (size_t)Hkv * dh * d * wb;
        buf.resize(qb + 2 * kb);
        memcpy(buf.data(), byname[p + "self_attn.q_proj.weight"]->data, qb);
        memcpy(buf.data() + qb, byname[p + "self_attn.k_proj.weight"]->data, kb);
        memcpy(buf.data() + qb + kb, byname[p + "self_attn.v_proj.weight"]->data, kb);
        if (!(L.wqkv = upload(buf.data(), buf.size()))) return oom();
        if (!(L.wo = upload(byname[p + "self_attn.o_proj.weight"]->data, (size_t)d * Hq * dh * wb))) return oom();
        // gate/up interleaved in blocks of 16 rows: gate rows 16j..16j+15 then the same up rows
        const size_t rowb = (size_t)d * wb;
        buf.resize((size_t)2 * F * rowb);
        const uint8_t* g = (const uint8_t*)byname[p + "mlp.gate_proj.weight"]->data;
        const uint8_t* u = (const uint8_t*)byname[p + "mlp.up_proj.weight"]->data;
        for (int j = 0; j < F / 16; ++j) {
            memcpy(buf.data() + (size_t)(32 * j) * rowb, g + (size_t)(16 * j) * rowb, 16 * rowb);
            memcpy(buf.data() + (size_t)(32 * j + 16) * rowb, u + (size_t)(16 * j) * rowb, 16 * rowb);
        }
        if (!(L.wgu = upload(buf.data(), buf.size()))) return oom();
        if (!(L.wd = upload(byname[p + "mlp.down_proj.weight"]->data, (size_t)d * F * wb))) return oom();
        if (!(L.in_norm = upload_norm(p + "input_layernorm.weight"))) return oom();
        if (!(L.post_norm = upload_norm(p + "post_attention_layernorm.weight"))) return oom();
        if (!(L.q_norm = upload_norm(p + "self_attn.q_norm.weight"))) return oom();
        if (!(L.k_norm = upload_norm(p + "self_attn.k_norm.weight"))) return oom();
    }
    // RoPE frequencies f_i = theta^(-i/64), evaluated in double and rounded once to float
    {
        std::vector<float> f(dh / 2);
        for (int i = 0; i < dh / 2; ++i) f[i] = (float)std::pow((double)c.rope_theta, -(double)i / (dh / 2));
        if (!(e->inv_freq = (float*)upload(f.data(), f.size() * 4))) return oom();
    }
    // KV-cache page pool and page table
    e->max_pages = (c.max_seq + kKvPage - 1) / kKvPage;
    e->n_pages = c.kv_pages > 0 ? c.kv_pages : c.max_batch * e->max_pages;
    e->page_elems = (size_t)Hkv * kKvPage * dh;
    e->kv_layer_elems = e->page_elems * (size_t)e->n_pages;
    const size_t kvb = e->kv_layer_elems * (size_t)(c.n_layers > 0 ? c.n_layers : 1) * e->kvbytes();
    if (!(e->kc = e->alloc(kvb)) || !(e->vc = e->alloc(kvb))) return oom();
    const size_t ptn = (size_t)c.max_batch * e->max_pages;
    e->h_pt.assign(ptn, 0);       // entry 0 until a sequence holds the page: never read
    if (!(e->d_pt = (int32_t*)upload(e->h_pt.data(), ptn * 4))) return oom();
    e->h_npages.assign(c.max_batch, 0);
    e->refs.assign(e->n_pages, 0);
    e->free_pages.resize(e->n_pages);
    for (int i = 0; i < e->n_pages; ++i) e->free_pages[i] = e->n_pages - 1 - i;   // page 0 handed out first
    if (!(e->d_len = (int32_t*)e->alloc(sizeof(int32_t) * c.max_batch))) return oom();
    if (hipMemset(e->d_len, 0, sizeof(int32_t) * c.max_batch) != hipSuccess) { q3_free(e); return Q3_ERR_HIP; }
    e->h_len.assign(c.max_batch, 0);
    if (!(e->d_err = (unsigned*)e->alloc(sizeof(unsigned)))) return oom();
    if (hipMemset(e->d_err, 0, sizeof(unsigned)) != hipSuccess) { q3_free(e); return Q3_ERR_HIP; }
    // decode workspace
    const int B = c.max_batch;
    if (!(e->x = (float*)e->alloc((size_t)B * d * 4))) return oom();
    if (!(e->h = (float*)e->alloc((size_t)B * (d > F ? d : F) * 4))) return oom();
    if (!(e->qkv = (float*)e->alloc((size_t)B * e->qkv_rows() * 4))) return oom();
    if (!(e->q = (float*)e->alloc((size_t)B * Hq * dh * 4))) return oom();
    if (!(e->o = (float*)e->alloc((size_t)B * Hq * dh * 4))) return oom();
    if (!(e->a = (float*)e->alloc((size_t)B * F * 4))) return oom();
    if (!(e->logits = (float*)e->alloc((size_t)B * V * 4))) return oom();
    if (!(e->amax = (unsigned long long*)e->alloc((size_t)B * 8))) return oom();
    if (!(e->sample_ws = e->alloc(sample_workspace_bytes(V, B)))) return oom();
    if (B > 8 && !(e->parts = (float*)e->alloc((size_t)q3_engine::kMaxSplits * B * d * 4))) return oom();
    if (hipMemset(e->sample_ws, 0, sample_workspace_bytes(V, B)) != hipSuccess) { q3_free(e); return Q3_ERR_HIP; }
    e->attn_ws_T = c.max_seq;
    if (!(e->attn_ws = (float*)e->alloc(attn_decode_workspace_bytes(B, Hkv, c.max_seq)))) return oom();
    // persistent decode kernel: fixed layer shape, bf16 weights and cache, one workgroup per CU
    {
        hipDeviceProp_t prop;
        int occ = 0;
        const bool shape = d == 1024 && Hq == 16 && Hkv == 8 && dh == 128 && F == 3072 &&
                           (c.weight_dtype == Q3_BF16 || i8) && c.kv_dtype == Q3_BF16 && c.n_layers > 0 &&
                           c.n_layers <= kMegaMaxLayers;
        if (shape && hipGetDeviceProperties(&prop, e->device) == hipSuccess && prop.multiProcessorCount == 256) {
            if (decode_mega_prepare() == hipSuccess) e->mega_ok = true;
            else (void)hipGetLastError();   // not usable here: clear the error, use the per-operation path
        }
        (void)occ;
        if (i8 && !e->mega_ok) {
            q3_free(e);
            return Q3_ERR_HIP;     // int8 / int4 decode runs only in the persistent kernel (a 256-CU GPU)
        }
        if (e->mega_ok) {
            std::vector<MegaLayer> hl(c.n_layers);
            for (int l = 0; l < c.n_layers; ++l) {
                const auto& L = e->layers[l];
                // (int8 / int4: the matrix buffers of codes + scales)
                hl[l] = i8 ? MegaLayer{(const uint16_t*)L.wqkv8, (const uint16_t*)L.wo8, (const uint16_t*)L.wgu8,
                                       (const uint16_t*)L.wd8, L.in_norm, L.post_norm, L.q_norm, L.k_norm}
                           : MegaLayer{(const uint16_t*)L.wqkv, (const uint16_t*)L.wo, (const uint16_t*)L.wgu,
                                       (const uint16_t*)L.wd, L.in_norm, L.post_norm, L.q_norm, L.k_norm};
            }
            if (!(e->d_layers = (MegaLayer*)upload(hl.data(), hl.size() * sizeof(MegaLayer)))) return oom();
            e->m_ex_layer = decode_mega_exchange_words_per_layer();
            const size_t exw = ((size_t)c.n_layers + 1) * e->m_ex_layer;
            if (!(e->m_ex = (float*)e->alloc(exw * 4))) return oom();
            if (launch_mega_fill(e->m_ex, exw, e->stream) != hipSuccess) { q3_free(e); return Q3_ERR_HIP; }
            if (!(e->m_cand = (unsigned long long*)e->alloc((size_t)kMegaMaxRows * kMegaWorkgroups * 8))) return oom();
        }
    }
    if (hipDeviceSynchronize() != hipSuccess) { q3_free(e); return Q3_ERR_HIP; }
    *out = e;
    return Q3_OK;
}

extern "C" void q3_free(q3_engine* e) {
    if (!e) return;
    hipStreamSynchronize(e->stream);
    for (hipEvent_t ev : e->prof.ev) hipEventDestroy(ev);
    for (void* p : e->allocs)
        if (p) hipFree(p);
    delete e;
}

extern "C" const char* q3_last_error(const q3_engine* e) { return e ? e->err.c_str() : "engine is NULL"; }

extern "C" int32_t q3_seq_len(const q3_engine* e, int32_t seq) {
    if (!e || seq < 0 || seq >= e->cfg.max_batch) return -1;
    return e->h_len[seq];
}

// Launch the deferred tail of the last persistent decode launch (greedy_out: also write the
// greedy tokens of its rows).
static q3_status flush_tail(q3_engine* e, int32_t* greedy_out = nullptr) {
    if (!e->tail_pending) return Q3_OK;
    e->tail_pending = false;
    HIPCHK(e, launch_mega_tail(e->m_cand, e->amax, e->d_len, e->tail_seq_base, e->tail_B, e->m_ex, e->m_ex_layer,
                               e->cfg.n_layers, e->tail_chunks, greedy_out, e->stream, e->tail_nout, e->tail_causal));
    return Q3_OK;
}

// Algorithmic K/V bytes read by one decode step (all layers): 2 * Hkv * 128 * kv bytes per
// visible slot and layer.
static double kv_read_bytes(const q3_engine* e, int seq_base, int B) {
    const q3_config& c = e->cfg;
    double slots = 0;
    for (int b = 0; b < B; ++b) slots += e->h_len[seq_base + b] + 1;
    return slots * 2.0 * c.n_kv_heads * c.head_dim * e->kvbytes() * c.n_layers;
}

// Algorithmic bytes of one decode step: every weight once (the tied embedding counted once,
// as the LM head), norm weights, K/V reads and writes, embedding rows and logits.
static double step_bytes(const q3_engine* e, int seq_base, int B) {
    const q3_config& c = e->cfg;
    const double wb = e->wbytes();
    const double per_layer = (double)e->qkv_rows() * c.hidden + (double)c.hidden * c.n_heads * c.head_dim +
                             3.0 * c.ffn * c.hidden;
    double weights = wb * (per_layer * c.n_layers + (double)c.vocab * c.hidden);
    if (e->quant())             // the row scales (float32) of every matrix
        weights += 4.0 * ((double)(e->qkv_rows() + c.hidden + 2 * c.ffn + c.hidden) * c.n_layers + c.vocab);
    const double norms = 4.0 * (c.n_layers * (2.0 * c.hidden + 2.0 * c.head_dim) + c.hidden);
    const double kv_write = (double)B * c.n_layers * 2.0 * c.n_kv_heads * c.head_dim * e->kvbytes();
    const double rows = (double)B * (c.hidden * wb + 4.0 * c.vocab);
    return weights + norms + kv_read_bytes(e, seq_base, B) + kv_write + rows;
}

static double attn_prefill_flops(int M, int t0, int Hq) {
    // QK^T and PV over the visible slots: 2 * 2 * 128 flops per (row, slot, head)
    const double vis = (double)M * t0 + (double)M * (M + 1) / 2.0;
    return 4.0 * 128.0 * Hq * vis;
}

// ---------------------------------------------------------------------------------
// KV-cache pages
// ---------------------------------------------------------------------------------

// Page-table entries [first, first + n) of sequence seq (from the host copy) to the device,
// and the sequence's device length when len >= 0, in stream order (kernels, not copies).
static q3_status push_pages(q3_engine* e, int seq, int first, int n, int len = -1) {
    if (n <= 0 && len < 0) return Q3_OK;
    do {
        const int k = std::min(n, 64);
        HIPCHK(e, launch_set_pages(e->d_pt, e->max_pages, seq, first,
                                   e->h_pt.data() + (size_t)seq * e->max_pages + first, std::max(k, 0), e->d_len,
                                   len, e->stream));
        first += k;
        n -= k;
        len = -1;
    } while (n > 0);
    return Q3_OK;
}

// Slots of page p that sequence seq has written.
static int page_valid(const q3_engine* e, int seq, int p) {
    return std::max(0, std::min(kKvPage, e->h_len[seq] - p * kKvPage));
}

// Pages taken from the pool to make slots [slot0, slot0 + n) of seq writable.
static size_t pages_needed(const q3_engine* e, int seq, int slot0, int n) {
    if (n <= 0) return 0;
    const int32_t* row = e->h_pt.data() + (size_t)seq * e->max_pages;
    size_t need = 0;
    for (int p = std::min(slot0 / kKvPage, e->h_npages[seq]); p <= (slot0 + n - 1) / kKvPage; ++p)
        need += p >= e->h_npages[seq] || e->refs[row[p]] > 1;
    return need;
}

// Pages of seq from index `keep` on back to the pool (a page another sequence still holds
// stays with it).
static void release_pages(q3_engine* e, int seq, int keep) {
    const int32_t* row = e->h_pt.data() + (size_t)seq * e->max_pages;
    for (int p = keep; p < e->h_npages[seq]; ++p)
        if (--e->refs[row[p]] == 0) e->free_pages.push_back(row[p]);
    e->h_npages[seq] = std::min(e->h_npages[seq], keep);
}

// Make the pages of slots [slot0, slot0 + n) of seq present and held by seq alone: a missing
// page comes from the pool, a shared one is first copied (the slots seq has written, every
// layer) into a page of its own. All of them or none (Q3_ERR_CAPACITY).
static q3_status claim_pages(q3_engine* e, int seq, int slot0, int n) {
    if (n <= 0) return Q3_OK;
    if (pages_needed(e, seq, slot0, n) > e->free_pages.size())
        return e->fail(Q3_ERR_CAPACITY, "KV cache full: no free page in the pool");
    int32_t* row = e->h_pt.data() + (size_t)seq * e->max_pages;
    const int p1 = (slot0 + n - 1) / kKvPage;
    int lo = -1, hi = -1;
    for (int p = std::min(slot0 / kKvPage, e->h_npages[seq]); p <= p1; ++p) {
        const bool missing = p >= e->h_npages[seq];
        if (!missing && e->refs[row[p]] == 1) continue;
        const int32_t pg = e->free_pages.back();
        e->free_pages.pop_back();
        e->refs[pg] = 1;
        if (!missing) {      // copy on write
            --e->refs[row[p]];
            HIPCHK(e, launch_kv_page_copy(e->kc, e->vc, e->page_elems, e->kv_layer_elems, e->cfg.n_layers,
                                          e->cfg.n_kv_heads, (int)e->kvbytes(), row[p], pg, page_valid(e, seq, p),
                                          e->stream));
        }
        row[p] = pg;
        if (lo < 0) lo = p;
        hi = p;
    }
    e->h_npages[seq] = std::max(e->h_npages[seq], p1 + 1);
    return lo < 0 ? Q3_OK : push_pages(e, seq, lo, hi - lo + 1);
}

static q3_status ensure_kv_dense(q3_engine* e, size_t bytes) {
    if (bytes <= e->kv_dense_bytes) return Q3_OK;
    if (e->kv_dense) e->release(e->kv_dense);
    e->kv_dense = nullptr;
    e->kv_dense_bytes = 0;
    if (!(e->kv_dense = e->alloc(bytes))) return e->fail(Q3_ERR_OOM, "KV staging buffer allocation failed");
    e->kv_dense_bytes = bytes;
    return Q3_OK;
}

extern "C" int32_t q3_kv_free_pages(const q3_engine* e) { return e ? (int32_t)e->free_pages.size() : -1; }

// ---------------------------------------------------------------------------------
// decode rows (also the tail of a prefill)
// ---------------------------------------------------------------------------------

// Persistent-kernel parameters shared by every launch (rows' slots left to the caller).
static MegaParams mega_params(const q3_engine* e, const int32_t* tokens, const int32_t* positions, int seq_base,
                              int B, float* logits) {
    const q3_config& c = e->cfg;
    MegaParams mp{};
    mp.n_layers = c.n_layers;
    mp.vocab = c.vocab;
    mp.B = B;
    mp.seq_base = seq_base;
    mp.t_cap = c.max_seq;
    mp.causal = 0;
    mp.head_first = 0;
    mp.eps = c.rms_eps;
    mp.layers = e->d_layers;
    mp.embed = e->quant() ? (const uint16_t*)e->embed8 : (const uint16_t*)e->embed;
    mp.wq = e->i8() ? 1 : e->i4() ? 2 : 0;
    mp.final_norm = e->final_norm;
    mp.inv_freq = e->inv_freq;
    mp.kc = (uint16_t*)e->kc;
    mp.vc = (uint16_t*)e->vc;
    mp.kv_layer_elems = e->kv_layer_elems;
    mp.kv = e->layout();
    mp.tokens = tokens;
    mp.positions = positions;
    mp.ex = e->m_ex;
    mp.ex_layer = e->m_ex_layer;
    mp.logits = logits;
    mp.cand = e->m_cand;
    mp.err = e->d_err;
    mp.trace = e->m_trace;
    mp.trace_n = e->m_trace_n;
    return mp;
}

// A short prompt through the persistent kernel: up to kMegaMaxRows consecutive tokens of
// sequence `seq` in one launch, row b at slot len + b, each row attending the rows before
// it in the launch as well as the cache (Step 5's causal mask). With want_logits, the last
// row's logits go to logits_out (or the engine's buffer); otherwise the launch has no LM
// head at all.
static q3_status run_prefill_mega(q3_engine* e, int seq, const int32_t* tokens, int n, float* logits_out,
                                  bool want_logits) {
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    float* lg = logits_out ? logits_out : e->logits;
    MegaParams mp = mega_params(e, tokens, nullptr, seq, n, lg);
    mp.causal = 1;
    mp.head_first = want_logits ? n - 1 : n;
    for (int b = 0; b < n; ++b) mp.slots[b] = e->h_len[seq] + b;
    HIPCHK(e, launch_decode_mega(mp, e->decode_path != 3, e->stream));
    e->tail_pending = true;
    e->tail_B = n;
    e->tail_nout = want_logits ? 1 : 0;
    e->tail_causal = 1;
    e->tail_seq_base = seq;
    e->tail_chunks = 0;                 // the short-context instance writes no chunk partials
    if (want_logits) {
        e->cur_logits = lg;
        e->cur_rows = 1;
    }
    e->h_len[seq] += n;
    return Q3_OK;
}

static q3_status run_decode(q3_engine* e, const int32_t* tokens, const int32_t* positions,
                            int seq_base, int B, float* logits_out, bool want_logits) {
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;   // the previous launch's tail first
    const q3_config& c = e->cfg;
    const int d = c.hidden, Hq = c.n_heads, Hkv = c.n_kv_heads, F = c.ffn, V = c.vocab;
    const int wdt = c.weight_dtype == Q3_BF16 ? DT_BF16 : DT_F32;
    const int kvbf = c.kv_dtype == Q3_BF16;
    hipStream_t s = e->stream;
    int maxT = 0;
    for (int b = 0; b < B; ++b) maxT = std::max(maxT, e->h_len[seq_base + b] + 1);
    const double wb = e->wbytes();
    // the persistent kernel always computes the logits (into the engine's buffer when the
    // caller does not want them)
    const bool use_mega = e->mega_ok && B <= kMegaMaxRows && maxT <= kMegaMaxSlots && e->decode_path != 1;
    if (!use_mega && e->decode_path == 2) return e->fail(Q3_ERR_STATE, "persistent decode kernel not usable here");
    if (!use_mega && e->quant())
        return e->fail(Q3_ERR_STATE, "int8 / int4 weights: decode runs only in the persistent kernel (at most 4 rows)");
    if (use_mega) {
        float* lg = logits_out ? logits_out : e->logits;
        MegaParams mp = mega_params(e, tokens, positions, seq_base, B, lg);
        for (int b = 0; b < B; ++b) mp.slots[b] = e->h_len[seq_base + b];
        prof_mark(e, Q3_PROF_DECODE_STEP, true, step_bytes(e, seq_base, B), 0);
        HIPCHK(e, launch_decode_mega(mp, e->decode_path != 3, s));
        prof_mark(e, Q3_PROF_DECODE_STEP, false);
        e->tail_pending = true;
        e->tail_B = B;
        e->tail_nout = B;
        e->tail_causal = 0;
        e->tail_seq_base = seq_base;
        {
            int vis[kMegaMaxRows];
            for (int b = 0; b < B; ++b) vis[b] = mp.slots[b] + 1;
            e->tail_chunks = decode_mega_chunks(vis, B);
        }
        e->cur_logits = lg;
        e->cur_rows = B;
        for (int b = 0; b < B; ++b) e->h_len[seq_base + b] += 1;
        return Q3_OK;
    }
    // More rows than one GEMV pass takes (8): the projections and the LM head run on the
    // matrix cores, activations handed over as bf16 hi/lo pairs, so every weight is read
    // once per step instead of once per 8 rows.
    const int HD = Hq * 128;
    const bool mm = c.weight_dtype == Q3_BF16 && B > 8 && e->qkv_rows() % 128 == 0 && d % 128 == 0 &&
                    (2 * F) % 128 == 0 && V % 128 == 0 && d % 64 == 0 && HD % 64 == 0 && F % 64 == 0;
    const int nmode = mm ? 2 : 0;   // RMSNorm output: bf16 pairs for the matrix cores, else float32
    // The residual projections (o, down) of few rows are split along K over enough blocks to
    // fill the GPU; their partials are added to x by the next RMSNorm, in a fixed order.
    // Split counts: enough blocks (>= 256) along K for each projection, within K / 64 and
    // the partials workspace (kMaxSplits x rows x hidden floats).
    int split = 1, split_qkv = 1, split_gu = 1, pending = 0;
    if (mm) {
        const int mblocks = (B + 63) / 64;
        auto pick = [&](int N, int K, int target = 256) {
            const int nb = (N / 128) * mblocks;
            int sp = std::max(1, (target + nb - 1) / nb);
            sp = std::min(sp, K / 64);
            while (sp > 1 && (size_t)sp * N > (size_t)q3_engine::kMaxSplits * d) --sp;
            return sp;
        };
        split = std::min(pick(d, HD, 128), pick(d, F, 128));
        split_qkv = pick(e->qkv_rows(), d);
        split_gu = pick(2 * F, d);
    }
    prof_mark(e, Q3_PROF_DECODE_STEP, true, step_bytes(e, seq_base, B), 0);
    HIPCHK(e, launch_embed(tokens, e->embed, wdt, e->x, B, d, V, e->d_err, s));
    for (int l = 0; l < c.n_layers; ++l) {
        const auto& L = e->layers[l];
        char* kcl = (char*)e->kc + (size_t)l * e->kv_layer_elems * e->kvbytes();
        char* vcl = (char*)e->vc + (size_t)l * e->kv_layer_elems * e->kvbytes();
        const KvLayout lay = e->layout();
        HIPCHK(e, launch_rmsnorm(e->x, L.in_norm, e->h, nmode, B, d, c.rms_eps, s, e->parts, pending));
        pending = 0;
        prof_mark(e, Q3_PROF_GEMV, true, wb * e->qkv_rows() * d + 4.0 * B * (d + e->qkv_rows()));
        if (mm && split_qkv > 1) {
            HIPCHK(e, launch_gemm(e->h, GEMM_A_PAIR, (const uint16_t*)L.wqkv, e->parts, B, e->qkv_rows(), d,
                                  GEMM_PARTIAL_F32, s, split_qkv));
        } else if (mm) {
            HIPCHK(e, launch_gemm(e->h, GEMM_A_PAIR, (const uint16_t*)L.wqkv, e->qkv, B, e->qkv_rows(), d, GEMM_F32, s));
        } else {
            HIPCHK(e, launch_gemv(L.wqkv, wdt, e->h, e->qkv, e->qkv_rows(), d, B, GEMV_STORE, s));
        }
        prof_mark(e, Q3_PROF_GEMV, false);
        HIPCHK(e, launch_qk_rope_decode(mm && split_qkv > 1 ? e->parts : e->qkv, positions, e->d_len, seq_base, B,
                                        L.q_norm, L.k_norm, e->inv_freq, c.rms_eps, e->q, kcl, vcl, kvbf, c.max_seq,
                                        lay, Hq, Hkv, s, mm ? split_qkv : 1));
        prof_mark(e, Q3_PROF_ATTN_DECODE, true, kv_read_bytes(e, seq_base, B) / c.n_layers);
        HIPCHK(e, launch_attn_decode(e->q, kcl, vcl, kvbf, c.max_seq, lay, e->d_len, 1, seq_base, B, Hq, Hkv,
                                     maxT, e->attn_ws, e->o, mm, s));
        prof_mark(e, Q3_PROF_ATTN_DECODE, false);
        prof_mark(e, Q3_PROF_GEMV, true, wb * d * HD + 4.0 * B * (HD + 2 * d));
        if (mm && split > 1) {
            HIPCHK(e, launch_gemm(e->o, GEMM_A_PAIR, (const uint16_t*)L.wo, e->parts, B, d, HD, GEMM_PARTIAL_F32, s, split));
            pending = split;
        } else if (mm) {
            HIPCHK(e, launch_gemm(e->o, GEMM_A_PAIR, (const uint16_t*)L.wo, e->x, B, d, HD, GEMM_RESID_F32, s));
        } else {
            HIPCHK(e, launch_gemv(L.wo, wdt, e->o, e->x, d, HD, B, GEMV_RESID, s));
        }
        prof_mark(e, Q3_PROF_GEMV, false);
        HIPCHK(e, launch_rmsnorm(e->x, L.post_norm, e->h, nmode, B, d, c.rms_eps, s, e->parts, pending));
        pending = 0;
        prof_mark(e, Q3_PROF_GEMV, true, wb * 2.0 * F * d + 4.0 * B * (d + F));
        if (mm && split_gu > 1) {
            HIPCHK(e, launch_gemm(e->h, GEMM_A_PAIR, (const uint16_t*)L.wgu, e->parts, B, 2 * F, d, GEMM_PARTIAL_F32, s,
                                  split_gu));
            HIPCHK(e, launch_swiglu_parts(e->parts, split_gu, B, F, e->a, s));
        } else if (mm) {
            HIPCHK(e, launch_gemm(e->h, GEMM_A_PAIR, (const uint16_t*)L.wgu, e->a, B, 2 * F, d, GEMM_SWIGLU_PAIR, s));
        } else {
            HIPCHK(e, launch_gemv(L.wgu, wdt, e->h, e->a, 2 * F, d, B, GEMV_SWIGLU, s));
        }
        prof_mark(e, Q3_PROF_GEMV, false);
        prof_mark(e, Q3_PROF_GEMV, true, wb * d * F + 4.0 * B * (F + 2 * d));
        if (mm && split > 1) {
            HIPCHK(e, launch_gemm(e->a, GEMM_A_PAIR, (const uint16_t*)L.wd, e->parts, B, d, F, GEMM_PARTIAL_F32, s, split));
            pending = split;
        } else if (mm) {
            HIPCHK(e, launch_gemm(e->a, GEMM_A_PAIR, (const uint16_t*)L.wd, e->x, B, d, F, GEMM_RESID_F32, s));
        } else {
            HIPCHK(e, launch_gemv(L.wd, wdt, e->a, e->x, d, F, B, GEMV_RESID, s));
        }
        prof_mark(e, Q3_PROF_GEMV, false);
    }
    if (pending && !want_logits) {   // x must be complete when the step ends
        HIPCHK(e, launch_rmsnorm(e->x, e->final_norm, e->h, nmode, B, d, c.rms_eps, s, e->parts, pending));
        pending = 0;
    }
    if (want_logits) {
        float* lg = logits_out ? logits_out : e->logits;
        HIPCHK(e, launch_rmsnorm(e->x, e->final_norm, e->h, nmode, B, d, c.rms_eps, s, e->parts, pending));
        pending = 0;
        prof_mark(e, Q3_PROF_LMHEAD, true, wb * V * d + 4.0 * B * (d + V));
        if (mm) {
            HIPCHK(e, launch_gemm(e->h, GEMM_A_PAIR, (const uint16_t*)e->embed, lg, B, V, d, GEMM_F32, s));
            HIPCHK(e, launch_argmax_rows(lg, e->amax, V, B, e->d_err, s));
        } else {
            HIPCHK(e, launch_fill_u64(e->amax, 0ull, B, s));
            HIPCHK(e, launch_lmhead(e->embed, wdt, e->h, lg, e->amax, V, d, B, e->d_err, s));
        }
        prof_mark(e, Q3_PROF_LMHEAD, false);
        e->cur_logits = lg;
        e->cur_rows = B;
    }
    HIPCHK(e, launch_len_advance(e->d_len, seq_base, B, 1, s));
    prof_mark(e, Q3_PROF_DECODE_STEP, false);
    for (int b = 0; b < B; ++b) e->h_len[seq_base + b] += 1;
    return Q3_OK;
}

static q3_status ensure_prefill_ws(q3_engine* e, int M) {
    if (M <= e->pf_cap) return Q3_OK;
    const q3_config& c = e->cfg;
    const int d = c.hidden, F = c.ffn, HD = c.n_heads * c.head_dim;
    for (void* p : {(void*)e->pf_x, (void*)e->pf_qkv, (void*)e->pf_h, (void*)e->pf_q, (void*)e->pf_o, (void*)e->pf_a,
                    (void*)e->pf_parts})
        if (p) e->release(p);
    e->pf_parts = nullptr;
    e->pf_cap = 0;
    if (!(e->pf_x = (float*)e->alloc((size_t)M * d * 4))) return Q3_ERR_OOM;
    if (!(e->pf_qkv = (float*)e->alloc((size_t)M * e->qkv_rows() * 4))) return Q3_ERR_OOM;
    // pf_h, pf_o, pf_a hold bf16 hi/lo pair rows (same bytes as float32)
    if (!(e->pf_h = (float*)e->alloc((size_t)M * d * 4))) return Q3_ERR_OOM;
    if (!(e->pf_q = (float*)e->alloc((size_t)M * HD * 4))) return Q3_ERR_OOM;
    if (!(e->pf_o = (float*)e->alloc((size_t)M * HD * 4))) return Q3_ERR_OOM;
    if (!(e->pf_a = (float*)e->alloc((size_t)M * F * 4))) return Q3_ERR_OOM;
    if (M < kPrefillSplitRows && !(e->pf_parts = (float*)e->alloc((size_t)kPrefillSplits * M * d * 4)))
        return Q3_ERR_OOM;
    e->pf_cap = M;
    return Q3_OK;
}

// Rows tokens[0..M) of sequence `seq` at slots t0 .. t0+M-1 through the matrix-core path.
// Only the last row's logits are wanted (Step 8 takes the last position), so the last
// layer stops after the K/V append of all rows: its attention, O projection and FFN feed
// nothing but the last row. With `logits` (bf16 weights) that row then finishes the last
// layer on the single-row kernels -- attention over the cache, O projection, RMSNorm,
// SwiGLU FFN, final RMSNorm and the LM head with its argmax -- in float32 activations;
// without, the caller runs the last prompt row through the decode path. Below kPrefillSplitRows rows
// the two hidden-width projections (N = 1024) would give too few 128-row tiles to fill the
// chip; they run split-K instead, and the next RMSNorm adds the partials to the residual
// in a fixed order.
static q3_status run_prefill_mfma(q3_engine* e, int seq, const int32_t* tokens, int M, float* logits = nullptr) {
    const q3_config& c = e->cfg;
    const int d = c.hidden, Hq = c.n_heads, Hkv = c.n_kv_heads, F = c.ffn, V = c.vocab;
    hipStream_t s = e->stream;
    q3_status st = ensure_prefill_ws(e, M);
    if (st != Q3_OK) return e->fail(st, "prefill workspace allocation failed");
    const int t0 = e->h_len[seq];
    HIPCHK(e, launch_embed(tokens, e->embed, DT_BF16, e->pf_x, M, d, V, e->d_err, s, e->escale));
    const bool sk = M < kPrefillSplitRows;
    const int split_o = sk ? std::min(kPrefillSplits, Hq * 128 / 512) : 1;
    const int split_d = sk ? std::min(kPrefillSplits, F / 512) : 1;
    int pending = 0;                                   // partials not yet added to pf_x
    for (int l = 0; l < c.n_layers; ++l) {
        const auto& L = e->layers[l];
        uint16_t* kcs = (uint16_t*)e->kc + (size_t)l * e->kv_layer_elems;
        uint16_t* vcs = (uint16_t*)e->vc + (size_t)l * e->kv_layer_elems;
        const KvLayout lay = e->layout();
        HIPCHK(e, launch_rmsnorm(e->pf_x, L.in_norm, e->pf_h, 2, M, d, c.rms_eps, s, e->pf_parts, pending));
        pending = 0;
        prof_mark(e, Q3_PROF_GEMM, true, 0, 2.0 * M * e->qkv_rows() * d);
        HIPCHK(e, launch_gemm(e->pf_h, GEMM_A_PAIR, (const uint16_t*)L.wqkv, e->pf_qkv, M, e->qkv_rows(), d,
                              GEMM_F32, s, 1, L.sqkv));
        prof_mark(e, Q3_PROF_GEMM, false);
        HIPCHK(e, launch_qk_rope_prefill(e->pf_qkv, M, t0, L.q_norm, L.k_norm, e->inv_freq, c.rms_eps,
                                         e->pf_q, kcs, vcs, lay, seq, Hq, Hkv, s));
        if (l + 1 == c.n_layers) {                    // the last layer's K/V are written
            if (!logits) break;
            // row M - 1 alone: its q gathered from the [Hq][M][128] prefill layout, attention
            // over its t0 + M visible slots (lens[seq] still holds t0), then the rest of the
            // layer and the LM head on that row of pf_x (complete: the input RMSNorm above
            // added every pending partial)
            const int HD = Hq * 128;
            float* xr = e->pf_x + (size_t)(M - 1) * d;
            HIPCHK(e, hipMemcpy2DAsync(e->q, 128 * sizeof(float), e->pf_q + (size_t)(M - 1) * 128,
                                       (size_t)M * 128 * sizeof(float), 128 * sizeof(float), Hq,
                                       hipMemcpyDeviceToDevice, s));
            HIPCHK(e, launch_attn_decode(e->q, kcs, vcs, 1, c.max_seq, lay, e->d_len, M, seq, 1, Hq, Hkv, t0 + M,
                                         e->attn_ws, e->o, 0, s));
            HIPCHK(e, launch_gemv(L.wo, DT_BF16, e->o, xr, d, HD, 1, GEMV_RESID, s));
            HIPCHK(e, launch_rmsnorm(xr, L.post_norm, e->h, 0, 1, d, c.rms_eps, s));
            HIPCHK(e, launch_gemv(L.wgu, DT_BF16, e->h, e->a, 2 * F, d, 1, GEMV_SWIGLU, s));
            HIPCHK(e, launch_gemv(L.wd, DT_BF16, e->a, xr, d, F, 1, GEMV_RESID, s));
            HIPCHK(e, launch_rmsnorm(xr, e->final_norm, e->h, 0, 1, d, c.rms_eps, s));
            HIPCHK(e, launch_fill_u64(e->amax, 0ull, 1, s));
            HIPCHK(e, launch_lmhead(e->embed, DT_BF16, e->h, logits, e->amax, V, d, 1, e->d_err, s));
            e->cur_logits = logits;
            e->cur_rows = 1;
            break;
        }
        prof_mark(e, Q3_PROF_ATTN_PREFILL, true, 0, attn_prefill_flops(M, t0, Hq));
        HIPCHK(e, launch_attn_prefill(e->pf_q, kcs, vcs, lay, seq, M, t0, Hq, Hkv, e->pf_o, 1, s));
        prof_mark(e, Q3_PROF_ATTN_PREFILL, false);
        prof_mark(e, Q3_PROF_GEMM, true, 0, 2.0 * M * d * Hq * 128);
        if (split_o > 1) {
            HIPCHK(e, launch_gemm(e->pf_o, GEMM_A_PAIR, (const uint16_t*)L.wo, e->pf_parts, M, d, Hq * 128,
                                  GEMM_PARTIAL_F32, s, split_o, L.so));
            pending = split_o;
        } else {
            HIPCHK(e, launch_gemm(e->pf_o, GEMM_A_PAIR, (const uint16_t*)L.wo, e->pf_x, M, d, Hq * 128, GEMM_RESID_F32, s,
                                  1, L.so));
        }
        prof_mark(e, Q3_PROF_GEMM, false);
        HIPCHK(e, launch_rmsnorm(e->pf_x, L.post_norm, e->pf_h, 2, M, d, c.rms_eps, s, e->pf_parts, pending));
        pending = 0;
        prof_mark(e, Q3_PROF_GEMM, true, 0, 2.0 * M * 2 * F * d);
        HIPCHK(e, launch_gemm(e->pf_h, GEMM_A_PAIR, (const uint16_t*)L.wgu, e->pf_a, M, 2 * F, d, GEMM_SWIGLU_PAIR, s,
                              1, L.sgu));
        prof_mark(e, Q3_PROF_GEMM, false);
        prof_mark(e, Q3_PROF_GEMM, true, 0, 2.0 * M * d * F);
        if (split_d > 1) {
            HIPCHK(e, launch_gemm(e->pf_a, GEMM_A_PAIR, (const uint16_t*)L.wd, e->pf_parts, M, d, F, GEMM_PARTIAL_F32, s,
                                  split_d, L.sd));
            pending = split_d;
        } else {
            HIPCHK(e, launch_gemm(e->pf_a, GEMM_A_PAIR, (const uint16_t*)L.wd, e->pf_x, M, d, F, GEMM_RESID_F32, s, 1,
                                  L.sd));
        }
        prof_mark(e, Q3_PROF_GEMM, false);
    }
    HIPCHK(e, launch_len_advance(e->d_len, seq, 1, M, s));
    e->h_len[seq] += M;
    return Q3_OK;
}

extern "C" q3_status q3_prefill(q3_engine* e, int32_t seq, const int32_t* tokens, int32_t n, float* logits) {
    if (!e) return Q3_ERR_ARG;
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    if (seq < 0 || seq >= e->cfg.max_batch) return e->fail(Q3_ERR_ARG, "seq out of range");
    if (!tokens || n < 1) return e->fail(Q3_ERR_ARG, "tokens is NULL or n < 1");
    if ((int64_t)e->h_len[seq] + n > e->cfg.max_seq) return e->fail(Q3_ERR_CAPACITY, "KV cache full");
    q3_status st = claim_pages(e, seq, e->h_len[seq], n);
    if (st != Q3_OK) return st;
    int done = 0;
    if (e->mega_ok && e->decode_path != 1 && n < kPrefillMfmaMin && e->h_len[seq] + n <= kMegaShortSlots) {
        // a short prompt: causal chunks of up to kMegaMaxRows rows per persistent launch, the
        // LM head only in the last one
        for (int i = 0; i < n; i += kMegaMaxRows) {
            const int cnt = std::min(kMegaMaxRows, n - i);
            if ((st = run_prefill_mega(e, seq, tokens + i, cnt, logits, i + cnt == n)) != Q3_OK) return st;
        }
        return Q3_OK;
    }
    if (e->cfg.weight_dtype == Q3_BF16 && e->cfg.kv_dtype == Q3_BF16 && n >= kPrefillMfmaMin) {
        // every row on the matrix cores, the last one finishing its last layer and the LM
        // head on the single-row kernels
        return run_prefill_mfma(e, seq, tokens, n, logits ? logits : e->logits);
    }
    if (e->quant() && e->cfg.kv_dtype == Q3_BF16 && n >= kPrefillMfmaMin) {
        // int8 / int4 weights (no single-row kernels for them): the last row through the decode path
        if ((st = run_prefill_mfma(e, seq, tokens, n - 1)) != Q3_OK) return st;
        done = n - 1;
    }
    for (int i = done; i < n; ++i) {
        if ((st = run_decode(e, tokens + i, nullptr, seq, 1, logits, i == n - 1)) != Q3_OK) return st;
    }
    return Q3_OK;
}

extern "C" q3_status q3_decode_step(q3_engine* e, const int32_t* tokens, const int32_t* positions,
                                    int32_t batch, float* logits) {
    if (!e) return Q3_ERR_ARG;
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    if (!tokens || batch < 1 || batch > e->cfg.max_batch) return e->fail(Q3_ERR_ARG, "bad tokens or batch");
    size_t need = 0;
    for (int b = 0; b < batch; ++b) {
        if (e->h_len[b] + 1 > e->cfg.max_seq) return e->fail(Q3_ERR_CAPACITY, "KV cache full");
        need += pages_needed(e, b, e->h_len[b], 1);
    }
    if (need > e->free_pages.size()) return e->fail(Q3_ERR_CAPACITY, "KV cache full: no free page in the pool");
    for (int b = 0; b < batch; ++b)
        if (q3_status st = claim_pages(e, b, e->h_len[b], 1); st != Q3_OK) return st;
    return run_decode(e, tokens, positions, 0, batch, logits, true);
}

extern "C" q3_status q3_sample(q3_engine* e, const float* logits, int32_t batch, float temperature,
                               float top_p, const float* uniforms, int32_t* tokens_out) {
    if (!e) return Q3_ERR_ARG;
    if (!tokens_out || batch < 1 || batch > e->cfg.max_batch) return e->fail(Q3_ERR_ARG, "bad output or batch");
    if (!(temperature >= 0.f)) return e->fail(Q3_ERR_ARG, "temperature must be >= 0");
    if (temperature > 0.f && !uniforms) return e->fail(Q3_ERR_ARG, "uniforms required when temperature > 0");
    const int V = e->cfg.vocab;
    if (e->tail_pending && temperature == 0.f && !logits && batch == e->tail_nout) {
        // greedy pick of the persistent launch's rows: fused into its tail
        return flush_tail(e, tokens_out);
    }
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    if (!logits) {
        if (!e->cur_logits || batch > e->cur_rows) return e->fail(Q3_ERR_STATE, "no current logits for that many rows");
        logits = e->cur_logits;
    } else {
        HIPCHK(e, launch_argmax_rows(logits, e->amax, V, batch, e->d_err, e->stream));
    }
    HIPCHK(e, launch_sample(logits, e->amax, V, batch, temperature, top_p, uniforms, tokens_out,
                            e->sample_ws, true, e->stream));
    return Q3_OK;
}

extern "C" q3_status q3_reset(q3_engine* e, int32_t seq) {
    if (!e) return Q3_ERR_ARG;
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    if (seq < 0 || seq >= e->cfg.max_batch) return e->fail(Q3_ERR_ARG, "seq out of range");
    release_pages(e, seq, 0);
    e->h_len[seq] = 0;
    return push_pages(e, seq, 0, 0, 0);
}

extern "C" q3_status q3_kv_import(q3_engine* e, int32_t seq, int32_t layer, const void* k, const void* v,
                                  int32_t len) {
    if (!e) return Q3_ERR_ARG;
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    const q3_config& c = e->cfg;
    if (seq < 0 || seq >= c.max_batch || layer < 0 || layer >= c.n_layers || !k || !v || len < 0)
        return e->fail(Q3_ERR_ARG, "bad kv_import arguments");
    if (len > c.max_seq) return e->fail(Q3_ERR_CAPACITY, "KV cache full");
    const int keep = (len + kKvPage - 1) / kKvPage;
    if (pages_needed(e, seq, 0, len) > e->free_pages.size())
        return e->fail(Q3_ERR_CAPACITY, "KV cache full: no free page in the pool");
    const size_t bytes = (size_t)c.n_kv_heads * len * c.head_dim * e->kvbytes();
    if (q3_status st = ensure_kv_dense(e, 2 * bytes); st != Q3_OK) return st;
    release_pages(e, seq, keep);
    if (q3_status st = claim_pages(e, seq, 0, len); st != Q3_OK) return st;
    char* dk = (char*)e->kv_dense;
    if (len > 0) {
        HIPCHK(e, hipMemcpyAsync(dk, k, bytes, hipMemcpyDefault, e->stream));
        HIPCHK(e, hipMemcpyAsync(dk + bytes, v, bytes, hipMemcpyDefault, e->stream));
        const size_t lo = (size_t)layer * e->kv_layer_elems * e->kvbytes();
        HIPCHK(e, launch_kv_dense((char*)e->kc + lo, (char*)e->vc + lo, e->layout(), seq, c.n_kv_heads,
                                  (int)e->kvbytes(), dk, dk + bytes, len, true, e->stream));
    }
    e->h_len[seq] = len;
    if (q3_status st = push_pages(e, seq, 0, 0, len); st != Q3_OK) return st;
    HIPCHK(e, hipStreamSynchronize(e->stream));
    return Q3_OK;
}

extern "C" q3_status q3_kv_fork(q3_engine* e, int32_t src, int32_t dst, int32_t len) {
    if (!e) return Q3_ERR_ARG;
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    const q3_config& c = e->cfg;
    if (src < 0 || src >= c.max_batch || dst < 0 || dst >= c.max_batch || src == dst || len < 0)
        return e->fail(Q3_ERR_ARG, "bad kv_fork arguments");
    if (len > e->h_len[src]) return e->fail(Q3_ERR_ARG, "kv_fork beyond the source sequence's length");
    release_pages(e, dst, 0);
    const int np = (len + kKvPage - 1) / kKvPage;
    for (int p = 0; p < np; ++p) {
        const int32_t pg = e->h_pt[(size_t)src * e->max_pages + p];
        e->h_pt[(size_t)dst * e->max_pages + p] = pg;
        ++e->refs[pg];
    }
    e->h_npages[dst] = np;
    e->h_len[dst] = len;
    return push_pages(e, dst, 0, np, len);
}

extern "C" q3_status q3_kv_export(q3_engine* e, int32_t seq, int32_t layer, void* k, void* v, int32_t len) {
    if (!e) return Q3_ERR_ARG;
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    const q3_config& c = e->cfg;
    if (seq < 0 || seq >= c.max_batch || layer < 0 || layer >= c.n_layers || !k || !v || len < 0)
        return e->fail(Q3_ERR_ARG, "bad kv_export arguments");
    if (len > e->h_len[seq]) return e->fail(Q3_ERR_ARG, "kv_export beyond the sequence's length");
    if (len == 0) return Q3_OK;
    const size_t bytes = (size_t)c.n_kv_heads * len * c.head_dim * e->kvbytes();
    if (q3_status st = ensure_kv_dense(e, 2 * bytes); st != Q3_OK) return st;
    char* dk = (char*)e->kv_dense;
    const size_t lo = (size_t)layer * e->kv_layer_elems * e->kvbytes();
    HIPCHK(e, launch_kv_dense((char*)e->kc + lo, (char*)e->vc + lo, e->layout(), seq, c.n_kv_heads,
                              (int)e->kvbytes(), dk, dk + bytes, len, false, e->stream));
    HIPCHK(e, hipMemcpyAsync(k, dk, bytes, hipMemcpyDefault, e->stream));
    HIPCHK(e, hipMemcpyAsync(v, dk + bytes, bytes, hipMemcpyDefault, e->stream));
    HIPCHK(e, hipStreamSynchronize(e->stream));
    return Q3_OK;
}

extern "C" q3_status q3_sync(q3_engine* e) {
    if (!e) return Q3_ERR_ARG;
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    HIPCHK(e, hipStreamSynchronize(e->stream));
    unsigned flags = 0, zero = 0;
    HIPCHK(e, hipMemcpyAsync(&flags, e->d_err, 4, hipMemcpyDeviceToHost, e->stream));
    HIPCHK(e, hipMemcpyAsync(e->d_err, &zero, 4, hipMemcpyHostToDevice, e->stream));
    HIPCHK(e, hipStreamSynchronize(e->stream));
    if (flags & Q3_DEVERR_SYNC) {
        // a wait timed out and every workgroup left the kernel. The tail kernel that follows
        // every launch has put the sentinel / zero back into the hand-over words, so later
        // launches start clean; the rows of that step are not: their lengths advanced while
        // the layers after the wait never appended K/V (q3.h asks the caller to reset them)
        return e->fail(Q3_ERR_HIP, "persistent decode kernel: a cross-workgroup wait timed out");
    }
    if (flags & Q3_DEVERR_TOKEN) return e->fail(Q3_ERR_TOKEN, "a token id outside [0, vocab) reached the device");
    if (flags & Q3_DEVERR_NONFINITE) return e->fail(Q3_ERR_NUMERIC, "non-finite logits");
    return Q3_OK;
}

extern "C" q3_status q3_profile_begin(q3_engine* e, int32_t kind) {
    if (!e) return Q3_ERR_ARG;
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    if (kind < Q3_PROF_OFF || kind > Q3_PROF_ATTN_PREFILL) return e->fail(Q3_ERR_ARG, "bad profile kind");
    HIPCHK(e, hipStreamSynchronize(e->stream));
    e->prof.kind = kind;
    e->prof.used = 0;
    e->prof.bytes = e->prof.flops = 0;
    e->prof.launches = 0;
    return Q3_OK;
}

extern "C" q3_status q3_profile_end(q3_engine* e, double* total_ms, int64_t* launches, double* bytes,
                                    double* flops) {
    if (!e) return Q3_ERR_ARG;
    if (q3_status st = flush_tail(e); st != Q3_OK) return st;
    HIPCHK(e, hipStreamSynchronize(e->stream));
    double ms = 0;
    for (size_t i = 0; i + 1 < e->prof.used; i += 2) {
        float t = 0;
        HIPCHK(e, hipEventElapsedTime(&t, e->prof.ev[i], e->prof.ev[i + 1]));
        ms += t;
    }
    if (total_ms) *total_ms = ms;
    if (launches) *launches = e->prof.launches;
    if (bytes) *bytes = e->prof.bytes;
    if (flops) *flops = e->prof.flops;
    e->prof.kind = -1;
    e->prof.used = 0;
    return Q3_OK;
}

extern "C" q3_status q3_set_decode_path(q3_engine* e, int32_t path) {
    if (!e) return Q3_ERR_ARG;
    if (path < 0 || path > 3) return e->fail(Q3_ERR_ARG, "decode path must be 0, 1, 2 or 3");
    if (path == 2 && !e->mega_ok) return e->fail(Q3_ERR_STATE, "persistent decode kernel not available for this model/GPU");
    if (path == 1 && e->quant()) return e->fail(Q3_ERR_STATE, "int8 / int4 weights: no per-operation decode path");
    e->decode_path = path;
    return Q3_OK;
}

extern "C" q3_status q3_profile_trace(q3_engine* e, unsigned long long* dev_out, int32_t n) {
    if (!e) return Q3_ERR_ARG;
    if (n < 0 || (n > 0 && !dev_out)) return e->fail(Q3_ERR_ARG, "bad trace buffer");
    e->m_trace = n > 0 ? dev_out : nullptr;
    e->m_trace_n = n;
    return Q3_OK;
}
