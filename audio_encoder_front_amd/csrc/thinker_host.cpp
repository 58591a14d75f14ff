// Host runtime of the audio splice + Qwen3 Thinker prefill behind the C ABI
// (qwenasr.cpp ARCHITECTURE.md, "Qwen3 Thinker decoder", "Prompt assembly
// and audio splice", "GGUF layout").  Weights are repacked once at create:
// q/k/v fused into one [(Hq + 2 Hkv) 128, hidden] matrix, gate and up
// interleaved in 16-row blocks for the fused SwiGLU epilogue, RMSNorm gains in
// fp32.  A prefill call plans the packed batch on the host (token -> embedding
// row or encoder state, positions, prompt boundaries, last rows), uploads the
// tables in one copy and enqueues the layer sequence.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/qa_encoder.h"
#include "qa_kernels.h"

#define QA_API extern "C" __attribute__((visibility("default")))

namespace {

using qa::bf16;

constexpr float kRmsEps = 1e-6f;          // rms_norm_eps is named on the page but not valued
constexpr double kRopeBase = 1e6;         // rope.freq_base
constexpr int kHeadDim = 128;             // key_length / value_length
constexpr int64_t kMaxPrompt = 65536;     // context_length
constexpr int64_t kMaxTokens = 1 << 20;   // packed tokens per call

void set_errf(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    qa::set_error_message(buf);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Element i of a host tensor given in the dims' dtype, as float (exact).
float elem(const void* p, int dtype, size_t i) {
    if (dtype == QA_DTYPE_F32) return static_cast<const float*>(p)[i];
    const uint32_t u = (uint32_t) static_cast<const uint16_t*>(p)[i] << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

struct LayerOff {
    size_t attn_norm, qkv, q_norm, k_norm, o, ffn_norm, gu, down;
};

}  // namespace

struct qa_thinker {
    qa_thinker_dims d{};
    int esize = 4;
    hipStream_t stream = nullptr;
    char* wbuf = nullptr;
    size_t embed = 0, out_norm = 0, zero = 0;
    std::vector<LayerOff> layers;
    char* ws = nullptr;
    size_t ws_size = 0;
    char* pinned = nullptr;
    size_t pinned_size = 0;
    float2* rope = nullptr;            // [rope_len][64] (cos, sin)
    int64_t rope_len = 0;

    template <typename P = void>
    P* W(size_t off) const { return reinterpret_cast<P*>(wbuf + off); }
};

namespace {

bool check_dims(const qa_thinker_dims* d) {
    if (!d) { set_errf("dims is NULL"); return false; }
    if (d->abi_version != QA_ABI_VERSION) {
        set_errf("abi_version %d does not match the library's %d", d->abi_version, QA_ABI_VERSION);
        return false;
    }
    if (d->head_dim != kHeadDim) { set_errf("head_dim must be 128"); return false; }
    if (d->hidden < 64 || d->hidden > 4096 || d->hidden % 64) { set_errf("hidden must be a multiple of 64 in 64..4096"); return false; }
    if (d->n_layers < 0) { set_errf("n_layers must be >= 0"); return false; }
    if (d->n_q_heads < 1 || d->n_kv_heads < 1 || d->n_q_heads % d->n_kv_heads || d->n_q_heads > 64) {
        set_errf("n_q_heads must be a multiple of n_kv_heads (1..64 heads)");
        return false;
    }
    if (d->ffn_dim < 16 || d->ffn_dim % 16 || d->ffn_dim > 65536) { set_errf("ffn_dim must be a multiple of 16 in 16..65536"); return false; }
    if (d->vocab < 1 || d->vocab > (1 << 24)) { set_errf("vocab must be in 1..2^24"); return false; }
    if (d->dtype != QA_DTYPE_F32 && d->dtype != QA_DTYPE_BF16) { set_errf("dtype must be QA_DTYPE_F32 or QA_DTYPE_BF16"); return false; }
    return true;
}

bool check_weights(const qa_thinker_weights* w, int L) {
    if (!w) { set_errf("weights is NULL"); return false; }
    if (!w->embed || !w->out_norm) { set_errf("embed / out_norm is NULL"); return false; }
    const void* const* arrs[] = {w->attn_norm, w->q_w, w->k_w, w->v_w, w->q_norm, w->k_norm, w->o_w, w->ffn_norm,
                                 w->gate_w, w->up_w, w->down_w};
    for (auto a : arrs) {
        if (L > 0 && !a) { set_errf("a per-layer weight array is NULL"); return false; }
        for (int l = 0; l < L; ++l)
            if (!a[l]) { set_errf("layer %d has a NULL weight pointer", l); return false; }
    }
    return true;
}

// Packs host tensors into one device buffer (256-byte aligned pieces).
struct Pack {
    std::vector<char> host;
    size_t reserve(size_t bytes) {
        const size_t off = align256(host.size());
        host.resize(off + bytes);
        return off;
    }
};

// Copies rows [r0, r0 + n) of a [*, cols] host matrix in the operand type.
void put_rows(Pack& pk, size_t off, size_t dst_row, const void* src, int dtype, int esize, size_t r0, size_t n,
              size_t cols) {
    char* dst = pk.host.data() + off + dst_row * cols * esize;
    const size_t se = dtype == QA_DTYPE_F32 ? 4 : 2;
    if ((int)se == esize) {
        memcpy(dst, static_cast<const char*>(src) + r0 * cols * se, n * cols * se);
    } else {   // never happens: weights arrive in the operand type
        for (size_t i = 0; i < n * cols; ++i) {
            const float v = elem(src, dtype, r0 * cols + i);
            memcpy(dst + i * esize, &v, esize);
        }
    }
}

size_t put_f32(Pack& pk, const void* src, int dtype, size_t n) {
    const size_t off = pk.reserve(n * 4);
    float* dst = reinterpret_cast<float*>(pk.host.data() + off);
    for (size_t i = 0; i < n; ++i) dst[i] = elem(src, dtype, i);
    return off;
}

template <typename T>
int run_prefill(qa_thinker* t, const int32_t* ids, const int64_t* lengths, int n, const float* audio,
                const int64_t* aoff, const int64_t* acnt, float* hidden_out, float* logits_out) {
    const qa_thinker_dims& d = t->d;
    const int H = d.hidden, F = d.ffn_dim, hq = d.n_q_heads, hkv = d.n_kv_heads, V = d.vocab;
    const int NQKV = (hq + 2 * hkv) * kHeadDim;
    // ---- plan
    int64_t M = 0, max_len = 0;
    for (int i = 0; i < n; ++i) { M += lengths[i]; max_len = std::max(max_len, lengths[i]); }
    const size_t tab_bytes = align256((size_t)M * 4) * 2 + align256((size_t)(n + 1) * 4) + align256((size_t)n * 4);
    if (t->pinned_size < tab_bytes) {
        if (t->pinned) (void)hipHostFree(t->pinned);
        t->pinned = nullptr;
        t->pinned_size = 0;
        if (hipHostMalloc((void**)&t->pinned, tab_bytes) != hipSuccess) {
            (void)hipGetLastError();
            set_errf("pinned host allocation of %zu bytes failed", tab_bytes);
            return QA_STATUS_OOM;
        }
        t->pinned_size = tab_bytes;
    }
    int* src = reinterpret_cast<int*>(t->pinned);
    int* pos = reinterpret_cast<int*>(t->pinned + align256((size_t)M * 4));
    int* cu = reinterpret_cast<int*>(t->pinned + 2 * align256((size_t)M * 4));
    int* last = reinterpret_cast<int*>(t->pinned + 2 * align256((size_t)M * 4) + align256((size_t)(n + 1) * 4));
    int64_t row = 0, arow = 0;
    for (int i = 0; i < n; ++i) {
        cu[i] = (int)row;
        for (int64_t p = 0; p < lengths[i]; ++p) {
            const bool is_audio = p >= aoff[i] && p < aoff[i] + acnt[i];
            src[row + p] = is_audio ? -(int)(arow + (p - aoff[i])) - 1 : ids[row + p];
            pos[row + p] = (int)p;
        }
        arow += acnt[i];
        row += lengths[i];
        last[i] = (int)row - 1;
    }
    cu[n] = (int)row;
    // ---- rope table (cos, sin of p base^(-i/64), fp64 trig), grown on demand
    if (t->rope_len < max_len) {
        const int64_t len = std::max<int64_t>(max_len, 1024);
        std::vector<float2> cs((size_t)len * 64);
        for (int64_t p = 0; p < len; ++p)
            for (int i = 0; i < 64; ++i) {
                const double a = (double)p * std::pow(kRopeBase, -(double)i / 64.0);
                cs[(size_t)p * 64 + i] = make_float2((float)std::cos(a), (float)std::sin(a));
            }
        if (t->rope) (void)hipFree(t->rope);
        t->rope = nullptr;
        t->rope_len = 0;
        if (hipMalloc((void**)&t->rope, cs.size() * sizeof(float2)) != hipSuccess ||
            hipMemcpy(t->rope, cs.data(), cs.size() * sizeof(float2), hipMemcpyHostToDevice) != hipSuccess) {
            (void)hipGetLastError();
            set_errf("rope table allocation failed");
            return QA_STATUS_OOM;
        }
        t->rope_len = len;
    }
    // ---- workspace
    const size_t e = sizeof(T);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
    const size_t o_tab = take(tab_bytes);
    const size_t o_x = take((size_t)M * H * 4);
    const size_t o_h = take((size_t)M * H * e);
    const size_t o_qkv = take((size_t)M * NQKV * e);
    const size_t o_att = take((size_t)M * hq * kHeadDim * e);
    const size_t o_u = take((size_t)M * F * e);
    if (t->ws_size < off) {
        if (t->ws) (void)hipFree(t->ws);
        t->ws = nullptr;
        t->ws_size = 0;
        if (hipMalloc((void**)&t->ws, off) != hipSuccess) {
            (void)hipGetLastError();
            set_errf("workspace allocation of %zu bytes failed", off);
            return QA_STATUS_OOM;
        }
        t->ws_size = off;
    }
    char* ws = t->ws;
    const int* d_src = reinterpret_cast<const int*>(ws + o_tab);
    const int* d_pos = reinterpret_cast<const int*>(ws + o_tab + align256((size_t)M * 4));
    const int* d_cu = reinterpret_cast<const int*>(ws + o_tab + 2 * align256((size_t)M * 4));
    const int* d_last = reinterpret_cast<const int*>(ws + o_tab + 2 * align256((size_t)M * 4) + align256((size_t)(n + 1) * 4));
    float* x = reinterpret_cast<float*>(ws + o_x);
    T* h = reinterpret_cast<T*>(ws + o_h);
    T* qkv = reinterpret_cast<T*>(ws + o_qkv);
    T* att = reinterpret_cast<T*>(ws + o_att);
    T* u = reinterpret_cast<T*>(ws + o_u);
    const float* zero = t->W<float>(t->zero);
    hipStream_t s = t->stream;
#define QA_TRY(label, expr)                                                        \
    do {                                                                           \
        const hipError_t st_ = (expr);                                             \
        if (st_ != hipSuccess) {                                                   \
            set_errf("%s: %s", label, hipGetErrorString(st_));                     \
            (void)hipGetLastError();                                               \
            return QA_STATUS_ENCODE_FAILED;                                        \
        }                                                                          \
    } while (0)
    QA_TRY("tables", hipMemcpyAsync(ws + o_tab, t->pinned, tab_bytes, hipMemcpyHostToDevice, s));
    QA_TRY("splice", qa::embed_splice<T>(s, t->W<T>(t->embed), audio, d_src, (int)M, H, x));
    for (int l = 0; l < d.n_layers; ++l) {
        const LayerOff& L = t->layers[l];
        QA_TRY("attn_norm", qa::rmsnorm<T>(s, x, (int)M, H, t->W<float>(L.attn_norm), kRmsEps, h));
        QA_TRY("qkv", qa::thinker_gemm<T>(s, qa::kThinkerSiteQKV, h, (int)M, H, t->W<T>(L.qkv), NQKV, zero, qkv, nullptr));
        QA_TRY("qk_norm_rope", qa::qknorm_rope<T>(s, qkv, (int)M, hq, hkv, d_pos, t->W<float>(L.q_norm),
                                                   t->W<float>(L.k_norm), t->rope, kRmsEps));
        QA_TRY("attention", qa::thinker_attention<T>(s, qkv, d_cu, n, hq, hkv, (int)max_len, att));
        QA_TRY("o_proj", qa::thinker_gemm<T>(s, qa::kThinkerSiteOProj, att, (int)M, hq * kHeadDim, t->W<T>(L.o), H, zero, nullptr, x));
        QA_TRY("ffn_norm", qa::rmsnorm<T>(s, x, (int)M, H, t->W<float>(L.ffn_norm), kRmsEps, h));
        QA_TRY("gate_up", qa::thinker_gemm<T>(s, qa::kThinkerSiteGateUp, h, (int)M, H, t->W<T>(L.gu), 2 * F, zero, u, nullptr));
        QA_TRY("down", qa::thinker_gemm<T>(s, qa::kThinkerSiteDown, u, (int)M, F, t->W<T>(L.down), H, zero, nullptr, x));
    }
    if (hidden_out) QA_TRY("out_norm", qa::rmsnorm<float>(s, x, (int)M, H, t->W<float>(t->out_norm), kRmsEps, hidden_out));
    if (logits_out) {
        QA_TRY("out_norm", qa::rmsnorm<T>(s, x, (int)M, H, t->W<float>(t->out_norm), kRmsEps, h));
        QA_TRY("logits", qa::thinker_logits<T>(s, h, d_last, n, H, t->W<T>(t->embed), V, zero, logits_out));
    }
#undef QA_TRY
    const hipError_t st = hipStreamSynchronize(s);
    if (st != hipSuccess) {
        set_errf("stream synchronize: %s", hipGetErrorString(st));
        return QA_STATUS_ENCODE_FAILED;
    }
    return QA_STATUS_OK;
}

}  // namespace

QA_API qa_thinker* qa_thinker_create(const qa_thinker_weights* w, const qa_thinker_dims* d) {
    if (!check_dims(d) || !check_weights(w, d->n_layers)) return nullptr;
    qa_thinker* t = new (std::nothrow) qa_thinker();
    if (!t) { set_errf("host allocation failed"); return nullptr; }
    t->d = *d;
    t->esize = d->dtype == QA_DTYPE_BF16 ? 2 : 4;
    const int H = d->hidden, F = d->ffn_dim, hq = d->n_q_heads, hkv = d->n_kv_heads, V = d->vocab;
    const size_t es = t->esize;
    Pack pk;
    t->embed = pk.reserve((size_t)V * H * es);
    put_rows(pk, t->embed, 0, w->embed, d->dtype, t->esize, 0, V, H);
    t->layers.resize(d->n_layers);
    for (int l = 0; l < d->n_layers; ++l) {
        LayerOff& L = t->layers[l];
        L.attn_norm = put_f32(pk, w->attn_norm[l], d->dtype, H);
        L.qkv = pk.reserve((size_t)(hq + 2 * hkv) * kHeadDim * H * es);
        put_rows(pk, L.qkv, 0, w->q_w[l], d->dtype, t->esize, 0, (size_t)hq * kHeadDim, H);
        put_rows(pk, L.qkv, (size_t)hq * kHeadDim, w->k_w[l], d->dtype, t->esize, 0, (size_t)hkv * kHeadDim, H);
        put_rows(pk, L.qkv, (size_t)(hq + hkv) * kHeadDim, w->v_w[l], d->dtype, t->esize, 0, (size_t)hkv * kHeadDim, H);
        L.q_norm = put_f32(pk, w->q_norm[l], d->dtype, kHeadDim);
        L.k_norm = put_f32(pk, w->k_norm[l], d->dtype, kHeadDim);
        L.o = pk.reserve((size_t)H * hq * kHeadDim * es);
        put_rows(pk, L.o, 0, w->o_w[l], d->dtype, t->esize, 0, H, (size_t)hq * kHeadDim);
        L.ffn_norm = put_f32(pk, w->ffn_norm[l], d->dtype, H);
        // gate / up interleaved in blocks of 16 rows: [g 0..15, u 0..15, g 16..31, u 16..31, ...]
        L.gu = pk.reserve((size_t)2 * F * H * es);
        for (int b = 0; b < F / 16; ++b) {
            put_rows(pk, L.gu, (size_t)32 * b, w->gate_w[l], d->dtype, t->esize, (size_t)16 * b, 16, H);
            put_rows(pk, L.gu, (size_t)32 * b + 16, w->up_w[l], d->dtype, t->esize, (size_t)16 * b, 16, H);
        }
        L.down = pk.reserve((size_t)H * F * es);
        put_rows(pk, L.down, 0, w->down_w[l], d->dtype, t->esize, 0, H, F);
    }
    t->out_norm = put_f32(pk, w->out_norm, d->dtype, H);
    const size_t nz = (size_t)std::max({V, 2 * F, (hq + 2 * hkv) * kHeadDim, H});
    t->zero = pk.reserve(nz * 4);
    memset(pk.host.data() + t->zero, 0, nz * 4);
    if (hipMalloc((void**)&t->wbuf, pk.host.size()) != hipSuccess ||
        hipMemcpy(t->wbuf, pk.host.data(), pk.host.size(), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipGetLastError();
        set_errf("device allocation or copy of %zu weight bytes failed", pk.host.size());
        if (t->wbuf) (void)hipFree(t->wbuf);
        delete t;
        return nullptr;
    }
    return t;
}

QA_API int qa_thinker_set_stream(qa_thinker* t, void* hip_stream) {
    if (!t) { set_errf("thinker is NULL"); return QA_STATUS_INVALID_PARAMS; }
    t->stream = static_cast<hipStream_t>(hip_stream);
    return QA_STATUS_OK;
}

QA_API int qa_thinker_prefill(qa_thinker* t, const int32_t* ids, const int64_t* lengths, int n_prompts,
                              const float* audio, const int64_t* audio_offsets, const int64_t* audio_counts,
                              float* hidden_out, float* logits_out) {
    if (!t) { set_errf("thinker is NULL"); return QA_STATUS_INVALID_PARAMS; }
    if (n_prompts < 0) { set_errf("n_prompts must be >= 0"); return QA_STATUS_INVALID_PARAMS; }
    if (n_prompts == 0) return QA_STATUS_OK;
    if (!ids || !lengths || !audio_offsets || !audio_counts) { set_errf("NULL host array"); return QA_STATUS_INVALID_PARAMS; }
    int64_t M = 0, A = 0;
    for (int i = 0; i < n_prompts; ++i) {
        if (lengths[i] < 1 || lengths[i] > kMaxPrompt) {
            set_errf("prompt %d has %lld tokens: must be in 1..%lld", i, (long long)lengths[i], (long long)kMaxPrompt);
            return QA_STATUS_INVALID_PARAMS;
        }
        if (audio_counts[i] < 0 || audio_offsets[i] < 0 || audio_offsets[i] + audio_counts[i] > lengths[i]) {
            set_errf("prompt %d: the audio span must lie inside the prompt", i);
            return QA_STATUS_INVALID_PARAMS;
        }
        for (int64_t p = 0; p < lengths[i]; ++p) {
            const bool is_audio = p >= audio_offsets[i] && p < audio_offsets[i] + audio_counts[i];
            const int32_t id = ids[M + p];
            if (!is_audio && (id < 0 || id >= t->d.vocab)) {
                set_errf("prompt %d token %lld: id %d outside 0..%d", i, (long long)p, id, t->d.vocab - 1);
                return QA_STATUS_INVALID_PARAMS;
            }
        }
        M += lengths[i];
        A += audio_counts[i];
        if (M > kMaxTokens) { set_errf("more than %lld packed tokens", (long long)kMaxTokens); return QA_STATUS_INVALID_PARAMS; }
    }
    if (A > 0 && !audio) { set_errf("audio is NULL but the prompts hold audio spans"); return QA_STATUS_INVALID_PARAMS; }
    if (!hidden_out && !logits_out) return QA_STATUS_OK;
    return t->d.dtype == QA_DTYPE_BF16
               ? run_prefill<bf16>(t, ids, lengths, n_prompts, audio, audio_offsets, audio_counts, hidden_out, logits_out)
               : run_prefill<float>(t, ids, lengths, n_prompts, audio, audio_offsets, audio_counts, hidden_out, logits_out);
}

QA_API void qa_thinker_free(qa_thinker* t) {
    if (!t) return;
    if (t->wbuf) (void)hipFree(t->wbuf);
    if (t->ws) (void)hipFree(t->ws);
    if (t->rope) (void)hipFree(t->rope);
    if (t->pinned) (void)hipHostFree(t->pinned);
    delete t;
}
