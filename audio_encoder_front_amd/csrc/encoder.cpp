// Host runtime behind the C ABI: argument validation, weight repacking,
// front-end constant tables, the per-call planner (frames -> chunks ->
// tokens -> windows), the device workspace and the launch sequence.
//
// Sources: qwenasr.cpp ARCHITECTURE.md ("GGUF layout" dims and tensors,
// "Mel frontend", "Conv2d subsampling stem" after-cnn length, "Windowed audio
// tower" chunk plan, PE table and block-diagonal windows, "Public API" status
// codes and thread-local last error); OneSpeech "Low-level recognition" and
// "Front end and graph numerics" (input rules, 100-frame chunks, bf16 policy);
// M* ASR page "Graph" / request length (one packed forward, one segment per
// window of every request, up to 20 minutes per request).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <utility>
#include <mutex>
#include <new>
#include <string>
#include <type_traits>
#include <vector>

#include "../../include/qa_encoder.h"
#include "qa_kernels.h"

#define QA_API extern "C" __attribute__((visibility("default")))

namespace {

using qa::bf16;

thread_local std::string g_err;

void set_err(const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
}

}  // namespace

namespace qa {
void set_error_message(const char* msg) { g_err = msg; }
}  // namespace qa

namespace {

constexpr int64_t kMaxSamples = 20LL * 60 * 16000;   // a request hears up to 20 minutes
constexpr int64_t kMaxFullInput = 30LL * 16000;      // bounded input of full-input attention (30 s)
constexpr int kHop = 160;
constexpr int kSplitKMaxTokens = 4096;   // residual GEMMs of smaller batches take split-K
constexpr int kMaxLanes = 4;             // streams a large batch's layers may run on
// lanes a batch past the split-K sizes runs as (at most the handle's
// maximum): 3 up to kMidLaneTokens tokens, whose GEMMs fill few rounds of
// CUs per lane, else 2 (measured: 4 lanes never paid; 3 against 2 was
// 5.38 / 5.51 ms at 5,986 tokens, 15.80 / 15.54 ms at 15,600)
constexpr int kMidLaneTokens = 8192;
constexpr int kNfft = 400;
constexpr int kBins = kNfft / 2 + 1;

int after_cnn(int m) {
    for (int i = 0; i < 3; ++i) m = (m - 1) / 2 + 1;
    return m;
}

int64_t tokens_of(int64_t n) {
    const int64_t fr = n / kHop;
    const int64_t tail = fr % qa::kChunk;
    return (fr / qa::kChunk) * qa::kChunkTok + (tail ? after_cnn((int)tail) : 0);
}

bool valid_len(int64_t n) { return n == 0 || (n > 200 && n <= kMaxSamples); }

// Workspace of qa_encode_noalloc: one fixed device array per GPU, held until
// the process ends.  In host code `scratch` is only a handle; its device
// address (different on every GPU) comes from hipGetSymbolAddress, taken once
// per device when an encoder is created there, and only that address is
// passed to kernels and copies.
constexpr size_t kScratchBytes = QA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
hipError_t g_scratch_err[kMaxDevices] = {};
bool g_scratch_tried[kMaxDevices] = {};

// With `device` current: the device address of its scratch array (taken on
// the first call for the device), or null with the error recorded.
void* scratch_address(int device) {
    if (device < 0 || device >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_tried[device]) {
        void* ptr = nullptr;
        const hipError_t st = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        g_scratch_tried[device] = true;
        g_scratch_err[device] = st;
        g_scratch_ptr[device] = st == hipSuccess ? ptr : nullptr;
        if (st != hipSuccess) (void)hipGetLastError();
    }
    return g_scratch_ptr[device];
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

float bf16_bits_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t f32_to_bf16_rne(float f) {   // finite inputs
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// v = hi + mid + lo exactly (each part a bf16; 3 x 8 significant bits cover
// fp32's 24): hi = rne(v), mid = rne(v - hi), lo = v - hi - mid.
void split3_bf16(float v, uint16_t* part) {
    part[0] = f32_to_bf16_rne(v);
    const float r1 = v - bf16_bits_to_f32(part[0]);
    part[1] = f32_to_bf16_rne(r1);
    const float r2 = r1 - bf16_bits_to_f32(part[1]);
    part[2] = f32_to_bf16_rne(r2);
}

// ---------------------------------------------------------------- front-end constants

double hz_to_mel(double f) {   // Slaney: linear below 1 kHz, 27 mels per factor 6.4 above
    return f < 1000.0 ? 3.0 * f / 200.0 : 15.0 + 27.0 * std::log(f / 1000.0) / std::log(6.4);
}
double mel_to_hz(double m) {
    return m < 15.0 ? 200.0 * m / 3.0 : 1000.0 * std::exp((m - 15.0) * std::log(6.4) / 27.0);
}

struct FrontConsts {
    std::vector<uint16_t> basis;   // bf16 A fragments [13][13][2][3][64][8] (see qa::frontend)
    std::vector<float> melw;    // [128][qa::kMelTaps] weights of bins melb0[m] ..
    std::vector<int> melb0;     // [128] first bin of each band
    bool ok = true;             // every band fits qa::kMelTaps bins
};

FrontConsts make_front_consts() {
    FrontConsts c;
    // Slaney-normalised mel filters, fmin 0, fmax 8000, 130 edges uniform in mel
    std::vector<double> fb((size_t)qa::kMels * kBins, 0.0);
    const double top = hz_to_mel(8000.0);
    std::vector<double> edge(qa::kMels + 2);
    for (int i = 0; i < qa::kMels + 2; ++i) edge[i] = mel_to_hz(top * i / (qa::kMels + 1));
    for (int m = 0; m < qa::kMels; ++m) {
        const double lo = edge[m], ce = edge[m + 1], hi = edge[m + 2];
        for (int k = 0; k < kBins; ++k) {
            const double f = 40.0 * k;
            const double v = std::max(0.0, std::min((f - lo) / (ce - lo), (hi - f) / (hi - ce)));
            fb[(size_t)m * kBins + k] = v * 2.0 / (hi - lo);
        }
    }
    // periodic Hann folded into the cos / sin basis (trig in fp64, rounded to
    // fp32), each fp32 value split exactly into bf16 hi + mid + lo and laid out
    // as MFMA A fragments: lane l holds bin 16 bc + l % 16, samples
    // 32 kb + 8 (l / 16) .. + 7
    c.basis.assign((size_t)qa::kBinChunks * qa::kDftKBlocks * 2 * 3 * 64 * 8, 0);
    for (int bc = 0; bc < qa::kBinChunks; ++bc)
        for (int kb = 0; kb < qa::kDftKBlocks; ++kb)
            for (int l = 0; l < 64; ++l)
                for (int e = 0; e < 8; ++e) {
                    const int bin = bc * 16 + l % 16, n = 32 * kb + 8 * (l / 16) + e;
                    if (bin >= kBins || n >= kNfft) continue;
                    const double w = 0.5 - 0.5 * std::cos(2.0 * M_PI * n / kNfft);
                    const double ang = 2.0 * M_PI * (double)((bin * n) % kNfft) / kNfft;
                    const float v[2] = {(float)(w * std::cos(ang)), (float)(w * std::sin(ang))};
                    for (int cs = 0; cs < 2; ++cs) {
                        uint16_t part[3];
                        split3_bf16(v[cs], part);
                        for (int pp = 0; pp < 3; ++pp)
                            c.basis[(((((size_t)bc * qa::kDftKBlocks + kb) * 2 + cs) * 3 + pp) * 64 + l) * 8 + e] = part[pp];
                    }
                }
    // each band's support (consecutive bins) in a kMelTaps-wide window
    c.melw.assign((size_t)qa::kMels * qa::kMelTaps, 0.f);
    c.melb0.assign(qa::kMels, 0);
    for (int m = 0; m < qa::kMels; ++m) {
        int lo = kBins, hi = -1;
        for (int k = 0; k < kBins; ++k)
            if (fb[(size_t)m * kBins + k] != 0.0) { lo = std::min(lo, k); hi = std::max(hi, k); }
        if (hi < lo) lo = hi = 0;
        if (hi - lo + 1 > qa::kMelTaps) c.ok = false;
        const int b0 = std::min(lo, qa::kBinChunks * 16 - qa::kMelTaps);
        c.melb0[m] = b0;
        for (int j = 0; j < qa::kMelTaps; ++j) {
            const int k = b0 + j;
            c.melw[(size_t)m * qa::kMelTaps + j] = k < kBins ? (float)fb[(size_t)m * kBins + k] : 0.f;
        }
    }
    return c;
}

std::vector<float> make_pe(int d) {   // sinusoidal table, rows 0..12, trig in fp64
    const int half = d / 2;
    std::vector<float> pe((size_t)qa::kChunkTok * d);
    for (int t = 0; t < qa::kChunkTok; ++t)
        for (int i = 0; i < half; ++i) {
            const double inv = std::exp(-std::log(10000.0) / (half - 1) * i);
            pe[(size_t)t * d + i] = (float)std::sin(t * inv);
            pe[(size_t)t * d + half + i] = (float)std::cos(t * inv);
        }
    return pe;
}

// ---------------------------------------------------------------- weights

struct LayerW {
    size_t ln1_w, ln1_b, qkv_w, qkv_b, o_w, o_b, ln2_w, ln2_b, fc1_w, fc1_b, fc2_w, fc2_b;
};

struct Profile {
    const char* label;
    hipEvent_t a, b;
};

}  // namespace

struct qa_encoder {
    qa_dims d{};
    int esize = 4;                      // bytes per operand element (4 fp32, 2 bf16)
    hipStream_t stream = nullptr;
    int device = 0;
    // further lanes of the layers (see run_encode): their streams and the fork/join events
    int max_lanes = kMaxLanes;
    hipStream_t lane[kMaxLanes - 1] = {};
    hipEvent_t ev_fork = nullptr, ev_join[kMaxLanes - 1] = {};
    // weights + constants in one device allocation
    char* wbuf = nullptr;
    size_t conv1_frag = 0;              // bf16 MFMA fragments of conv1 (0: VALU kernel)
    size_t conv1_w = 0, conv1_b = 0, conv2_w = 0, conv2_b = 0, conv3_w = 0, conv3_b = 0, conv_out_w = 0;
    std::vector<LayerW> layers;
    size_t post_ln_w = 0, post_ln_b = 0, proj1_w = 0, proj1_b = 0, proj2_w = 0, proj2_b = 0;
    size_t basis = 0, melw = 0, melb0 = 0, pe = 0;
    // per-call workspace
    char* ws = nullptr;
    size_t ws_size = 0;
    char* pinned = nullptr;
    size_t pinned_size = 0;
    int* flag_host = nullptr;
    // taps
    bool taps = false;
    int64_t tap_frames = -1, tap_tokens = -1;
    float *tap_logmel = nullptr, *tap_stem = nullptr, *tap_layer0 = nullptr;
    // profiling
    bool profiling = false;
    std::string prof_only;                  // non-empty: time only launches with this label
    std::vector<hipEvent_t> ev_pool;
    std::vector<Profile> prof_cur;
    std::map<std::string, std::pair<double, int64_t>> prof_acc;
    std::vector<std::string> prof_labels;   // stable storage for returned labels

    template <typename P = void>
    P* W(size_t off) const { return reinterpret_cast<P*>(wbuf + off); }
};

namespace {

// Packs host weights into one device buffer.
struct Packer {
    std::vector<char> host;
    size_t put(const void* p, size_t bytes) {
        const size_t off = align256(host.size());
        host.resize(off + bytes);
        memcpy(host.data() + off, p, bytes);
        return off;
    }
};

// Reads element i of a host weight tensor given in dims.dtype.
struct Src {
    const void* p;
    int dtype;
    float operator[](size_t i) const {
        return dtype == QA_DTYPE_BF16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i])
                                      : static_cast<const float*>(p)[i];
    }
};

// A matrix of operand elements (fp32 or bf16 bit patterns); values given as
// floats are exactly representable in the operand type.
void push_elems(std::vector<char>& out, const std::vector<float>& v, int esize) {
    out.resize(v.size() * esize);
    if (esize == 4) {
        memcpy(out.data(), v.data(), v.size() * 4);
    } else {
        uint16_t* o = reinterpret_cast<uint16_t*>(out.data());
        for (size_t i = 0; i < v.size(); ++i) {
            uint32_t u;
            memcpy(&u, &v[i], 4);
            o[i] = (uint16_t)(u >> 16);   // exact: values came from bf16
        }
    }
}

bool check_dims(const qa_dims* d) {
    if (!d) { set_err("dims is NULL"); return false; }
    if (d->abi_version != QA_ABI_VERSION) {
        set_err("abi_version %d does not match the library's %d", d->abi_version, QA_ABI_VERSION);
        return false;
    }
    if (d->n_mels != 128) { set_err("n_mels must be 128"); return false; }
    if (d->chunk_frames != 100) { set_err("chunk_frames must be 100"); return false; }
    if (d->head_dim != 64) { set_err("head_dim must be 64"); return false; }
    if (d->window_chunks < 0 || d->window_chunks * qa::kChunkTok > qa::kMaxWindow) {
        set_err("window_chunks must be 0 (full-input attention) or in 1..%d", qa::kMaxWindow / qa::kChunkTok);
        return false;
    }
    if (d->conv_channels < 32 || d->conv_channels > 1024 || d->conv_channels % 32) {
        set_err("conv_channels must be a multiple of 32 in 32..1024");
        return false;
    }
    if (d->d_model < 64 || d->d_model > 2048 || d->d_model % 64) {
        set_err("d_model must be a multiple of 64 in 64..2048");
        return false;
    }
    if (d->n_heads < 1 || d->n_heads * d->head_dim != d->d_model) {
        set_err("n_heads * head_dim must equal d_model");
        return false;
    }
    if (d->ffn_dim < 64 || d->ffn_dim % 64 || d->ffn_dim > 65536) { set_err("ffn_dim must be a multiple of 64"); return false; }
    if (d->output_dim < 64 || d->output_dim % 64 || d->output_dim > 65536) {
        set_err("output_dim must be a multiple of 64");
        return false;
    }
    if (d->n_layers < 0 || d->n_layers > 1024) { set_err("n_layers out of range"); return false; }
    if (d->dtype != QA_DTYPE_F32 && d->dtype != QA_DTYPE_BF16) { set_err("unknown dtype"); return false; }
    return true;
}

bool check_weights(const qa_weights* w, int n_layers) {
    if (!w) { set_err("weights is NULL"); return false; }
    const void* top[] = {w->conv1_w, w->conv1_b, w->conv2_w, w->conv2_b, w->conv3_w, w->conv3_b, w->conv_out_w,
                         w->post_ln_w, w->post_ln_b, w->proj1_w, w->proj1_b, w->proj2_w, w->proj2_b};
    for (const void* p : top)
        if (!p) { set_err("a weight pointer is NULL"); return false; }
    const void* const* arr[] = {w->ln1_w, w->ln1_b, w->q_w, w->q_b, w->k_w, w->k_b, w->v_w, w->v_b,
                                w->o_w, w->o_b, w->ln2_w, w->ln2_b, w->fc1_w, w->fc1_b, w->fc2_w, w->fc2_b};
    for (const void* const* a : arr) {
        if (n_layers > 0 && !a) { set_err("a per-layer weight array is NULL"); return false; }
        for (int l = 0; l < n_layers; ++l)
            if (!a[l]) { set_err("layer %d has a NULL weight pointer", l); return false; }
    }
    return true;
}

#define HIP_TRY(call, status)                                                               \
    do {                                                                                    \
        hipError_t e_ = (call);                                                             \
        if (e_ != hipSuccess) {                                                             \
            set_err("%s failed: %s", #call, hipGetErrorString(e_));                        \
            return status;                                                                  \
        }                                                                                   \
    } while (0)

}  // namespace

// =====================================================================  C ABI

QA_API int qa_abi_version(void) { return QA_ABI_VERSION; }

QA_API const char* qa_last_error(void) { return g_err.c_str(); }

QA_API int64_t qa_encode_num_tokens(int64_t n_samples) {
    if (!valid_len(n_samples)) {
        set_err("clip length %lld: must be 0 or in 201..%lld samples", (long long)n_samples,
                (long long)kMaxSamples);
        return -1;
    }
    return tokens_of(n_samples);
}

QA_API qa_encoder* qa_encoder_create(const qa_weights* w, const qa_dims* d) {
    if (!check_dims(d) || !check_weights(w, d ? d->n_layers : 0)) return nullptr;
    const int C = d->conv_channels, D = d->d_model, F = d->ffn_dim, O = d->output_dim, L = d->n_layers;
    const int esz = d->dtype == QA_DTYPE_BF16 ? 2 : 4;
    auto f32vec = [&](const void* p, size_t n) {
        std::vector<float> v(n);
        Src s{p, d->dtype};
        for (size_t i = 0; i < n; ++i) v[i] = s[i];
        return v;
    };
    qa_encoder* e = new (std::nothrow) qa_encoder();
    if (!e) { set_err("host allocation failed"); return nullptr; }
    e->d = *d;
    e->esize = esz;
    Packer pk;
    std::vector<char> tmp;
    auto put_f32 = [&](const std::vector<float>& v) { return pk.put(v.data(), v.size() * 4); };
    auto put_op = [&](const std::vector<float>& v) {
        push_elems(tmp, v, esz);
        return pk.put(tmp.data(), tmp.size());
    };
    // conv1 [C][1][3][3] -> [9][C] fp32
    {
        auto v = f32vec(w->conv1_w, (size_t)C * 9);
        std::vector<float> r((size_t)9 * C);
        for (int c = 0; c < C; ++c)
            for (int k = 0; k < 9; ++k) r[(size_t)k * C + c] = v[(size_t)c * 9 + k];
        e->conv1_w = put_f32(r);
        e->conv1_b = put_f32(f32vec(w->conv1_b, C));
        if (d->dtype == QA_DTYPE_BF16 && C <= qa::kStemFusedMaxC) {
            // A operand of lane l for channel tile t: channel 32 (t / 2) + 8 (r / 4) +
            // 4 (t % 2) + r % 4 with r = l % 16, K entries k = 8 (l / 16) + e: tap
            // k / 3 for k < 27 (three copies, one per input part), the bias at
            // k = 27, zero beyond.
            const uint16_t* wb = static_cast<const uint16_t*>(w->conv1_w);
            const uint16_t* bb = static_cast<const uint16_t*>(w->conv1_b);
            std::vector<uint16_t> fr((size_t)(C / 16) * 64 * 8, 0);
            for (int t = 0; t < C / 16; ++t)
                for (int l = 0; l < 64; ++l)
                    for (int el = 0; el < 8; ++el) {
                        const int r = l % 16, k = 8 * (l / 16) + el;
                        const int c = 32 * (t / 2) + 8 * (r / 4) + 4 * (t % 2) + r % 4;
                        uint16_t v = 0;
                        if (k < 27) v = wb[(size_t)c * 9 + k / 3];
                        else if (k == 27) v = bb[c];
                        fr[((size_t)t * 64 + l) * 8 + el] = v;
                    }
            e->conv1_frag = pk.put(fr.data(), fr.size() * 2);
        }
    }
    // conv2/conv3 [Co][Ci][3][3] -> [Co][K], K index (ci / 32, tap, ci % 32)
    auto conv_pack = [&](const void* p) {
        auto v = f32vec(p, (size_t)C * C * 9);
        std::vector<float> r((size_t)C * 9 * C);
        const int cb = qa::kConvCB;
        for (int co = 0; co < C; ++co)
            for (int ci = 0; ci < C; ++ci)
                for (int k = 0; k < 9; ++k)
                    r[(size_t)co * 9 * C + (size_t)(ci / cb) * 9 * cb + k * cb + ci % cb] =
                        v[((size_t)co * C + ci) * 9 + k];
        return put_op(r);
    };
    e->conv2_w = conv_pack(w->conv2_w);
    e->conv2_b = put_f32(f32vec(w->conv2_b, C));
    e->conv3_w = conv_pack(w->conv3_w);
    e->conv3_b = put_f32(f32vec(w->conv3_b, C));
    // conv_out [D][c*16 + f] -> [D][f*C + c]  (the stem stores frequency outer, channel inner)
    {
        auto v = f32vec(w->conv_out_w, (size_t)D * C * 16);
        std::vector<float> r(v.size());
        for (int n = 0; n < D; ++n)
            for (int c = 0; c < C; ++c)
                for (int f = 0; f < 16; ++f) r[(size_t)n * C * 16 + f * C + c] = v[(size_t)n * C * 16 + c * 16 + f];
        e->conv_out_w = put_op(r);
    }
    e->layers.resize(L);
    for (int l = 0; l < L; ++l) {
        LayerW& lw = e->layers[l];
        lw.ln1_w = put_f32(f32vec(w->ln1_w[l], D));
        lw.ln1_b = put_f32(f32vec(w->ln1_b[l], D));
        std::vector<float> qkv((size_t)3 * D * D), qkvb((size_t)3 * D);
        const void* mats[3] = {w->q_w[l], w->k_w[l], w->v_w[l]};
        const void* bs[3] = {w->q_b[l], w->k_b[l], w->v_b[l]};
        for (int j = 0; j < 3; ++j) {
            auto m = f32vec(mats[j], (size_t)D * D);
            std::copy(m.begin(), m.end(), qkv.begin() + (size_t)j * D * D);
            auto b = f32vec(bs[j], D);
            std::copy(b.begin(), b.end(), qkvb.begin() + (size_t)j * D);
        }
        lw.qkv_w = put_op(qkv);
        lw.qkv_b = put_f32(qkvb);
        lw.o_w = put_op(f32vec(w->o_w[l], (size_t)D * D));
        lw.o_b = put_f32(f32vec(w->o_b[l], D));
        lw.ln2_w = put_f32(f32vec(w->ln2_w[l], D));
        lw.ln2_b = put_f32(f32vec(w->ln2_b[l], D));
        lw.fc1_w = put_op(f32vec(w->fc1_w[l], (size_t)F * D));
        lw.fc1_b = put_f32(f32vec(w->fc1_b[l], F));
        lw.fc2_w = put_op(f32vec(w->fc2_w[l], (size_t)D * F));
        lw.fc2_b = put_f32(f32vec(w->fc2_b[l], D));
    }
    e->post_ln_w = put_f32(f32vec(w->post_ln_w, D));
    e->post_ln_b = put_f32(f32vec(w->post_ln_b, D));
    e->proj1_w = put_op(f32vec(w->proj1_w, (size_t)D * D));
    e->proj1_b = put_f32(f32vec(w->proj1_b, D));
    e->proj2_w = put_op(f32vec(w->proj2_w, (size_t)O * D));
    e->proj2_b = put_f32(f32vec(w->proj2_b, O));
    FrontConsts fc = make_front_consts();
    if (!fc.ok) {   // a mel band wider than the kernel's tap window: a build defect, not an input error
        set_err("internal: mel filter support exceeds the front-end tap window");
        delete e;
        return nullptr;
    }
    e->basis = pk.put(fc.basis.data(), fc.basis.size() * sizeof(uint16_t));
    e->melw = put_f32(fc.melw);
    e->melb0 = pk.put(fc.melb0.data(), fc.melb0.size() * sizeof(int));
    e->pe = put_f32(make_pe(D));

    hipError_t st = hipGetDevice(&e->device);
    if (st == hipSuccess) (void)scratch_address(e->device);   // failure is reported by qa_encode_noalloc
    if (st == hipSuccess) st = hipMalloc(&e->wbuf, pk.host.size());
    if (st == hipSuccess) st = hipMemcpy(e->wbuf, pk.host.data(), pk.host.size(), hipMemcpyHostToDevice);
    if (st == hipSuccess) st = hipHostMalloc(&e->flag_host, sizeof(int), hipHostMallocDefault);
    for (int g = 0; g + 1 < kMaxLanes && st == hipSuccess; ++g) {
        st = hipStreamCreateWithFlags(&e->lane[g], hipStreamNonBlocking);
        if (st == hipSuccess) st = hipEventCreateWithFlags(&e->ev_join[g], hipEventDisableTiming);
    }
    if (st == hipSuccess) st = hipEventCreateWithFlags(&e->ev_fork, hipEventDisableTiming);
    if (st != hipSuccess) {
        set_err("loading weights to the device failed: %s", hipGetErrorString(st));
        qa_encoder_free(e);
        return nullptr;
    }
    return e;
}

QA_API int qa_encoder_set_stream(qa_encoder* e, void* hip_stream) {
    if (!e) { set_err("encoder is NULL"); return QA_STATUS_INVALID_PARAMS; }
    e->stream = static_cast<hipStream_t>(hip_stream);
    return QA_STATUS_OK;
}

QA_API int qa_encoder_enable_taps(qa_encoder* e, int enable) {
    if (!e || (enable != 0 && enable != 1)) { set_err("bad arguments"); return QA_STATUS_INVALID_PARAMS; }
    e->taps = enable != 0;
    return QA_STATUS_OK;
}

QA_API int qa_encoder_set_profiling(qa_encoder* e, int enable) {
    if (!e || (enable != 0 && enable != 1)) { set_err("bad arguments"); return QA_STATUS_INVALID_PARAMS; }
    e->profiling = enable != 0;
    e->prof_acc.clear();
    return QA_STATUS_OK;
}

QA_API int qa_encoder_set_max_lanes(qa_encoder* e, int n) {
    if (!e) { set_err("encoder is NULL"); return QA_STATUS_INVALID_PARAMS; }
    if (n < 1 || n > kMaxLanes) { set_err("max lanes must be 1 .. %d, got %d", kMaxLanes, n); return QA_STATUS_INVALID_PARAMS; }
    e->max_lanes = n;
    return QA_STATUS_OK;
}

QA_API int qa_encoder_set_profiling_label(qa_encoder* e, const char* label) {
    if (!e) { set_err("encoder is NULL"); return QA_STATUS_INVALID_PARAMS; }
    e->prof_only = label ? label : "";
    return QA_STATUS_OK;
}

QA_API int qa_encoder_kernel_times(qa_encoder* e, const char** labels, double* total_ms, int64_t* launches,
                                   int cap) {
    if (!e || cap < 0 || (cap > 0 && (!labels || !total_ms || !launches))) {
        set_err("bad arguments");
        return -1;
    }
    e->prof_labels.clear();
    for (auto& kv : e->prof_acc) e->prof_labels.push_back(kv.first);
    int i = 0;
    for (auto& kv : e->prof_acc) {
        if (i < cap) {
            labels[i] = e->prof_labels[i].c_str();
            total_ms[i] = kv.second.first;
            launches[i] = kv.second.second;
        }
        ++i;
    }
    return (int)e->prof_acc.size();
}

QA_API int64_t qa_encoder_tap(qa_encoder* e, int tap, float* dst, int64_t capacity) {
    if (!e) { set_err("encoder is NULL"); return -1; }
    if (!e->taps || e->tap_tokens < 0) { set_err("taps are not enabled or no encode ran with taps"); return -1; }
    const float* src = nullptr;
    int64_t n = 0;
    switch (tap) {
        case QA_TAP_LOG_MEL: src = e->tap_logmel; n = e->tap_frames * qa::kMels; break;
        case QA_TAP_STEM: src = e->tap_stem; n = e->tap_tokens * e->d.d_model; break;
        case QA_TAP_LAYER0: src = e->tap_layer0; n = e->tap_tokens * e->d.d_model; break;
        default: set_err("unknown tap %d", tap); return -1;
    }
    if (tap == QA_TAP_LAYER0 && e->d.n_layers == 0) { set_err("no layer 0"); return -1; }
    if (capacity < n || (n > 0 && !dst)) { set_err("tap needs %lld floats", (long long)n); return -1; }
    if (n > 0) {
        HIP_TRY(hipMemcpyAsync(dst, src, (size_t)n * 4, hipMemcpyDeviceToDevice, e->stream), -1);
        HIP_TRY(hipStreamSynchronize(e->stream), -1);
    }
    return n;
}

QA_API void qa_encoder_free(qa_encoder* e) {
    if (!e) return;
    if (e->wbuf) (void)hipFree(e->wbuf);
    if (e->ws) (void)hipFree(e->ws);
    if (e->pinned) (void)hipHostFree(e->pinned);
    if (e->flag_host) (void)hipHostFree(e->flag_host);
    for (hipEvent_t ev : e->ev_pool) (void)hipEventDestroy(ev);
    for (int g = 0; g + 1 < kMaxLanes; ++g) {
        if (e->lane[g]) (void)hipStreamDestroy(e->lane[g]);
        if (e->ev_join[g]) (void)hipEventDestroy(e->ev_join[g]);
    }
    if (e->ev_fork) (void)hipEventDestroy(e->ev_fork);
    delete e;
}

namespace {

// A caller-fixed workspace (qa_encode_noalloc): nothing is allocated, the
// tables go up from pageable host memory, and neither taps nor profiling
// events are recorded.
struct FixedWorkspace {
    char* base;
    size_t bytes;
};

template <typename T>
int run_encode(qa_encoder* e, const float* pcm, const int64_t* lengths, int n_clips, float* out,
               const FixedWorkspace* fixed = nullptr) {
    const qa_dims& d = e->d;
    const bool taps = e->taps && !fixed;
    const bool profiling = e->profiling && !fixed;
    if (fixed) e->tap_tokens = -1;      // the taps of an earlier call pointed into the growable workspace
    const int C = d.conv_channels, D = d.d_model, F = d.ffn_dim, O = d.output_dim;
    // ---------------- plan
    std::vector<qa::ClipInfo> clips(n_clips);
    std::vector<qa::FrontTile> tiles;
    std::vector<qa::ChunkInfo> chunks;
    std::vector<int> tok_src, cu{0};
    {   // capacities from the frame counts (one pass over the lengths)
        int64_t frames = 0;
        for (int i = 0; i < n_clips; ++i) frames += lengths[i] / kHop;
        tiles.reserve((size_t)(frames / qa::kFrontFrames + 2 * n_clips));
        chunks.reserve((size_t)(frames / qa::kChunk + n_clips));
        tok_src.reserve((size_t)((frames / qa::kChunk + n_clips) * qa::kChunkTok));
    }
    int64_t sample_off = 0;
    int64_t frame_row = 0;
    // window_chunks == 0: one attention segment per clip (full-input attention)
    const int win_tok = d.window_chunks > 0 ? d.window_chunks * qa::kChunkTok : (1 << 30);
    for (int i = 0; i < n_clips; ++i) {
        const int64_t len = lengths[i];
        const int nf = (int)(len / kHop);
        clips[i] = qa::ClipInfo{sample_off, (int32_t)len, (int32_t)frame_row};
        // front-end tiles cover the nf kept frames and the final STFT frame:
        // the front end computes that frame (not stored) so that every sample
        // of the clip is read and checked, and its power too
        const int nf_all = len > 0 ? nf + 1 : 0;
        for (int f0 = 0; f0 < nf_all; f0 += qa::kFrontFrames)
            tiles.push_back(qa::FrontTile{i, f0, std::min(qa::kFrontFrames, nf_all - f0), 0});
        const int tok0 = (int)tok_src.size();
        for (int c0 = 0; c0 < nf; c0 += qa::kChunk) {
            const int m = std::min(qa::kChunk, nf - c0);
            const int ch = (int)chunks.size();
            chunks.push_back(qa::ChunkInfo{(int32_t)(frame_row + c0), m});
            const int nt = after_cnn(m);
            for (int j = 0; j < nt; ++j) tok_src.push_back(ch * qa::kChunkTok + j);
        }
        const int ntok = (int)tok_src.size() - tok0;
        for (int s = 0; s < ntok; s += win_tok) cu.push_back(tok0 + std::min(s + win_tok, ntok));
        sample_off += len;
        frame_row += nf;
    }
    const int n_frames = (int)frame_row, n_chunks = (int)chunks.size(), n_tok = (int)tok_src.size();
    const int n_win = (int)cu.size() - 1, n_tiles = (int)tiles.size();
    int max_seg = 0;
    for (int i = 0; i < n_win; ++i) max_seg = std::max(max_seg, cu[i + 1] - cu[i]);
    if (n_tok > 0 && !out) { set_err("out is NULL but the batch has %d tokens", n_tok); return QA_STATUS_INVALID_PARAMS; }
    if (sample_off > 0 && !pcm) { set_err("pcm is NULL"); return QA_STATUS_INVALID_PARAMS; }
    if (n_tok == 0) {
        if (taps) { e->tap_frames = 0; e->tap_tokens = 0; }
        return QA_STATUS_OK;
    }

    // ---------------- tables (one pinned staging buffer, one H2D copy)
    size_t off = 0;
    auto slot = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    const size_t o_clips = slot(clips.size() * sizeof(qa::ClipInfo));
    const size_t o_tiles = slot(tiles.size() * sizeof(qa::FrontTile));
    const size_t o_chunks = slot(chunks.size() * sizeof(qa::ChunkInfo));
    const size_t o_src = slot(tok_src.size() * 4);
    const size_t o_cu = slot(cu.size() * 4);
    const size_t table_bytes = off;
    // ---------------- workspace
    const size_t o_logmel = slot((size_t)n_frames * qa::kMels * 4);
    const size_t o_key = slot((size_t)n_clips * 4);
    const size_t o_flag = slot(8);                 // the nonfinite-input flag, the fused stem's tile counter
    // bf16 with the MFMA conv1: conv1 and conv2 run as one kernel and conv1's
    // output is never stored
    const bool fused_stem = std::is_same<T, qa::bf16>::value && e->conv1_frag != 0;
    const size_t o_c1 = slot(fused_stem ? 0 : (size_t)n_chunks * 64 * 50 * C * sizeof(T));
    const size_t o_c2 = slot((size_t)n_chunks * 32 * 25 * C * sizeof(T));
    const size_t o_c3 = slot((size_t)n_chunks * 13 * 16 * C * sizeof(T));
    const size_t o_x = slot((size_t)n_tok * D * 4);
    const size_t o_h = slot((size_t)n_tok * D * sizeof(T));
    const size_t o_qkv = slot((size_t)n_tok * 3 * D * sizeof(T));
    const size_t o_att = slot((size_t)n_tok * D * sizeof(T));
    const size_t o_u = slot((size_t)n_tok * std::max(F, D) * sizeof(T));
    // split-K partial sums of the residual GEMMs (small batches only: up to
    // 8 splits of [n_tok][D] fp32)
    const size_t part_elems = n_tok <= kSplitKMaxTokens ? (size_t)8 * n_tok * D : 0;
    const size_t o_part = slot(part_elems * 4);
    size_t o_tstem = 0, o_tl0 = 0;
    if (taps) {
        o_tstem = slot((size_t)n_tok * D * 4);
        o_tl0 = slot((size_t)n_tok * D * 4);
    }
    const size_t need = off;
    if (fixed) {
        if (need > fixed->bytes) {
            set_err("this batch needs %zu bytes of workspace; qa_encode_noalloc holds at most %zu "
                    "(use qa_encode, or a smaller batch)", need, fixed->bytes);
            return QA_STATUS_INVALID_PARAMS;
        }
    } else if (need > e->ws_size) {
        if (e->ws) { (void)hipFree(e->ws); e->ws = nullptr; e->ws_size = 0; }
        hipError_t st = hipMalloc(&e->ws, need);
        if (st != hipSuccess) {
            (void)hipGetLastError();
            set_err("workspace of %zu bytes: %s", need, hipGetErrorString(st));
            return QA_STATUS_OOM;
        }
        e->ws_size = need;
    }
    // the tables, laid out as in the workspace: in the pinned staging buffer
    // (grown on demand), or with a fixed workspace in pageable host memory
    std::vector<char> host_tables;
    char* tables = nullptr;
    if (fixed) {
        host_tables.resize(table_bytes);
        tables = host_tables.data();
    } else {
        if (table_bytes > e->pinned_size) {
            if (e->pinned) { (void)hipHostFree(e->pinned); e->pinned = nullptr; e->pinned_size = 0; }
            hipError_t st = hipHostMalloc(&e->pinned, table_bytes, hipHostMallocDefault);
            if (st != hipSuccess) { set_err("pinned staging: %s", hipGetErrorString(st)); return QA_STATUS_OOM; }
            e->pinned_size = table_bytes;
        }
        tables = e->pinned;
    }
    memcpy(tables + o_clips, clips.data(), clips.size() * sizeof(qa::ClipInfo));
    memcpy(tables + o_tiles, tiles.data(), tiles.size() * sizeof(qa::FrontTile));
    memcpy(tables + o_chunks, chunks.data(), chunks.size() * sizeof(qa::ChunkInfo));
    memcpy(tables + o_src, tok_src.data(), tok_src.size() * 4);
    memcpy(tables + o_cu, cu.data(), cu.size() * 4);

    char* ws = fixed ? fixed->base : e->ws;
    auto P = [&](size_t o) { return ws + o; };
    const auto* d_clips = reinterpret_cast<const qa::ClipInfo*>(P(o_clips));
    const auto* d_tiles = reinterpret_cast<const qa::FrontTile*>(P(o_tiles));
    const auto* d_chunks = reinterpret_cast<const qa::ChunkInfo*>(P(o_chunks));
    const int* d_src = reinterpret_cast<const int*>(P(o_src));
    const int* d_cu = reinterpret_cast<const int*>(P(o_cu));
    float* logmel = reinterpret_cast<float*>(P(o_logmel));
    int* key = reinterpret_cast<int*>(P(o_key));
    int* flag = reinterpret_cast<int*>(P(o_flag));
    T* c1 = reinterpret_cast<T*>(P(o_c1));
    T* c2 = reinterpret_cast<T*>(P(o_c2));
    T* c3 = reinterpret_cast<T*>(P(o_c3));
    float* x = reinterpret_cast<float*>(P(o_x));
    T* h = reinterpret_cast<T*>(P(o_h));
    T* qkv = reinterpret_cast<T*>(P(o_qkv));
    T* att = reinterpret_cast<T*>(P(o_att));
    T* u = reinterpret_cast<T*>(P(o_u));
    float* tstem = taps ? reinterpret_cast<float*>(P(o_tstem)) : nullptr;
    float* tl0 = taps ? reinterpret_cast<float*>(P(o_tl0)) : nullptr;
    float* part = part_elems ? reinterpret_cast<float*>(P(o_part)) : nullptr;
    hipStream_t s = e->stream;

    // ---------------- launches
    e->prof_cur.clear();
    size_t ev_next = 0;
    // events go on the stream the launch is enqueued on (a lane's, past the fork)
    auto launch = [&](const char* label, hipStream_t ls, auto&& fn) -> hipError_t {
        if (!profiling || (!e->prof_only.empty() && e->prof_only != label)) return fn();
        while (e->ev_pool.size() < ev_next + 2) {
            hipEvent_t ev;
            hipError_t st = hipEventCreate(&ev);
            if (st != hipSuccess) return st;
            e->ev_pool.push_back(ev);
        }
        hipEvent_t a = e->ev_pool[ev_next++], b = e->ev_pool[ev_next++];
        hipError_t st = hipEventRecord(a, ls);
        if (st == hipSuccess) st = fn();
        if (st == hipSuccess) st = hipEventRecord(b, ls);
        e->prof_cur.push_back(Profile{label, a, b});
        return st;
    };
#define QA_LAUNCH(label, expr)                                                              \
    do {                                                                                    \
        hipError_t st_ = launch(label, s, [&]() { return (expr); });                       \
        if (st_ != hipSuccess) {                                                            \
            set_err("%s: %s", label, hipGetErrorString(st_));                              \
            (void)hipGetLastError();                                                        \
            return QA_STATUS_ENCODE_FAILED;                                                 \
        }                                                                                   \
    } while (0)

    // (from pageable memory the copy is staged before the call returns;
    // host_tables outlives the stream synchronisation below either way)
    QA_LAUNCH("tables", hipMemcpyAsync(ws, tables, table_bytes, hipMemcpyHostToDevice, s));
    QA_LAUNCH("init", qa::init_flags(s, key, n_clips, flag));
    QA_LAUNCH("frontend", qa::frontend(s, pcm, d_clips, d_tiles, n_tiles, e->W<uint4>(e->basis), e->W<float>(e->melw),
                                       e->W<int>(e->melb0), logmel, key, flag));
    QA_LAUNCH("normalize", qa::normalize(s, logmel, d_clips, d_tiles, n_tiles, key));
    // The first stem kernel (the fused conv1 + conv2, or conv1) over every chunk
    if constexpr (std::is_same<T, qa::bf16>::value) {
        if (fused_stem)
            QA_LAUNCH("stem12", qa::stem12(s, logmel, d_chunks, n_chunks, e->W<uint4>(e->conv1_frag), e->W<T>(e->conv2_w),
                                           e->W<float>(e->conv2_b), C, c2, flag + 1));
        else
            QA_LAUNCH("conv1", qa::conv1<T>(s, logmel, d_chunks, n_chunks, e->W<float>(e->conv1_w), e->W<float>(e->conv1_b), C, c1));
    } else {
        QA_LAUNCH("conv1", qa::conv1<T>(s, logmel, d_chunks, n_chunks, e->W<float>(e->conv1_w), e->W<float>(e->conv1_b), C, c1));
    }
    // From there on a large batch runs as two or three lanes: the tokens
    // split at the attention windows whose starts are nearest the even split
    // points (chunk boundaries), and each part runs the rest of its stem
    // chunks, conv_out, the layers and the projection on a stream of its own
    // (the caller's, then the encoder's own streams).  One part's tiles then
    // fill the CUs that another part's last round of tiles leaves idle.  Rows (chunks, tokens) are
    // independent in every kernel and no window crosses the split, so the
    // outputs are bit-identical to one lane's.  Not with taps or with
    // profiling of every launch (one lane: each kernel's time is its own; with
    // profiling restricted to one label the lanes stay, and a launch in a lane
    // is timed on that lane's stream), nor for the small batches that take
    // split-K (one workspace for the partial sums).
    const bool every_launch = profiling && e->prof_only.empty();
    const int lanes = (e->max_lanes > 1 && !taps && !every_launch && n_tok > kSplitKMaxTokens)
                          ? std::min({e->max_lanes, n_win, n_tok <= kMidLaneTokens ? 3 : 2}) : 1;
    // If a launch fails after the fork, the call returns early: wait for what
    // the other streams already hold, so that no work of this call outlives it
    // (the next call may grow, and so free, the workspace).
    struct LaneGuard {
        hipStream_t lane[kMaxLanes - 1] = {};
        ~LaneGuard() {
            for (hipStream_t l : lane)
                if (l) (void)hipStreamSynchronize(l);
        }
    } lane_guard;
    // lane g takes windows [gw[g], gw[g + 1]): the split points are the window
    // starts nearest g n_tok / lanes (distinct, increasing)
    int gw[kMaxLanes + 1] = {0};
    gw[lanes] = n_win;
    for (int g = 1; g < lanes; ++g) {
        int best = gw[g - 1] + 1;
        for (int w = best + 1; w <= n_win - (lanes - g); ++w)
            if (std::abs((int64_t)lanes * cu[w] - (int64_t)g * n_tok) < std::abs((int64_t)lanes * cu[best] - (int64_t)g * n_tok))
                best = w;
        gw[g] = best;
    }
    hipStream_t gs[kMaxLanes] = {s};
    if (lanes > 1) {
        QA_LAUNCH("fork", hipEventRecord(e->ev_fork, s));
        for (int g = 1; g < lanes; ++g) {
            lane_guard.lane[g - 1] = e->lane[g - 1];
            gs[g] = e->lane[g - 1];
            QA_LAUNCH("fork", hipStreamWaitEvent(gs[g], e->ev_fork, 0));
        }
    }
    float* gpart = lanes > 1 ? nullptr : part;
    const size_t gpe = lanes > 1 ? 0 : part_elems;
    const int UF = std::max(F, D);
    // The LayerNorm after a residual GEMM (conv_out, O-proj, FC2) runs inside
    // that GEMM's split-K reduction when it splits K (small batches); ln_ready
    // says that lane's h already holds the next LayerNorm's output.
    bool ln_ready[kMaxLanes] = {};
    auto ln_of = [&](int l, bool second) -> std::pair<const float*, const float*> {
        if (l >= d.n_layers) return {e->W<float>(e->post_ln_w), e->W<float>(e->post_ln_b)};
        const LayerW& lw = e->layers[l];
        return second ? std::make_pair(e->W<float>(lw.ln2_w), e->W<float>(lw.ln2_b))
                      : std::make_pair(e->W<float>(lw.ln1_w), e->W<float>(lw.ln1_b));
    };
    // layer l of lane g; l == -2: the stem, -1: conv_out, n_layers: the final LN and projection
    for (int l = -2; l <= d.n_layers; ++l) {
        for (int g = 0; g < lanes; ++g) {
            const hipStream_t s = gs[g];
            const int w0 = gw[g], nw = gw[g + 1] - w0, t0 = cu[w0], nt = cu[gw[g + 1]] - t0;
            if (l == -2) {   // the lane's chunks: windows start at chunk boundaries
                const int k0 = tok_src[t0] / qa::kChunkTok;
                const int nk = (g + 1 < lanes ? tok_src[cu[gw[g + 1]]] / qa::kChunkTok : n_chunks) - k0;
                T* c1g = c1 + (size_t)k0 * 64 * 50 * C;
                T* c2g = c2 + (size_t)k0 * 32 * 25 * C;
                if (!fused_stem)   // NHWC conv1 output (VALU conv1)
                    QA_LAUNCH("conv2", qa::conv3x3s2<T>(s, c1g, nk, 64, 50, C, e->W<T>(e->conv2_w), e->W<float>(e->conv2_b),
                                                        c2g, false, lanes));
                QA_LAUNCH("conv3", qa::conv3x3s2<T>(s, c2g, nk, 32, 25, C, e->W<T>(e->conv3_w), e->W<float>(e->conv3_b),
                                                    c3 + (size_t)k0 * 13 * 16 * C, true, lanes));
                if (taps)   // one lane
                    QA_LAUNCH("tap_stem", qa::conv_out<T>(s, c3, d_src, n_tok, 16 * C, e->W<T>(e->conv_out_w), D,
                                                          e->W<float>(e->pe), tl0, tstem, part, part_elems));
                continue;
            }
            float* xg = x + (size_t)t0 * D;
            T* hg = h + (size_t)t0 * D;
            T* qg = qkv + (size_t)t0 * 3 * D;
            T* ag = att + (size_t)t0 * D;
            T* ug = u + (size_t)t0 * UF;   // fc1 rows of F, the projection's of D
            if (l < 0) {
                const auto nx = ln_of(0, false);
                qa::LnAfter<T> after{nx.first, nx.second, hg, false};
                QA_LAUNCH("conv_out", qa::conv_out<T>(s, c3, d_src + t0, nt, 16 * C, e->W<T>(e->conv_out_w), D,
                                                      e->W<float>(e->pe), xg, nullptr, gpart, gpe, lanes, &after));
                ln_ready[g] = after.done;
                continue;
            }
            if (l == d.n_layers) {
                if (!ln_ready[g])
                    QA_LAUNCH("ln", qa::layernorm<T>(s, xg, nt, D, e->W<float>(e->post_ln_w), e->W<float>(e->post_ln_b), hg));
                QA_LAUNCH("proj1", qa::gemm_bias<T>(s, hg, nt, D, e->W<T>(e->proj1_w), D, e->W<float>(e->proj1_b), ug,
                                                    true, lanes));
                QA_LAUNCH("proj2", qa::gemm_bias_f32<T>(s, ug, nt, D, e->W<T>(e->proj2_w), O, e->W<float>(e->proj2_b),
                                                        out + (size_t)t0 * O, lanes));
                continue;
            }
            const LayerW& lw = e->layers[l];
            if (!ln_ready[g])
                QA_LAUNCH("ln", qa::layernorm<T>(s, xg, nt, D, e->W<float>(lw.ln1_w), e->W<float>(lw.ln1_b), hg));
            QA_LAUNCH("qkv", qa::gemm_bias<T>(s, hg, nt, D, e->W<T>(lw.qkv_w), 3 * D, e->W<float>(lw.qkv_b), qg, false,
                                              lanes));
            // window offsets are absolute token rows
            QA_LAUNCH("attention", qa::attention<T>(s, qkv, d_cu + w0, nw, d.n_heads, D, max_seg, att));
            qa::LnAfter<T> after2{e->W<float>(lw.ln2_w), e->W<float>(lw.ln2_b), hg, false};
            QA_LAUNCH("o_proj", qa::gemm_bias_resid<T>(s, ag, nt, D, e->W<T>(lw.o_w), D, e->W<float>(lw.o_b), xg,
                                                       gpart, gpe, lanes, &after2));
            if (!after2.done)
                QA_LAUNCH("ln", qa::layernorm<T>(s, xg, nt, D, e->W<float>(lw.ln2_w), e->W<float>(lw.ln2_b), hg));
            QA_LAUNCH("fc1", qa::gemm_bias<T>(s, hg, nt, D, e->W<T>(lw.fc1_w), F, e->W<float>(lw.fc1_b), ug, true,
                                              lanes));
            const auto nx = ln_of(l + 1, false);
            qa::LnAfter<T> after1{nx.first, nx.second, hg, false};
            QA_LAUNCH("fc2", qa::gemm_bias_resid<T>(s, ug, nt, F, e->W<T>(lw.fc2_w), D, e->W<float>(lw.fc2_b), xg,
                                                    gpart, gpe, lanes, &after1));
            ln_ready[g] = after1.done;
            if (l == 0 && taps)
                QA_LAUNCH("tap_layer0", hipMemcpyAsync(tl0, x, (size_t)n_tok * D * 4, hipMemcpyDeviceToDevice, s));
        }
    }
    for (int g = 1; g < lanes; ++g) {
        QA_LAUNCH("join", hipEventRecord(e->ev_join[g - 1], gs[g]));
        QA_LAUNCH("join", hipStreamWaitEvent(s, e->ev_join[g - 1], 0));
        lane_guard.lane[g - 1] = nullptr;   // the caller's stream now waits for this one
    }
    QA_LAUNCH("flag", hipMemcpyAsync(e->flag_host, flag, sizeof(int), hipMemcpyDeviceToHost, s));
#undef QA_LAUNCH
    hipError_t st = hipStreamSynchronize(s);
    if (st != hipSuccess) {
        set_err("stream synchronize: %s", hipGetErrorString(st));
        return QA_STATUS_ENCODE_FAILED;
    }
    if (profiling) {
        for (const Profile& p : e->prof_cur) {
            float ms = 0.f;
            if (hipEventElapsedTime(&ms, p.a, p.b) == hipSuccess) {
                auto& acc = e->prof_acc[p.label];
                acc.first += ms;
                acc.second += 1;
            }
        }
    }
    if (taps) {
        e->tap_frames = n_frames;
        e->tap_tokens = n_tok;
        e->tap_logmel = logmel;
        e->tap_stem = tstem;
        e->tap_layer0 = tl0;
    }
    if (*e->flag_host) {
        set_err("input rejected: a nonfinite sample or a mel energy beyond float32 range");
        return QA_STATUS_INVALID_PARAMS;
    }
    return QA_STATUS_OK;
}

}  // namespace

namespace {

int encode_entry(qa_encoder* e, const float* pcm, const int64_t* lengths, int n_clips, float* out, bool noalloc) {
    if (!e) { set_err("encoder is NULL"); return QA_STATUS_INVALID_PARAMS; }
    if (n_clips < 0) { set_err("n_clips < 0"); return QA_STATUS_INVALID_PARAMS; }
    if (n_clips > 0 && !lengths) { set_err("lengths is NULL"); return QA_STATUS_INVALID_PARAMS; }
    int64_t total = 0, frames = 0;
    for (int i = 0; i < n_clips; ++i) {
        if (!valid_len(lengths[i])) {
            set_err("clip %d has %lld samples: must be 0 or in 201..%lld", i, (long long)lengths[i],
                    (long long)kMaxSamples);
            return QA_STATUS_INVALID_PARAMS;
        }
        if (e->d.window_chunks == 0 && lengths[i] > kMaxFullInput) {
            set_err("clip %d has %lld samples: full-input attention takes clips of at most 30 s (%lld)", i,
                    (long long)lengths[i], (long long)kMaxFullInput);
            return QA_STATUS_INVALID_PARAMS;
        }
        total += lengths[i];
        frames += lengths[i] / kHop;
    }
    // the kernels index frames, chunk rows and tokens with 32-bit integers
    if (frames * qa::kMels > INT32_MAX || total > ((int64_t)1 << 40)) {
        set_err("batch too large: %lld frames", (long long)frames);
        return QA_STATUS_INVALID_PARAMS;
    }
    hipError_t st = hipSetDevice(e->device);
    if (st != hipSuccess) { set_err("hipSetDevice: %s", hipGetErrorString(st)); return QA_STATUS_ENCODE_FAILED; }
    FixedWorkspace fw{nullptr, 0};
    if (noalloc) {
        fw.base = static_cast<char*>(scratch_address(e->device));
        if (!fw.base) {
            std::lock_guard<std::mutex> lock(g_scratch_mu);
            set_err("no scratch array on device %d: %s", e->device,
                    e->device >= 0 && e->device < kMaxDevices ? hipGetErrorString(g_scratch_err[e->device])
                                                              : "device id out of range");
            return QA_STATUS_ENCODE_FAILED;
        }
        fw.bytes = kScratchBytes;
    }
    const FixedWorkspace* f = noalloc ? &fw : nullptr;
    if (e->d.dtype == QA_DTYPE_BF16) return run_encode<bf16>(e, pcm, lengths, n_clips, out, f);
    return run_encode<float>(e, pcm, lengths, n_clips, out, f);
}

}  // namespace

QA_API int qa_encode(qa_encoder* e, const float* pcm, const int64_t* lengths, int n_clips, float* out) {
    return encode_entry(e, pcm, lengths, n_clips, out, false);
}

QA_API int qa_encode_noalloc(qa_encoder* e, const float* pcm, const int64_t* lengths, int n_clips, float* out) {
    return encode_entry(e, pcm, lengths, n_clips, out, true);
}
