// Resampling to 16 kHz, the step in front of the log-mel front end
// (qwenasr.cpp ARCHITECTURE.md, "Upstream model": any input is resampled to
// 16 kHz mono before the frontend; "Module map": a Kaiser polyphase
// resampler).  The page names the method only; the filter is this library's
// reading:
//   * up / down = 16000 / rate reduced by their gcd;
//   * a linear-phase low-pass FIR of 2 half + 1 taps, half = 10 max(up, down),
//     cut-off 1 / max(up, down) of the upsampled Nyquist frequency, Kaiser
//     window beta = 5, unit gain at DC, then scaled by up;
//   * output n is the filtered zero-stuffed input at upsampled index n down
//     (zero delay), with zeros outside the clip; n_out = ceil(n_in up / down).
//
// Two kernels compute it: resample_phase_kernel (tables of at most 64 taps per
// phase and 1,024 phases, i.e. the common rates: each thread keeps one
// phase's row in registers, see there) and resample_kernel (any table).
//
// Polyphase form: of the 2 half + 1 taps only those landing on original
// samples contribute, i.e. taps p + j up with p = (n down + half) mod up, so
// output n is a dot product of one table row hp[p][0..L) (L = ceil(taps / up),
// zero padded) with the input samples q, q - 1, ..., q = (n down + half) / up.
// Each output reads its L taps and L samples from LDS, so the kernel is bound
// by LDS reads, not by HBM (4 bytes read per input sample, 4 written per
// output sample).  Neighbouring outputs use different table rows; the LDS
// copy of the table has a row stride of 4 x (an odd number) floats, so the
// 16-byte tap reads of 16 lanes land in 16 different bank groups whenever
// their phases differ modulo 16 (for 44.1 kHz the phase steps by 121 of 160
// per output).
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <new>
#include <numeric>
#include <vector>

#include "../../include/qa_encoder.h"
#include "qa_device.h"
#include "qa_kernels.h"

#define QA_API extern "C" __attribute__((visibility("default")))

namespace qa {

constexpr int kResampleTarget = 16000;
constexpr int kResampleMinRate = 1000, kResampleMaxRate = 768000;
constexpr double kResampleBeta = 5.0;
constexpr int kResampleHalfFactor = 10;

constexpr int kResampleThreads = 256;
constexpr int kResampleMaxWindow = 16384;      // staged input samples per workgroup (64 KB of LDS)
constexpr int kResampleMaxLdsTable = 12288;    // tables up to 48 KB (padded rows) are staged in LDS too
constexpr int kResamplePhaseWindow = 8192;     // the phase-major kernel's window target (32 KB of LDS)

// LDS row stride of the table: L (a multiple of 4) rounded up to 4 x an odd number.
__host__ __device__ constexpr int resample_lds_row(int L) { return (L / 4) % 2 ? L : L + 4; }

// A block of opb = 256 OPT consecutive outputs reads a contiguous input
// window; each thread forms OPT of them as dot products of one table row (L
// taps, a multiple of 4, zero padded; read as float4) with the window staged
// in LDS (zeros outside the clip, so the taps need no bounds checks), in four
// partial sums.  The grid is persistent: a workgroup stages the table once
// and then walks the output blocks blockIdx.x, blockIdx.x + gridDim.x, ...
template <int OPT, bool TLDS>
__global__ __launch_bounds__(kResampleThreads) void resample_kernel(const float* __restrict__ x, int64_t n_in,
                                                                    float* __restrict__ y, int64_t n_out,
                                                                    const float* __restrict__ hp, int up, int down,
                                                                    int half, int L, int64_t n_blocks) {
    extern __shared__ float xs[];
    constexpr int opb = kResampleThreads * OPT;
    // table first (16-byte aligned at the start of LDS, rows of LT floats),
    // then the window
    const int LT = resample_lds_row(L);
    float* tab = xs;
    float* win = TLDS ? xs + up * LT : xs;
    if (TLDS) {
        const float4* src = reinterpret_cast<const float4*>(hp);
        float4* dst = reinterpret_cast<float4*>(tab);
        for (int i = threadIdx.x; i < up * L / 4; i += kResampleThreads) {
            const int row = i / (L / 4), c = i - row * (L / 4);
            dst[row * (LT / 4) + c] = src[i];
        }
    }
    for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x) {
        const int64_t n0 = blk * opb;
        const int64_t n_last = (n0 + opb < n_out ? n0 + opb : n_out) - 1;
        const int64_t lo = (n0 * down + half) / up - (L - 1);           // lowest input sample read
        const int cnt = (int)((n_last * down + half) / up - lo + 1);   // <= kResampleMaxWindow (host-checked)
        __syncthreads();                                                // previous window consumed
        // eight loads in flight per thread before their LDS stores
        for (int i0 = 0; i0 < cnt; i0 += 8 * kResampleThreads) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kResampleThreads + threadIdx.x;
                const int64_t g = lo + i;
                v[u] = i < cnt && g >= 0 && g < n_in ? x[g] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = i0 + u * kResampleThreads + threadIdx.x;
                if (i < cnt) win[i] = v[u];
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < OPT; ++k) {
            const int64_t n = n0 + threadIdx.x + k * kResampleThreads;
            if (n > n_last) break;
            const int64_t t = n * down + half;          // upsampled index met by tap 0
            const int p = (int)(t % up);
            const int qs = (int)(t / up - lo);           // staged index of input sample q = t / up
            const float4* hr =
                reinterpret_cast<const float4*>(TLDS ? tab + (size_t)p * LT : hp + (size_t)p * L);
            float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
            for (int j4 = 0; j4 < L / 4; ++j4) {         // tap p + j up meets sample q - j
                const float4 h = hr[j4];
                const int b = qs - 4 * j4;
                a0 = fmaf(h.x, win[b], a0);
                a1 = fmaf(h.y, win[b - 1], a1);
                a2 = fmaf(h.z, win[b - 2], a2);
                a3 = fmaf(h.w, win[b - 3], a3);
            }
            y[n] = (a0 + a1) + (a2 + a3);
        }
    }
}

// Tables of up to 64 taps per phase and up to 1,024 phases (every rate the
// front end meets in practice: 44.1, 48, 22.05, 11.025, 8 kHz ...): outputs
// n and n + up use the same table row, so each thread takes the outputs of
// one phase and holds that row in registers for the whole kernel, and only
// the input window is read from LDS (half the LDS traffic of
// resample_kernel, whose table reads cost as much LDS time as its window
// reads).  A workgroup of T = up C threads (C = ceil(256 / up) columns)
// covers blocks of M = T rows consecutive outputs (M a multiple of up, so
// thread (i, c) = (tid % up, tid / up) always has phase (i down + half) mod
// up) and stages each block's input window in LDS; the dot products and
// their summation order are resample_kernel's, so the outputs are the same.
template <int LQ>
__global__ __launch_bounds__(1024) void resample_phase_kernel(const float* __restrict__ x, int64_t n_in,
                                                              float* __restrict__ y, int64_t n_out,
                                                              const float* __restrict__ hp, int up, int down,
                                                              int half, int C, int rows, int64_t n_blocks) {
    extern __shared__ float win[];
    constexpr int L = 4 * LQ;
    const int T = (int)blockDim.x, tid = (int)threadIdx.x;
    const int i = tid % up, c = tid / up;
    const int64_t M = (int64_t)T * rows;
    const int p = (int)(((int64_t)i * down + half) % up);
    float4 h[LQ];
    const float4* hr = reinterpret_cast<const float4*>(hp + (size_t)p * L);
#pragma unroll
    for (int j4 = 0; j4 < LQ; ++j4) h[j4] = hr[j4];
    for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x) {
        const int64_t n0 = blk * M;
        const int64_t n_last = (n0 + M < n_out ? n0 + M : n_out) - 1;
        const int64_t lo = (n0 * down + half) / up - (L - 1);           // lowest input sample read
        const int cnt = (int)((n_last * down + half) / up - lo + 1);   // <= the staged window (host-checked)
        __syncthreads();                                                // previous window consumed
        for (int i0 = 0; i0 < cnt; i0 += 8 * T) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = i0 + u * T + tid;
                const int64_t g = lo + k;
                v[u] = k < cnt && g >= 0 && g < n_in ? x[g] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = i0 + u * T + tid;
                if (k < cnt) win[k] = v[u];
            }
        }
        __syncthreads();
        for (int r = 0; r < rows; ++r) {
            const int64_t n = n0 + ((int64_t)r * C + c) * up + i;
            if (n > n_last) break;
            const int64_t t = n * down + half;           // upsampled index met by tap 0
            const int qs = (int)(t / up - lo);           // staged index of input sample q = t / up
            float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
#pragma unroll
            for (int j4 = 0; j4 < LQ; ++j4) {            // tap p + j up meets sample q - j
                const int b = qs - 4 * j4;
                a0 = fmaf(h[j4].x, win[b], a0);
                a1 = fmaf(h[j4].y, win[b - 1], a1);
                a2 = fmaf(h[j4].z, win[b - 2], a2);
                a3 = fmaf(h[j4].w, win[b - 3], a3);
            }
            y[n] = (a0 + a1) + (a2 + a3);
        }
    }
}

}  // namespace qa

struct qa_resampler {
    int rate = 0, up = 1, down = 1, half = 0, L = 0;
    float* table = nullptr;     // device [up][L]
};

namespace {

// I0 by its power series sum_k ((z / 2)^k / k!)^2.
double bessel_i0(double z) {
    double term = 1.0, total = 1.0;
    for (int k = 1; k < 500; ++k) {
        term *= (z / (2.0 * k)) * (z / (2.0 * k));
        total += term;
        if (term <= 1e-17 * total) break;
    }
    return total;
}

bool valid_rate(int rate) { return rate >= qa::kResampleMinRate && rate <= qa::kResampleMaxRate; }

}  // namespace

QA_API int64_t qa_resample_length(int64_t n_in, int rate_in) {
    if (n_in < 0 || !valid_rate(rate_in)) {
        qa::set_error_message("qa_resample_length: n_in must be >= 0 and rate_in in 1000..768000");
        return -1;
    }
    const int64_t g = std::gcd(qa::kResampleTarget, rate_in);
    const int64_t up = qa::kResampleTarget / g, down = rate_in / g;
    return (n_in * up + down - 1) / down;
}

QA_API qa_resampler* qa_resampler_create(int rate_in) {
    if (!valid_rate(rate_in)) {
        qa::set_error_message("qa_resampler_create: rate_in must be in 1000..768000 Hz");
        return nullptr;
    }
    qa_resampler* r = new (std::nothrow) qa_resampler();
    if (!r) { qa::set_error_message("qa_resampler_create: host allocation failed"); return nullptr; }
    const int g = std::gcd(qa::kResampleTarget, rate_in);
    r->rate = rate_in;
    r->up = qa::kResampleTarget / g;
    r->down = rate_in / g;
    const int mx = r->up > r->down ? r->up : r->down;
    r->half = qa::kResampleHalfFactor * mx;
    const int taps = 2 * r->half + 1;
    r->L = ((taps + r->up - 1) / r->up + 3) / 4 * 4;   // taps per phase, padded to a multiple of 4
    // Kaiser-windowed sinc low-pass, cut-off fc = 1 / max(up, down), unit DC gain
    std::vector<double> h(taps);
    const double fc = 1.0 / mx, i0b = bessel_i0(qa::kResampleBeta);
    double sum = 0.0;
    for (int k = 0; k < taps; ++k) {
        const double m = k - r->half;
        const double arg = M_PI * fc * m;
        const double sinc = m == 0 ? 1.0 : std::sin(arg) / arg;
        const double rr = 2.0 * k / (taps - 1) - 1.0;
        const double w = bessel_i0(qa::kResampleBeta * std::sqrt(std::max(0.0, 1.0 - rr * rr))) / i0b;
        h[k] = fc * sinc * w;
        sum += h[k];
    }
    std::vector<float> table((size_t)r->up * r->L, 0.0f);
    for (int k = 0; k < taps; ++k) table[(size_t)(k % r->up) * r->L + k / r->up] = (float)(h[k] / sum * r->up);
    if (hipMalloc(&r->table, table.size() * sizeof(float)) != hipSuccess ||
        hipMemcpy(r->table, table.data(), table.size() * sizeof(float), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipGetLastError();
        if (r->table) (void)hipFree(r->table);
        delete r;
        qa::set_error_message("qa_resampler_create: device allocation or copy failed");
        return nullptr;
    }
    return r;
}

QA_API int qa_resample(qa_resampler* r, void* hip_stream, const float* in, int64_t n_in, float* out) {
    if (!r || n_in < 0 || (n_in > 0 && (!in || !out))) {
        qa::set_error_message("qa_resample: bad arguments");
        return QA_STATUS_INVALID_PARAMS;
    }
    const int64_t n_out = qa_resample_length(n_in, r->rate);
    if (n_out == 0) return QA_STATUS_OK;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    hipStream_t s = static_cast<hipStream_t>(hip_stream);
    if (r->L <= 64 && r->up <= 1024) {
        // phase-major kernel: T = up C threads, blocks of T rows outputs whose
        // window stays within kResamplePhaseWindow samples
        const int C = r->up >= 256 ? 1 : (256 + r->up - 1) / r->up, T = r->up * C;
        auto window = [&](int64_t m) { return (m - 1) * r->down / r->up + 2 + r->L; };
        int rows = 8;
        while (rows > 1 && window((int64_t)T * rows) > qa::kResamplePhaseWindow) --rows;
        if (window((int64_t)T * rows) <= qa::kResampleMaxWindow) {
            const int64_t M = (int64_t)T * rows, blocks = (n_out + M - 1) / M;
            const size_t lds = (size_t)window(M) * sizeof(float);
            const int per_cu = std::max(1, std::min({8, (int)(160 * 1024 / lds), 2048 / T}));
            const unsigned grid = (unsigned)std::min<int64_t>(blocks, (int64_t)cus * per_cu);
            switch (r->L / 4) {
#define QA_RSP(q) case q: qa::resample_phase_kernel<q><<<grid, T, lds, s>>>(in, n_in, out, n_out, r->table, r->up, \
                                                                        r->down, r->half, C, rows, blocks); break;
                QA_RSP(1) QA_RSP(2) QA_RSP(3) QA_RSP(4) QA_RSP(5) QA_RSP(6) QA_RSP(7) QA_RSP(8)
                QA_RSP(9) QA_RSP(10) QA_RSP(11) QA_RSP(12) QA_RSP(13) QA_RSP(14) QA_RSP(15) QA_RSP(16)
#undef QA_RSP
                default: break;
            }
            const hipError_t st = hipGetLastError();
            if (st != hipSuccess) {
                qa::set_error_message(hipGetErrorString(st));
                return QA_STATUS_ENCODE_FAILED;
            }
            return QA_STATUS_OK;
        }
    }
    // outputs per thread: the largest of 4, 2, 1 whose input window fits the LDS stage
    auto window = [&](int opb) { return (int64_t)(opb - 1) * r->down / r->up + 2 + r->L; };
    int opt = 4;
    while (opt > 1 && window(qa::kResampleThreads * opt) > qa::kResampleMaxWindow) opt /= 2;
    if (window(qa::kResampleThreads * opt) > qa::kResampleMaxWindow) {
        qa::set_error_message("qa_resample: filter too long for the staged window");
        return QA_STATUS_INVALID_PARAMS;
    }
    const int64_t opb = (int64_t)qa::kResampleThreads * opt;
    const int64_t blocks = (n_out + opb - 1) / opb;
    const int64_t lt = (int64_t)r->up * qa::resample_lds_row(r->L);
    const bool tlds = lt <= qa::kResampleMaxLdsTable;
    const size_t lds = ((size_t)window(qa::kResampleThreads * opt) + (tlds ? (size_t)lt : 0)) * sizeof(float);
    // persistent grid: a few workgroups per CU (as many as the LDS allows, at
    // most 4), each staging the table once
    const int per_cu = std::max(1, std::min(4, (int)(160 * 1024 / std::max<size_t>(lds, 1))));
    const unsigned grid = (unsigned)std::min<int64_t>(blocks, (int64_t)cus * per_cu);
#define QA_RS(o, t) qa::resample_kernel<o, t><<<grid, qa::kResampleThreads, lds, s>>>( \
        in, n_in, out, n_out, r->table, r->up, r->down, r->half, r->L, blocks)
    if (tlds) {
        if (opt == 4) QA_RS(4, true); else if (opt == 2) QA_RS(2, true); else QA_RS(1, true);
    } else {
        if (opt == 4) QA_RS(4, false); else if (opt == 2) QA_RS(2, false); else QA_RS(1, false);
    }
#undef QA_RS
    const hipError_t st = hipGetLastError();
    if (st != hipSuccess) {
        qa::set_error_message(hipGetErrorString(st));
        return QA_STATUS_ENCODE_FAILED;
    }
    return QA_STATUS_OK;
}

QA_API void qa_resampler_free(qa_resampler* r) {
    if (!r) return;
    if (r->table) (void)hipFree(r->table);
    delete r;
}
