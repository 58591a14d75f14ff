// MFMA GEMM family for gfx950: out = A . W^T with fused epilogues.
//
// One kernel template serves every contraction of the encoder:
//   * conv2 / conv3 of the stem as implicit GEMMs (A rows are output pixels,
//     K = 9 taps x C input channels gathered from NHWC input), + bias + GELU
//     (qwenasr.cpp ARCHITECTURE.md "Conv2d subsampling stem", "Conv2d stem");
//   * conv_out with a row gather (token -> chunk row) and the per-chunk
//     sinusoidal position table added in the epilogue ("Windowed audio tower";
//     OneSpeech "Front end and graph numerics": positions reset per chunk);
//   * q/k/v, FC1 (+GELU), proj1 (+GELU) with bias, bf16 out; O-proj and FC2
//     with bias added into the fp32 residual stream; proj2 to fp32 output.
//
// Layout: both operands are K-contiguous rows (activations [M][K], PyTorch
// Linear weights [N][K]).  A workgroup of WM x WN waves computes a BM x BN
// tile; LDS holds two stages of 128-byte K slices per row (64 bf16 or 32
// fp32 elements) with a 16-byte pad per row, so the 16-byte fragment reads of
// 8 consecutive rows hit disjoint banks.  The MFMA is issued transposed
// (weights as the A operand): lane l then holds 4 consecutive output columns
// of one output row, which makes bias loads and stores 8/16-byte vectors.
// Global loads of stage k+1 are in flight while stage k is multiplied.
#include "qa_device.h"
#include "qa_kernels.h"

namespace qa {

constexpr int kRowBytes = 144;   // 128 data bytes + 16 pad per LDS row

// ------------------------------------------------------------ A loaders
// prep(m) is evaluated once per thread and row; load(ctx, k0) returns the 16
// bytes of elements [k0, k0 + per16) of row m, or zeros outside the matrix.

template <typename T>
struct DenseA {
    const T* a;
    int M, K, lda;
    struct Ctx { const T* p; };
    __device__ Ctx prep(int m) const { return Ctx{m < M ? a + (size_t)m * lda : nullptr}; }
    __device__ uint4 load(const Ctx& c, int k0) const {
        return (c.p && k0 < K) ? ld16(c.p + k0) : zero16();
    }
};

template <typename T>
struct GatherA {   // row m of the GEMM is row src[m] of a
    const T* a;
    const int* src;
    int M, K;
    struct Ctx { const T* p; };
    __device__ Ctx prep(int m) const { return Ctx{m < M ? a + (size_t)src[m] * K : nullptr}; }
    __device__ uint4 load(const Ctx& c, int k0) const {
        return (c.p && k0 < K) ? ld16(c.p + k0) : zero16();
    }
};

template <typename T>
struct ConvA {     // implicit im2col of a 3x3 stride-2 pad-1 conv over NHWC input
    const T* in;
    int M, Hin, Win, C, Hout, Wout;
    bool time_major;                  // output row order (chunk, j, i) instead of (chunk, i, j)
    struct Ctx { const T* base; int r0, c0; };
    __device__ Ctx prep(int m) const {
        if (m >= M) return Ctx{nullptr, 0, 0};
        const int per = Hout * Wout;
        const int chunk = m / per, rem = m - chunk * per;
        int i, j;
        if (time_major) { j = rem / Hout; i = rem - j * Hout; }
        else            { i = rem / Wout; j = rem - i * Wout; }
        return Ctx{in + (size_t)chunk * Hin * Win * C, 2 * i - 1, 2 * j - 1};
    }
    __device__ uint4 load(const Ctx& c, int k0) const {
        if (!c.base || k0 >= 9 * C) return zero16();
        const int tap = k0 / C, ci = k0 - tap * C;
        const int a = tap / 3, b = tap - a * 3;
        const int r = c.r0 + a, col = c.c0 + b;
        if ((unsigned)r >= (unsigned)Hin || (unsigned)col >= (unsigned)Win) return zero16();
        return ld16(c.base + ((size_t)r * Win + col) * C + ci);
    }
};

// ------------------------------------------------------------ epilogues
// op(m, n, v): v holds out[m][n..n+3] before bias; n is a multiple of 4.

template <typename T>
struct EpiBias {           // out = acc + bias (optionally GELU), stored as T
    T* out;
    const float* bias;
    int M, N;
    bool gelu;
    __device__ void operator()(int m, int n, f32x4 v) const {
        if (m >= M || n >= N) return;
        const float4 b = *reinterpret_cast<const float4*>(bias + n);
        float x0 = v[0] + b.x, x1 = v[1] + b.y, x2 = v[2] + b.z, x3 = v[3] + b.w;
        if (gelu) { x0 = gelu_erf(x0); x1 = gelu_erf(x1); x2 = gelu_erf(x2); x3 = gelu_erf(x3); }
        store4(out + (size_t)m * N + n, x0, x1, x2, x3);
    }
};

struct EpiResid {          // x += acc + bias (fp32 residual stream)
    float* x;
    const float* bias;
    int M, N;
    __device__ void operator()(int m, int n, f32x4 v) const {
        if (m >= M || n >= N) return;
        const float4 b = *reinterpret_cast<const float4*>(bias + n);
        float4* p = reinterpret_cast<float4*>(x + (size_t)m * N + n);
        float4 r = *p;
        r.x += v[0] + b.x; r.y += v[1] + b.y; r.z += v[2] + b.z; r.w += v[3] + b.w;
        *p = r;
    }
};

struct EpiF32Bias {        // out = acc + bias, fp32
    float* out;
    const float* bias;
    int M, N;
    __device__ void operator()(int m, int n, f32x4 v) const {
        if (m >= M || n >= N) return;
        const float4 b = *reinterpret_cast<const float4*>(bias + n);
        store4(out + (size_t)m * N + n, v[0] + b.x, v[1] + b.y, v[2] + b.z, v[3] + b.w);
    }
};

struct EpiPE {             // x = acc + pe[src[m] % 13]; tap = acc
    float* x;
    float* tap;
    const float* pe;
    const int* src;
    int M, N;
    __device__ void operator()(int m, int n, f32x4 v) const {
        if (m >= M || n >= N) return;
        const int j = src[m] % kChunkTok;
        const float4 p = *reinterpret_cast<const float4*>(pe + (size_t)j * N + n);
        store4(x + (size_t)m * N + n, v[0] + p.x, v[1] + p.y, v[2] + p.z, v[3] + p.w);
        if (tap) store4(tap + (size_t)m * N + n, v[0], v[1], v[2], v[3]);
    }
};

// ------------------------------------------------------------ kernel

template <typename T, int BM, int BN, int WM, int WN, class AL, class EP>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(AL al, const T* __restrict__ w, int N, int K,
                                                            int tiles_m, EP ep) {
    constexpr int NT = WM * WN * 64;
    constexpr int TM = BM / WM / 16;          // 16-row MFMA tiles per wave along M
    constexpr int TN = BN / WN / 16;          // along N
    constexpr int PER = Elem<T>::per16;
    constexpr int ACH = BM * 8 / NT;          // 16-byte chunks per thread per stage
    constexpr int BCH = BN * 8 / NT;
    static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/threads mismatch");
    __shared__ __align__(16) char smem[2 * (BM + BN) * kRowBytes];
    char* As = smem;
    char* Bs = smem + 2 * BM * kRowBytes;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;
    const int bm = blockIdx.x % tiles_m, bn = blockIdx.x / tiles_m;
    const int m0 = bm * BM, n0 = bn * BN;

    const int col = tid & 7;                  // 16-byte column of the 128-byte slice
    typename AL::Ctx actx[ACH];
    const T* wrow[BCH];
#pragma unroll
    for (int q = 0; q < ACH; ++q) actx[q] = al.prep(m0 + tid / 8 + q * (NT / 8));
#pragma unroll
    for (int q = 0; q < BCH; ++q) {
        const int n = n0 + tid / 8 + q * (NT / 8);
        wrow[q] = n < N ? w + (size_t)n * K : nullptr;
    }
    uint4 ra[ACH], rb[BCH];
    auto gload = [&](int kt) {
        const int k0 = kt * (8 * PER) + col * PER;
#pragma unroll
        for (int q = 0; q < ACH; ++q) ra[q] = al.load(actx[q], k0);
#pragma unroll
        for (int q = 0; q < BCH; ++q) rb[q] = (wrow[q] && k0 < K) ? ld16(wrow[q] + k0) : zero16();
    };
    auto lstore = [&](int buf) {
        char* a = As + buf * BM * kRowBytes;
        char* b = Bs + buf * BN * kRowBytes;
#pragma unroll
        for (int q = 0; q < ACH; ++q) st16(a + (tid / 8 + q * (NT / 8)) * kRowBytes + col * 16, ra[q]);
#pragma unroll
        for (int q = 0; q < BCH; ++q) st16(b + (tid / 8 + q * (NT / 8)) * kRowBytes + col * 16, rb[q]);
    };

    f32x4 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = (K + 8 * PER - 1) / (8 * PER);
    gload(0);
    lstore(0);
    __syncthreads();
    const int fr = lane & 15, fg = lane >> 4;
    for (int kt = 0; kt < nk; ++kt) {
        if (kt + 1 < nk) gload(kt + 1);
        const char* a = As + (kt & 1) * BM * kRowBytes + (wm * TM * 16 + fr) * kRowBytes + fg * 16;
        const char* b = Bs + (kt & 1) * BN * kRowBytes + (wn * TN * 16 + fr) * kRowBytes + fg * 16;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            uint4 fa[TM], fb[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) fa[i] = ld16(a + i * 16 * kRowBytes + kb * 64);
#pragma unroll
            for (int j = 0; j < TN; ++j) fb[j] = ld16(b + j * 16 * kRowBytes + kb * 64);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) mfma_kblock(T(), fb[j], fa[i], acc[i][j]);
        }
        if (kt + 1 < nk) lstore((kt + 1) & 1);
        __syncthreads();
    }
    // acc[i][j] lane holds out[m = row fr][n = 4 fg + r] of tile (i, j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            ep(m0 + (wm * TM + i) * 16 + fr, n0 + (wn * TN + j) * 16 + 4 * fg, acc[i][j]);
}

template <typename T, int BM, int BN, int WM, int WN, class AL, class EP>
static hipError_t run(hipStream_t s, const AL& al, int M, const T* w, int N, int K, const EP& ep) {
    if (M <= 0 || N <= 0) return hipSuccess;
    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    gemm_kernel<T, BM, BN, WM, WN, AL, EP><<<tm * tn, WM * WN * 64, 0, s>>>(al, w, N, K, tm, ep);
    return hipGetLastError();
}

// ------------------------------------------------------------ entry points

template <typename T>
hipError_t conv3x3s2(hipStream_t s, const T* in, int n_chunks, int Hin, int Win, int C,
                     const T* w, const float* bias, T* out, bool time_major) {
    const int Hout = (Hin + 1) / 2, Wout = (Win + 1) / 2;
    const int M = n_chunks * Hout * Wout;
    ConvA<T> al{in, M, Hin, Win, C, Hout, Wout, time_major};
    EpiBias<T> ep{out, bias, M, C, true};
    return run<T, 128, 128, 2, 2>(s, al, M, w, C, 9 * C, ep);
}

template <typename T>
hipError_t conv_out(hipStream_t s, const T* a, const int* src, int n_tok, int K, const T* w, int N,
                    const float* pe, float* x, float* tap) {
    GatherA<T> al{a, src, n_tok, K};
    EpiPE ep{x, tap, pe, src, n_tok, N};
    return run<T, 128, 128, 2, 2>(s, al, n_tok, w, N, K, ep);
}

template <typename T>
hipError_t gemm_bias(hipStream_t s, const T* a, int M, int K, const T* w, int N, const float* bias,
                     T* out, bool gelu) {
    DenseA<T> al{a, M, K, K};
    EpiBias<T> ep{out, bias, M, N, gelu};
    return run<T, 128, 128, 2, 2>(s, al, M, w, N, K, ep);
}

template <typename T>
hipError_t gemm_bias_resid(hipStream_t s, const T* a, int M, int K, const T* w, int N,
                           const float* bias, float* x) {
    DenseA<T> al{a, M, K, K};
    EpiResid ep{x, bias, M, N};
    return run<T, 128, 128, 2, 2>(s, al, M, w, N, K, ep);
}

template <typename T>
hipError_t gemm_bias_f32(hipStream_t s, const T* a, int M, int K, const T* w, int N,
                         const float* bias, float* out) {
    DenseA<T> al{a, M, K, K};
    EpiF32Bias ep{out, bias, M, N};
    return run<T, 128, 128, 2, 2>(s, al, M, w, N, K, ep);
}

#define QA_INST(T)                                                                                    \
    template hipError_t conv3x3s2<T>(hipStream_t, const T*, int, int, int, int, const T*, const float*, \
                                     T*, bool);                                                       \
    template hipError_t conv_out<T>(hipStream_t, const T*, const int*, int, int, const T*, int,        \
                                    const float*, float*, float*);                                    \
    template hipError_t gemm_bias<T>(hipStream_t, const T*, int, int, const T*, int, const float*, T*, \
                                     bool);                                                           \
    template hipError_t gemm_bias_resid<T>(hipStream_t, const T*, int, int, const T*, int,            \
                                           const float*, float*);                                     \
    template hipError_t gemm_bias_f32<T>(hipStream_t, const T*, int, int, const T*, int, const float*, \
                                         float*);
QA_INST(float)
QA_INST(bf16)

}  // namespace qa
