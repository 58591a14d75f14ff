// First convolution of the conv stem: conv2d k3 s2 p1 (1 -> C channels) + bias
// + erf-GELU over each 100-frame chunk of the normalised log-mel, seen as a
// one-channel image [128 mel, 100 time] (qwenasr.cpp ARCHITECTURE.md "Conv2d
// subsampling stem"; OneSpeech "Front end and graph numerics": chunks of 100
// frames, each padded independently -- the frames past a tail chunk's end are
// zeros).
//
// K = 9 per output, so this is VALU work: each thread owns 8 output channels
// (weights in registers) and walks pixels; the 17 input mel rows a block of 8
// output rows needs are staged in LDS.  Output is NHWC [chunk][64][50][C], the
// layout the implicit-GEMM conv2 reads 16 bytes at a time.
#include "qa_device.h"
#include "qa_kernels.h"

namespace qa {

constexpr int kC1RowsPerBlock = 8;                   // output mel rows per workgroup
constexpr int kC1InRows = 2 * kC1RowsPerBlock + 1;   // input mel rows needed
constexpr int kC1Hout = 64, kC1Wout = 50;

template <typename T>
__global__ __launch_bounds__(256) void conv1_kernel(const float* __restrict__ logmel,
                                                    const ChunkInfo* __restrict__ chunks,
                                                    const float* __restrict__ w9c,
                                                    const float* __restrict__ bias, int C,
                                                    T* __restrict__ out) {
    __shared__ float img[kC1InRows][kChunk + 4];     // [mel row][time], time index + 1 (pad col 0)
    const int chunk = blockIdx.x;
    const int rb = blockIdx.y;
    const ChunkInfo ci = chunks[chunk];
    const int r0 = 2 * rb * kC1RowsPerBlock - 1;     // first input mel row (may be -1)
    for (int idx = threadIdx.x; idx < kC1InRows * (kChunk + 2); idx += blockDim.x) {
        const int rr = idx / (kChunk + 2), tt = idx % (kChunk + 2) - 1;   // tt in [-1, 100]
        const int f = r0 + rr;
        float v = 0.0f;
        if (f >= 0 && f < kMels && tt >= 0 && tt < ci.m) v = logmel[(size_t)(ci.frame_row0 + tt) * kMels + f];
        img[rr][tt + 1] = v;
    }
    __syncthreads();

    const int cg_n = C / 8;
    const int lanes_px = blockDim.x / cg_n;
    const int cg = threadIdx.x % cg_n;
    const int pl = threadIdx.x / cg_n;
    if (pl >= lanes_px) return;
    const int c0 = cg * 8;
    float w[9][8], b[8];
#pragma unroll
    for (int k = 0; k < 9; ++k)
#pragma unroll
        for (int j = 0; j < 8; ++j) w[k][j] = w9c[k * C + c0 + j];
#pragma unroll
    for (int j = 0; j < 8; ++j) b[j] = bias[c0 + j];

    T* obase = out + (size_t)chunk * kC1Hout * kC1Wout * C;
    for (int p = pl; p < kC1RowsPerBlock * kC1Wout; p += lanes_px) {
        const int il = p / kC1Wout, j = p % kC1Wout;
        const int i = rb * kC1RowsPerBlock + il;
        float acc[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = b[q];
#pragma unroll
        for (int a = 0; a < 3; ++a)
#pragma unroll
            for (int bb = 0; bb < 3; ++bb) {
                // input (mel 2i+a-1, time 2j+bb-1); LDS row 2*il+a, column 2j+bb
                const float v = img[2 * il + a][2 * j + bb];
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[q] = fmaf(w[a * 3 + bb][q], v, acc[q]);
            }
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[q] = gelu_for<T>(acc[q]);
        store8(obase + ((size_t)i * kC1Wout + j) * C + c0, acc);
    }
}

// bf16 operand mode: the 9 taps as one v_mfma_f32_16x16x32_bf16 per 16
// channels x 16 pixels.  The weights (bf16) are exact bf16 operands; each fp32
// input sample is split into three bf16 parts hi + mid + lo that add up to it
// (to within one fp32 ulp), so K = 9 taps x 3 parts + 1 bias slot (input 1.0,
// weight = bias, itself a bf16 value) = 28 <= 32 and the MFMA returns the fp32
// dot product of the VALU form.  The MFMA frees the VALU for the GELU, which
// is the bulk of this kernel's work.
//
// Weight fragments come pre-laid-out (wfrag[tile][lane][8] bf16, the A operand
// of lane l: K entries 8 (l / 16) .. + 7 of channel 32 (t / 2) + 8 (r / 4) +
// 4 (t % 2) + r % 4, r = l % 16, so that the results of tiles 2 cb and 2 cb + 1
// give each lane 8 consecutive channels) and stay in registers: C / 16 <= 32
// tiles (C <= 512).  A workgroup covers one half
// of a chunk's output rows (32 x 50 pixels); its input rows sit in LDS.  The
// output is channel-blocked, [chunk][C / 32][64][50][32], so that each store
// instruction of a wave covers 1 KB of contiguous memory.
constexpr int kC1HalfRows = 32;                        // output mel rows per workgroup
constexpr int kC1ImgRows = 2 * kC1HalfRows + 1;        // 65 input rows
constexpr int kC1ImgPitch = kChunk + 2;                // time -1 .. 100

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int NT>   // channel tiles, C = 16 NT
__global__ __launch_bounds__(256) void conv1_mfma_kernel(const float* __restrict__ logmel,
                                                         const ChunkInfo* __restrict__ chunks,
                                                         const uint4* __restrict__ wfrag,
                                                         bf16* __restrict__ out) {
    constexpr int C = 16 * NT;
    __shared__ float img[kC1ImgRows * kC1ImgPitch];
    const int chunk = blockIdx.x, half = blockIdx.y;
    const ChunkInfo ci = chunks[chunk];
    const int r0 = 2 * kC1HalfRows * half - 1;          // first input mel row (may be -1)
    // stage: idx -> (time tt in -1..100, row rr), row fastest (mel rows are contiguous in logmel)
    for (int idx = threadIdx.x; idx < kC1ImgRows * kC1ImgPitch; idx += blockDim.x) {
        const int tt = idx / kC1ImgRows - 1, rr = idx % kC1ImgRows;
        const int f = r0 + rr;
        float v = 0.0f;
        if (f >= 0 && f < kMels && tt >= 0 && tt < ci.m) v = logmel[(size_t)(ci.frame_row0 + tt) * kMels + f];
        img[rr * kC1ImgPitch + tt + 1] = v;
    }

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, px = lane & 15;
    uint4 wa[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) wa[t] = wfrag[(size_t)t * 64 + lane];
    // B entries of this lane: k = 8 g + e -> tap k / 3 (offset a * pitch + b) and part k % 3;
    // k = 27 is the constant 1 of the bias slot, k > 27 zero.
    int off[8], part[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int k = 8 * g + e;
        const int tap = k / 3;
        off[e] = k < 27 ? (tap / 3) * kC1ImgPitch + tap % 3 : 0;
        part[e] = k < 27 ? k % 3 : (k == 27 ? 3 : 4);
    }
    __syncthreads();

    constexpr int kPix = kC1HalfRows * kC1Wout;         // 1600 pixels, 100 groups of 16
    constexpr int kPlane = kC1Hout * kC1Wout * kConvCB;  // one 32-channel block of a chunk
    bf16* obase = out + (size_t)chunk * kC1Hout * kC1Wout * C + half * kPix * kConvCB;
    for (int grp = wave; grp < kPix / 16; grp += 4) {
        const int p = grp * 16 + px;
        const int il = p / kC1Wout, j = p - il * kC1Wout;
        const int base = 2 * il * kC1ImgPitch + 2 * j;  // tap (0, 0) of pixel (il, j)
        bf16 bv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = img[base + off[e]];
            const bf16 hi = (bf16)x;
            const float r1 = x - (float)hi;
            const bf16 mid = (bf16)r1;
            const bf16 lo = (bf16)(r1 - (float)mid);
            const int q = part[e];
            bv[e] = q == 0 ? hi : q == 1 ? mid : q == 2 ? lo : q == 3 ? (bf16)1.0f : (bf16)0.0f;
        }
        const bf16x8 b = {bv[0], bv[1], bv[2], bv[3], bv[4], bv[5], bv[6], bv[7]};
        bf16* orow = obase + p * kConvCB + 8 * g;
#pragma unroll
        for (int cb = 0; cb < NT / 2; ++cb) {
            // tiles 2 cb and 2 cb + 1 hold channels 32 cb + 8 g + (0..3) and + (4..7)
            // of pixel p in this lane: one 16-byte store; the wave writes 1 KB
            // contiguously (16 pixels x 32 channels of block cb)
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            const f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa[2 * cb]), b, z, 0, 0, 0);
            const f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa[2 * cb + 1]), b, z, 0, 0, 0);
            float v[8];
#pragma unroll
            for (int r = 0; r < 4; ++r) { v[r] = gelu_erf_bf16(a0[r]); v[4 + r] = gelu_erf_bf16(a1[r]); }
            // non-temporal: the 3.7 GB output is read back by conv2 long after
            // any cache could hold it (measured: conv2 runs ~2 % faster after it)
            const bf16x8 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3],
                              (bf16)v[4], (bf16)v[5], (bf16)v[6], (bf16)v[7]};
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, o), reinterpret_cast<u32x4*>(orow + cb * kPlane));
        }
    }
}

hipError_t conv1_mfma(hipStream_t s, const float* logmel, const ChunkInfo* chunks, int n_chunks,
                      const uint4* wfrag, int C, bf16* out) {
    if (n_chunks <= 0) return hipSuccess;
    const dim3 grid(n_chunks, kC1Hout / kC1HalfRows);
    switch (C) {   // C is a multiple of 32 (checked with the dims)
#define QA_C1(nt) case 16 * nt: conv1_mfma_kernel<nt><<<grid, 256, 0, s>>>(logmel, chunks, wfrag, out); break;
        QA_C1(2) QA_C1(4) QA_C1(6) QA_C1(8) QA_C1(10) QA_C1(12) QA_C1(14) QA_C1(16)
        QA_C1(18) QA_C1(20) QA_C1(22) QA_C1(24) QA_C1(26) QA_C1(28) QA_C1(30) QA_C1(32)
#undef QA_C1
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T>
hipError_t conv1(hipStream_t s, const float* logmel, const ChunkInfo* chunks, int n_chunks,
                 const float* w9c, const float* bias, int C, T* out) {
    if (n_chunks <= 0) return hipSuccess;
    const int cg_n = C / 8;
    int lanes_px = 256 / cg_n;
    if (lanes_px < 1) return hipErrorInvalidValue;
    dim3 grid(n_chunks, kC1Hout / kC1RowsPerBlock);
    conv1_kernel<T><<<grid, cg_n * lanes_px, 0, s>>>(logmel, chunks, w9c, bias, C, out);
    return hipGetLastError();
}

template hipError_t conv1<float>(hipStream_t, const float*, const ChunkInfo*, int, const float*, const float*, int, float*);
template hipError_t conv1<bf16>(hipStream_t, const float*, const ChunkInfo*, int, const float*, const float*, int, bf16*);

}  // namespace qa
