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
// layout the implicit-GEMM conv2 reads 16 bytes at a time.  This path serves
// fp32 encoders and bf16 stems wider than 512 channels; other bf16 stems run
// conv1 inside conv2 (stem_fused.hip).
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
