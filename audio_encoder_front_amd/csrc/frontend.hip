// Front end: framing + periodic-Hann 400-point real DFT as an fp32 MFMA GEMM,
// power spectrum, 128-filter Slaney mel GEMM, 1e-10 floor, log10 and the
// per-clip maximum; then the peak-minus-8 clip and (x+4)/4 affine.
//
// Follows qwenasr.cpp ARCHITECTURE.md "Mel frontend" / "Mel DFT without an FFT
// op" (the DFT as real matmuls against precomputed cos/sin matrices, fp32) and
// OneSpeech "Front end and graph numerics" (periodic Hann, centered
// reflection, Slaney mel, power floor 1e-10, log10 peak-minus-eight, (x+4)/4,
// floor(len/160) frames).
//
// Kernel design (two waves per 64-frame tile, splitting the DFT bins):
//  * the tile's samples (with mirror padding) sit in LDS, two pad words every
//    160 samples so that the 16 frames x 4 samples a fragment reads fall in
//    distinct banks;
//  * GEMM 1 is computed transposed, D[bin][frame] = sum_n basis[n][bin] x[frame][n],
//    with the Hann window folded into the basis; for each block of 16 bins the
//    cos and sin products land in matching registers, so the power needs no
//    data movement;
//  * the lane layout of D is exactly the A-operand layout GEMM 2 needs
//    (frame = lane%16, bin = 4*(lane/16) + r at k-step r), so the power feeds
//    the mel MFMA straight from registers;
//  * mel tiles with no nonzero filter weight for a bin block are skipped;
//  * the two waves take alternate 16-bin blocks; their partial mel energies
//    meet in LDS (the sample buffer is free by then) before the log.
#include "qa_device.h"
#include "qa_kernels.h"

namespace qa {

constexpr int kSpan = 160 * (kFrontFrames - 1) + 400;          // samples per tile
constexpr int kLdsSamples = kSpan + 2 * (kSpan / 160) + 4;

__device__ __forceinline__ int pad_index(int s) { return s + 2 * (s / 160); }

__global__ void init_flags_kernel(int* clip_key, int n_clips, int* flag) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_clips) clip_key[i] = float_key(-INFINITY);
    if (i == 0) *flag = 0;
}

__global__ __launch_bounds__(128) __attribute__((amdgpu_waves_per_eu(2))) void frontend_kernel(
    const float* __restrict__ pcm, const ClipInfo* __restrict__ clips,
    const FrontTile* __restrict__ tiles, const float* __restrict__ basis,
    const float* __restrict__ fbB, const int* __restrict__ fb_range,
    float* __restrict__ logmel, int* __restrict__ clip_key, int* __restrict__ flag) {
    __shared__ float xs[kLdsSamples];
    const FrontTile t = tiles[blockIdx.x];
    const ClipInfo c = clips[t.clip];
    const float* x = pcm + c.sample_off;
    const int L = c.len;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nsamp = 160 * (t.nframes - 1) + 400;
    bool bad = false;
    for (int s = threadIdx.x; s < kSpan; s += 128) {
        float v = 0.0f;
        if (s < nsamp) {
            int i = 160 * t.frame0 + s - 200;     // centered: frame j starts 200 samples early
            if (i < 0) i = -i;                      // mirror without repeating the edge
            if (i >= L) i = 2 * (L - 1) - i;
            v = x[i];
            bad |= !isfinite(v);
        }
        xs[pad_index(s)] = v;
    }
    __syncthreads();

    const int g = lane >> 4, li = lane & 15;
    f32x4 E[4][8];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) E[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    int fbase[4];
#pragma unroll
    for (int ft = 0; ft < 4; ++ft) fbase[ft] = 162 * (ft * 16 + li);   // pad_index(160*frame)

    for (int bc = wave; bc < kBinChunks; bc += 2) {
        f32x4 re[4], im[4];
#pragma unroll
        for (int ft = 0; ft < 4; ++ft) { re[ft] = f32x4{0.f, 0.f, 0.f, 0.f}; im[ft] = re[ft]; }
        const float* bp = basis + (size_t)bc * 100 * 128 + g * 16 + li;
#pragma unroll 4
        for (int kk = 0; kk < 100; ++kk) {
            const float bcos = bp[kk * 128];
            const float bsin = bp[kk * 128 + 64];
            const int n = 4 * kk + g;
            const int off = n + 2 * (n / 160);
#pragma unroll
            for (int ft = 0; ft < 4; ++ft) {
                const float xv = xs[fbase[ft] + off];
                re[ft] = __builtin_amdgcn_mfma_f32_16x16x4f32(bcos, xv, re[ft], 0, 0, 0);
                im[ft] = __builtin_amdgcn_mfma_f32_16x16x4f32(bsin, xv, im[ft], 0, 0, 0);
            }
        }
        // power P[bin 4g+r][frame ft*16+li] = re^2 + im^2 (no sqrt)
#pragma unroll
        for (int ft = 0; ft < 4; ++ft) re[ft] = re[ft] * re[ft] + im[ft] * im[ft];
        const int lo = fb_range[2 * bc], hi = fb_range[2 * bc + 1];
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            if (mt < lo || mt >= hi) continue;      // wave-uniform: all-zero filter tile
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float fb = fbB[(((size_t)bc * 4 + r) * 8 + mt) * 64 + lane];
#pragma unroll
                for (int ft = 0; ft < 4; ++ft)
                    E[ft][mt] = __builtin_amdgcn_mfma_f32_16x16x4f32(re[ft][r], fb, E[ft][mt], 0, 0, 0);
            }
        }
    }

    // combine the two waves' partial mel energies through LDS
    __syncthreads();
    float4* ex = reinterpret_cast<float4*>(xs);
    if (wave == 1) {
#pragma unroll
        for (int ft = 0; ft < 4; ++ft)
#pragma unroll
            for (int mt = 0; mt < 8; ++mt)
                ex[(ft * 8 + mt) * 64 + lane] = make_float4(E[ft][mt][0], E[ft][mt][1], E[ft][mt][2], E[ft][mt][3]);
    }
    __syncthreads();
    if (wave == 1) {
        if (__any(bad) && lane == 0) atomicOr(flag, 1);
        return;
    }
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
            const float4 o = ex[(ft * 8 + mt) * 64 + lane];
            E[ft][mt][0] += o.x; E[ft][mt][1] += o.y; E[ft][mt][2] += o.z; E[ft][mt][3] += o.w;
        }

    // E[ft][mt] lane holds mel energy of frame ft*16 + 4g + r, mel mt*16 + li.
    float vmax = -INFINITY;
    float* outp = logmel + (size_t)(c.frame_row0 + t.frame0) * kMels;
#pragma unroll
    for (int ft = 0; ft < 4; ++ft)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int fi = ft * 16 + 4 * g + r;
            if (fi < t.nframes) {
#pragma unroll
                for (int mt = 0; mt < 8; ++mt) {
                    const float e = E[ft][mt][r];
                    bad |= !isfinite(e);             // power beyond float32 range
                    const float lg = log10f(fmaxf(e, 1e-10f));
                    outp[(size_t)fi * kMels + mt * 16 + li] = lg;
                    vmax = fmaxf(vmax, lg);
                }
            }
        }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, o));
    if (lane == 0) atomicMax(clip_key + t.clip, float_key(vmax));
    if (__any(bad) && lane == 0) atomicOr(flag, 1);
}

__global__ __launch_bounds__(256) void normalize_kernel(float* __restrict__ logmel,
                                                        const ClipInfo* __restrict__ clips,
                                                        const FrontTile* __restrict__ tiles,
                                                        const int* __restrict__ clip_key) {
    const FrontTile t = tiles[blockIdx.x];
    const float mx = key_float(clip_key[t.clip]);
    const float lo = mx - 8.0f;
    float4* p = reinterpret_cast<float4*>(logmel + (size_t)(clips[t.clip].frame_row0 + t.frame0) * kMels);
    const int n4 = t.nframes * kMels / 4;
    for (int i = threadIdx.x; i < n4; i += 256) {
        float4 v = p[i];
        v.x = (fmaxf(v.x, lo) + 4.0f) * 0.25f;
        v.y = (fmaxf(v.y, lo) + 4.0f) * 0.25f;
        v.z = (fmaxf(v.z, lo) + 4.0f) * 0.25f;
        v.w = (fmaxf(v.w, lo) + 4.0f) * 0.25f;
        p[i] = v;
    }
}

hipError_t init_flags(hipStream_t s, int* clip_key, int n_clips, int* flag) {
    int n = n_clips > 1 ? n_clips : 1;
    init_flags_kernel<<<(n + 255) / 256, 256, 0, s>>>(clip_key, n_clips, flag);
    return hipGetLastError();
}

hipError_t frontend(hipStream_t s, const float* pcm, const ClipInfo* clips, const FrontTile* tiles,
                    int n_tiles, const float* basis, const float* fbB, const int* fb_range,
                    float* logmel, int* clip_key, int* flag) {
    if (n_tiles <= 0) return hipSuccess;
    frontend_kernel<<<n_tiles, 128, 0, s>>>(pcm, clips, tiles, basis, fbB, fb_range, logmel, clip_key, flag);
    return hipGetLastError();
}

hipError_t normalize(hipStream_t s, float* logmel, const ClipInfo* clips, const FrontTile* tiles,
                     int n_tiles, const int* clip_key) {
    if (n_tiles <= 0) return hipSuccess;
    normalize_kernel<<<n_tiles, 256, 0, s>>>(logmel, clips, tiles, clip_key);
    return hipGetLastError();
}

}  // namespace qa
