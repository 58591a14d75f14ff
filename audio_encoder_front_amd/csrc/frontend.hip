// Front end: framing + periodic-Hann 400-point real DFT as an MFMA GEMM,
// power spectrum, 128-filter Slaney mel GEMM, 1e-10 floor, log10 and the
// per-clip maximum; then the peak-minus-8 clip and (x+4)/4 affine.
//
// Follows qwenasr.cpp ARCHITECTURE.md "Mel frontend" / "Mel DFT without an FFT
// op" (the DFT as real matmuls against precomputed cos/sin matrices, fp32) and
// OneSpeech "Front end and graph numerics" (periodic Hann, centered
// reflection, Slaney mel, power floor 1e-10, log10 peak-minus-eight, (x+4)/4,
// floor(len/160) frames).
//
// Kernel design (four waves per 64-frame tile):
//  * the DFT runs on the bf16 MFMA at fp32 accuracy: every fp32 sample and
//    every fp32 basis value (Hann window folded in) is split exactly into
//    three bf16 parts, hi + mid + lo, and each product keeps the six part
//    products whose exponents reach the fp32 result (hi.hi, hi.mid, mid.hi,
//    hi.lo, mid.mid, lo.hi); the three dropped ones are below 2^-24 of it.
//    Six 16x16x32 bf16 MFMAs replace eight 16x16x4 fp32 ones per 32 samples
//    (96 instead of 256 MFMA cycles);
//  * the tile's samples, split, sit in LDS as three bf16 planes with 8 pad
//    samples after every 160, so the 16 frames x 8 samples a fragment reads
//    hit 16 distinct 4-bank groups;
//  * D[bin][frame] = sum_n basis[n][bin] x[frame][n]: wave w takes the
//    16-bin chunks w, w + 4, w + 8, w + 12 for all 64 frames (cos and sin of
//    a bin in the same registers, so the power needs no data movement), the
//    basis fragments come pre-split and pre-laid-out from global memory;
//  * the power goes to LDS frame-major (the sample planes are free by then);
//    a Slaney filter covers at most 9 consecutive bins, so each thread sums
//    one mel band of 32 frames directly (kMelTaps weights in registers, fp32
//    FMAs): 402 multiply-adds per frame instead of a mostly-zero dense GEMM;
//    then log10, the clip maximum and the store (a workgroup writes whole
//    512-byte log-mel rows).
#include "qa_device.h"
#include "qa_kernels.h"

namespace qa {

constexpr int kDftKB = 13;                                     // 32-sample K blocks (416 >= 400)
constexpr int kSpan = 160 * (kFrontFrames - 1) + 32 * kDftKB;  // samples a tile reads (K padded)
constexpr int kPlane = kSpan + 8 * (kSpan / 160) + 8;          // padded bf16 samples per plane
constexpr int kPStride = kBinChunks * 16 + 4;                  // floats per power row (one frame): 212
constexpr int kFrontLds = 3 * kPlane * 2 > kFrontFrames * kPStride * 4 ? 3 * kPlane * 2 : kFrontFrames * kPStride * 4;

__device__ __forceinline__ int pad_index(int s) { return s + 8 * (s / 160); }

__global__ void init_flags_kernel(int* clip_key, int n_clips, int* flag) {
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_clips) clip_key[i] = float_key(-INFINITY);
    if (i == 0) {
        flag[0] = 0;
        flag[1] = 0;   // the fused stem's tile counter
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void frontend_kernel(
    const float* __restrict__ pcm, const ClipInfo* __restrict__ clips,
    const FrontTile* __restrict__ tiles, const uint4* __restrict__ basis,
    const float* __restrict__ melw, const int* __restrict__ melb0,
    float* __restrict__ logmel, int* __restrict__ clip_key, int* __restrict__ flag) {
    __shared__ __align__(16) char lds[kFrontLds];
    bf16* planes = reinterpret_cast<bf16*>(lds);          // [3][kPlane]
    float* pw = reinterpret_cast<float*>(lds);            // [64 frames][kPStride], after the DFT
    const FrontTile t = tiles[blockIdx.x];
    const ClipInfo c = clips[t.clip];
    const float* x = pcm + c.sample_off;
    const int L = c.len;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nsamp = 160 * (t.nframes - 1) + 400;
    // frames past the clip's kept range (the final STFT frame, which the
    // planner gives to the clip's last tile so that every sample is read and
    // its power checked) are computed but neither stored nor in the maximum
    const int nkeep = min(t.nframes, L / 160 - t.frame0);
    bool bad = false;
    // Samples in pairs (a pair never straddles a pad): every load of the tile
    // is issued before the first split, then each part plane gets one
    // 4-byte write per pair.
    constexpr int NP = (kSpan / 2 + 255) / 256;
    float va[NP], vb[NP];
    auto sample = [&](int s) {
        if (s >= nsamp) return 0.0f;
        int i = 160 * t.frame0 + s - 200;         // centered: frame j starts 200 samples early
        if (i < 0) i = -i;                          // mirror without repeating the edge
        if (i >= L) i = 2 * (L - 1) - i;
        return x[i];
    };
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        const int s = 2 * ((int)threadIdx.x + 256 * k);
        va[k] = s < kSpan ? sample(s) : 0.0f;
        vb[k] = s < kSpan ? sample(s + 1) : 0.0f;
    }
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int k = 0; k < NP; ++k) {
        const int s = 2 * ((int)threadIdx.x + 256 * k);
        if (s >= kSpan) continue;
        float v[2] = {va[k], vb[k]};
        bf16x2 part[3];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            bad |= !isfinite(v[e]);
            if (!isfinite(v[e])) v[e] = 0.0f;       // reported through the flag; keep the MFMA finite
            const bf16 hi = (bf16)v[e];
            const float r1 = v[e] - (float)hi;
            const bf16 mid = (bf16)r1;
            part[0][e] = hi;
            part[1][e] = mid;
            part[2][e] = (bf16)(r1 - (float)mid);
        }
        const int q = pad_index(s);
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) *reinterpret_cast<bf16x2*>(planes + pp * kPlane + q) = part[pp];
    }
    __syncthreads();

    const int g = lane >> 4, li = lane & 15;
    // acc[slot][cs][ft]: bins 16 bc + 4 g + r, bc = wave + 4 slot, of frame 16 ft + li (cs: cos, sin)
    f32x4 acc[4][2][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[a][b][f] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (K block, chunk slot) units of this wave in order; the basis fragments
    // of the next unit are loaded while the current one multiplies.
    const int nslots = (kBinChunks - wave + 3) / 4;   // 4 for wave 0, 3 for the others
    const int nunits = kDftKB * nslots;
    auto load_basis = [&](int u, uint4* b) {
        const int kb = u / nslots, bc = wave + 4 * (u % nslots);
        const uint4* bp = basis + (size_t)((bc * kDftKB + kb) * 2) * 3 * 64 + lane;
#pragma unroll
        for (int q = 0; q < 6; ++q) b[q] = bp[q * 64];   // cos hi, mid, lo, sin hi, mid, lo
    };
    uint4 bcur[6], bnxt[6];
    load_basis(0, bcur);
    bf16x8 xf[4][3];
    for (int u = 0; u < nunits; ++u) {
        const int kb = u / nslots, slot = u % nslots;
        if (u + 1 < nunits) load_basis(u + 1, bnxt);
        if (slot == 0) {
            // B operand: 8 consecutive samples 32 kb + 8 g .. of frame 16 ft + li, per part
#pragma unroll
            for (int ft = 0; ft < 4; ++ft) {
                const int q = pad_index(160 * (16 * ft + li) + 32 * kb + 8 * g);
#pragma unroll
                for (int p = 0; p < 3; ++p) xf[ft][p] = __builtin_bit_cast(bf16x8, ld16(planes + p * kPlane + q));
            }
        }
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
            if (sl != slot) continue;                 // register-indexed accumulators stay static
#pragma unroll
            for (int cs = 0; cs < 2; ++cs) {
                const bf16x8 bh = __builtin_bit_cast(bf16x8, bcur[3 * cs]);
                const bf16x8 bm = __builtin_bit_cast(bf16x8, bcur[3 * cs + 1]);
                const bf16x8 bl = __builtin_bit_cast(bf16x8, bcur[3 * cs + 2]);
#pragma unroll
                for (int ft = 0; ft < 4; ++ft) {
                    f32x4 a = acc[sl][cs][ft];
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bl, xf[ft][0], a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bm, xf[ft][1], a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh, xf[ft][2], a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bm, xf[ft][0], a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh, xf[ft][1], a, 0, 0, 0);
                    a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bh, xf[ft][0], a, 0, 0, 0);
                    acc[sl][cs][ft] = a;
                }
            }
        }
#pragma unroll
        for (int q = 0; q < 6; ++q) bcur[q] = bnxt[q];
    }
    __syncthreads();                                  // every wave is done with the sample planes

    // power P[frame][bin] = re^2 + im^2 (no sqrt): a lane's four bins of a
    // frame are consecutive, one 16-byte write
#pragma unroll
    for (int slot = 0; slot < 4; ++slot) {
        const int bc = wave + 4 * slot;
        if (bc >= kBinChunks) continue;
#pragma unroll
        for (int ft = 0; ft < 4; ++ft) {
            f32x4 pwr;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float re = acc[slot][0][ft][r], im = acc[slot][1][ft][r];
                pwr[r] = re * re + im * im;
                bad |= !isfinite(pwr[r]);              // power beyond float32 range
            }
            *reinterpret_cast<f32x4*>(pw + (16 * ft + li) * kPStride + 16 * bc + 4 * g) = pwr;
        }
    }
    __syncthreads();

    // mel band m of frames fo, fo + 2, ..: E = sum_j w[j] P[frame][b0 + j]
    const int m = threadIdx.x & (kMels - 1), fo = threadIdx.x / kMels;
    const int b0 = melb0[m];
    float w[kMelTaps];
#pragma unroll
    for (int j = 0; j < kMelTaps; ++j) w[j] = melw[m * kMelTaps + j];
    float vmax = -INFINITY;
    float* outp = logmel + (size_t)(c.frame_row0 + t.frame0) * kMels + m;
    for (int f = fo; f < t.nframes; f += 256 / kMels) {
        const float* pr = pw + f * kPStride + b0;
        float e = 0.0f;
#pragma unroll
        for (int j = 0; j < kMelTaps; ++j) e = fmaf(w[j], pr[j], e);
        bad |= !isfinite(e);                     // mel energy beyond float32 range
        if (f >= nkeep) continue;                // the dropped final frame
        const float lg = log10f(fmaxf(e, 1e-10f));
        outp[(size_t)f * kMels] = lg;
        vmax = fmaxf(vmax, lg);
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
    const ClipInfo c = clips[t.clip];
    float4* p = reinterpret_cast<float4*>(logmel + (size_t)(c.frame_row0 + t.frame0) * kMels);
    const int n4 = max(0, min(t.nframes, c.len / 160 - t.frame0)) * kMels / 4;   // kept frames only
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
                    int n_tiles, const uint4* basis, const float* melw, const int* melb0,
                    float* logmel, int* clip_key, int* flag) {
    if (n_tiles <= 0) return hipSuccess;
    frontend_kernel<<<n_tiles, 256, 0, s>>>(pcm, clips, tiles, basis, melw, melb0, logmel, clip_key, flag);
    return hipGetLastError();
}

hipError_t normalize(hipStream_t s, float* logmel, const ClipInfo* clips, const FrontTile* tiles,
                     int n_tiles, const int* clip_key) {
    if (n_tiles <= 0) return hipSuccess;
    normalize_kernel<<<n_tiles, 256, 0, s>>>(logmel, clips, tiles, clip_key);
    return hipGetLastError();
}

}  // namespace qa
