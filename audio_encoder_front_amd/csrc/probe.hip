// Ceiling probes measured beside the encoder in the same run: the bf16 MFMA
// rate of a register-only loop (random and constant operands; the operand
// bits toggle the multipliers, and the power they draw sets the clock the
// chip sustains) and the HBM rate of plain streaming reads and copies.  The
// benchmark reports every kernel's roofline fraction against the published
// peaks and against these measured ceilings.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qa_probe.h"

#define QA_PROBE_API extern "C" __attribute__((visibility("default")))

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mix32(uint32_t x) {   // a 32-bit integer hash (xorshift-multiply)
    x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
    return x;
}

// Each lane holds four A and four B operands (random bf16 in [-2, 2) with
// full mantissas, or all 1.0) and runs `iters` rounds of 4 x 8 independent
// 16x16x32 MFMAs, cycling through the operand pairs so the inputs change
// every instruction.
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, int random, float* out) {
    bf16x8 a[4], b[4];
    const uint32_t tid = blockIdx.x * 256u + threadIdx.x;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t h = mix32(tid * 64u + r * 8u + e);
            const float va = random ? ((float)(h & 0xffff) / 16384.0f - 2.0f) : 1.0f;
            const float vb = random ? ((float)(h >> 16) / 16384.0f - 2.0f) : 1.0f;
            a[r][e] = (__bf16)va;
            b[r][e] = (__bf16)vb;
        }
    f32x4 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int u = 0; u < 4; ++u)            // static operand indices (no indexed register arrays)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[j & 3], b[(j + u) & 3], acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    if (s == 1.2345e-30f) out[0] = s;      // keeps the loop live; never true in practice
}

// Grid-stride streaming over n4 16-byte elements.
__global__ __launch_bounds__(256) void read_probe_kernel(const float4* __restrict__ in, int64_t n4, float* out) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        const float4 v = in[i];
        s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
    if (s.x + s.y + s.z + s.w == 1.2345e-30f) out[0] = s.x;
}

__global__ __launch_bounds__(256) void copy_probe_kernel(const float4* __restrict__ in, float4* __restrict__ dst,
                                                         int64_t n4) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) dst[i] = in[i];
}

}  // namespace

QA_PROBE_API int qa_probe_mfma_bf16(void* stream, int blocks, int iters, int random, float* scratch) {
    if (blocks <= 0 || iters <= 0 || !scratch) return -1;
    mfma_probe_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(iters, random, scratch);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

QA_PROBE_API double qa_probe_mfma_flops(int blocks, int iters) {
    return (double)blocks * 4 /* waves */ * iters * 32 * (16.0 * 16 * 32 * 2);
}

QA_PROBE_API int qa_probe_read(void* stream, const void* src, int64_t bytes, float* scratch) {
    if (!src || !scratch || bytes < 16) return -1;
    read_probe_kernel<<<4096, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const float4*>(src), bytes / 16,
                                                                          scratch);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

QA_PROBE_API int qa_probe_copy(void* stream, const void* src, void* dst, int64_t bytes) {
    if (!src || !dst || bytes < 16) return -1;
    copy_probe_kernel<<<4096, 256, 0, static_cast<hipStream_t>(stream)>>>(static_cast<const float4*>(src),
                                                                          static_cast<float4*>(dst), bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}
