// Device-side helpers shared by the gfx950 kernels: element types, 16-byte
// fragment moves and the MFMA step over one 64-byte K block.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int per16 = 4; };   // elements per 16 bytes
template <> struct Elem<bf16>  { static constexpr int per16 = 8; };

__device__ __forceinline__ uint4 zero16() { return make_uint4(0u, 0u, 0u, 0u); }

__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// One MFMA pass over a 64-byte K block held as 16 bytes per lane.
//   bf16: v_mfma_f32_16x16x32_bf16, lane l holds A[l%16][8g..8g+7] and
//         B[8g..8g+7][l%16] (g = l/16).
//   fp32: four v_mfma_f32_16x16x4_f32; float s of the lane's 16 bytes is the
//         k index 4g+s of the block, identically for A and B, so the product
//         is the same sum in a permuted order.
// The result lane l holds D[4g + r][l % 16], r = 0..3.
// Row of head dimension d in the transposed-V LDS tiles of the attention
// kernels: dims are XOR-permuted within each group of 8 by the group index.
// One store instruction writes dims 8 c + e of many 16-byte chunks c at once,
// rows a multiple of 8 apart that an unpermuted layout maps to few LDS banks;
// the permutation spreads them.  The fragment reads (16 consecutive dims)
// are unaffected.  The row paddings that go with it were chosen by timing.
__device__ __forceinline__ int vt_row(int d) { return d ^ ((d >> 3) & 7); }

__device__ __forceinline__ void mfma_kblock(bf16, const uint4& a, const uint4& b, f32x4& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
__device__ __forceinline__ void mfma_kblock(float, const uint4& a, const uint4& b, f32x4& acc) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

// GELU with the erf (not tanh) form, gelu(z) = z (1 + erf(z / sqrt 2)) / 2,
// written as relu(z) - a erfc(a / sqrt 2) / 2 with a = min(|z|, A), and
// erfc(a / sqrt 2) / 2 = exp2(P(a)) for a polynomial P fitted to
// log2(erfc(a / sqrt 2)) - 1, weighted by the GELU error it causes
// (gelu_coeffs.py in this package derives and checks the coefficients).
// Horner in fp32, one exp2, relu as a median (one instruction, no NaN
// canonicalisation).
//   gelu_erf:      degree 6, A = 6, absolute error <= 2.7e-7 over the fp32
//                  range (float32 emulation against the exact erf); the tail
//                  past |z| = 6 is below 1e-8.  For results kept in fp32.
//   gelu_erf_bf16: degree 4, A = 5, absolute error <= 6.4e-6; the tail past
//                  |z| = 5 is below 1.5e-6.  For results rounded to bf16 at
//                  once (two fused multiply-adds fewer per element).
// +inf maps to +inf, -inf to -0 (gelu_erf) or -1.4e-6 (gelu_erf_bf16).
__device__ __forceinline__ float gelu_erf(float z) {
    const float a = __builtin_amdgcn_fmed3f(fabsf(z), 0.0f, 6.0f);
    float y = 3.454265243e-05f;
    y = fmaf(y, a, -7.817276055e-04f);
    y = fmaf(y, a, 8.121271618e-03f);
    y = fmaf(y, a, -5.347414687e-02f);
    y = fmaf(y, a, -4.587250352e-01f);
    y = fmaf(y, a, -1.151216626e+00f);
    y = fmaf(y, a, -9.999914765e-01f);
    return fmaf(-a, __builtin_amdgcn_exp2f(y), __builtin_amdgcn_fmed3f(z, 0.0f, __builtin_inff()));
}
__device__ __forceinline__ float gelu_erf_bf16(float z) {
    const float a = __builtin_amdgcn_fmed3f(fabsf(z), 0.0f, 5.0f);
    float y = 3.872423200e-03f;
    y = fmaf(y, a, -4.409601539e-02f);
    y = fmaf(y, a, -4.680127501e-01f);
    y = fmaf(y, a, -1.147355437e+00f);
    y = fmaf(y, a, -1.000486970e+00f);
    return fmaf(-a, __builtin_amdgcn_exp2f(y), __builtin_amdgcn_fmed3f(z, 0.0f, __builtin_inff()));
}
// The GELU for a result stored as T.
template <typename T> __device__ __forceinline__ float gelu_for(float z) { return gelu_erf(z); }
template <> __device__ __forceinline__ float gelu_for<bf16>(float z) { return gelu_erf_bf16(z); }

// Store 4 consecutive values (fp32 -> 16 bytes, bf16 -> 8 bytes, RNE).
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
    *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 v = {(bf16)a, (bf16)b, (bf16)c, (bf16)d};
    *reinterpret_cast<bf16x4*>(p) = v;
}
// Store 8 consecutive values (bf16: one 16-byte store).
__device__ __forceinline__ void store8(float* p, const float* v) {
    store4(p, v[0], v[1], v[2], v[3]);
    store4(p + 4, v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(bf16* p, const float* v) {
    bf16x8 o = {(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3], (bf16)v[4], (bf16)v[5], (bf16)v[6], (bf16)v[7]};
    *reinterpret_cast<bf16x8*>(p) = o;
}
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// ---- direct-to-LDS loads (global -> LDS without a register round trip)
typedef __attribute__((address_space(3))) void lds_void;

// Direct-to-LDS loads written as inline asm: the compiler's wait-count pass
// cannot tell the LDS stages apart and would otherwise wait for the
// in-flight loads of later stages before every LDS read of stage k.
// Completion is awaited explicitly (s_waitcnt vmcnt(n), leaving the n loads
// of the stage two ahead in flight) before the barrier that publishes a
// stage.  M0 carries the wave's LDS destination; no other code in these
// kernels uses M0.
//
// Two forms.  buffer_load_dwordx4 ... lds reads through a buffer resource
// (base and size in four SGPRs) at a 32-bit lane offset: one VGPR per load
// and no 64-bit address arithmetic, and any offset at or past the resource
// size reads zeros, which covers ragged rows and conv padding for free.  The
// loaders that can keep their per-workgroup range under 4 GB (dense rows, conv
// chunks) use it; the row-gather loader uses global_load_lds_dwordx4 with
// 64-bit addresses and a zero block.
typedef int i32x4 __attribute__((ext_vector_type(4)));
constexpr unsigned kOobOffset = 0xFFFFFFF0u;     // >= every resource size below: reads zeros

__device__ __forceinline__ void dma16(const void* src, unsigned lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(lds_addr), "v"(src) : "m0");
}
__device__ __forceinline__ void dma16_buf(i32x4 rsrc, unsigned voff, unsigned lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds_addr), "v"(voff),
                 "s"(rsrc) : "m0");
}
// One dword per lane: the wave's 64 dwords land at lds_addr + 4 * lane.
__device__ __forceinline__ void dma4_buf(i32x4 rsrc, unsigned voff, unsigned lds_addr) {
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds_addr), "v"(voff),
                 "s"(rsrc) : "m0");
}
// Raw buffer resource (stride 0) over [base, base + bytes), bytes clamped
// below kOobOffset; the fourth word is the gfx9 raw-buffer format.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint64_t bytes) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const unsigned n = bytes < 0xFFFFFF00ull ? (unsigned)bytes : 0xFFFFFF00u;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)b);
    r[1] = __builtin_amdgcn_readfirstlane((int)(unsigned)(b >> 32));
    r[2] = __builtin_amdgcn_readfirstlane((int)n);
    r[3] = 0x00020000;
    return r;
}

// Order-preserving int key of a float, for atomicMax over floats.
__device__ __forceinline__ int float_key(float f) {
    int i = __float_as_int(f);
    return i >= 0 ? i : (i ^ 0x7fffffff);
}
__device__ __forceinline__ float key_float(int k) {
    return __int_as_float(k >= 0 ? k : (k ^ 0x7fffffff));
}

// ---- LayerNorm of one row held by one wave (fp32 statistics)
constexpr float kLnEps = 1e-5f;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// Lane `lane` holds the row's float4 chunks i = lane + 64 q (q < NQ, i < d/4)
// in v, and gamma / beta's in g / b; writes (v - mean) / sqrt(var + eps) *
// gamma + beta to o[0 .. d).  Every LayerNorm of the encoder goes through
// this one sequence, so a fused and a separate LayerNorm agree bit for bit.
template <typename T, int NQ>
__device__ __forceinline__ void ln_row(const float4 (&v)[NQ], const float4 (&g)[NQ], const float4 (&b)[NQ],
                                       int lane, int d, T* __restrict__ o) {
    const int d4 = d >> 2;
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i = lane + 64 * q;
        if (i < d4) s += (v[q].x + v[q].y) + (v[q].z + v[q].w);
    }
    const float mean = wave_sum(s) / (float)d;
    float ss = 0.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i = lane + 64 * q;
        if (i < d4) {
            const float a = v[q].x - mean, e1 = v[q].y - mean, c = v[q].z - mean, e = v[q].w - mean;
            ss += (a * a + e1 * e1) + (c * c + e * e);
        }
    }
    const float rstd = rsqrtf(wave_sum(ss) / (float)d + kLnEps);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i = lane + 64 * q;
        if (i < d4)
            store4(o + 4 * i, (v[q].x - mean) * rstd * g[q].x + b[q].x, (v[q].y - mean) * rstd * g[q].y + b[q].y,
                   (v[q].z - mean) * rstd * g[q].z + b[q].z, (v[q].w - mean) * rstd * g[q].w + b[q].w);
    }
}

}  // namespace qa
