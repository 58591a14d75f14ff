// Kernels of the step after the encoder: the audio splice into the prompt
// embeddings and the Qwen3 Thinker prefill (qwenasr.cpp ARCHITECTURE.md,
// "Qwen3 Thinker decoder" and "Prompt assembly and audio splice").  The
// projections run on the GEMM family (gemm.hip); this file holds the
// splice, RMSNorm, the per-head QK-RMSNorm fused with the NEOX RoPE, and the
// causal grouped-query attention with head_dim 128.
#include "qa_device.h"
#include "qa_kernels.h"

namespace qa {

namespace {

__device__ __forceinline__ float wsum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

}  // namespace

// ---------------------------------------------------------------- splice
// x[t] = embed[src[t]] for src[t] >= 0 (token id), audio[-src[t] - 1] otherwise.
// One wave per row, float4 / 8-byte vectors.
template <typename T>
__global__ __launch_bounds__(256) void embed_splice_kernel(const T* __restrict__ embed, const float* __restrict__ audio,
                                                           const int* __restrict__ src, int M, int H,
                                                           float* __restrict__ x) {
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= M) return;
    const int s = src[row];
    float* xr = x + (size_t)row * H;
    if (s < 0) {
        const float4* a = reinterpret_cast<const float4*>(audio + (size_t)(-s - 1) * H);
        for (int i = lane; i < H / 4; i += 64) reinterpret_cast<float4*>(xr)[i] = a[i];
    } else {
        const T* e = embed + (size_t)s * H;
        for (int i = lane; i < H / 4; i += 64) {
            const int c = 4 * i;
            reinterpret_cast<float4*>(xr)[i] =
                make_float4(to_f32(e[c]), to_f32(e[c + 1]), to_f32(e[c + 2]), to_f32(e[c + 3]));
        }
    }
}

// ---------------------------------------------------------------- RMSNorm
// out[r] = x[r] / sqrt(mean(x[r]^2) + eps) * g, one wave per row (H <= 4096:
// up to 16 float4 per lane), persistent over rows.
constexpr int kRmsMaxVec = 16;

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int M, int H,
                                                      const float* __restrict__ g, float eps, T* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int h4 = H >> 2;
    const float4* g4 = reinterpret_cast<const float4*>(g);
    for (int row = blockIdx.x * 4 + (threadIdx.x >> 6); row < M; row += gridDim.x * 4) {
        const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * H);
        float4 v[kRmsMaxVec];
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < kRmsMaxVec; ++q) {
            const int i = lane + 64 * q;
            if (i < h4) {
                v[q] = xr[i];
                ss += (v[q].x * v[q].x + v[q].y * v[q].y) + (v[q].z * v[q].z + v[q].w * v[q].w);
            }
        }
        const float r = rsqrtf(wsum(ss) / (float)H + eps);
        T* orow = out + (size_t)row * H;
#pragma unroll
        for (int q = 0; q < kRmsMaxVec; ++q) {
            const int i = lane + 64 * q;
            if (i < h4) {
                const float4 gg = g4[i];
                store4(orow + 4 * i, v[q].x * r * gg.x, v[q].y * r * gg.y, v[q].z * r * gg.z, v[q].w * r * gg.w);
            }
        }
    }
}

// ---------------------------------------------------------------- QK-norm + RoPE
// In place on the fused projection rows [q (Hq x 128) | k (Hkv x 128) | v]:
// for every query and key head, RMSNorm over the 128 values with the
// [128] gain, then the rotate-half RoPE at the token's position:
// (a, b) = (x[i], x[i + 64]) -> (a c - b s, b c + a s), c, s = cos, sin of
// pos * base^(-i / 64), taken from a table computed in double on the host.
// One wave per (token, head); lane i holds the pair (i, i + 64).
template <typename T>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(T* __restrict__ qkv, int M, int hq, int hkv,
                                                          const int* __restrict__ pos,
                                                          const float* __restrict__ qg, const float* __restrict__ kg,
                                                          const float2* __restrict__ cs, float eps) {
    const int item = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int heads = hq + hkv;
    if (item >= M * heads) return;
    const int t = item / heads, h = item - t * heads;
    T* p = qkv + (size_t)t * (hq + 2 * hkv) * 128 + h * 128;
    const float a = to_f32(p[lane]), b = to_f32(p[lane + 64]);
    const float r = rsqrtf(wsum(a * a + b * b) / 128.0f + eps);
    const float* gg = h < hq ? qg : kg;
    const float an = a * r * gg[lane], bn = b * r * gg[lane + 64];
    const float2 c = cs[(size_t)pos[t] * 64 + lane];
    p[lane] = from_f32<T>(an * c.x - bn * c.y);
    p[lane + 64] = from_f32<T>(bn * c.x + an * c.y);
}

// ---------------------------------------------------------------- attention
// Causal grouped-query attention, head_dim 128, over packed prompts
// [cu[i], cu[i + 1]); query head h reads KV head h / (hq / hkv).  One
// workgroup per (prompt, query head, 64 queries), one 16-query tile per wave.
// Per key block of 64: S^T = K Q^T on MFMA (a lane holds one query column),
// the causal mask, an online softmax (running max / sum, the partial output
// rescaled when the max grows) and O^T = V^T P^T with V^T transposed in LDS;
// the workgroup stops at the block holding its last query.  When a KV head
// serves an even number of query heads, a workgroup takes two of them (8
// waves) so each K/V block is staged once for both.
constexpr int kTHd = 128;
constexpr int kTKB = 64;                     // keys per block

template <typename T> struct TAttnLds;
template <> struct TAttnLds<bf16> {
    static constexpr int krow = kTHd * 2 + 16;      // bytes per K row (padded)
    static constexpr int vrow = kTKB * 2 + 8;       // bytes per V^T row (d index)
};
template <> struct TAttnLds<float> {
    static constexpr int krow = kTHd * 4 + 16;
    static constexpr int vrow = kTKB * 4 + 16;
};

__device__ __forceinline__ void tpv_step(bf16, const char* vt, int kbase, int fr, int fg, const f32x4* p, int t0,
                                         f32x4* o) {
    // slots 0..3: keys kbase + 4g + r (tile t0), 4..7: kbase + 16 + 4g + r (tile t0 + 1)
    bf16x8 pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) { pb[r] = (bf16)p[t0][r]; pb[4 + r] = (bf16)p[t0 + 1][r]; }
#pragma unroll
    for (int dt = 0; dt < kTHd / 16; ++dt) {
        const char* row = vt + (dt * 16 + fr) * TAttnLds<bf16>::vrow;
        const uint2 lo = *reinterpret_cast<const uint2*>(row + 2 * (kbase + 4 * fg));
        const uint2 hi = *reinterpret_cast<const uint2*>(row + 2 * (kbase + 16 + 4 * fg));
        const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pb, o[dt], 0, 0, 0);
    }
}
__device__ __forceinline__ void tpv_step(float, const char* vt, int kbase, int fr, int fg, const f32x4* p, int t0,
                                         f32x4* o) {
#pragma unroll
    for (int dt = 0; dt < kTHd / 16; ++dt) {
        const char* row = vt + (dt * 16 + fr) * TAttnLds<float>::vrow;
        const float4 va = *reinterpret_cast<const float4*>(row + 4 * (kbase + 4 * fg));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.x, p[t0][0], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.y, p[t0][1], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.z, p[t0][2], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.w, p[t0][3], o[dt], 0, 0, 0);
    }
}

template <typename T, int HPW>
__global__ __launch_bounds__(256 * HPW) void thinker_attention_kernel(const T* __restrict__ qkv,
                                                                      const int* __restrict__ cu, int hq, int hkv,
                                                                      int qgroups, T* __restrict__ out) {
    constexpr int KR = TAttnLds<T>::krow, VR = TAttnLds<T>::vrow;
    constexpr int PER = Elem<T>::per16;
    constexpr int CPR = kTHd / PER;                          // 16-byte chunks per head row
    constexpr int KBN = kTHd * (int)sizeof(T) / 64;          // 64-byte MFMA K blocks per head row
    constexpr int NT = 256 * HPW;                            // threads
    constexpr int NCH = kTKB * CPR / NT;                     // chunks per thread per key block
    __shared__ __align__(16) char ks[kTKB * KR];
    __shared__ __align__(16) char vts[kTHd * VR];

    // workgroup = (prompt, HPW consecutive query heads of one KV head, 64 queries);
    // waves 4 i .. 4 i + 3 take query head i of the group, 16 queries each.
    // Causal work grows with the query group, so the groups are dispatched
    // longest first (all (prompt, head group) pairs of the last query group,
    // then the one before, ...): the short ones fill the tail.
    const int hgroups = hq / HPW;
    const int nph = (int)(gridDim.x / qgroups);              // (prompt, head group) pairs
    const int qg = qgroups - 1 - (int)(blockIdx.x / nph);
    const int ph = (int)(blockIdx.x % nph);
    const int seg = ph / hgroups;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = (ph % hgroups) * HPW + (wave >> 2);
    const int kvh = h / (hq / hkv);                          // the same for all HPW heads
    const int s0 = cu[seg], n = cu[seg + 1] - s0;
    if (qg * 64 >= n) return;                                // whole workgroup idle (uniform)
    const int fr = lane & 15, fg = lane >> 4;
    const size_t ld = (size_t)(hq + 2 * hkv) * kTHd;
    const T* kbase_p = qkv + (size_t)hq * kTHd + (size_t)kvh * kTHd;
    const T* vbase_p = kbase_p + (size_t)hkv * kTHd;
    const int qt = qg * 4 + (wave & 3);
    const bool active = qt * 16 < n;                         // wave-uniform
    const int q = qt * 16 + fr;                              // this lane's query (within the prompt)
    uint4 qf[KBN];
    {
        const T* row = qkv + (size_t)(s0 + q) * ld + h * kTHd + fg * PER;
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) qf[kb] = q < n ? ld16(row + kb * (64 / (int)sizeof(T))) : zero16();
    }
    const float sc = 0.08838834764831845f * 1.4426950408889634f;   // 1/sqrt(128) * log2(e)
    float m = -INFINITY, l = 0.f;
    f32x4 o[kTHd / 16];
#pragma unroll
    for (int dt = 0; dt < kTHd / 16; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int kend = min(n, qg * 64 + 64);                   // causal: no key beyond the group's last query
    // K / V rows of a key block go global -> registers one block ahead (the
    // loads of block k0 + kTKB are in flight while block k0 is multiplied),
    // then registers -> LDS (V transposed) at the top of the next iteration.
    // Chunk c of this thread is key row key_of(c), 16-byte column tid % CPR.
    // bf16: the thread's keys come in adjacent pairs (2 p, 2 p + 1), so the
    // transposed V store writes both keys of a dimension as one 4-byte word.
    static_assert(sizeof(T) != 2 || NCH % 2 == 0, "key pairs");
    auto key_of = [&](int c) {
        if constexpr (sizeof(T) == 2) return 2 * (tid / CPR + (c / 2) * (NT / CPR)) + (c & 1);
        else return (tid + c * NT) / CPR;
    };
    uint4 kv[NCH], vv[NCH];
    auto load_block = [&](int k0) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int t = key_of(c), ch = tid % CPR;
            kv[c] = vv[c] = zero16();
            if (k0 + t < n) {
                const size_t off = (size_t)(s0 + k0 + t) * ld + ch * PER;
                kv[c] = ld16(kbase_p + off);
                vv[c] = ld16(vbase_p + off);
            }
        }
    };
    load_block(0);
    for (int k0 = 0; k0 < kend; k0 += kTKB) {
        __syncthreads();                                     // previous block consumed
        {
            const int ch = tid % CPR;
#pragma unroll
            for (int c = 0; c < NCH; ++c) st16(ks + key_of(c) * KR + ch * 16, kv[c]);
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int c = 0; c < NCH; c += 2) {
                    const int t = key_of(c);              // even; t + 1 is chunk c + 1's key
                    const unsigned* va = reinterpret_cast<const unsigned*>(&vv[c]);
                    const unsigned* vb = reinterpret_cast<const unsigned*>(&vv[c + 1]);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {         // dims 2 w, 2 w + 1 of the chunk
                        const unsigned lo = __builtin_amdgcn_perm(vb[w], va[w], 0x05040100u);   // (a.d0, b.d0)
                        const unsigned hi = __builtin_amdgcn_perm(vb[w], va[w], 0x07060302u);   // (a.d1, b.d1)
                        *reinterpret_cast<unsigned*>(vts + (ch * PER + 2 * w) * VR + t * 2) = lo;
                        *reinterpret_cast<unsigned*>(vts + (ch * PER + 2 * w + 1) * VR + t * 2) = hi;
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const T* ve = reinterpret_cast<const T*>(&vv[c]);
#pragma unroll
                    for (int e = 0; e < PER; ++e)
                        *reinterpret_cast<T*>(vts + (ch * PER + e) * VR + key_of(c) * sizeof(T)) = ve[e];
                }
            }
        }
        __syncthreads();
        if (k0 + kTKB < kend) load_block(k0 + kTKB);
        if (!active || k0 > qt * 16 + 15) continue;          // this wave's queries precede the block
        f32x4 sacc[kTKB / 16];
#pragma unroll
        for (int kt = 0; kt < kTKB / 16; ++kt) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
#pragma unroll
            for (int kt = 0; kt < kTKB / 16; ++kt) {
                const uint4 kf = ld16(ks + (kt * 16 + fr) * KR + fg * 16 + kb * 64);
                mfma_kblock(T(), kf, qf[kb], sacc[kt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane holds S^T[key k0 + 16 kt + 4 fg + r][query fr]
        float bm = -INFINITY;
        if (k0 + kTKB - 1 <= qt * 16 && k0 + kTKB <= n) {   // whole block visible to every query of the wave
#pragma unroll
            for (int kt = 0; kt < kTKB / 16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    sacc[kt][r] *= sc;
                    bm = fmaxf(bm, sacc[kt][r]);
                }
        } else {
#pragma unroll
            for (int kt = 0; kt < kTKB / 16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = k0 + kt * 16 + 4 * fg + r;
                    const float v = (key <= q && key < n) ? sacc[kt][r] * sc : -INFINITY;
                    sacc[kt][r] = v;
                    bm = fmaxf(bm, v);
                }
        }
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mn = fmaxf(m, bm);
        // a query past the prompt end (q >= n) sees no key: keep it finite
        const float mref = mn == -INFINITY ? 0.f : mn;
        const float alpha = __builtin_amdgcn_exp2f(m - mref);
        float bs = 0.f;
#pragma unroll
        for (int kt = 0; kt < kTKB / 16; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(sacc[kt][r] - mref);
                sacc[kt][r] = p;
                bs += p;
            }
        bs += __shfl_xor(bs, 16);
        bs += __shfl_xor(bs, 32);
        l = l * alpha + bs;
        m = mn;
#pragma unroll
        for (int dt = 0; dt < kTHd / 16; ++dt) o[dt] = o[dt] * alpha;
        if (sizeof(T) == 2) {
#pragma unroll
            for (int st = 0; st < kTKB / 32; ++st) {
                tpv_step(T(), vts, 32 * st, fr, fg, sacc, 2 * st, o);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < kTKB / 16; ++kt) {
                tpv_step(T(), vts, 16 * kt, fr, fg, sacc, kt, o);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    if (active && q < n) {
        const float inv = 1.0f / l;
        T* orow = out + (size_t)(s0 + q) * hq * kTHd + h * kTHd;
#pragma unroll
        for (int dt = 0; dt < kTHd / 16; ++dt)
            store4(orow + dt * 16 + 4 * fg, o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
    }
}

// ---------------------------------------------------------------- launches

template <typename T>
hipError_t embed_splice(hipStream_t s, const T* embed, const float* audio, const int* src, int M, int H, float* x) {
    if (M <= 0) return hipSuccess;
    if (H % 4) return hipErrorInvalidValue;
    embed_splice_kernel<T><<<(M + 3) / 4, 256, 0, s>>>(embed, audio, src, M, H, x);
    return hipGetLastError();
}

template <typename T>
hipError_t rmsnorm(hipStream_t s, const float* x, int M, int H, const float* g, float eps, T* out) {
    if (M <= 0) return hipSuccess;
    if (H % 4 || H > 4 * 64 * kRmsMaxVec) return hipErrorInvalidValue;
    const int blocks = min((M + 3) / 4, 1024);
    rmsnorm_kernel<T><<<blocks, 256, 0, s>>>(x, M, H, g, eps, out);
    return hipGetLastError();
}

template <typename T>
hipError_t qknorm_rope(hipStream_t s, T* qkv, int M, int hq, int hkv, const int* pos, const float* qg,
                       const float* kg, const float2* cs, float eps) {
    if (M <= 0) return hipSuccess;
    const int64_t items = (int64_t)M * (hq + hkv);
    qknorm_rope_kernel<T><<<(unsigned)((items + 3) / 4), 256, 0, s>>>(qkv, M, hq, hkv, pos, qg, kg, cs, eps);
    return hipGetLastError();
}

template <typename T>
hipError_t thinker_attention(hipStream_t s, const T* qkv, const int* cu, int n_prompts, int hq, int hkv,
                             int max_len, T* out) {
    if (n_prompts <= 0) return hipSuccess;
    if (hkv <= 0 || hq % hkv) return hipErrorInvalidValue;
    const int qgroups = (max_len + 63) / 64;
    // two query heads of one KV head per workgroup when the group size is even
    const int hpw = (hq / hkv) % 2 == 0 ? 2 : 1;
    const int64_t blocks = (int64_t)n_prompts * (hq / hpw) * qgroups;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (hpw == 2)
        thinker_attention_kernel<T, 2><<<(unsigned)blocks, 512, 0, s>>>(qkv, cu, hq, hkv, qgroups, out);
    else
        thinker_attention_kernel<T, 1><<<(unsigned)blocks, 256, 0, s>>>(qkv, cu, hq, hkv, qgroups, out);
    return hipGetLastError();
}

#define QA_TINST(T)                                                                                          \
    template hipError_t embed_splice<T>(hipStream_t, const T*, const float*, const int*, int, int, float*);  \
    template hipError_t rmsnorm<T>(hipStream_t, const float*, int, int, const float*, float, T*);           \
    template hipError_t qknorm_rope<T>(hipStream_t, T*, int, int, int, const int*, const float*, const float*, \
                                       const float2*, float);                                                \
    template hipError_t thinker_attention<T>(hipStream_t, const T*, const int*, int, int, int, int, T*);
QA_TINST(float)
QA_TINST(bf16)
#undef QA_TINST

}  // namespace qa
