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
// out[r] = x[r] / sqrt(mean(x[r]^2) + eps) * g, one wave per row (a row of
// H <= 256 NQ values is NQ float4 per lane).  The grid normally covers every
// row at once (each wave walks rows row0, row0 + stride, ... past that); the
// gain is loaded once per wave, with the first row.
constexpr int kRmsMaxVec = 16;

template <typename T, int NQ>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int M, int H,
                                                      const float* __restrict__ g, float eps, T* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int h4 = H >> 2;
    const float4* g4 = reinterpret_cast<const float4*>(g);
    int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    float4 gg[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i = lane + 64 * q;
        if (i < h4) gg[q] = g4[i];
    }
    for (; row < M; row += gridDim.x * 4) {
        const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * H);
        float4 v[NQ];
        float ss = 0.f;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int i = lane + 64 * q;
            if (i < h4) {
                v[q] = xr[i];
                ss += (v[q].x * v[q].x + v[q].y * v[q].y) + (v[q].z * v[q].z + v[q].w * v[q].w);
            }
        }
        const float r = rsqrtf(wsum(ss) / (float)H + eps);
        T* orow = out + (size_t)row * H;
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int i = lane + 64 * q;
            if (i < h4)
                store4(orow + 4 * i, v[q].x * r * gg[q].x, v[q].y * r * gg[q].y, v[q].z * r * gg[q].z,
                       v[q].w * r * gg[q].w);
        }
    }
}

// ---------------------------------------------------------------- QK-norm + RoPE
// In place on the fused projection rows [q (Hq x 128) | k (Hkv x 128) | v]:
// for every query and key head, RMSNorm over the 128 values with the
// [128] gain, then the rotate-half RoPE at the token's position:
// (a, b) = (x[i], x[i + 64]) -> (a c - b s, b c + a s), c, s = cos, sin of
// pos * base^(-i / 64), taken from a table computed in double on the host.
// 16 lanes per (token, head), 4 per wave: lane j of a group holds the pairs
// (i, i + 64) for i = 4 j .. 4 j + 3, read and written as 4-element vectors.
__device__ __forceinline__ void load4f(const float* p, float* v) {
    const float4 t = *reinterpret_cast<const float4*>(p);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
__device__ __forceinline__ void load4f(const bf16* p, float* v) {
    const uint2 t = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(t.x << 16); v[1] = __uint_as_float(t.x & 0xffff0000u);
    v[2] = __uint_as_float(t.y << 16); v[3] = __uint_as_float(t.y & 0xffff0000u);
}

template <typename T>
__global__ __launch_bounds__(256) void qknorm_rope_kernel(T* __restrict__ qkv, int M, int hq, int hkv,
                                                          const int* __restrict__ pos,
                                                          const float* __restrict__ qg, const float* __restrict__ kg,
                                                          const float2* __restrict__ cs, float eps) {
    const int lane = threadIdx.x & 63, j = lane & 15;
    const int64_t item = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 4 + (lane >> 4);
    const int heads = hq + hkv;
    if (item >= (int64_t)M * heads) return;              // uniform within the 16-lane group
    const int t = (int)(item / heads), h = (int)(item - (int64_t)t * heads);
    T* p = qkv + (size_t)t * (hq + 2 * hkv) * 128 + h * 128 + 4 * j;
    float a[4], b[4];
    load4f(p, a);
    load4f(p + 64, b);
    const float* gp = (h < hq ? qg : kg) + 4 * j;
    const float4 ga = *reinterpret_cast<const float4*>(gp), gb = *reinterpret_cast<const float4*>(gp + 64);
    const float4* c4 = reinterpret_cast<const float4*>(cs + (size_t)pos[t] * 64 + 4 * j);
    const float4 c01 = c4[0], c23 = c4[1];                // (cos, sin) of i = 4 j .. 4 j + 3
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) ss += a[e] * a[e] + b[e] * b[e];
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
    const float r = rsqrtf(ss / 128.0f + eps);
    const float gA[4] = {ga.x, ga.y, ga.z, ga.w}, gB[4] = {gb.x, gb.y, gb.z, gb.w};
    const float cc[4] = {c01.x, c01.z, c23.x, c23.z}, sn[4] = {c01.y, c01.w, c23.y, c23.w};
    float oa[4], ob[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float an = a[e] * r * gA[e], bn = b[e] * r * gB[e];
        oa[e] = an * cc[e] - bn * sn[e];
        ob[e] = bn * cc[e] + an * sn[e];
    }
    store4(p, oa[0], oa[1], oa[2], oa[3]);
    store4(p + 64, ob[0], ob[1], ob[2], ob[3]);
}

// ---------------------------------------------------------------- attention
// Causal grouped-query attention, head_dim 128, over packed prompts
// [cu[i], cu[i + 1]); query head h reads KV head h / (hq / hkv).  One
// workgroup per (prompt, query heads, query block): 128 queries in bf16 (two
// 16-query tiles per wave), 64 in fp32 (one tile per wave).  Per key block of
// 64: S^T = K Q^T on MFMA (a lane holds one query column), the causal mask,
// an online softmax (running max / sum, the partial output rescaled when the
// max grows past a margin) and O^T = V^T P^T with V^T transposed in LDS; the
// workgroup stops at the block holding its last query.  When a KV head serves
// an even number of query heads, a workgroup takes two of them so each K/V
// block is staged once for both.
constexpr int kTHd = 128;
constexpr int kTKB = 64;                     // keys per block
constexpr int kTQB = 128;                    // queries per workgroup (bf16)

// bf16: LDS row of key k within its 32-key step.  The S^T MFMA gives lane
// group g the rows 4 g .. 4 g + 3 of each 16-row tile; storing key
// 8 g + 4 h + r at row 16 h + 4 g + r makes the 8 probabilities a lane feeds
// to the P.V MFMA those of 8 consecutive keys, so their V^T values are one
// 16-byte read.
__device__ __forceinline__ int tkey_row(int k) {
    return (k & ~31) | (((k >> 2) & 1) << 4) | (((k >> 3) & 3) << 2) | (k & 3);
}
// The inverse: the key held at LDS row rho.
__device__ __forceinline__ int trow_key(int rho) {
    return (rho & ~31) | (((rho >> 2) & 3) << 3) | (((rho >> 4) & 1) << 2) | (rho & 3);
}

template <typename T> struct TAttnLds;
template <> struct TAttnLds<bf16> {
    static constexpr int krow = kTHd * 2 + 16;      // bytes per K row (padded)
    static constexpr int vrow = kTKB * 2 + 16;      // bytes per V^T row (row vt_row(d) for dim d; 16-byte reads)
};
template <> struct TAttnLds<float> {
    static constexpr int krow = kTHd * 4 + 16;
    static constexpr int vrow = kTKB * 4 + 16;
};

// P.V for the QT query tiles of a wave over one 32-key step (bf16) or one
// 16-key tile (fp32): each V^T fragment is read from LDS once and multiplied
// into every query tile.  bf16: o[u][kTHd / 16] (the extra tile) accumulates
// the probability sums; its A operand is all ones, so each of its rows is
// sum_k p[k][query], taken over the same bf16-rounded probabilities that
// weight V.
template <int QT>
__device__ __forceinline__ void tpv_step(bf16, const char* vt, int kbase, int fr, int fg,
                                         const f32x4 (*p)[kTKB / 16], int t0, f32x4 (*o)[kTHd / 16 + 1]) {
    // slots 0..3: LDS rows kbase + 4g + r (tile t0), 4..7: kbase + 16 + 4g + r
    // (tile t0 + 1), i.e. keys kbase + 8 g .. kbase + 8 g + 7 (tkey_row)
    bf16x8 pb[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) { pb[u][r] = (bf16)p[u][t0][r]; pb[u][4 + r] = (bf16)p[u][t0 + 1][r]; }
    const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);   // bf16 1.0 x 8
#pragma unroll
    for (int u = 0; u < QT; ++u)
        o[u][kTHd / 16] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), pb[u], o[u][kTHd / 16], 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < kTHd / 16; ++dt) {
        const char* row = vt + vt_row(dt * 16 + fr) * TAttnLds<bf16>::vrow;
        const bf16x8 va = __builtin_bit_cast(bf16x8, ld16(row + 2 * (kbase + 8 * fg)));
#pragma unroll
        for (int u = 0; u < QT; ++u) o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[u], o[u][dt], 0, 0, 0);
    }
}
template <int QT>
__device__ __forceinline__ void tpv_step(float, const char* vt, int kbase, int fr, int fg,
                                         const f32x4 (*p)[kTKB / 16], int t0, f32x4 (*o)[kTHd / 16 + 1]) {
#pragma unroll
    for (int dt = 0; dt < kTHd / 16; ++dt) {
        const char* row = vt + vt_row(dt * 16 + fr) * TAttnLds<float>::vrow;
        const float4 va = *reinterpret_cast<const float4*>(row + 4 * (kbase + 4 * fg));
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.x, p[u][t0][0], o[u][dt], 0, 0, 0);
            o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.y, p[u][t0][1], o[u][dt], 0, 0, 0);
            o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.z, p[u][t0][2], o[u][dt], 0, 0, 0);
            o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.w, p[u][t0][3], o[u][dt], 0, 0, 0);
        }
    }
}

// Workgroup = (prompt, HPW consecutive query heads of one KV head, QB
// queries); each head has QB / 16 / QT waves, each taking QT consecutive
// 16-query tiles, so every K and V fragment read from LDS feeds QT MFMAs.
// Each workgroup streams every K/V block up to its diagonal, so the K/V
// traffic (from L2 / the last-level cache) scales as 1 / QB.
template <typename T, int HPW, int QT, int QB>
__global__ __launch_bounds__(HPW * QB / QT * 4) __attribute__((amdgpu_waves_per_eu(2))) void thinker_attention_kernel(const T* __restrict__ qkv,
                                                                                const int* __restrict__ cu, int hq,
                                                                                int hkv, int qgroups,
                                                                                T* __restrict__ out) {
    constexpr int KR = TAttnLds<T>::krow, VR = TAttnLds<T>::vrow;
    constexpr int PER = Elem<T>::per16;
    constexpr int CPR = kTHd / PER;                          // 16-byte chunks per head row
    constexpr int KBN = kTHd * (int)sizeof(T) / 64;          // 64-byte MFMA K blocks per head row
    constexpr int WPH = QB / 16 / QT;                        // waves per head
    constexpr int NT = 64 * HPW * WPH;                       // threads
    constexpr int NCH = kTKB * CPR / NT;                     // chunks per thread per key block
    static_assert(QB % (16 * QT) == 0 && kTKB * CPR % NT == 0, "tiling");
    __shared__ __align__(16) char ks[kTKB * KR];
    __shared__ __align__(16) char vts[kTHd * VR];

    // Causal work grows with the query group, so the groups are dispatched
    // longest first (all (prompt, head group) pairs of the last query group,
    // then the one before, ...): the short ones fill the tail.
    const int hgroups = hq / HPW;
    const int nph = (int)(gridDim.x / qgroups);              // (prompt, head group) pairs
    const int qg = qgroups - 1 - (int)(blockIdx.x / nph);
    const int ph = (int)(blockIdx.x % nph);
    const int seg = ph / hgroups;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = (ph % hgroups) * HPW + wave / WPH;
    const int kvh = h / (hq / hkv);                          // the same for all HPW heads
    const int s0 = cu[seg], n = cu[seg + 1] - s0;
    if (qg * QB >= n) return;                                // whole workgroup idle (uniform)
    const int fr = lane & 15, fg = lane >> 4;
    const size_t ld = (size_t)(hq + 2 * hkv) * kTHd;
    const T* kbase_p = qkv + (size_t)hq * kTHd + (size_t)kvh * kTHd;
    const T* vbase_p = kbase_p + (size_t)hkv * kTHd;
    const int qt0 = qg * (QB / 16) + (wave % WPH) * QT;      // this wave's first query tile
    const bool active = qt0 * 16 < n;                        // wave-uniform
    uint4 qf[QT][KBN];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        const int q = (qt0 + u) * 16 + fr;
        const T* row = qkv + (size_t)(s0 + q) * ld + h * kTHd + fg * PER;
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) qf[u][kb] = q < n ? ld16(row + kb * (64 / (int)sizeof(T))) : zero16();
    }
    const float sc = 0.08838834764831845f * 1.4426950408889634f;   // 1/sqrt(128) * log2(e)
    // Online softmax in log2 units.  m is the reference the probabilities are
    // taken against, 2^(s sc - m); it moves to the running maximum only when
    // some lane's block maximum exceeds it by more than kLazy (the decision is
    // wave-uniform), so most blocks skip the rescaling of o and keep p below
    // 2^kLazy.  -inf while the lane's query has seen no key.
    constexpr float kLazy = 8.f;
    constexpr bool kSumMfma = sizeof(T) == 2;                // row sums in o[u][kTHd / 16] (bf16)
    float m[QT], l[QT];
    f32x4 o[QT][kTHd / 16 + 1];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        m[u] = -INFINITY;
        l[u] = 0.f;
#pragma unroll
        for (int dt = 0; dt <= kTHd / 16; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    const int kend = min(n, qg * QB + QB);                   // causal: no key beyond the group's last query
    // K / V rows of a key block go global -> registers two blocks ahead (the
    // loads of blocks k0 + kTKB and k0 + 2 kTKB are in flight while block k0
    // is multiplied; two register sets alternate), then registers -> LDS (V
    // transposed) at the top of the block's own iteration.
    // Chunk c of this thread is key row key_of(c), 16-byte column tid % CPR.
    // bf16: the thread's keys come in adjacent pairs (2 p, 2 p + 1), so the
    // transposed V store writes both keys of a dimension as one 4-byte word.
    static_assert(sizeof(T) != 2 || NCH % 2 == 0, "key pairs");
    auto key_of = [&](int c) {
        if constexpr (sizeof(T) == 2) return 2 * (tid / CPR + (c / 2) * (NT / CPR)) + (c & 1);
        else return (tid + c * NT) / CPR;
    };
    using Regs = uint4[NCH];
    Regs kvA, vvA, kvB, vvB;
    auto load_block = [&](int k0, Regs& kv, Regs& vv) {
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
    auto process = [&](int k0, Regs& kv, Regs& vv) {
        __syncthreads();                                     // previous block consumed
        {
            const int ch = tid % CPR;
#pragma unroll
            for (int c = 0; c < NCH; ++c)
                st16(ks + (sizeof(T) == 2 ? tkey_row(key_of(c)) : key_of(c)) * KR + ch * 16, kv[c]);
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
                        *reinterpret_cast<unsigned*>(vts + vt_row(ch * PER + 2 * w) * VR + t * 2) = lo;
                        *reinterpret_cast<unsigned*>(vts + vt_row(ch * PER + 2 * w + 1) * VR + t * 2) = hi;
                    }
                }
            } else {
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const T* ve = reinterpret_cast<const T*>(&vv[c]);
#pragma unroll
                    for (int e = 0; e < PER; ++e)
                        *reinterpret_cast<T*>(vts + vt_row(ch * PER + e) * VR + key_of(c) * sizeof(T)) = ve[e];
                }
            }
        }
        __syncthreads();
        if (k0 + 2 * kTKB < kend) load_block(k0 + 2 * kTKB, kv, vv);
        if (!active || k0 > (qt0 + QT) * 16 - 1) return;     // every query of the wave precedes the block
        f32x4 sacc[QT][kTKB / 16];
#pragma unroll
        for (int u = 0; u < QT; ++u)
#pragma unroll
            for (int kt = 0; kt < kTKB / 16; ++kt) sacc[u][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
#pragma unroll
            for (int kt = 0; kt < kTKB / 16; ++kt) {
                const uint4 kf = ld16(ks + (kt * 16 + fr) * KR + fg * 16 + kb * 64);
#pragma unroll
                for (int u = 0; u < QT; ++u) mfma_kblock(T(), kf, qf[u][kb], sacc[u][kt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane holds S^T[LDS row 16 kt + 4 fg + r][query (qt0 + u) 16 + fr] (unscaled);
        // the row is key k0 + trow_key(row) in bf16, key k0 + row in fp32
        const bool full = k0 + kTKB - 1 <= qt0 * 16 && k0 + kTKB <= n;   // visible to every query of the wave
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            const int q = (qt0 + u) * 16 + fr;
            float bm = -INFINITY;
            if (full) {
#pragma unroll
                for (int kt = 0; kt < kTKB / 16; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) bm = fmaxf(bm, sacc[u][kt][r]);
            } else {
#pragma unroll
                for (int kt = 0; kt < kTKB / 16; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rho = kt * 16 + 4 * fg + r;
                        const int key = k0 + (sizeof(T) == 2 ? trow_key(rho) : rho);
                        const float v = (key <= q && key < n) ? sacc[u][kt][r] : -INFINITY;
                        sacc[u][kt][r] = v;
                        bm = fmaxf(bm, v);
                    }
            }
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            const float bms = bm * sc;                       // block maximum in log2 units (sc > 0)
            if (__builtin_amdgcn_ballot_w64(bms > m[u] + kLazy) != 0) {
                const float mn = fmaxf(m[u], bms);
                // alpha = 0 while nothing has been accumulated (m = -inf)
                const float alpha = m[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[u] - mn);
#pragma unroll
                for (int dt = 0; dt <= kTHd / 16; ++dt) o[u][dt] = o[u][dt] * alpha;
                l[u] *= alpha;
                m[u] = mn;
            }
            // a query that has seen no key keeps m = -inf: take 0 as the reference
            const float mref = m[u] == -INFINITY ? 0.f : m[u];
            float bs = 0.f;
#pragma unroll
            for (int kt = 0; kt < kTKB / 16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sacc[u][kt][r], sc, -mref));
                    sacc[u][kt][r] = p;
                    if constexpr (!kSumMfma) bs += p;
                }
            if constexpr (!kSumMfma) {
                bs += __shfl_xor(bs, 16);
                bs += __shfl_xor(bs, 32);
                l[u] += bs;
            }
        }
        if (sizeof(T) == 2) {
#pragma unroll
            for (int st = 0; st < kTKB / 32; ++st) {
                tpv_step<QT>(T(), vts, 32 * st, fr, fg, sacc, 2 * st, o);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < kTKB / 16; ++kt) {
                tpv_step<QT>(T(), vts, 16 * kt, fr, fg, sacc, kt, o);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        };
    load_block(0, kvA, vvA);
    if (kTKB < kend) load_block(kTKB, kvB, vvB);
    for (int k0 = 0; k0 < kend; k0 += 2 * kTKB) {
        process(k0, kvA, vvA);
        if (k0 + kTKB < kend) process(k0 + kTKB, kvB, vvB);
    }
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        const int q = (qt0 + u) * 16 + fr;
        if (active && q < n) {
            const float inv = 1.0f / (kSumMfma ? o[u][kTHd / 16][0] : l[u]);
            T* orow = out + (size_t)(s0 + q) * hq * kTHd + h * kTHd;
#pragma unroll
            for (int dt = 0; dt < kTHd / 16; ++dt)
                store4(orow + dt * 16 + 4 * fg, o[u][dt][0] * inv, o[u][dt][1] * inv, o[u][dt][2] * inv,
                       o[u][dt][3] * inv);
        }
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
    const int blocks = min((M + 3) / 4, 16384);             // one wave per row up to 64K rows
    if (H <= 1024) rmsnorm_kernel<T, 4><<<blocks, 256, 0, s>>>(x, M, H, g, eps, out);
    else if (H <= 2048) rmsnorm_kernel<T, 8><<<blocks, 256, 0, s>>>(x, M, H, g, eps, out);
    else rmsnorm_kernel<T, kRmsMaxVec><<<blocks, 256, 0, s>>>(x, M, H, g, eps, out);
    return hipGetLastError();
}

template <typename T>
hipError_t qknorm_rope(hipStream_t s, T* qkv, int M, int hq, int hkv, const int* pos, const float* qg,
                       const float* kg, const float2* cs, float eps) {
    if (M <= 0) return hipSuccess;
    const int64_t items = (int64_t)M * (hq + hkv);          // 16 per workgroup (4 per wave)
    if ((items + 15) / 16 > 0x7fffffff) return hipErrorInvalidValue;
    qknorm_rope_kernel<T><<<(unsigned)((items + 15) / 16), 256, 0, s>>>(qkv, M, hq, hkv, pos, qg, kg, cs, eps);
    return hipGetLastError();
}

template <typename T>
hipError_t thinker_attention(hipStream_t s, const T* qkv, const int* cu, int n_prompts, int hq, int hkv,
                             int max_len, T* out) {
    if (n_prompts <= 0) return hipSuccess;
    if (hkv <= 0 || hq % hkv) return hipErrorInvalidValue;
    // bf16: two 16-query tiles per wave, 128 queries per workgroup; fp32
    // (register-heavy): one tile per wave, 64 queries
    constexpr int QT = sizeof(T) == 2 ? 2 : 1;
    constexpr int QB = sizeof(T) == 2 ? kTQB : 64;
    const int qgroups = (max_len + QB - 1) / QB;
    // two query heads of one KV head per workgroup when the group size is even
    const int hpw = (hq / hkv) % 2 == 0 ? 2 : 1;
    const int64_t blocks = (int64_t)n_prompts * (hq / hpw) * qgroups;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    if (hpw == 2)
        thinker_attention_kernel<T, 2, QT, QB><<<(unsigned)blocks, 2 * QB / QT * 4, 0, s>>>(qkv, cu, hq, hkv, qgroups, out);
    else
        thinker_attention_kernel<T, 1, QT, QB><<<(unsigned)blocks, QB / QT * 4, 0, s>>>(qkv, cu, hq, hkv, qgroups, out);
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
