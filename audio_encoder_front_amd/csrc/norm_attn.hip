// LayerNorm (fp32 statistics, one wave per row) and block-diagonal windowed
// multi-head attention (one workgroup per (window, head)), plus the
// full-input variant with one attention segment per clip (OneSpeech "Front
// end and graph numerics": CPU graphs attend over the whole bounded input).
//
// qwenasr.cpp ARCHITECTURE.md "Windowed audio tower": pre-norm blocks with
// LayerNorm carrying a bias; bidirectional attention without RoPE, scaled by
// 1/sqrt(head_dim), confined by a block-diagonal mask to windows of 13 * 8 =
// 104 tokens; M* ASR page "Graph": one attention segment per window of every
// request, all in one packed ragged batch (cu_seqlens).  OneSpeech "Front end
// and graph numerics": scores and softmax stay fp32, the attended output is
// rounded to bf16.
#include <algorithm>

#include "qa_device.h"
#include "qa_kernels.h"

#include <type_traits>

namespace qa {

// ------------------------------------------------------------ LayerNorm

template <typename T, int NQ>
__global__ __launch_bounds__(256) void layernorm_kernel(const float* __restrict__ x, int M, int d,
                                                        const float* __restrict__ g,
                                                        const float* __restrict__ b, T* __restrict__ out) {
    // One wave per row (a row of d <= 256 NQ values is NQ float4 per lane).
    // The grid normally covers every row at once; past that, each wave walks
    // rows row0, row0 + stride, ... with the next row's loads issued before
    // the current row is reduced.  gamma / beta are loaded with the row, so
    // their (L2) latency hides under the row's.
    const int lane = threadIdx.x & 63;
    const int stride = gridDim.x * 4;
    const int d4 = d >> 2;
    const float4* g4 = reinterpret_cast<const float4*>(g);
    const float4* b4 = reinterpret_cast<const float4*>(b);
    auto load_row = [&](int row, float4* v) {
        const float4* xr = reinterpret_cast<const float4*>(x + (size_t)row * d);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int i = lane + 64 * q;
            if (i < d4) v[q] = xr[i];
        }
    };
    int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= M) return;
    float4 cur[NQ], nxt[NQ], gg[NQ], bb[NQ];
    load_row(row, cur);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i = lane + 64 * q;
        if (i < d4) { gg[q] = g4[i]; bb[q] = b4[i]; }
    }
    for (; row < M; row += stride) {
        if (row + stride < M) load_row(row + stride, nxt);
        ln_row<T, NQ>(cur, gg, bb, lane, d, out + (size_t)row * d);
#pragma unroll
        for (int q = 0; q < NQ; ++q) cur[q] = nxt[q];
    }
}

template <typename T>
hipError_t layernorm(hipStream_t s, const float* x, int M, int d, const float* g, const float* b, T* out) {
    if (M <= 0) return hipSuccess;
    if (d % 4 || d > 2048) return hipErrorInvalidValue;
    // One wave per row up to 64K rows (every row's loads in flight at once).
    const int blocks = std::min((M + 3) / 4, 16384);
    if (d <= 1024) layernorm_kernel<T, 4><<<blocks, 256, 0, s>>>(x, M, d, g, b, out);
    else layernorm_kernel<T, 8><<<blocks, 256, 0, s>>>(x, M, d, g, b, out);
    return hipGetLastError();
}

// ------------------------------------------------------------ attention
//
// Per wave and 16-query tile: S^T = K Q^T on MFMA (keys as rows), so each lane
// holds one query column and 4 keys per 16-key tile; the softmax over keys
// reduces in-lane, then across the 4 lane groups with two xor shuffles.  The
// probabilities then feed O^T = V^T P^T straight from registers: for a
// 32-key MFMA step the lane's 8 k-slots are its keys {4g..4g+3} of two key
// tiles, and V^T (kept transposed in LDS) is read at the same keys.

constexpr int kHd = 64;

// LDS rows: K rows of the head (64 values + 16 bytes of padding) and V^T
// rows (head dimension d at row vt_row(d), ROWS keys + padding), for ROWS
// keys.
template <typename T, int ROWS> struct AttnLds {
    static constexpr int qrow = 64 * (int)sizeof(T) + 16;
    static constexpr int vrow = (int)sizeof(T) * ROWS + (sizeof(T) == 2 ? 40 : 16);
};

// P.V over one 32-key step (bf16) or one 16-key tile (fp32), accumulate o[dt].
// HALF: the step's second key tile lies past the LDS rows (an odd number of
// key tiles); its V values are taken as zero, its probabilities are zero.
template <int VR, bool HALF = false>
__device__ __forceinline__ void pv_step(bf16, const char* vt, int kbase, int fr, int fg, const f32x4* p,
                                        int t0, f32x4* o) {
    // slots 0..3: keys kbase + 4g + r (tile t0), slots 4..7: kbase + 16 + 4g + r (tile t0 + 1)
    bf16x8 pb;
#pragma unroll
    for (int r = 0; r < 4; ++r) { pb[r] = (bf16)p[t0][r]; pb[4 + r] = (bf16)p[t0 + 1][r]; }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const char* row = vt + vt_row(dt * 16 + fr) * VR;
        const uint2 lo = *reinterpret_cast<const uint2*>(row + 2 * (kbase + 4 * fg));
        const uint2 hi = HALF ? make_uint2(0u, 0u) : *reinterpret_cast<const uint2*>(row + 2 * (kbase + 16 + 4 * fg));
        const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pb, o[dt], 0, 0, 0);
    }
}
template <int VR>
__device__ __forceinline__ void pv_step(float, const char* vt, int kbase, int fr, int fg, const f32x4* p,
                                        int t0, f32x4* o) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const char* row = vt + vt_row(dt * 16 + fr) * VR;
        const float4 va = *reinterpret_cast<const float4*>(row + 4 * (kbase + 4 * fg));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.x, p[t0][0], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.y, p[t0][1], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.z, p[t0][2], o[dt], 0, 0, 0);
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.w, p[t0][3], o[dt], 0, 0, 0);
    }
}

template <typename T, int KT>
__global__ __launch_bounds__(256) void attention_kernel(const T* __restrict__ qkv, const int* __restrict__ cu,
                                                        int n_heads, int d, T* __restrict__ out) {
    constexpr int ROWS = KT * 16;                  // keys held in LDS
    constexpr int QR = AttnLds<T, ROWS>::qrow, VR = AttnLds<T, ROWS>::vrow;
    constexpr int PER = Elem<T>::per16;
    constexpr int CPR = kHd / PER;                 // 16-byte chunks per head row
    constexpr int KBN = kHd * (int)sizeof(T) / 64; // 64-byte MFMA K blocks per head row
    __shared__ __align__(16) char ks[ROWS * QR];
    __shared__ __align__(16) char vts[kHd * VR];

    const int win = blockIdx.x / n_heads, h = blockIdx.x % n_heads;
    const int s0 = cu[win], n = cu[win + 1] - s0;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
    const int fr = lane & 15, fg = lane >> 4;
    const int nt = (n + 15) >> 4;                  // 16-row tiles in this window
    const size_t ld = 3 * (size_t)d;

    // Query fragments of this wave's first tile come straight from global
    // memory (B operand: lane holds query row fr, K chunk fg of each block).
    auto load_q = [&](int qt, uint4* qf) {
        const int q = qt * 16 + fr;
        const T* row = qkv + (size_t)(s0 + q) * ld + h * kHd + fg * PER;
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) qf[kb] = q < n ? ld16(row + kb * (64 / (int)sizeof(T))) : zero16();
    };
    uint4 qf[KBN];
    if (wave < nt) load_q(wave, qf);

    // K and V rows of this head (16 bytes per load, every load issued before
    // any LDS store); rows at or beyond n are zeros.  V is stored transposed.
    constexpr int NCH = (ROWS * CPR + 255) / 256;  // 16-byte chunks per thread per matrix
    // Chunk q of this thread is key row key_of(q), 16-byte column tid % CPR;
    // bf16 keys come in adjacent pairs (2 p, 2 p + 1) so that the transposed
    // V store writes both keys of a dimension as one 4-byte word.
    static_assert(sizeof(T) != 2 || NCH % 2 == 0, "key pairs");
    auto key_of = [&](int q) {
        if constexpr (sizeof(T) == 2) return 2 * (tid / CPR + (q / 2) * (256 / CPR)) + (q & 1);
        else return (tid + q * 256) / CPR;
    };
    const int c = tid % CPR;
    uint4 kv[NCH], vv[NCH];
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
        const int t = key_of(q);
        kv[q] = vv[q] = zero16();
        if (t < n) {
            const T* row = qkv + (size_t)(s0 + t) * ld + d + h * kHd + c * PER;
            kv[q] = ld16(row);
            vv[q] = ld16(row + d);
        }
    }
#pragma unroll
    for (int q = 0; q < NCH; ++q) {
        const int t = key_of(q);
        if (t < ROWS) st16(ks + t * QR + c * 16, kv[q]);
    }
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int q = 0; q < NCH; q += 2) {
            const int t = key_of(q);                   // even; t + 1 is chunk q + 1's key
            if (t >= ROWS) continue;                   // ROWS is even: the pair is in or out together
            const unsigned* va = reinterpret_cast<const unsigned*>(&vv[q]);
            const unsigned* vb = reinterpret_cast<const unsigned*>(&vv[q + 1]);
#pragma unroll
            for (int w = 0; w < 4; ++w) {              // dimensions 2 w, 2 w + 1 of the chunk
                *reinterpret_cast<unsigned*>(vts + vt_row(c * PER + 2 * w) * VR + t * 2) =
                    __builtin_amdgcn_perm(vb[w], va[w], 0x05040100u);   // (key t, key t + 1) of dim 2 w
                *reinterpret_cast<unsigned*>(vts + vt_row(c * PER + 2 * w + 1) * VR + t * 2) =
                    __builtin_amdgcn_perm(vb[w], va[w], 0x07060302u);   // ... of dim 2 w + 1
            }
        }
    } else {
#pragma unroll
        for (int q = 0; q < NCH; ++q) {
            const int t = key_of(q);
            if (t >= ROWS) continue;
            const T* ve = reinterpret_cast<const T*>(&vv[q]);
#pragma unroll
            for (int e = 0; e < PER; ++e)
                *reinterpret_cast<T*>(vts + vt_row(c * PER + e) * VR + t * sizeof(T)) = ve[e];
        }
    }
    __syncthreads();

    const float sc = 0.125f * 1.4426950408889634f; // 1/sqrt(64) * log2(e)
    // KT key tiles of 16 hold every key of the longest window (7 for the
    // 104-token windows); an unused 8th tile only pairs tiles into 32-key
    // P.V steps and stays zero.
    static_assert(KT >= 1 && KT * 16 <= kMaxWindow, "key tiles");
    for (int qt = wave; qt < nt; qt += 4) {
        f32x4 sacc[8];
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {   // rows past n are zeros, masked below
                const uint4 kf = ld16(ks + (kt * 16 + fr) * QR + fg * 16 + kb * 64);
                mfma_kblock(T(), kf, qf[kb], sacc[kt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (qt + 4 < nt) load_q(qt + 4, qf);       // next tile's queries, in flight during softmax and P.V
        // sacc[kt][r] = score(key kt*16 + 4fg + r, query qt*16 + fr).  Keys
        // at or past n exist only in the tiles that reach n (a uniform test
        // per tile); the max is taken on the unscaled scores (sc > 0) and
        // the scale folded into one fma per probability.
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            if (kt * 16 + 16 > n) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (kt * 16 + 4 * fg + r >= n) sacc[kt][r] = -INFINITY;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kt][r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float off = -mx * sc;
        float sum = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], sc, off));
                sacc[kt][r] = p;
                sum += p;
            }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        f32x4 o[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (sizeof(T) == 2) {
#pragma unroll
            for (int st = 0; st < (KT + 1) / 2; ++st) {   // keys past n have p = 0 and zero V rows
                if (2 * st + 1 < KT) pv_step<VR>(T(), vts, 32 * st, fr, fg, sacc, 2 * st, o);
                else pv_step<VR, true>(T(), vts, 32 * st, fr, fg, sacc, 2 * st, o);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                pv_step<VR>(T(), vts, 16 * kt, fr, fg, sacc, kt, o);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        const int q = qt * 16 + fr;
        if (q < n) {
            const float inv = 1.0f / sum;
            T* orow = out + (size_t)(s0 + q) * d + h * kHd;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                store4(orow + dt * 16 + 4 * fg, o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
        }
    }
}

// bf16 windows, two heads per workgroup (four waves each): K and V go
// global -> LDS by direct-to-LDS loads (no register round trip), both
// row-major with their 16-byte chunks XOR-swizzled per row, and the P.V
// operand V^T comes from LDS transpose reads (ds_read_b64_tr_b16: within each
// 16-lane group the 4-element reads of lanes 4 r .. 4 r + 3 form row r of a
// 4 x 16 matrix and lane i receives column i, so two reads give a lane one
// head dimension at 4 + 4 keys).  The two heads of a window read neighbouring
// 128-byte pieces of the same token rows.  Key slots are those of
// attention_kernel (slots 0..3 of a 32-key step: keys 4 g + r, slots 4..7:
// 16 + 4 g + r), so the results are identical to it.
__device__ __forceinline__ int vchunk_swz(int j) { return 2 * (j & 3); }   // keeps chunk pairs adjacent

typedef short lds_s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) lds_s16x4 lds_s16x4_p;
__device__ __forceinline__ uint2 lds_tr_read(const char* p) {
    const lds_s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_p*)p);
    return __builtin_bit_cast(uint2, v);
}

constexpr int kAttnHpw = 2;                      // heads per workgroup of attention_dma_kernel

template <int KT>
__global__ __launch_bounds__(256 * kAttnHpw) void attention_dma_kernel(const bf16* __restrict__ qkv,
                                                                       const int* __restrict__ cu, int n_heads, int d,
                                                                       bf16* __restrict__ out) {
    constexpr int ROWS = KT * 16;                  // keys held in LDS
    constexpr int RB = kHd * 2;                    // bytes per K / V row
    constexpr int BLK = ROWS * RB;                 // bytes per K or V block of one head
    constexpr int NLD = BLK / 1024;                // 1 KB direct-to-LDS loads per block (8 rows each)
    constexpr int KBN = kHd * 2 / 64;              // 64-byte MFMA K blocks per head row
    static_assert(ROWS % 8 == 0, "rows per load");
    __shared__ __align__(1024) char smem_all[kAttnHpw * 2 * BLK];
    const int hw = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8);   // head within the workgroup
    const char* ks = smem_all + hw * 2 * BLK;
    const char* vs = ks + BLK;
    const int hg = n_heads / kAttnHpw;
    const int win = blockIdx.x / hg, h = (blockIdx.x % hg) * kAttnHpw + hw;
    const int s0 = cu[win], n = cu[win + 1] - s0;
    const int tid = threadIdx.x & 255;
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fr = lane & 15, fg = lane >> 4;
    const int nt = (n + 15) >> 4;
    const size_t ld = 3 * (size_t)d;
    const unsigned row_bytes = (unsigned)(ld * 2);

    // query fragments (B operand: lane holds query row fr, K chunk fg of each block)
    auto load_q = [&](int qt, uint4* qf) {
        const int q = qt * 16 + fr;
        const bf16* row = qkv + (size_t)(s0 + q) * ld + h * kHd + fg * 8;
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) qf[kb] = q < n ? ld16(row + kb * 32) : zero16();
    };
    uint4 qf[KBN];
    if (wave < nt) load_q(wave, qf);

    // K and V rows of this head: load q of a block fills rows 8 q .. 8 q + 7,
    // lane l row 8 q + l / 8 at LDS chunk l % 8, which holds source chunk
    // (l % 8) ^ swizzle(row); rows at or past n read zeros (buffer range).
    {
        const i32x4 rk = buffer_rsrc(qkv + (size_t)s0 * ld + d + h * kHd, (uint64_t)n * row_bytes);
        const i32x4 rv = buffer_rsrc(qkv + (size_t)s0 * ld + 2 * d + h * kHd, (uint64_t)n * row_bytes);
        const unsigned lds0 = (unsigned)(uintptr_t)(lds_void*)ks;
        const int lr = lane >> 3, p = lane & 7;
#pragma unroll
        for (int q = wave; q < 2 * NLD; q += 4) {  // wave-uniform: K loads, then V loads
            if (q < NLD) {
                const int row = 8 * q + lr;
                dma16_buf(rk, row < n ? (unsigned)row * row_bytes + (unsigned)((p ^ (row & 7)) << 4) : kOobOffset,
                          lds0 + q * 1024);
            } else {
                const int row = 8 * (q - NLD) + lr;
                dma16_buf(rv, row < n ? (unsigned)row * row_bytes + (unsigned)((p ^ vchunk_swz(row)) << 4) : kOobOffset,
                          lds0 + BLK + (q - NLD) * 1024);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);            // vmcnt(0): this wave's queries and K / V loads
    __syncthreads();

    const float sc = 0.125f * 1.4426950408889634f; // 1/sqrt(64) * log2(e)
    const int tr_r = (lane & 15) >> 2, tr_c = lane & 3;   // transpose-read source row / 8-byte column
    for (int qt = wave; qt < nt; qt += 4) {
        f32x4 sacc[8];
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) sacc[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {      // rows past n are zeros, masked below
                const int row = kt * 16 + fr;
                const uint4 kf = ld16(ks + row * RB + (((4 * kb + fg) ^ (row & 7)) << 4));
                mfma_kblock(bf16(), kf, qf[kb], sacc[kt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (qt + 4 < nt) load_q(qt + 4, qf);       // next tile's queries, in flight during softmax and P.V
        float mx = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            if (kt * 16 + 16 > n) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (kt * 16 + 4 * fg + r >= n) sacc[kt][r] = -INFINITY;
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[kt][r]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float off = -mx * sc;
        float sum = 0.f;
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[kt][r], sc, off));
                sacc[kt][r] = pr;
                sum += pr;
            }
        sum += __shfl_xor(sum, 16);
        sum += __shfl_xor(sum, 32);
        f32x4 o[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        // P.V per 32-key step: rows j0 and j0 + 16 (j0 = 32 st + 4 g + tr_r) of V
#pragma unroll
        for (int st = 0; st < (KT + 1) / 2; ++st) {
            bf16x8 pb;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pb[r] = (bf16)sacc[2 * st][r];
                pb[4 + r] = 2 * st + 1 < KT ? (bf16)sacc[2 * st + 1][r] : (bf16)0.f;
            }
            const int j0 = 32 * st + 4 * fg + tr_r, j1 = j0 + 16;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const int c = 2 * dt + (tr_c >> 1), half = (tr_c & 1) * 8;
                const uint2 lo = lds_tr_read(vs + j0 * RB + ((c ^ vchunk_swz(j0)) << 4) + half);
                // an odd key-tile count leaves the last step's second tile outside the LDS rows
                const uint2 hi = 2 * st + 1 < KT ? lds_tr_read(vs + j1 * RB + ((c ^ vchunk_swz(j1)) << 4) + half)
                                                 : make_uint2(0u, 0u);
                const uint4 va = make_uint4(lo.x, lo.y, hi.x, hi.y);
                o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, va), pb, o[dt], 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const int q = qt * 16 + fr;
        if (q < n) {
            const float inv = 1.0f / sum;
            bf16* orow = out + (size_t)(s0 + q) * d + h * kHd;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                store4(orow + dt * 16 + 4 * fg, o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
        }
    }
}

// Segments longer than 128 tokens (full-input attention over a whole clip):
// one workgroup per (segment, head, block of QB queries): 128 queries in bf16
// with two 16-query tiles per wave (each K / V fragment read from LDS feeds
// two MFMAs), 64 in fp32 with one.  Keys stream through LDS in blocks of 64,
// loaded into registers two blocks ahead (two register sets alternate), with
// an online softmax in log2 units: the 1/sqrt(64) scale folded into the exp2
// argument, and the reference maximum moved (and the partial output
// rescaled) only when some lane's block maximum exceeds it by more than
// kLazy, so the probabilities stay below 2^kLazy.  bf16: V goes to LDS
// transposed as key pairs (one 4-byte write per two keys of a dimension),
// the K rows of each 32-key step sit permuted (key 8 g + 4 h + r at row
// 16 h + 4 g + r) so that the 8 probabilities a lane feeds to the P.V MFMA
// are 8 consecutive keys and their V^T values one 16-byte read, and the row
// sums come from one more MFMA against an all-ones operand (the same
// bf16-rounded probabilities that weight V).
constexpr int kLKB = 64;                         // keys per block
constexpr float kLazy = 8.f;

__device__ __forceinline__ int lkey_row(int k) {   // LDS row of key k (bf16)
    return (k & ~31) | (((k >> 2) & 1) << 4) | (((k >> 3) & 3) << 2) | (k & 3);
}
__device__ __forceinline__ int lrow_key(int rho) { // key held at LDS row rho (bf16)
    return (rho & ~31) | (((rho >> 2) & 3) << 3) | (((rho >> 4) & 1) << 2) | (rho & 3);
}

template <typename T> struct LAttnLds;
template <> struct LAttnLds<bf16> {
    static constexpr int krow = kHd * 2 + 16;
    static constexpr int vrow = kLKB * 2 + 16;   // 16-byte V^T reads
};
template <> struct LAttnLds<float> {
    static constexpr int krow = kHd * 4 + 16;
    static constexpr int vrow = kLKB * 4 + 16;
};

template <int QT, int VR>
__device__ __forceinline__ void lpv_step(bf16, const char* vt, int kbase, int fr, int fg,
                                         const f32x4 (*p)[kLKB / 16], int t0, f32x4 (*o)[kHd / 16 + 1]) {
    // slots 0..3: LDS rows kbase + 4 g + r, 4..7: kbase + 16 + 4 g + r, i.e.
    // keys kbase + 8 g .. + 7
    bf16x8 pb[QT];
#pragma unroll
    for (int u = 0; u < QT; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) { pb[u][r] = (bf16)p[u][t0][r]; pb[u][4 + r] = (bf16)p[u][t0 + 1][r]; }
    const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);   // bf16 1.0 x 8
#pragma unroll
    for (int u = 0; u < QT; ++u)
        o[u][kHd / 16] =
            __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), pb[u], o[u][kHd / 16], 0, 0, 0);
#pragma unroll
    for (int dt = 0; dt < kHd / 16; ++dt) {
        const bf16x8 va = __builtin_bit_cast(bf16x8, ld16(vt + vt_row(dt * 16 + fr) * VR + 2 * (kbase + 8 * fg)));
#pragma unroll
        for (int u = 0; u < QT; ++u) o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[u], o[u][dt], 0, 0, 0);
    }
}
template <int QT, int VR>
__device__ __forceinline__ void lpv_step(float, const char* vt, int kbase, int fr, int fg,
                                         const f32x4 (*p)[kLKB / 16], int t0, f32x4 (*o)[kHd / 16 + 1]) {
#pragma unroll
    for (int dt = 0; dt < kHd / 16; ++dt) {
        const float4 va = *reinterpret_cast<const float4*>(vt + vt_row(dt * 16 + fr) * VR + 4 * (kbase + 4 * fg));
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.x, p[u][t0][0], o[u][dt], 0, 0, 0);
            o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.y, p[u][t0][1], o[u][dt], 0, 0, 0);
            o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.z, p[u][t0][2], o[u][dt], 0, 0, 0);
            o[u][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(va.w, p[u][t0][3], o[u][dt], 0, 0, 0);
        }
    }
}

template <typename T, int QT, int QB>
__global__ __launch_bounds__(QB / QT * 4) __attribute__((amdgpu_waves_per_eu(2))) void attention_long_kernel(
    const T* __restrict__ qkv, const int* __restrict__ cu, int n_heads, int d, int qgroups, T* __restrict__ out) {
    constexpr bool kB = sizeof(T) == 2;
    constexpr int KR = LAttnLds<T>::krow, VR = LAttnLds<T>::vrow;
    constexpr int PER = Elem<T>::per16;
    constexpr int CPR = kHd / PER;                   // 16-byte chunks per head row
    constexpr int KBN = kHd * (int)sizeof(T) / 64;   // 64-byte MFMA K blocks per head row
    constexpr int NW = QB / 16 / QT, NT = 64 * NW;
    constexpr int NCH = kLKB * CPR / NT;             // chunks per thread per key block
    static_assert(QB % (16 * QT) == 0 && (kLKB * CPR) % NT == 0 && (!kB || NCH % 2 == 0), "tiling");
    __shared__ __align__(16) char ks[kLKB * KR];
    __shared__ __align__(16) char vts[kHd * VR];

    const int qg = blockIdx.x % qgroups;
    const int sh = blockIdx.x / qgroups;
    const int seg = sh / n_heads, h = sh % n_heads;
    const int s0 = cu[seg], n = cu[seg + 1] - s0;
    if (qg * QB >= n) return;                        // whole workgroup idle (uniform)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
    const int fr = lane & 15, fg = lane >> 4;
    const size_t ld = 3 * (size_t)d;
    const T* kbase_p = qkv + (size_t)s0 * ld + d + h * kHd;
    const T* vbase_p = kbase_p + d;
    const int qt0 = qg * (QB / 16) + wave * QT;      // this wave's first query tile
    const bool active = qt0 * 16 < n;                // wave-uniform
    uint4 qf[QT][KBN];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        const int q = qt0 * 16 + u * 16 + fr;
        const T* row = qkv + (size_t)(s0 + q) * ld + h * kHd + fg * PER;
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) qf[u][kb] = q < n ? ld16(row + kb * (64 / (int)sizeof(T))) : zero16();
    }
    const float sc = 0.125f * 1.4426950408889634f;   // 1/sqrt(64) * log2(e)
    float m[QT], l[QT];
    f32x4 o[QT][kHd / 16 + 1];
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        m[u] = -INFINITY;
        l[u] = 0.f;
#pragma unroll
        for (int dt = 0; dt <= kHd / 16; ++dt) o[u][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // chunk c of this thread: key row key_of(c), 16-byte column tid % CPR;
    // bf16 keys come in adjacent pairs (2 p, 2 p + 1)
    auto key_of = [&](int c) {
        if constexpr (kB) return 2 * (tid / CPR + (c / 2) * (NT / CPR)) + (c & 1);
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
                const size_t off = (size_t)(k0 + t) * ld + ch * PER;
                kv[c] = ld16(kbase_p + off);
                vv[c] = ld16(vbase_p + off);
            }
        }
    };
    auto process = [&](int k0, Regs& kv, Regs& vv) {
        __syncthreads();                             // previous block consumed
        {
            const int ch = tid % CPR;
#pragma unroll
            for (int c = 0; c < NCH; ++c) st16(ks + (kB ? lkey_row(key_of(c)) : key_of(c)) * KR + ch * 16, kv[c]);
            if constexpr (kB) {
#pragma unroll
                for (int c = 0; c < NCH; c += 2) {
                    const int t = key_of(c);         // even; t + 1 is chunk c + 1's key
                    const unsigned* va = reinterpret_cast<const unsigned*>(&vv[c]);
                    const unsigned* vb = reinterpret_cast<const unsigned*>(&vv[c + 1]);
#pragma unroll
                    for (int w = 0; w < 4; ++w) {    // dims 2 w, 2 w + 1 of the chunk
                        *reinterpret_cast<unsigned*>(vts + vt_row(ch * PER + 2 * w) * VR + t * 2) =
                            __builtin_amdgcn_perm(vb[w], va[w], 0x05040100u);
                        *reinterpret_cast<unsigned*>(vts + vt_row(ch * PER + 2 * w + 1) * VR + t * 2) =
                            __builtin_amdgcn_perm(vb[w], va[w], 0x07060302u);
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
        if (k0 + 2 * kLKB < n) load_block(k0 + 2 * kLKB, kv, vv);
        if (!active) return;
        f32x4 sacc[QT][kLKB / 16];
#pragma unroll
        for (int u = 0; u < QT; ++u)
#pragma unroll
            for (int kt = 0; kt < kLKB / 16; ++kt) sacc[u][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KBN; ++kb) {
#pragma unroll
            for (int kt = 0; kt < kLKB / 16; ++kt) {
                const uint4 kf = ld16(ks + (kt * 16 + fr) * KR + fg * 16 + kb * 64);
#pragma unroll
                for (int u = 0; u < QT; ++u) mfma_kblock(T(), kf, qf[u][kb], sacc[u][kt]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // lane holds S^T[LDS row 16 kt + 4 fg + r][query] (unscaled); the row is
        // key k0 + lrow_key(row) in bf16, key k0 + row in fp32
        const bool full = k0 + kLKB <= n;
#pragma unroll
        for (int u = 0; u < QT; ++u) {
            float bm = -INFINITY;
            if (full) {
#pragma unroll
                for (int kt = 0; kt < kLKB / 16; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) bm = fmaxf(bm, sacc[u][kt][r]);
            } else {
#pragma unroll
                for (int kt = 0; kt < kLKB / 16; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rho = kt * 16 + 4 * fg + r;
                        const float v = k0 + (kB ? lrow_key(rho) : rho) < n ? sacc[u][kt][r] : -INFINITY;
                        sacc[u][kt][r] = v;
                        bm = fmaxf(bm, v);
                    }
            }
            bm = fmaxf(bm, __shfl_xor(bm, 16));
            bm = fmaxf(bm, __shfl_xor(bm, 32));
            const float bms = bm * sc;
            if (__builtin_amdgcn_ballot_w64(bms > m[u] + kLazy) != 0) {
                const float mn = fmaxf(m[u], bms);
                const float alpha = m[u] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[u] - mn);
#pragma unroll
                for (int dt = 0; dt <= kHd / 16; ++dt) o[u][dt] = o[u][dt] * alpha;
                l[u] *= alpha;
                m[u] = mn;
            }
            const float mref = m[u] == -INFINITY ? 0.f : m[u];
            float bs = 0.f;
#pragma unroll
            for (int kt = 0; kt < kLKB / 16; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float p = __builtin_amdgcn_exp2f(fmaf(sacc[u][kt][r], sc, -mref));
                    sacc[u][kt][r] = p;
                    if constexpr (!kB) bs += p;
                }
            if constexpr (!kB) {
                bs += __shfl_xor(bs, 16);
                bs += __shfl_xor(bs, 32);
                l[u] += bs;
            }
        }
        if constexpr (kB) {
#pragma unroll
            for (int st = 0; st < kLKB / 32; ++st) {
                lpv_step<QT, VR>(T(), vts, 32 * st, fr, fg, sacc, 2 * st, o);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int kt = 0; kt < kLKB / 16; ++kt) {
                lpv_step<QT, VR>(T(), vts, 16 * kt, fr, fg, sacc, kt, o);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };
    load_block(0, kvA, vvA);
    if (kLKB < n) load_block(kLKB, kvB, vvB);
    for (int k0 = 0; k0 < n; k0 += 2 * kLKB) {
        process(k0, kvA, vvA);
        if (k0 + kLKB < n) process(k0 + kLKB, kvB, vvB);
    }
#pragma unroll
    for (int u = 0; u < QT; ++u) {
        const int q = qt0 * 16 + u * 16 + fr;
        if (active && q < n) {
            const float inv = 1.0f / (kB ? o[u][kHd / 16][0] : l[u]);
            T* orow = out + (size_t)(s0 + q) * d + h * kHd;
#pragma unroll
            for (int dt = 0; dt < kHd / 16; ++dt)
                store4(orow + dt * 16 + 4 * fg, o[u][dt][0] * inv, o[u][dt][1] * inv, o[u][dt][2] * inv,
                       o[u][dt][3] * inv);
        }
    }
}

template <typename T>
hipError_t attention(hipStream_t s, const T* qkv, const int* cu_seqlens, int n_windows, int n_heads,
                     int d, int max_len, T* out) {
    if (n_windows <= 0) return hipSuccess;
    if (std::is_same<T, bf16>::value && n_heads % kAttnHpw == 0 && max_len <= kMaxWindow) {
        // bf16, an even number of heads: direct-to-LDS kernel, two heads per workgroup
        const unsigned blocks = (unsigned)(n_windows * (n_heads / kAttnHpw));
        const bf16* q = reinterpret_cast<const bf16*>(qkv);
        bf16* o = reinterpret_cast<bf16*>(out);
        if (max_len <= 112) attention_dma_kernel<7><<<blocks, 256 * kAttnHpw, 0, s>>>(q, cu_seqlens, n_heads, d, o);
        else attention_dma_kernel<kMaxWindow / 16><<<blocks, 256 * kAttnHpw, 0, s>>>(q, cu_seqlens, n_heads, d, o);
    } else if (max_len <= 112) {          // every window fits 7 key tiles (104-token windows)
        attention_kernel<T, 7><<<n_windows * n_heads, 256, 0, s>>>(qkv, cu_seqlens, n_heads, d, out);
    } else if (max_len <= kMaxWindow) {
        attention_kernel<T, kMaxWindow / 16><<<n_windows * n_heads, 256, 0, s>>>(qkv, cu_seqlens, n_heads, d, out);
    } else {
        // bf16: 128 queries per workgroup, two 16-query tiles per wave; fp32: 64, one
        constexpr int QT = sizeof(T) == 2 ? 2 : 1, QB = sizeof(T) == 2 ? 128 : 64;
        const int qgroups = (max_len + QB - 1) / QB;
        const int64_t blocks = (int64_t)n_windows * n_heads * qgroups;
        if (blocks > 0x7fffffff) return hipErrorInvalidValue;
        attention_long_kernel<T, QT, QB><<<(unsigned)blocks, QB / QT * 4, 0, s>>>(qkv, cu_seqlens, n_heads, d,
                                                                                  qgroups, out);
    }
    return hipGetLastError();
}

template hipError_t layernorm<float>(hipStream_t, const float*, int, int, const float*, const float*, float*);
template hipError_t layernorm<bf16>(hipStream_t, const float*, int, int, const float*, const float*, bf16*);
template hipError_t attention<float>(hipStream_t, const float*, const int*, int, int, int, int, float*);
template hipError_t attention<bf16>(hipStream_t, const bf16*, const int*, int, int, int, int, bf16*);

}  // namespace qa
