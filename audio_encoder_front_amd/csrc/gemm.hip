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
// tile in stages of 128 bytes of K (64 bf16 or 32 fp32 elements).
//
// Staging: every 16-byte chunk moves global -> LDS with one direct-to-LDS
// load, no register round trip.  Such a load writes 64 lanes x 16 B
// contiguously, i.e. 8 LDS rows of 128 B; lane l therefore fetches K-chunk
// (l%8) ^ (row%8) of its row, an XOR swizzle that makes the 16-byte fragment
// reads of 8 consecutive rows hit 8 different 16-byte bank groups.  Chunks
// outside the matrix (ragged M/N/K, conv padding) read as zeros.  While
// stage k is multiplied, stage k+1 of one operand and stage k+2 of the other
// are in flight: a ring of three stages for the operand that runs two ahead
// and two for the other.  The conv and gather loaders run A two ahead (their
// input streams from HBM); the dense loader runs the weights two ahead.  With
// dense activations every concurrent tile of an XCD asks for the same weight
// slice at the same moment, so one L2 miss stalls up to eight workgroups.
//
// The MFMA is issued transposed (weights as the A operand): lane l then holds
// 4 consecutive output columns of one output row.  After the K loop the tile
// is staged row-major through LDS and written as whole rows (see the
// epilogues).  Workgroups are remapped so that each of the 8 XCDs works
// through a contiguous, M-grouped range of tiles (L2 reuse of both operand
// tiles).
#include "qa_device.h"
#include "qa_kernels.h"

namespace qa {

__device__ __align__(16) uint4 g_zero16[2];

// ------------------------------------------------------------ A loaders
// A loader keeps a compact per-lane state for the AI rows the lane fetches
// (rows r, r + RS, ..., r + RS (AI-1) of the tile); kprep(k0) is evaluated
// once per stage.  Buffer loaders (kBuffer) give rsrc(tile0), the workgroup's
// resource, and boff(lane, q, kx), the byte offset of elements [k0, k0 + per16)
// of row q or kOobOffset outside the matrix; the gather loader gives
// addr(lane, q, kx), a global address or g_zero16.

template <typename T>
struct DenseA {
    static constexpr bool kBuffer = true;
    static constexpr bool kWeightsAhead = true;     // weights two stages ahead, A one
    const T* a;
    int M, K, lda;
    template <int AI, int RS>
    struct Lane { unsigned off; };             // byte offset of the lane's first row from row tile0
    struct KCtx { unsigned off; bool ok; };
    __device__ i32x4 rsrc(int tile0) const {
        return buffer_rsrc(a + (size_t)tile0 * lda, (uint64_t)(M > tile0 ? M - tile0 : 0) * lda * sizeof(T));
    }
    template <int AI, int RS>
    __device__ Lane<AI, RS> init(int tile0, int m) const {
        return Lane<AI, RS>{(unsigned)((m - tile0) * lda * (int)sizeof(T))};
    }
    __device__ KCtx kprep(int k0) const { return KCtx{(unsigned)(k0 * (int)sizeof(T)), k0 < K}; }
    template <int AI, int RS>
    __device__ unsigned boff(const Lane<AI, RS>& l, int q, const KCtx& k) const {
        return k.ok ? l.off + (unsigned)(q * RS * lda * (int)sizeof(T)) + k.off : kOobOffset;
    }
};

template <typename T>
struct GatherA {   // row m of the GEMM is row src[m] of a
    static constexpr bool kBuffer = false;
    static constexpr bool kWeightsAhead = false;
    const T* a;
    const int* src;
    int M, K;
    template <int AI, int RS>
    struct Lane { int row[AI]; };
    struct KCtx { int off; bool ok; };
    template <int AI, int RS>
    __device__ Lane<AI, RS> init(int, int m) const {
        Lane<AI, RS> l;
#pragma unroll
        for (int q = 0; q < AI; ++q) l.row[q] = m + RS * q < M ? src[m + RS * q] : -1;
        return l;
    }
    __device__ KCtx kprep(int k0) const { return KCtx{k0 * (int)sizeof(T), k0 < K}; }
    template <int AI, int RS>
    __device__ const void* addr(const Lane<AI, RS>& l, int q, const KCtx& k) const {
        return (l.row[q] >= 0 && k.ok)
                   ? (const void*)(reinterpret_cast<const char*>(a + (size_t)l.row[q] * K) + k.off)
                   : (const void*)g_zero16;
    }
};

template <typename T>
struct ConvA {     // implicit im2col of a 3x3 stride-2 pad-1 conv
    static constexpr bool kBuffer = true;
    static constexpr bool kWeightsAhead = false;
    const T* in;
    int M, Hin, Win, C, Hout, Wout;
    bool time_major;                  // output row order (chunk, j, i) instead of (chunk, i, j)
    // input layout per chunk: NHWC [Hin][Win][C]
    // A tile of up to 256 output rows touches at most 3 chunks, so offsets from
    // the tile's first chunk stay far below 4 GB.
    template <int AI, int RS>
    struct Lane { int cofs[AI]; int rc[AI]; };    // chunk offset (elements) from the tile's first chunk, or -1;
                                                  // rc = (2i-1) << 16 | (2j-1) & 0xffff
    struct KCtx { int a, b; unsigned off; bool ok; };
    __device__ int chunk_elems() const { return Hin * Win * C; }
    __device__ i32x4 rsrc(int tile0) const {
        const int per = Hout * Wout, c0 = tile0 / per, nch = M / per;
        return buffer_rsrc(in + (size_t)c0 * chunk_elems(), (uint64_t)(nch - c0) * chunk_elems() * sizeof(T));
    }
    template <int AI, int RS>
    __device__ Lane<AI, RS> init(int tile0, int m0) const {
        Lane<AI, RS> l;
        const int per = Hout * Wout, c0 = tile0 / per;
#pragma unroll
        for (int q = 0; q < AI; ++q) {
            const int m = m0 + RS * q;
            const int chunk = m / per, rem = m - chunk * per;
            int i, j;
            if (time_major) { j = rem / Hout; i = rem - j * Hout; }
            else            { i = rem / Wout; j = rem - i * Wout; }
            l.cofs[q] = m < M ? (chunk - c0) * chunk_elems() : -1;
            l.rc[q] = ((2 * i - 1) << 16) | ((2 * j - 1) & 0xffff);
        }
        return l;
    }
    // K order (channel block of 32, tap, channel in block): the 9 taps of a
    // 32-channel slab are consecutive K stages, so the input slab a tile
    // gathers is reused from L2 before the next slab is fetched.
    __device__ KCtx kprep(int k0) const {
        const int cb = k0 / (9 * kConvCB), rem = k0 - cb * (9 * kConvCB);
        const int tap = rem / kConvCB, ci = cb * kConvCB + (rem - tap * kConvCB);
        const int a = tap / 3;
        return KCtx{a, tap - 3 * a, (unsigned)(ci * (int)sizeof(T)), k0 < 9 * C};
    }
    template <int AI, int RS>
    __device__ unsigned boff(const Lane<AI, RS>& l, int q, const KCtx& k) const {
        const int r = (l.rc[q] >> 16) + k.a;
        const int col = (int)(short)(l.rc[q] & 0xffff) + k.b;
        if (l.cofs[q] < 0 || !k.ok || (unsigned)r >= (unsigned)Hin || (unsigned)col >= (unsigned)Win)
            return kOobOffset;
        return (unsigned)((l.cofs[q] + (r * Win + col) * C) * (int)sizeof(T)) + k.off;
    }
};

// ------------------------------------------------------------ epilogues
// op(m, n, v): v holds out[m][n..n+3] before bias; n is a multiple of 4.

// Epilogues.  Every epilogue but EpiPE is "staged": after the K loop the
// workgroup converts its accumulators (frag / pair), writes them row-major
// into the idle LDS stages and then streams whole rows out with 16-byte
// stores (row), so a wave writes 1 KB of contiguous rows per instruction
// instead of 16 scattered 32-byte pieces.  S is the staged element type,
// kDiv the ratio of accumulator columns to staged columns.  Bias terms are
// folded into the accumulators' initial value (init) where the staged value
// already includes them.

// 4 consecutive fp32 values of v[n..n+3]; entries at or past N read as 0.
__device__ __forceinline__ f32x4 load4_tail(const float* v, int n, int N) {
    if (n + 4 <= N) {
        const float4 b = *reinterpret_cast<const float4*>(v + n);
        return f32x4{b.x, b.y, b.z, b.w};
    }
    f32x4 r = {0.f, 0.f, 0.f, 0.f};
    for (int e = 0; e < 4 && n + e < N; ++e) r[e] = v[n + e];
    return r;
}

// Store the 16-byte staged chunk c (elements of type S) at p; only the first
// `valid` elements when the chunk runs past the end of the row.
template <typename S>
__device__ __forceinline__ void store_chunk(S* p, uint4 c, int valid) {
    constexpr int E = Elem<S>::per16;
    if (valid >= E) { st16(p, c); return; }
    const S* e = reinterpret_cast<const S*>(&c);
#pragma unroll
    for (int i = 0; i < E; ++i)                  // constant indices: c stays in registers
        if (i < valid) p[i] = e[i];
}

template <typename T, bool kGelu>
struct EpiBias {           // out = acc + bias (GELU if kGelu), stored as T
    using S = T;
    static constexpr bool kStaged = true;
    static constexpr int kDiv = 1;
    T* out;
    const float* bias;
    int M, N;
    __device__ f32x4 init(int n) const { return n < N ? load4_tail(bias, n, N) : f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ void frag(f32x4 v, float* o) const {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = kGelu ? gelu_for<T>(v[r]) : v[r];
    }
    __device__ uint4 pre(int, int) const { return zero16(); }
    __device__ void row(int m, int n, uint4 c, uint4) const {
        if (m < M && n < N) store_chunk(out + (size_t)m * N + n, c, N - n);
    }
};

struct EpiResid {          // x = x + bias + acc (fp32 residual stream)
    using S = float;
    static constexpr bool kStaged = true;
    static constexpr int kDiv = 1;
    float* x;
    const float* bias;
    int M, N;
    __device__ f32x4 init(int) const { return f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ void frag(f32x4 v, float* o) const {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = v[r];
    }
    // The residual is read in whole rows per wave by pre(), issued for a
    // band before its values are staged so the loads overlap the staging.
    __device__ uint4 pre(int m, int n) const {
        if (m >= M || n >= N) return zero16();
        return __builtin_bit_cast(uint4, load4_tail(x + (size_t)m * N, n, N));
    }
    __device__ void row(int m, int n, uint4 c, uint4 pv) const {
        if (m >= M || n >= N) return;
        float* p = x + (size_t)m * N + n;
        const f32x4 a = __builtin_bit_cast(f32x4, c), r = __builtin_bit_cast(f32x4, pv);
        const f32x4 b = load4_tail(bias, n, N);
        if (n + 4 <= N) {
            *reinterpret_cast<float4*>(p) = make_float4(r[0] + (b[0] + a[0]), r[1] + (b[1] + a[1]), r[2] + (b[2] + a[2]),
                                                        r[3] + (b[3] + a[3]));
        } else {
            for (int e = 0; n + e < N; ++e) p[e] = r[e] + (b[e] + a[e]);
        }
    }
};

struct EpiF32Bias {        // out = acc + bias, fp32
    using S = float;
    static constexpr bool kStaged = true;
    static constexpr int kDiv = 1;
    float* out;
    const float* bias;
    int M, N;
    __device__ f32x4 init(int n) const { return n < N ? load4_tail(bias, n, N) : f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ void frag(f32x4 v, float* o) const {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = v[r];
    }
    __device__ uint4 pre(int, int) const { return zero16(); }
    __device__ void row(int m, int n, uint4 c, uint4) const {
        if (m < M && n < N) store_chunk(out + (size_t)m * N + n, c, N - n);
    }
};

// One K split of a split-K GEMM: the fp32 partial sum of the split's K range,
// part[blockIdx.y][m][n] = acc (no bias; resid_reduce adds the splits).
struct EpiPartial {
    using S = float;
    static constexpr bool kStaged = true;
    static constexpr int kDiv = 1;
    float* part;
    int M, N;
    __device__ f32x4 init(int) const { return f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ void frag(f32x4 v, float* o) const {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = v[r];
    }
    __device__ uint4 pre(int, int) const { return zero16(); }
    __device__ void row(int m, int n, uint4 c, uint4) const {
        if (m < M && n < N) store_chunk(part + ((size_t)blockIdx.y * M + m) * N + n, c, N - n);
    }
};

// SwiGLU of the Thinker FFN (qwenasr.cpp ARCHITECTURE.md, "Qwen3 Thinker
// decoder": silu(gate) * up).  The gate and up weights are interleaved in
// blocks of 16 rows (gate rows f..f+15, then up rows f..f+15, ...), so MFMA
// column tiles 2k and 2k + 1 hold gate and up of the same 16 features and the
// epilogue sees both in one lane: out[m][f] = silu(g) * u, f = 16 (n / 32) + n % 16.
template <typename T>
struct EpiSwiGLU {
    using S = T;
    static constexpr bool kStaged = true;
    static constexpr bool kPaired = true;
    static constexpr int kDiv = 2;
    T* out;
    int M, F;
    __device__ f32x4 init(int) const { return f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ void pair(f32x4 g, f32x4 u, float* o) const {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] = g[r] / (1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g[r])) * u[r];
    }
    __device__ uint4 pre(int, int) const { return zero16(); }
    __device__ void row(int m, int f, uint4 c, uint4) const {
        if (m < M && f < F) store_chunk(out + (size_t)m * F + f, c, F - f);
    }
};

template <class EP, class = void>
struct EpiIsPaired { static constexpr bool value = false; };
template <class EP>
struct EpiIsPaired<EP, decltype((void)EP::kPaired)> { static constexpr bool value = EP::kPaired; };

struct EpiPE {             // x = acc + pe[src[m] % 13]; tap = acc (stored from the lanes)
    static constexpr bool kStaged = false;
    float* x;
    float* tap;
    const float* pe;
    const int* src;
    int M, N;
    __device__ f32x4 init(int) const { return f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ void operator()(int m, int n, f32x4 v) const {
        if (m >= M || n >= N) return;
        const int j = src[m] % kChunkTok;
        const float4 p = *reinterpret_cast<const float4*>(pe + (size_t)j * N + n);
        store4(x + (size_t)m * N + n, v[0] + p.x, v[1] + p.y, v[2] + p.z, v[3] + p.w);
        if (tap) store4(tap + (size_t)m * N + n, v[0], v[1], v[2], v[3]);
    }
};

// ------------------------------------------------------------ kernel

// Launch-site tags: one kernel symbol per call site, so profilers attribute
// time per site.  The tag changes nothing in the generated code.
enum Site { kQKV = 1, kFC1, kProj1, kOProj, kFC2, kProj2, kConv2, kConv3, kConvOut,
            kTQKV, kTOProj, kTGateUp, kTDown, kTLogits };

// Swizzled 16-byte column of K-chunk c in LDS row r: rows of 128 B hold 8
// chunks (XOR with r % 8), rows of 64 B hold 4 (XOR with (r / 2) % 4); either
// way the fragment reads of 8 consecutive rows cover all 32 banks.
template <int BKB>
__device__ __forceinline__ int swz(int r, int c) {
    return BKB == 128 ? (c ^ (r & 7)) : (c ^ ((r >> 1) & 3));
}

template <typename T, int BM, int BN, int WM, int WN, int BKB, int SITE, class AL, class EP>
__global__ __launch_bounds__(WM * WN * 64) void gemm_kernel(AL al, const T* __restrict__ w, int N, int K,
                                                            int tiles_m, int tiles_n, EP ep) {
    constexpr int NW = WM * WN;               // waves
    constexpr int TM = BM / WM / 16;          // 16-row MFMA tiles per wave along M
    constexpr int TN = BN / WN / 16;          // along N
    constexpr int PER = Elem<T>::per16;       // elements per 16-byte chunk
    constexpr int CPR = BKB / 16;             // 16-byte chunks per LDS row (per stage)
    constexpr int RPD = 64 / CPR;             // rows filled by one direct-to-LDS load (1 KB)
    constexpr int KB = BKB / 64;              // 64-byte MFMA K blocks per stage
    constexpr int AI = BM / (RPD * NW);       // direct-to-LDS loads per wave per stage (A)
    constexpr int BI = BN / (RPD * NW);
    constexpr int ASTAGE = BM * BKB;          // bytes per LDS stage of A
    constexpr int BSTAGE = BN * BKB;          // of the weights
    constexpr int STAGE = ASTAGE + BSTAGE;
    static_assert(BM % (RPD * NW) == 0 && BN % (RPD * NW) == 0, "tile/waves mismatch");
    static_assert(TN >= 3, "the two-ahead weight prefetch needs at least 3 weight tiles");
    // The operand that runs two stages ahead has a ring of three LDS stages,
    // the other two: 160 KB for the 256 x 256 tile.  Rings: A at the start of
    // the LDS, the weights after it.
    constexpr bool WA = AL::kWeightsAhead;
    constexpr int ARING = WA ? 2 : 3, BRING = WA ? 3 : 2;
    __shared__ __align__(1024) char smem[ARING * ASTAGE + BRING * BSTAGE];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave % WM, wn = wave / WM;

    // XCD-aware tile order: dispatch sends workgroup b to XCD b % 8; give each
    // XCD a contiguous range of logical tiles, walked in groups of 8 M-tiles.
    const int G = tiles_m * tiles_n;
    const int b = blockIdx.x;
    const int per_xcd = (G + 7) / 8;
    const int xcd = b % 8, slot = b / 8;
    const int full = G - 8 * (per_xcd - 1);   // XCDs that get per_xcd tiles (the rest get one less)
    int t = xcd < full ? xcd * per_xcd + slot : full * per_xcd + (xcd - full) * (per_xcd - 1) + slot;
    const int GM = 8;
    const int group = t / (GM * tiles_n);
    const int first_m = group * GM;
    const int gm = min(GM, tiles_m - first_m);
    const int in_group = t - group * GM * tiles_n;
    const int bm = first_m + in_group % gm, bn = in_group / gm;
    const int m0 = bm * BM, n0 = bn * BN;

    // This lane's rows and K-chunk for the direct-to-LDS loads: a load fills
    // 1 KB = RPD rows of BKB bytes, lane l landing in row l / CPR, column
    // l % CPR, so it fetches the chunk that the swizzle puts there.
    const int lrow = lane / CPR;
    const int kc = swz<BKB>(lrow, lane % CPR);
    const auto alane = al.template init<AI, RPD>(m0, m0 + wave * AI * RPD + lrow);
    const DenseA<T> wl{w, N, K, K};
    const auto wlane = wl.template init<BI, RPD>(n0, n0 + wave * BI * RPD + lrow);
    i32x4 ra = {0, 0, 0, 0};
    if constexpr (AL::kBuffer) ra = al.rsrc(m0);
    const i32x4 rw = wl.rsrc(n0);
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_void*)smem;
    const unsigned wave_u = (unsigned)__builtin_amdgcn_readfirstlane(wave);
    constexpr int KSTEP = BKB / (int)sizeof(T);   // K elements per stage
    auto issue_a = [&](int kt, int buf) {
        const auto kx = al.kprep(kt * KSTEP + kc * PER);
        const unsigned sa = lds0 + buf * ASTAGE + wave_u * (AI * 1024);
#pragma unroll
        for (int q = 0; q < AI; ++q) {
            if constexpr (AL::kBuffer) dma16_buf(ra, al.boff(alane, q, kx), sa + q * 1024);
            else dma16(al.addr(alane, q, kx), sa + q * 1024);
        }
    };
    auto issue_b = [&](int kt, int buf) {
        const auto kw = wl.kprep(kt * KSTEP + kc * PER);
        const unsigned sb = lds0 + ARING * ASTAGE + buf * BSTAGE + wave_u * (BI * 1024);
#pragma unroll
        for (int q = 0; q < BI; ++q) dma16_buf(rw, wl.boff(wlane, q, kw), sb + q * 1024);
    };

    // K range of this workgroup: all of K, or split blockIdx.y of gridDim.y
    // (split-K; its partial sums go to EpiPartial)
    const int nk_all = (K + KSTEP - 1) / KSTEP;
    const int kper = (nk_all + (int)gridDim.y - 1) / (int)gridDim.y;
    const int kt0 = (int)blockIdx.y * kper;
    const int nk = max(0, min(nk_all, kt0 + kper) - kt0);
    if constexpr (WA) {
        issue_b(kt0, 0);
        issue_a(kt0, 0);
        issue_b(kt0 + 1, 1);
    } else {
        issue_a(kt0, 0);
        issue_b(kt0, 0);
        issue_a(kt0 + 1, 1);
    }
    const int fr = lane & 15, fg = lane >> 4;
    f32x4 acc[TM][TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const f32x4 a0 = ep.init(n0 + (wn * TN + j) * 16 + 4 * fg);   // per output column
#pragma unroll
        for (int i = 0; i < TM; ++i) acc[i][j] = a0;
    }

    // vmcnt(0) through the builtin, not inline asm: the compiler then knows
    // that the accumulator initial values loaded above have landed, and does
    // not wait for vector memory (i.e. for the next stage's loads) at the top
    // of every K-loop iteration.
    __builtin_amdgcn_s_waitcnt(0x0F70);           // vmcnt(0), expcnt and lgkmcnt untouched
    __syncthreads();
    int sw[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sw[kb] = swz<BKB>(fr, kb * 4 + fg) * 16;
    constexpr int MPK = sizeof(T) == 2 ? 1 : 4;   // MFMAs per 64-byte K block
    for (int i = 0; i < nk; ++i) {
        // Loads of the next stage (past the last stage of K they fetch zeros
        // into the idle buffer, past the last of a split they fetch the next
        // split's first stage unused), kept in this basic block so that the
        // scheduling below can spread them between the MFMA groups.
        // The two-ahead loads are issued after the one-ahead ones so that the
        // wait at the end of the iteration can leave them in flight:
        // vector-memory loads complete in issue order.
        const int kt = kt0 + i;
        const int r3 = i % 3, r3n = r3 == 0 ? 2 : r3 - 1;   // slots i and i + 2 of a three-stage ring
        const int abuf = WA ? (i & 1) : r3, bbuf = WA ? r3 : (i & 1);
        if constexpr (WA) {
            issue_a(kt + 1, (i + 1) & 1);
            issue_b(kt + 2, r3n);
        } else {
            issue_b(kt + 1, (i + 1) & 1);
            issue_a(kt + 2, r3n);
        }
        const char* a = smem + abuf * ASTAGE + (wm * TM * 16 + fr) * BKB;
        const char* bp = smem + ARING * ASTAGE + bbuf * BSTAGE + (wn * TN * 16 + fr) * BKB;
        // Fragments: the TM activation fragments of a 64-byte K block stay in
        // registers while the TN weight fragments stream through a two-ahead
        // prefetch; the next K block's activation fragments are fetched during
        // the current block's third-from-last weight tile.  The
        // sched_group_barriers pin this order, so each LDS read has two MFMA
        // groups (2 TM MFMAs) to land.
        uint4 fa[KB][TM], fb[KB][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) fa[0][i] = ld16(a + i * 16 * BKB + sw[0]);
        fb[0][0] = ld16(bp + sw[0]);
        fb[0][1] = ld16(bp + 16 * BKB + sw[0]);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if (j + 2 < TN) {
                    fb[kb][j + 2] = ld16(bp + (j + 2) * 16 * BKB + sw[kb]);
                } else if (kb + 1 < KB) {
                    if (j + 2 == TN) {
#pragma unroll
                        for (int i = 0; i < TM; ++i) fa[kb + 1][i] = ld16(a + i * 16 * BKB + sw[kb + 1]);
                        fb[kb + 1][0] = ld16(bp + sw[kb + 1]);
                    } else {
                        fb[kb + 1][1] = ld16(bp + 16 * BKB + sw[kb + 1]);
                    }
                }
#pragma unroll
                for (int i = 0; i < TM; ++i) mfma_kblock(T(), fb[kb][j], fa[kb][i], acc[i][j]);
            }
        }
        // One MFMA group per weight tile; the next stage's direct-to-LDS loads
        // are dealt out over the groups so they never issue as a burst.
        constexpr int VPG = (AI + BI + KB * TN - 1) / (KB * TN);
        __builtin_amdgcn_sched_group_barrier(0x100, TM + 2, 0);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                if (j + 2 < TN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                else if (kb + 1 < KB && j + 2 == TN) __builtin_amdgcn_sched_group_barrier(0x100, TM + 1, 0);
                else if (kb + 1 < KB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x020, VPG, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, TM * MPK, 0);
            }
        }
        // everything but this iteration's two-ahead loads: stage i + 1 has landed
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(WA ? BI : AI) : "memory");
        __syncthreads();
    }
    // the last two-ahead loads (zeros or an unused stage) land before the epilogue
    // reuses the LDS
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // acc[i][j] lane holds out[m = row fr][n = 4 fg + r] of tile (i, j)
    if constexpr (EP::kStaged) {
        // Staged epilogue: the lanes write their converted values row-major
        // into the two (now idle) LDS stages, rows of RB bytes whose 16-byte
        // chunks are XOR-swizzled by row (conflict-free writes from 16 rows
        // at once and conflict-free row reads); then every thread stores
        // whole 16-byte chunks of consecutive rows.  A tile whose staged rows
        // exceed the LDS goes out in PASSES bands of wave rows.
        using S = typename EP::S;
        constexpr bool kPair = EpiIsPaired<EP>::value;
        constexpr int SB = (int)sizeof(S);
        constexpr int RB = BN / EP::kDiv * SB;     // bytes per staged row
        constexpr int CPO = RB / 16;               // 16-byte chunks per staged row
        constexpr int XM = CPO < 16 ? CPO : 16;    // swizzle period
        constexpr int PASSES = (BM * RB + 2 * STAGE - 1) / (2 * STAGE);
        constexpr int WPP = WM / PASSES;           // wave rows per pass
        constexpr int RPP = BM / PASSES;           // tile rows per pass
        constexpr int NT = NW * 64;
        static_assert(WM % PASSES == 0 && RB % 16 == 0 && (RPP * CPO) % NT == 0, "staging layout");
        static_assert(!kPair || TN % 2 == 0, "paired epilogue needs an even number of column tiles per wave");
        auto lds_at = [&](int r, int byte) {
            return smem + r * RB + ((((byte >> 4) ^ (r & (XM - 1))) << 4) | (byte & 15));
        };
        constexpr int Q = RPP * CPO / NT;          // row-phase chunks per thread per band
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            uint4 pv[Q];                           // per-chunk operands of the row phase (the residual)
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int idx = q * NT + tid;
                pv[q] = ep.pre(m0 + p * RPP + idx / CPO, n0 / EP::kDiv + (idx % CPO) * (16 / SB));
            }
            if (p) __syncthreads();                // the previous band has been read
            if (wm / WPP == p) {
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; j += kPair ? 2 : 1) {
                        const int r = (wm % WPP) * TM * 16 + i * 16 + fr;
                        const int c = (kPair ? (wn * TN + j) / 2 : wn * TN + j) * 16 + 4 * fg;
                        float v[4];
                        if constexpr (kPair) ep.pair(acc[i][j], acc[i][j + 1], v);
                        else ep.frag(acc[i][j], v);
                        store4(reinterpret_cast<S*>(lds_at(r, c * SB)), v[0], v[1], v[2], v[3]);
                    }
            }
            __syncthreads();
#pragma unroll
            for (int q = 0; q < Q; ++q) {
                const int idx = q * NT + tid, r = idx / CPO, c = idx % CPO;
                ep.row(m0 + p * RPP + r, n0 / EP::kDiv + c * (16 / SB), ld16(lds_at(r, c * 16)), pv[q]);
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
                ep(m0 + (wm * TM + i) * 16 + fr, n0 + (wn * TN + j) * 16 + 4 * fg, acc[i][j]);
    }
}

template <typename T, int BM, int BN, int WM, int WN, int BKB, int SITE, class AL, class EP>
static hipError_t launch(hipStream_t s, const AL& al, int M, const T* w, int N, int K, const EP& ep,
                         int splits = 1) {
    const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
    gemm_kernel<T, BM, BN, WM, WN, BKB, SITE, AL, EP><<<dim3(tm * tn, splits), WM * WN * 64, 0, s>>>(al, w, N, K, tm,
                                                                                                   tn, ep);
    return hipGetLastError();
}

// Tile choice: 256 x 256 with 8 waves of 128 x 64 (two waves per SIMD hide
// LDS and MFMA latency) when the problem fills the GPU with it, else
// 128 x 128 with 4 waves of 64 x 64.  `lanes` launches of the same shape
// running side by side on separate streams fill it together.
template <int SITE, typename T, class AL, class EP>
static hipError_t run(hipStream_t s, const AL& al, int M, const T* w, int N, int K, const EP& ep,
                      int lanes = 1) {
    if (M <= 0 || N <= 0) return hipSuccess;
    if (K % Elem<T>::per16) return hipErrorInvalidValue;
    const long big = (long)((M + 255) / 256) * ((N + 255) / 256);
    if (big * lanes >= 200) return launch<T, 256, 256, 2, 4, 128, SITE>(s, al, M, w, N, K, ep);
    return launch<T, 128, 128, 2, 2, 128, SITE>(s, al, M, w, N, K, ep);
}

// ------------------------------------------------------------ entry points

template <typename T>
hipError_t conv3x3s2(hipStream_t s, const T* in, int n_chunks, int Hin, int Win, int C,
                     const T* w, const float* bias, T* out, bool time_major, int lanes) {
    const int Hout = (Hin + 1) / 2, Wout = (Win + 1) / 2;
    const int M = n_chunks * Hout * Wout;
    if (C % kConvCB) return hipErrorInvalidValue;
    ConvA<T> al{in, M, Hin, Win, C, Hout, Wout, time_major};
    EpiBias<T, true> ep{out, bias, M, C};
    if (C % Elem<T>::per16) return hipErrorInvalidValue;
    return time_major ? run<kConv3>(s, al, M, w, C, 9 * C, ep, lanes) : run<kConv2>(s, al, M, w, C, 9 * C, ep, lanes);
}

// Split-K for the residual GEMMs and conv_out of small batches: when the
// 128 x 128 tiling leaves most of the CUs idle and K is long, the K range is
// cut into up to 8 splits (each at least 4 stages), the partial sums go to
// `part`, and a reduction kernel adds them in a fixed order and applies the
// epilogue (resid_reduce: into the residual; pe_reduce: plus the position
// table).  Returns the number of splits (1: none).
constexpr int kMaxSplits = 8;

template <typename T>
static int resid_splits(int M, int K, int N, size_t part_elems) {
    constexpr int KSTEP = 128 / (int)sizeof(T);
    const int nk = (K + KSTEP - 1) / KSTEP;
    const long big = (long)((M + 255) / 256) * ((N + 255) / 256);
    const long tiles = (long)((M + 127) / 128) * ((N + 127) / 128);
    if (big >= 200 || tiles >= 128 || nk < 8 || N % 4) return 1;
    int sp = (int)std::min<long>(kMaxSplits, 256 / tiles);
    sp = std::min(sp, nk / 4);
    if (sp < 2) return 1;
    const int kper = (nk + sp - 1) / sp;
    sp = (nk + kper - 1) / kper;                                     // every split has a stage
    if ((size_t)sp * M * N > part_elems) return 1;
    return sp;
}

// x[m][n] = (part[0][m][n] + part[1][m][n] + ...) + pe[src[m] % 13][n], the
// splits added in a fixed order; tap[m][n] = the sum without the PE.
__global__ __launch_bounds__(256) void pe_reduce_kernel(float* __restrict__ x, float* __restrict__ tap,
                                                        const float* __restrict__ part, int splits, int M, int N,
                                                        const float* __restrict__ pe, const int* __restrict__ src) {
    const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_row = N / 4;
    if (i4 >= (int64_t)M * per_row) return;
    const int64_t m = i4 / per_row;
    const int n = (int)(i4 - m * per_row) * 4;
    const size_t o = (size_t)m * N + n, plane = (size_t)M * N;
    float4 acc = *reinterpret_cast<const float4*>(part + o);
    for (int sp = 1; sp < splits; ++sp) {
        const float4 p = *reinterpret_cast<const float4*>(part + sp * plane + o);
        acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
    }
    const float4 p = *reinterpret_cast<const float4*>(pe + (size_t)(src[m] % kChunkTok) * N + n);
    *reinterpret_cast<float4*>(x + o) = make_float4(acc.x + p.x, acc.y + p.y, acc.z + p.z, acc.w + p.w);
    if (tap) *reinterpret_cast<float4*>(tap + o) = acc;
}

// x[m][n] += bias[n] + (part[0][m][n] + part[1][m][n] + ...), the splits
// added in a fixed order (deterministic), 4 values per thread.
__global__ __launch_bounds__(256) void resid_reduce_kernel(float* __restrict__ x, const float* __restrict__ part,
                                                           int splits, int M, int N, const float* __restrict__ bias) {
    const int64_t i4 = (int64_t)blockIdx.x * 256 + threadIdx.x;      // index of a 4-value group
    const int64_t per_row = N / 4;
    if (i4 >= (int64_t)M * per_row) return;
    const int64_t m = i4 / per_row;
    const int n = (int)(i4 - m * per_row) * 4;
    const size_t o = (size_t)m * N + n, plane = (size_t)M * N;
    float4 acc = *reinterpret_cast<const float4*>(part + o);
    for (int sp = 1; sp < splits; ++sp) {
        const float4 p = *reinterpret_cast<const float4*>(part + sp * plane + o);
        acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
    }
    const float4 b = *reinterpret_cast<const float4*>(bias + n);
    float4* px = reinterpret_cast<float4*>(x + o);
    const float4 r = *px;
    *px = make_float4(r.x + (b.x + acc.x), r.y + (b.y + acc.y), r.z + (b.z + acc.z), r.w + (b.w + acc.w));
}

// The split-K reductions with the LayerNorm that follows them fused in: one
// wave per row, the splits added in the same order as resid_reduce_kernel
// (PE = false: x += bias + sum) or pe_reduce_kernel (PE = true: x = sum +
// pe, tap = sum), then ln = LayerNorm(x) through the same row routine as
// layernorm.  Both results are bit-identical to the two kernels run one
// after the other; the row stays in registers between them.
template <typename T, int NQ, bool PE>
__global__ __launch_bounds__(256) void reduce_ln_kernel(float* __restrict__ x, float* __restrict__ tap,
                                                        const float* __restrict__ part, int splits, int M, int N,
                                                        const float* __restrict__ add, const int* __restrict__ src,
                                                        const float* __restrict__ g, const float* __restrict__ b,
                                                        T* __restrict__ ln) {
    const int lane = threadIdx.x & 63;
    const int m = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (m >= M) return;
    const int n4 = N >> 2;
    const size_t plane = (size_t)M * N;
    const float* addr = PE ? add + (size_t)(src[m] % kChunkTok) * N : add;
    // every split of the row in flight at once (one wave holds a whole row)
    float4 p[NQ][kMaxSplits];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i = lane + 64 * q;
        if (i >= n4) continue;
        const float* pq = part + (size_t)m * N + 4 * i;
#pragma unroll
        for (int sp = 0; sp < kMaxSplits; ++sp)
            if (sp < splits) p[q][sp] = *reinterpret_cast<const float4*>(pq + sp * plane);
    }
    float4 v[NQ], gg[NQ], bb[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int i = lane + 64 * q;
        if (i >= n4) continue;
        float4 acc = p[q][0];
#pragma unroll
        for (int sp = 1; sp < kMaxSplits; ++sp)
            if (sp < splits) { acc.x += p[q][sp].x; acc.y += p[q][sp].y; acc.z += p[q][sp].z; acc.w += p[q][sp].w; }
        const size_t o = (size_t)m * N + 4 * i;
        const float4 a4 = reinterpret_cast<const float4*>(addr)[i];
        float4* px = reinterpret_cast<float4*>(x + o);
        if constexpr (PE) {
            v[q] = make_float4(acc.x + a4.x, acc.y + a4.y, acc.z + a4.z, acc.w + a4.w);
            if (tap) *reinterpret_cast<float4*>(tap + o) = acc;
        } else {
            const float4 r = *px;
            v[q] = make_float4(r.x + (a4.x + acc.x), r.y + (a4.y + acc.y), r.z + (a4.z + acc.z), r.w + (a4.w + acc.w));
        }
        *px = v[q];
        gg[q] = reinterpret_cast<const float4*>(g)[i];
        bb[q] = reinterpret_cast<const float4*>(b)[i];
    }
    ln_row<T, NQ>(v, gg, bb, lane, N, ln + (size_t)m * N);
}

// The reduction of a split-K residual GEMM (PE: conv_out's), with the
// following LayerNorm fused in when `after` asks for one and the row fits.
template <typename T, bool PE>
static hipError_t reduce_split(hipStream_t s, float* x, float* tap, const float* part, int sp, int M, int N,
                               const float* add, const int* src, LnAfter<T>* after) {
    if (after && N % 4 == 0 && N <= 1024 && sp <= kMaxSplits) {
        reduce_ln_kernel<T, 4, PE><<<(unsigned)((M + 3) / 4), 256, 0, s>>>(x, tap, part, sp, M, N, add, src,
                                                                          after->g, after->b, after->out);
        after->done = true;
    } else if (PE) {
        const unsigned blocks = (unsigned)(((int64_t)M * (N / 4) + 255) / 256);
        pe_reduce_kernel<<<blocks, 256, 0, s>>>(x, tap, part, sp, M, N, add, src);
    } else {
        const int64_t groups = (int64_t)M * (N / 4);
        resid_reduce_kernel<<<(unsigned)((groups + 255) / 256), 256, 0, s>>>(x, part, sp, M, N, add);
    }
    return hipGetLastError();
}

template <typename T>
hipError_t conv_out(hipStream_t s, const T* a, const int* src, int n_tok, int K, const T* w, int N,
                    const float* pe, float* x, float* tap, float* part, size_t part_elems, int lanes,
                    LnAfter<T>* after) {
    GatherA<T> al{a, src, n_tok, K};
    if (n_tok <= 0 || N <= 0) return hipSuccess;
    const int sp = part ? resid_splits<T>(n_tok, K, N, part_elems) : 1;
    if (sp > 1) {   // split-K (see resid_splits), the PE added in the reduction
        if (K % Elem<T>::per16) return hipErrorInvalidValue;
        const hipError_t st =
            launch<T, 128, 128, 2, 2, 128, kConvOut>(s, al, n_tok, w, N, K, EpiPartial{part, n_tok, N}, sp);
        if (st != hipSuccess) return st;
        return reduce_split<T, true>(s, x, tap, part, sp, n_tok, N, pe, src, after);
    }
    EpiPE ep{x, tap, pe, src, n_tok, N};
    return run<kConvOut>(s, al, n_tok, w, N, K, ep, lanes);
}

template <typename T>
hipError_t gemm_bias(hipStream_t s, const T* a, int M, int K, const T* w, int N, const float* bias,
                     T* out, bool gelu, int lanes) {
    DenseA<T> al{a, M, K, K};
    if (!gelu) return run<kQKV>(s, al, M, w, N, K, EpiBias<T, false>{out, bias, M, N}, lanes);
    if (N != K) return run<kFC1>(s, al, M, w, N, K, EpiBias<T, true>{out, bias, M, N}, lanes);
    return run<kProj1>(s, al, M, w, N, K, EpiBias<T, true>{out, bias, M, N}, lanes);
}

template <typename T>
hipError_t gemm_bias_resid(hipStream_t s, const T* a, int M, int K, const T* w, int N,
                           const float* bias, float* x, float* part, size_t part_elems, int lanes,
                           LnAfter<T>* after) {
    DenseA<T> al{a, M, K, K};
    if (M <= 0 || N <= 0) return hipSuccess;
    const int sp = part ? resid_splits<T>(M, K, N, part_elems) : 1;
    if (sp > 1) {
        if (K % Elem<T>::per16) return hipErrorInvalidValue;
        const EpiPartial ep{part, M, N};
        const hipError_t st = N == K ? launch<T, 128, 128, 2, 2, 128, kOProj>(s, al, M, w, N, K, ep, sp)
                                     : launch<T, 128, 128, 2, 2, 128, kFC2>(s, al, M, w, N, K, ep, sp);
        if (st != hipSuccess) return st;
        return reduce_split<T, false>(s, x, nullptr, part, sp, M, N, bias, nullptr, after);
    }
    EpiResid ep{x, bias, M, N};
    if (N == K) return run<kOProj>(s, al, M, w, N, K, ep, lanes);
    return run<kFC2>(s, al, M, w, N, K, ep, lanes);
}

template <typename T>
hipError_t gemm_bias_f32(hipStream_t s, const T* a, int M, int K, const T* w, int N,
                         const float* bias, float* out, int lanes) {
    DenseA<T> al{a, M, K, K};
    EpiF32Bias ep{out, bias, M, N};
    return run<kProj2>(s, al, M, w, N, K, ep, lanes);
}

template <typename T>
hipError_t thinker_gemm(hipStream_t s, int site, const T* a, int M, int K, const T* w, int N,
                        const float* zero, T* out_t, float* x) {
    DenseA<T> al{a, M, K, K};
    switch (site) {
        case kTQKV: return run<kTQKV>(s, al, M, w, N, K, EpiBias<T, false>{out_t, zero, M, N});
        case kTOProj: return run<kTOProj>(s, al, M, w, N, K, EpiResid{x, zero, M, N});
        case kTDown: return run<kTDown>(s, al, M, w, N, K, EpiResid{x, zero, M, N});
        case kTGateUp:
            if (N % 32) return hipErrorInvalidValue;
            return run<kTGateUp>(s, al, M, w, N, K, EpiSwiGLU<T>{out_t, M, N / 2});
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t thinker_logits(hipStream_t s, const T* a, const int* rows, int n_rows, int K, const T* w, int N,
                          const float* zero, float* out) {
    GatherA<T> al{a, rows, n_rows, K};
    return run<kTLogits>(s, al, n_rows, w, N, K, EpiF32Bias{out, zero, n_rows, N});
}

#define QA_INST(T)                                                                                    \
    template hipError_t conv3x3s2<T>(hipStream_t, const T*, int, int, int, int, const T*, const float*, \
                                     T*, bool, int);                                                  \
    template hipError_t conv_out<T>(hipStream_t, const T*, const int*, int, int, const T*, int,        \
                                    const float*, float*, float*, float*, size_t, int, LnAfter<T>*);  \
    template hipError_t gemm_bias<T>(hipStream_t, const T*, int, int, const T*, int, const float*, T*, \
                                     bool, int);                                                      \
    template hipError_t gemm_bias_resid<T>(hipStream_t, const T*, int, int, const T*, int,            \
                                           const float*, float*, float*, size_t, int, LnAfter<T>*);   \
    template hipError_t gemm_bias_f32<T>(hipStream_t, const T*, int, int, const T*, int, const float*, \
                                         float*, int);
template hipError_t thinker_gemm<float>(hipStream_t, int, const float*, int, int, const float*, int, const float*,
                                        float*, float*);
template hipError_t thinker_gemm<bf16>(hipStream_t, int, const bf16*, int, int, const bf16*, int, const float*,
                                       bf16*, float*);
template hipError_t thinker_logits<float>(hipStream_t, const float*, const int*, int, int, const float*, int,
                                          const float*, float*);
template hipError_t thinker_logits<bf16>(hipStream_t, const bf16*, const int*, int, int, const bf16*, int,
                                         const float*, float*);
QA_INST(float)
QA_INST(bf16)

}  // namespace qa
