// conv1 -> conv2 of the conv stem in one kernel (bf16 encoders): conv2's
// implicit GEMM takes its A operand from a conv1 patch that the workgroup
// computes into LDS, one 32-channel slab at a time, so conv1's output (two
// bytes per channel and pixel, 3.7 GB for 20 minutes of audio) never goes to
// HBM (qwenasr.cpp ARCHITECTURE.md "Conv2d subsampling stem": conv2d k3 s2 p1
// 1 -> C, GELU, conv2d k3 s2 p1 C -> C, GELU, per 100-frame chunk; OneSpeech
// "Front end and graph numerics": chunks padded independently).
//
// Tile: one chunk, 5 of conv2's 25 time columns x all 32 frequency rows (160
// output pixels, row order (column, row) inside the tile) x every output
// channel: 8 waves of 160 pixels x 64 channels (stems of more than 256
// channels, up to 512) or x 32 channels (up to 256).  The K order is conv2's
// (32-channel slab, tap, channel), so every 32-wide MFMA K block is one (slab,
// tap).  Per slab the MFMAs read a conv1 patch from LDS: conv1's outputs of
// the tile's receptive field for the slab's 32 channels (11 conv1 columns x
// 65 conv1 rows, -1 .. 63; row -1 and column -1 are conv2's zero padding),
// computed by a split-input MFMA (below) and the GELU, once per pixel tile
// for all output channels.  The patch is double-buffered: while the waves
// multiply slab s they compute slab s + 1's patch into the other buffer (one
// barrier per slab).  With 32 channels per wave a wave interleaves its patch
// groups with its MFMAs; with 64 (160 accumulator registers) waves 0-3 compute
// theirs before their MFMAs and waves 4-7 after, so that the two waves of a
// SIMD (w and w + 4) overlap one's VALU work with the other's MFMAs.  A wave's
// weight rows are its own, so they go global -> registers (buffer loads),
// three taps ahead (one with 64 channels), with no LDS and no barrier.
//
// conv1 on MFMA: K = 9 taps x 3 bf16 parts (hi + mid + lo, which add up to
// the fp32 log-mel value to within one fp32 ulp) + 1 bias slot = 28 <= 32, so
// one v_mfma_f32_16x16x32_bf16 gives 16 channels x 16 pixels of conv1 in fp32;
// the fragments' channel order (see the weight packing) gives each lane 8
// consecutive channels of one pixel from two MFMAs, one 16-byte patch store.
// conv2's accumulators take the (slab, tap) blocks in K order, as gemm_kernel
// with ConvA does over a stored conv1 output (the path of fp32 and of stems
// wider than 512 channels), and the output was checked bit-identical to that
// route when both existed.
//
// LDS: two patches (46,464 B each), the tile's log-mel window (11,868 B), the
// conv1 B operands of every wave's pixel groups (49,152 B; the same for every
// slab, built once, kept out of the registers) and two slabs' conv1 A
// fragments (4,096 B, loaded global -> LDS directly, slab s + 2's during slab
// s).  With 32 channels per wave the first two fragments of the next tap are
// read during the current tap's MFMAs; with 64 the slab's 90 (tap, fragment)
// reads run two fragments ahead of their MFMAs.
// Patch layout: [conv1 column 11][row parity 2][row / 2 33][32 channels]: a
// conv2 tap reads the conv1 rows 2 i + a of 16 consecutive output rows i,
// which this layout keeps 64 bytes apart; the 16-byte channel chunks are
// XOR-swizzled by (row / 2) / 2 so that the reads of 8 consecutive rows hit 8
// different bank groups.  Slot (parity 1, row / 2 = 32) of column 0 is never
// read: pixel groups past the patch write their results there.
#include <algorithm>
#include <type_traits>

#include "qa_device.h"
#include "qa_kernels.h"

namespace qa {

constexpr int kFsCols = 5;                              // conv2 time columns per tile
constexpr int kFsTilesPerChunk = 25 / kFsCols;          // 5
constexpr int kFsM = kFsCols * 32;                      // 160 output pixels
constexpr int kFsPcol = 2 * kFsCols + 1;                // 11 conv1 columns
constexpr int kFsProw = 65;                             // conv1 rows -1 .. 63
constexpr int kFsRi = 33;                               // patch rows per parity
constexpr int kFsPix = kFsPcol * kFsProw;               // 715 patch pixels
constexpr int kFsGroups = (kFsPix + 15) / 16;           // 45 MFMA pixel groups
constexpr int kFsGpw = (kFsGroups + 7) / 8;             // pixel groups per wave (6)
constexpr int kFsPatchBytes = kFsPcol * 2 * kFsRi * 64; // 46,464
constexpr int kFsMelRows = kMels + 1;                   // mel rows -1 .. 127
constexpr int kFsMelT = 4 * kFsCols + 3;                // 23 frames
constexpr int kFsMelBytes = kFsMelRows * kFsMelT * 4;   // 11,868
constexpr int kFsMelDma = (kFsMelRows * kFsMelT + 63) / 64;   // 47 direct-to-LDS dword loads of 64 lanes
constexpr int kFsOffMel = 2 * kFsPatchBytes;
constexpr int kFsOffBop = kFsOffMel + kFsMelDma * 256;       // (the last load's 41 spare dwords land before it)
constexpr int kFsOffWa = kFsOffBop + 8 * kFsGpw * 64 * 16;   // + the conv1 B operands
constexpr int kFsOffBias = kFsOffWa + 2 * 2048;        // + two slabs' conv1 A fragments
constexpr int kFsOffNext = kFsOffBias + 512 * 4;       // + conv2's bias (512 channels)
constexpr int kFsLds = kFsOffNext + 16;                 // + the next tile handed out: 160,272 B
constexpr int kFsPrefetch = 2;                          // fragments of the next tap read ahead
constexpr int kFsWAhead = 3;                            // weight taps in flight per wave (256-channel tiles)
constexpr int kFsWAheadWide = 1;                        // (512-channel tiles: 64 channels per wave)
constexpr int kFsStream = 2;                            // patch fragments read ahead (512-channel tiles)
static_assert(kFsM * 256 * 2 <= 2 * kFsPatchBytes, "epilogue staging fits the patches");
static_assert(9 % kFsWAhead == 0 && 9 % kFsWAheadWide == 0,
              "the weight ring position of a tap is the same in every slab");

__device__ __forceinline__ int fs_patch_off(int pcol, int prow, int chunk) {
    const int par = prow & 1, ri = prow >> 1;
    return ((pcol * 2 + par) * kFsRi + ri) * 64 + ((chunk ^ ((ri >> 1) & 3)) << 4);
}
constexpr int kFsDummy = (1 * kFsRi + 32) * 64;         // column 0, parity 1, row / 2 32: never read

// NCB: 32-channel slabs of conv1's output = conv2's input (C = 32 NCB).
// NJ: 16-channel fragments per wave, 2 (a workgroup covers 256 output
// channels) or 4 (512: every channel of the stem, so each slab's conv1 patch
// is computed once per pixel tile instead of once per 256-channel half).
//
// With 512-channel tiles the grid is persistent: one workgroup per CU takes
// tile blockIdx.x, then the tiles an atomic counter hands out (gridDim.x +
// the counter's old value), one ahead: the tile after next is asked for
// during a tile's epilogue, so the faster CUs take more tiles and the grid
// ends within about one tile time.  A tile's set-up runs inside the tile
// before it.  The last slab of a tile builds the next tile's
// conv1 B operands and its slab-0 patch in the VALU phase that the other
// slabs spend on their successor's patch (so it overlaps the sibling wave's
// MFMAs); the log-mel window of the tile after next goes global -> LDS by
// direct loads at the start of the epilogue (the window is only read when B
// operands are built); the conv1 fragments of the next tile's first two
// slabs arrive during the current tile's last two, and the weight ring runs
// on into the next tile's first K blocks.  The patch and fragment buffers
// alternate with a slab counter that runs on across tiles, and the epilogue
// stages its rows through the patch buffer the last slab read (four passes
// of 128 channels): the other one holds the next tile's first patch.
template <int NCB, int NJ>
__global__ __launch_bounds__(512) void stem12_kernel(const float* __restrict__ logmel,
                                                     const ChunkInfo* __restrict__ chunks, int n_tiles,
                                                     const uint4* __restrict__ wfrag,
                                                     const bf16* __restrict__ w2,
                                                     const float* __restrict__ b2,
                                                     bf16* __restrict__ out, int* __restrict__ tile_counter) {
    constexpr int C = 32 * NCB, K = 9 * C, NT = 9 * NCB;   // NT: (slab, tap) K blocks
    constexpr int WN = 16 * NJ, BN = 8 * WN;              // output channels per wave / per workgroup
    constexpr int WAH = NJ == 2 ? kFsWAhead : kFsWAheadWide;
    constexpr bool PERSIST = NJ == 4;
    __shared__ __align__(1024) char smem[kFsLds];
    float* img = reinterpret_cast<float*>(smem + kFsOffMel);
    float* bias_lds = reinterpret_cast<float*>(smem + kFsOffBias);
    int* next_lds = reinterpret_cast<int*>(smem + kFsOffNext);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int fr = lane & 15, fg = lane >> 4;
    const int n0 = wave * WN;                             // this wave's first output channel
    int tile = blockIdx.x;

    // ---- this wave's weight rows n0 + 16 j + fr (rows past C repeat row C - 1:
    // their outputs are never stored); K block t = (slab, tap) at element 32 t
    // (buffer loads: one 32-bit byte offset per row instead of a 64-bit address).
    // Blocks past the last one are the next tile's first blocks (the same
    // weights: the ring runs on across tiles; unused after the last tile).
    const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc((void*)w2, (short)0, C * K * 2, 0x00020000);
    int wrow[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) wrow[j] = (min(n0 + 16 * j + fr, C - 1) * K + 8 * fg) * 2;
    uint4 wb[WAH][NJ];
    // (the block's offset goes in the scalar offset operand: no per-block
    // vector address arithmetic, and nothing for the compiler to precompute
    // per block and hold in registers)
    auto load_w = [&](int t, uint4* dst) __attribute__((always_inline)) {
        const int tc = t < NT ? t : t - NT;
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            dst[j] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(wres, wrow[j], 64 * tc, 0));
    };
#pragma unroll
    for (int r = 0; r < WAH; ++r) load_w(r, wb[r]);
    // conv1's A fragments (2 x 64 lanes x 16 B per slab, the same for every
    // wave and every tile) go global -> LDS: slab q's into buffer (global slab
    // index of q) & 1, loaded two slabs ahead by waves 0 and 1 (after the
    // slab that last read that buffer)
    char* wab = smem + kFsOffWa;
    const unsigned wab_lds = (unsigned)(uintptr_t)(lds_void*)wab;
    const i32x4 wares = buffer_rsrc(wfrag, (uint64_t)NCB * 2 * 64 * 16);
    auto load_wa = [&](int frag_slab, int buf) __attribute__((always_inline)) {
        if (wave < 2) {
            int lx = lane;                               // opaque: the offset is recomputed, not kept per slab
            asm volatile("" : "+v"(lx));
            dma16_buf(wares, (unsigned)(lx * 16 + (2 * frag_slab + wave) * 1024), wab_lds + buf * 2048 + wave * 1024);
        }
    };
    load_wa(0, 0);
    if (NCB > 1 && wave >= 2 && wave < 4)
        dma16_buf(wares, (unsigned)(((2 + wave - 2) * 64 + lane) * 16), wab_lds + 2048 + (wave - 2) * 1024);

    // ---- a tile's log-mel window: rows -1 .. 127, frames 4 j0 - 3 .. 4 j0 + 19
    // (zeros outside the chunk's frames), [frame][row], loaded through a buffer
    // resource over the chunk's frames (out-of-range offsets read zeros).  All
    // of a thread's loads are issued before its first store: one memory
    // latency for the window.
    constexpr int NV = (kFsMelRows * kFsMelT + 511) / 512;
    // (valid = false: tile t does not exist, every value reads as zero)
    auto mel_load = [&](int t, float (&v)[NV], int tid, bool valid) __attribute__((always_inline)) {
        const ChunkInfo cx = chunks[valid ? t / kFsTilesPerChunk : 0];
        const int j0x = (t % kFsTilesPerChunk) * kFsCols;
        const __amdgpu_buffer_rsrc_t mres = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(logmel + (size_t)cx.frame_row0 * kMels), (short)0, valid ? cx.m * kMels * 4 : 0, 0x00020000);
#pragma unroll
        for (int k = 0; k < NV; ++k) {
            const int idx = tid + 512 * k;
            const int tt = idx / kFsMelRows, rr = idx - tt * kFsMelRows;
            const int f = rr - 1, fi = 4 * j0x - 3 + tt;
            const bool in = idx < kFsMelRows * kFsMelT && f >= 0 && fi >= 0;
            v[k] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 mres, in ? (fi * kMels + f) * 4 : (int)kOobOffset, 0, 0));
        }
    };
    auto mel_store = [&](const float (&v)[NV], int tid) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < NV; ++k)
            if (tid + 512 * k < kFsMelRows * kFsMelT) img[tid + 512 * k] = v[k];
    };
    // the same window by direct-to-LDS dword loads (no registers held; the
    // loads land by the next vmcnt(0) wait): load k of kFsMelDma (by wave
    // k % 8) fills img[64 k .. 64 k + 63]
    const unsigned img_lds = (unsigned)(uintptr_t)(lds_void*)img;
    auto mel_dma = [&](int t) __attribute__((always_inline)) {
        const ChunkInfo cx = chunks[t / kFsTilesPerChunk];
        const int j0x = (t % kFsTilesPerChunk) * kFsCols;
        const i32x4 mres = buffer_rsrc(logmel + (size_t)cx.frame_row0 * kMels, (uint64_t)cx.m * kMels * 4);
        int lx = lane;
        asm volatile("" : "+v"(lx));
        for (int k = wave; k < kFsMelDma; k += 8) {
            const int idx = 64 * k + lx;
            const int tt = idx / kFsMelRows, rr = idx - tt * kFsMelRows;
            const int f = rr - 1, fi = 4 * j0x - 3 + tt;
            const bool in = idx < kFsMelRows * kFsMelT && f >= 0 && fi >= 0;
            dma4_buf(mres, in ? (unsigned)((fi * kMels + f) * 4) : kOobOffset, img_lds + 256 * k);
        }
    };
    {
        float v[NV];
        mel_load(tile, v, tid, true);
        mel_store(v, tid);
    }
    // conv2's bias, zero past C (the accumulators' start value of every tile)
    for (int n = tid; n < BN; n += 512) bias_lds[n] = n < C ? b2[n] : 0.f;
    // the second tile
    if (PERSIST && tid == 0) *next_lds = (int)gridDim.x + atomicAdd(tile_counter, 1);

    __builtin_amdgcn_s_waitcnt(0x0F70);                  // vmcnt(0): this wave's conv1 fragment loads
    __syncthreads();                                     // the mel window and the fragments are in LDS
    int next = PERSIST ? __builtin_amdgcn_readfirstlane(*next_lds) : n_tiles;

    // ---- conv1 B operands of this wave's pixel groups (the same for every
    // slab): lane (px, g) holds K entries 8 g .. 8 g + 7 of pixel px: tap k / 3
    // (dy = tap / 3, dx = tap % 3), part k % 3 of the 3-way bf16 split, k = 27
    // the constant 1 of the bias slot.  Each group's LDS destination in the
    // patch (the dummy slot for pixels past it) and its padding flag.
    uint4* bop_lds = reinterpret_cast<uint4*>(smem + kFsOffBop) + wave * kFsGpw * 64 + lane;
    // group u's pixel, its patch destination (the dummy slot past the patch)
    // and whether it is conv2's zero padding (recomputed per use: registers)
    auto gpix = [&](int u, int& pc, int& pr, int frx) __attribute__((always_inline)) {
        const int p = (wave + 8 * u) * 16 + frx;
        const bool in = p < kFsPix;
        pc = in ? p / kFsProw : 0;
        pr = in ? p - pc * kFsProw : 1;
        return in;
    };
    // from the window in img (a wave writes and reads only its own groups);
    // lx: the lane id (an opaque copy in the tile loop, so that these
    // addresses are not held in registers between tiles)
    auto build_bop = [&](int lx) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < kFsGpw; ++u) {
            int pc, pr;
            gpix(u, pc, pr, lx & 15);
            const int base = 2 * pc * kFsMelRows + 2 * max(pr, 1) - 2;   // rows past the top are padding
            bf16 bv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int k = 8 * ((lx >> 4) & 3) + e;
                const int tap = k / 3, q = k - 3 * tap;
                const float x = k < 27 ? img[base + (tap % 3) * kFsMelRows + tap / 3] : 0.f;
                const bf16 hi = (bf16)x;
                const float r1 = x - (float)hi;
                const bf16 mid = (bf16)r1;
                const bf16 lo = (bf16)(r1 - (float)mid);
                bv[e] = k < 27 ? (q == 0 ? hi : q == 1 ? mid : lo) : (k == 27 ? (bf16)1.0f : (bf16)0.0f);
            }
            const bf16x8 b8 = {bv[0], bv[1], bv[2], bv[3], bv[4], bv[5], bv[6], bv[7]};
            bop_lds[u * 64] = __builtin_bit_cast(uint4, b8);
            __builtin_amdgcn_sched_barrier(0);           // one group's registers at a time
        }
    };
    // one pixel group of a slab's patch into buffer pb (j0x: the tile's first
    // conv2 column; column -1 is padding only in a chunk's first tile).  The
    // group's pixel is derived from an opaque copy of the lane id, so that the
    // compiler recomputes it (a few integer operations) instead of keeping
    // every group's destination in registers through the slab loop.
    auto conv1_group = [&](int u, const char* wa, char* pb, int j0x) __attribute__((always_inline)) {
        const uint4 wa0 = ld16(wa + lane * 16), wa1 = ld16(wa + 1024 + lane * 16);
        const uint4 bu = bop_lds[u * 64];
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        const f32x4 a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa0),
                                                                 __builtin_bit_cast(bf16x8, bu), z, 0, 0, 0);
        const f32x4 a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa1),
                                                                 __builtin_bit_cast(bf16x8, bu), z, 0, 0, 0);
        const bf16x8 o = {(bf16)gelu_erf_bf16(a0[0]), (bf16)gelu_erf_bf16(a0[1]), (bf16)gelu_erf_bf16(a0[2]),
                          (bf16)gelu_erf_bf16(a0[3]), (bf16)gelu_erf_bf16(a1[0]), (bf16)gelu_erf_bf16(a1[1]),
                          (bf16)gelu_erf_bf16(a1[2]), (bf16)gelu_erf_bf16(a1[3])};
        int frx = fr, pc, pr;
        asm volatile("" : "+v"(frx));
        const bool in = gpix(u, pc, pr, frx);
        const int dst = in ? fs_patch_off(pc, pr, fg) : kFsDummy + (fg << 4);
        const bool pad = pr == 0 || (pc == 0 && j0x == 0);
        *reinterpret_cast<uint4*>(pb + dst) = pad ? make_uint4(0u, 0u, 0u, 0u) : __builtin_bit_cast(uint4, o);
    };
    build_bop(lane);
#pragma unroll
    for (int u = 0; u < kFsGpw; ++u) conv1_group(u, wab, smem, (tile % kFsTilesPerChunk) * kFsCols);
    __syncthreads();                                     // slab 0's patch; every wave has read the window
    // the window of the second tile (read in the first tile's last slab)
    if (PERSIST && next < n_tiles) mel_dma(next);

    const int fbase0 = fr * 64 + ((fg ^ ((fr >> 1) & 3)) << 4);
    const int fbase1 = fr * 64 + ((fg ^ (((fr + 1) >> 1) & 3)) << 4);
    int g = 0;                                           // global index of this tile's slab 0 (buffer parity)
    for (;;) {
        const int chunk = tile / kFsTilesPerChunk, j0 = (tile % kFsTilesPerChunk) * kFsCols;
        const bool has_next = PERSIST && next < n_tiles;
        const int j0n = (next % kFsTilesPerChunk) * kFsCols;
        // lane indices of the per-tile code outside the slabs (accumulator
        // start, window loads, epilogue) come from opaque copies of the thread
        // id taken where they are used, so that the compiler recomputes them
        // per tile instead of holding them in registers through the slabs
        int tid_a = tid;
        asm volatile("" : "+v"(tid_a));

        // ---- accumulators, bias as the start value: lane holds out[m = fr][n = 4 fg + r]
        f32x4 acc[10][NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const f32x4 b = *reinterpret_cast<const f32x4*>(bias_lds + n0 + j * 16 + 4 * ((tid_a >> 4) & 3));
#pragma unroll
            for (int f = 0; f < 10; ++f) acc[f][j] = b;
        }
        // one slab: 9 taps of MFMAs from patch buffer gs & 1 (gs: the global
        // slab index); with NEXT, slab s + 1's patch into the other buffer; in
        // a tile's last slab, the next tile's B operands and slab-0 patch
        auto slab = [&](int s, auto next_tag) __attribute__((always_inline)) {
            constexpr bool NEXT = decltype(next_tag)::value;
            const int gs = g + s;
            const char* pa = smem + (gs & 1) * kFsPatchBytes;
            char* pn = smem + ((gs + 1) & 1) * kFsPatchBytes;
            const char* wan = wab + ((gs + 1) & 1) * 2048;    // conv1 fragments of the patch computed here
            const bool work = NEXT || has_next;               // a patch is computed during this slab
            const bool wa_next = s + 2 < NCB || has_next;     // fragments two slabs ahead are loaded
            if (wa_next) load_wa(s + 2 < NCB ? s + 2 : s + 2 - NCB, gs & 1);
            // fragment f of tap (a, b): conv1 rows 2 i + a, i = 16 (f & 1) + fr, of
            // column 2 (f >> 1) + b, i.e. patch row ri = fr + 16 (f & 1) + a / 2 of
            // parity a & 1.  The swizzle ((ri >> 1) & 3) then depends on the lane
            // and on a / 2 only, so every read is one of two per-lane bases plus a
            // constant offset (the 90 reads of a slab need no address registers).
            auto read_frag = [&](int tap, int f) __attribute__((always_inline)) {
                const int a = tap / 3, bb = tap - 3 * a, pcol = 2 * (f >> 1) + bb;
                const int cofs = ((pcol * 2 + (a & 1)) * kFsRi + 16 * (f & 1) + (a >> 1)) * 64;
                return ld16(pa + ((a >> 1) ? fbase1 : fbase0) + cofs);
            };
            if constexpr (NJ == 2) {
                uint4 fn[kFsPrefetch];
#pragma unroll
                for (int f = 0; f < kFsPrefetch; ++f) fn[f] = read_frag(0, f);
#pragma unroll
                for (int tap = 0; tap < 9; ++tap) {
                    const uint4 fb0 = wb[tap % WAH][0], fb1 = wb[tap % WAH][1];
                    load_w(9 * s + tap + WAH, wb[tap % WAH]);
                    uint4 fa[10];
#pragma unroll
                    for (int f = 0; f < kFsPrefetch; ++f) fa[f] = fn[f];
#pragma unroll
                    for (int f = kFsPrefetch; f < 10; ++f) fa[f] = read_frag(tap, f);
                    if (tap + 1 < 9) {
#pragma unroll
                        for (int f = 0; f < kFsPrefetch; ++f) fn[f] = read_frag(tap + 1, f);
                    }
#pragma unroll
                    for (int f = 0; f < 10; ++f) mfma_kblock(bf16(), fb0, fa[f], acc[f][0]);
#pragma unroll
                    for (int f = 0; f < 10; ++f) mfma_kblock(bf16(), fb1, fa[f], acc[f][1]);
                    if constexpr (NEXT) {
                        if (tap % 3 != 2) conv1_group(2 * (tap / 3) + tap % 3, wan, pn, j0);
                    }
                }
            } else {
                // 64 channels per wave: each patch fragment feeds NJ MFMAs, read
                // kFsStream fragments ahead through the slab's 90 (tap, fragment)
                // steps.  The next patch's work is not interleaved (its registers
                // would not fit beside 160 accumulators): waves 0-3 do their pixel
                // groups before their MFMAs, waves 4-7 after theirs, so on every
                // SIMD (waves w and w + 4) one wave runs the VALU work while the
                // other keeps the matrix core busy.
                auto conv1_phase = [&]() __attribute__((always_inline)) {
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (!NEXT) {                        // the next tile's, from its window
                        int lx = lane;
                        asm volatile("" : "+v"(lx));
                        build_bop(lx);
                        __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                    for (int u = 0; u < kFsGpw; ++u) conv1_group(u, wan, pn, NEXT ? j0 : j0n);
                    __builtin_amdgcn_sched_barrier(0);
                };
                if (work && wave < 4) conv1_phase();
                // The MFMA section runs at wave priority 1: when both waves of
                // the SIMD can issue, the matrix instruction goes first and the
                // sibling's VALU phase takes the cycles in between.
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(1);
                __builtin_amdgcn_sched_barrier(0);
                uint4 ring[kFsStream];
#pragma unroll
                for (int q = 0; q < kFsStream; ++q) ring[q] = read_frag(q / 10, q % 10);
#pragma unroll
                for (int tap = 0; tap < 9; ++tap) {
                    uint4 fb[NJ];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) fb[j] = wb[tap % WAH][j];
                    load_w(9 * s + tap + WAH, wb[tap % WAH]);
#pragma unroll
                    for (int f = 0; f < 10; ++f) {
                        const int q = tap * 10 + f;
                        const uint4 fa = ring[q % kFsStream];
                        if (q + kFsStream < 90) ring[q % kFsStream] = read_frag((q + kFsStream) / 10, (q + kFsStream) % 10);
#pragma unroll
                        for (int j = 0; j < NJ; ++j) mfma_kblock(bf16(), fb[j], fa, acc[f][j]);
                        __builtin_amdgcn_sched_barrier(0);   // keeps the register ring from being hoisted
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_setprio(0);
                __builtin_amdgcn_sched_barrier(0);
                if (work && wave >= 4) conv1_phase();
            }
            if (wa_next) __builtin_amdgcn_s_waitcnt(0x0F70);   // the conv1 fragments two slabs ahead landed
            __syncthreads();   // reads of buffer gs & 1 done; the next patch complete
        };
        for (int s = 0; s + 1 < NCB; ++s) slab(s, std::true_type{});
        slab(NCB - 1, std::false_type{});

        int tid_t = tid;
        asm volatile("" : "+v"(tid_t));
        const int fr_t = tid_t & 15, fg_t = (tid_t >> 4) & 3;

        // ---- epilogue: GELU, bf16, staged row-major through LDS (rows of PW
        // channels, 16-byte chunks XOR-swizzled by row % 16), then whole
        // 16-byte chunks of output rows: pixel (column jj, row i) of the tile
        // is row (chunk, i, j0 + jj) of conv2's NHWC output.  256-channel
        // tiles stage all rows at once in both patch buffers; 512-channel
        // tiles go out in four passes of 128 channels (waves 2h and 2h + 1 in
        // pass h) through the patch buffer the last slab read.  Every wave
        // converts its outputs first, so that the GELUs run on all SIMDs at
        // once.  The tile after next is asked for now (its index is read
        // after the first staging barrier), and its window goes in then: the
        // last slab has built the next tile's B operands from img.
        int grab = 0;
        if (has_next && tid_t == 0) grab = atomicAdd(tile_counter, 1);
        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
        bf16x4 ov[10][NJ];
#pragma unroll
        for (int f = 0; f < 10; ++f)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                ov[f][j] = bf16x4{(bf16)gelu_erf_bf16(acc[f][j][0]), (bf16)gelu_erf_bf16(acc[f][j][1]),
                                  (bf16)gelu_erf_bf16(acc[f][j][2]), (bf16)gelu_erf_bf16(acc[f][j][3])};
        bf16* obase = out + (size_t)chunk * 800 * C;
        constexpr int PASSES = PERSIST ? 4 : BN / 256;
        constexpr int PW = BN / PASSES, RB = 2 * PW, CPR = PW / 8, WPP = 8 / PASSES;
        static_assert(kFsM * RB <= (PERSIST ? kFsPatchBytes : 2 * kFsPatchBytes), "epilogue staging fits");
        char* stg = smem + (PERSIST ? ((g + NCB - 1) & 1) * kFsPatchBytes : 0);
        if (has_next && tid_t == 0) *next_lds = (int)gridDim.x + grab;
        int next2 = n_tiles;
#pragma unroll
        for (int h = 0; h < PASSES; ++h) {
            if (h == 1 && has_next) {
                next2 = __builtin_amdgcn_readfirstlane(*next_lds);
                if (next2 < n_tiles) mel_dma(next2);
            }
            if (h > 0) __syncthreads();                      // the previous pass's rows are out
            if (wave / WPP == h) {
#pragma unroll
                for (int f = 0; f < 10; ++f) {
                    const int m = f * 16 + fr_t;
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const int n = (wave * WN) % PW + j * 16 + 4 * fg_t;   // 4 channels = half of chunk n / 8
                        const int c16 = (n >> 3) ^ (m & 15);
                        *reinterpret_cast<bf16x4*>(stg + m * RB + (c16 << 4) + ((n & 4) << 1)) = ov[f][j];
                    }
                }
            }
            __syncthreads();
            const int nt0 = h * PW;
            for (int idx = tid_t; idx < kFsM * CPR; idx += 512) {
                const int m = idx / CPR, c = idx % CPR;
                const int n = nt0 + 8 * c;
                if (n >= C) continue;
                const int jj = m >> 5, i = m & 31;
                const uint4 v = ld16(stg + m * RB + ((c ^ (m & 15)) << 4));
                *reinterpret_cast<uint4*>(obase + ((size_t)i * 25 + j0 + jj) * C + n) = v;
            }
        }
        if (!has_next) break;
        __syncthreads();                                 // the staging buffer takes the next tile's slab-1 patch
        tile = next;
        next = next2;
        g += NCB;
    }
}

hipError_t stem12(hipStream_t s, const float* logmel, const ChunkInfo* chunks, int n_chunks, const uint4* wfrag,
                  const bf16* w2, const float* b2, int C, bf16* out, int* tile_counter) {
    if (n_chunks <= 0) return hipSuccess;
    // 256-channel tiles (8 waves of 32) for stems of up to 256 channels: one
    // workgroup per pixel tile; 512-channel tiles (8 waves of 64) above: one
    // workgroup per CU (160 KB of LDS each) walking the tiles
    const int n_tiles = n_chunks * kFsTilesPerChunk;
    int grid = n_tiles;
    if (C > 256) {
        int dev = 0, cus = 0;
        hipError_t st = hipGetDevice(&dev);
        if (st == hipSuccess) st = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (st != hipSuccess) return st;
        grid = std::min(n_tiles, std::max(cus, 1));
    }
    switch (C) {   // C is a multiple of 32, at most 512 (the MFMA conv1's limit)
#define QA_S12(ncb)                                                                                             \
    case 32 * ncb:                                                                                              \
        stem12_kernel<ncb, (ncb > 8 ? 4 : 2)><<<grid, 512, 0, s>>>(logmel, chunks, n_tiles, wfrag, w2, b2, out, tile_counter); \
        break;
        QA_S12(1) QA_S12(2) QA_S12(3) QA_S12(4) QA_S12(5) QA_S12(6) QA_S12(7) QA_S12(8)
        QA_S12(9) QA_S12(10) QA_S12(11) QA_S12(12) QA_S12(13) QA_S12(14) QA_S12(15) QA_S12(16)
#undef QA_S12
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace qa
