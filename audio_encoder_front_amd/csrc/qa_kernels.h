// Host-side launch interface of the gfx950 kernels (no device code here).
// Every function enqueues on `s` and returns hipGetLastError() of its launch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qa {

typedef __bf16 bf16;

// Per-clip bookkeeping: first sample in the packed PCM, sample count, and the
// global row of the clip's first log-mel frame.
struct ClipInfo {
    int64_t sample_off;
    int32_t len;
    int32_t frame_row0;
};

// A front-end tile: up to 64 consecutive STFT frames of one clip.  A clip of
// L samples has floor(L/160) kept frames plus the final frame, which its last
// tile computes (so every sample is read and its power checked) but does not
// store.
struct FrontTile {
    int32_t clip;
    int32_t frame0;      // first frame, counted within the clip
    int32_t nframes;     // 1..64, kept and final frames
    int32_t pad_;
};

// A 100-frame conv chunk: global log-mel row of its first frame and the
// number of real frames (the rest of the 100 are zeros).
struct ChunkInfo {
    int32_t frame_row0;
    int32_t m;
};

constexpr int kMels = 128;
constexpr int kFrontFrames = 64;     // frames per front-end tile
constexpr int kBinChunks = 13;       // 13 x 16 = 208 >= 201 DFT bins
constexpr int kChunk = 100;          // frames per conv chunk
constexpr int kChunkTok = 13;        // tokens per full chunk
constexpr int kMaxWindow = 128;      // attention kernel capacity (tokens per window)
constexpr int kConvCB = 32;          // input-channel block of the conv2/conv3 K order

// Sets the thread-local message returned by qa_last_error.
void set_error_message(const char* msg);

// ---- front end
// clip_key[i] = the key of -inf (per-clip maxima start there); flag[0] = 0
// (the nonfinite-input flag) and flag[1] = 0 (the fused stem's tile counter).
hipError_t init_flags(hipStream_t s, int* clip_key, int n_clips, int* flag);
// basis: the Hann-windowed cos / sin DFT basis as bf16 MFMA A fragments, each
// fp32 value split exactly into hi + mid + lo: [13 bin chunks][13 K blocks of
// 32 samples][cos, sin][hi, mid, lo][64 lanes] x 8 bf16 (lane l: bin
// 16 chunk + l % 16, samples 32 kb + 8 (l / 16) .. + 7; zero past bin 200 and
// sample 399).
// melw / melb0: mel band m weighs power bins melb0[m] .. + kMelTaps - 1 with
// melw[m][0 .. kMelTaps - 1] (zero past the filter's support).
constexpr int kDftKBlocks = 13;
constexpr int kMelTaps = 12;
hipError_t frontend(hipStream_t s, const float* pcm, const ClipInfo* clips, const FrontTile* tiles,
                    int n_tiles, const uint4* basis, const float* melw, const int* melb0,
                    float* logmel, int* clip_key, int* flag);
hipError_t normalize(hipStream_t s, float* logmel, const ClipInfo* clips, const FrontTile* tiles,
                     int n_tiles, const int* clip_key);

// ---- stem
template <typename T>
hipError_t conv1(hipStream_t s, const float* logmel, const ChunkInfo* chunks, int n_chunks,
                 const float* w9c, const float* bias, int C, T* out);
// conv1 and conv2 in one kernel (bf16, C a multiple of 32 and at most 512):
// conv2's output NHWC [n_chunks][32][25][C] from the normalised log-mel, with
// conv1 as bf16 MFMA fragments wfrag[C / 16][64][8] (3-way split input, bias in
// K slot 27) and conv2's weights w2 [C][9C] (K order as conv3x3s2) and bias b2;
// conv1's output is never stored.
constexpr int kStemFusedMaxC = 512;
// tile_counter: an int that is 0 when the kernel starts (512-channel tiles
// hand out their tiles from it).
hipError_t stem12(hipStream_t s, const float* logmel, const ChunkInfo* chunks, int n_chunks, const uint4* wfrag,
                  const bf16* w2, const float* b2, int C, bf16* out, int* tile_counter);
// conv 3x3 stride 2 pad 1 as an implicit GEMM over NHWC input [n_chunks][Hin][Win][C];
// weights [C_out][9*C]
// with k = (ci/32)*288 + (a*3+b)*32 + ci%32.  Output is NHWC
// [n_chunks][Hout][Wout][C] (time_major=false) or [n_chunks][Wout][Hout][C].
template <typename T>
hipError_t conv3x3s2(hipStream_t s, const T* in, int n_chunks, int Hin, int Win, int C,
                     const T* w, const float* bias, T* out, bool time_major, int lanes = 1);
// x[t][:] = A[src[t]][:] . Wout^T + pe[src[t] % 13][:]  (fp32), and optionally
// tap[t][:] without the PE.
// part (part_elems floats, may be null): workspace for split-K, used when
// the batch is too small to fill the GPU with tiles.
// lanes (all GEMMs here): how many launches of this shape the caller runs side
// by side on separate streams; the 256 x 256 tiling is taken when lanes times
// its tile count fills the GPU.  It changes the tiling only, never a value.
// after (conv_out, gemm_bias_resid; may be null): the LayerNorm that follows
// (gamma g, beta b, output out [rows][N]).  When the GEMM splits K its
// reduction also writes out = LayerNorm(x), bit-identical to layernorm on
// the new x, and sets done; otherwise done is left false and the caller runs
// layernorm itself.
template <typename T>
struct LnAfter {
    const float* g;
    const float* b;
    T* out;
    bool done;
};
template <typename T>
hipError_t conv_out(hipStream_t s, const T* a, const int* src, int n_tok, int K, const T* w, int N,
                    const float* pe, float* x, float* tap, float* part = nullptr, size_t part_elems = 0,
                    int lanes = 1, LnAfter<T>* after = nullptr);

// ---- dense GEMMs: out[M][N] = A[M][K] . W[N][K]^T + bias
template <typename T>
hipError_t gemm_bias(hipStream_t s, const T* a, int M, int K, const T* w, int N, const float* bias,
                     T* out, bool gelu, int lanes = 1);
// x += A . W^T + bias.  part (part_elems floats, may be null): workspace for
// split-K, used when the batch is too small to fill the GPU with tiles.
template <typename T>
hipError_t gemm_bias_resid(hipStream_t s, const T* a, int M, int K, const T* w, int N,
                           const float* bias, float* x, float* part = nullptr, size_t part_elems = 0,
                           int lanes = 1, LnAfter<T>* after = nullptr);
template <typename T>
hipError_t gemm_bias_f32(hipStream_t s, const T* a, int M, int K, const T* w, int N,
                         const float* bias, float* out, int lanes = 1);

// ---- LayerNorm (fp32 in, T out) and windowed attention
template <typename T>
hipError_t layernorm(hipStream_t s, const float* x, int M, int d, const float* g, const float* b, T* out);
// Attention over independent segments [cu[i], cu[i+1]) of at most max_len
// tokens (any length; segments over 128 tokens take the online-softmax path).
template <typename T>
hipError_t attention(hipStream_t s, const T* qkv, const int* cu_seqlens, int n_windows, int n_heads,
                     int d, int max_len, T* out);

// ---- Thinker prefill (audio splice, RMSNorm, QK-norm + RoPE, causal GQA)
constexpr int kThinkerSiteQKV = 10, kThinkerSiteOProj = 11, kThinkerSiteGateUp = 12, kThinkerSiteDown = 13;
template <typename T>
hipError_t embed_splice(hipStream_t s, const T* embed, const float* audio, const int* src, int M, int H, float* x);
template <typename T>
hipError_t rmsnorm(hipStream_t s, const float* x, int M, int H, const float* g, float eps, T* out);
template <typename T>
hipError_t qknorm_rope(hipStream_t s, T* qkv, int M, int hq, int hkv, const int* pos, const float* qg,
                       const float* kg, const float2* cs, float eps);
template <typename T>
hipError_t thinker_attention(hipStream_t s, const T* qkv, const int* cu, int n_prompts, int hq, int hkv,
                             int max_len, T* out);
// site kThinkerSiteQKV: out_t = a . w^T (no bias); kThinkerSiteOProj / Down: x += a . w^T;
// kThinkerSiteGateUp: out_t[M][N/2] = silu(gate) * up with w rows interleaved in 16-row blocks.
template <typename T>
hipError_t thinker_gemm(hipStream_t s, int site, const T* a, int M, int K, const T* w, int N,
                        const float* zero, T* out_t, float* x);
// out[i][:] = a[rows[i]] . w^T (fp32), i < n_rows.
template <typename T>
hipError_t thinker_logits(hipStream_t s, const T* a, const int* rows, int n_rows, int K, const T* w, int N,
                          const float* zero, float* out);

}  // namespace qa
