/*
 * qa_encoder.h -- C ABI of the MI355X (gfx950) AuT audio-encoder forward.
 *
 * Plain C99, no PyTorch or HIP types.  The library computes, for a packed
 * batch of 16 kHz mono clips, the Qwen3-ASR audio tower:
 *
 *   PCM -> 128-bin Whisper log-mel (n_fft 400, hop 160, periodic Hann,
 *          centered reflection, Slaney mel 0-8 kHz, floor 1e-10, log10,
 *          peak-minus-8 clip, (x+4)/4; the last STFT frame is dropped)
 *       -> per 100-frame chunk: three conv2d (k3, s2, p1) + bias + erf-GELU,
 *          flatten channel-outer / frequency-inner, conv_out Linear (no bias),
 *          plus a sinusoidal position table that restarts at every chunk
 *       -> n_layers pre-LN transformer blocks whose bidirectional attention is
 *          confined to windows of 13 * window_chunks tokens of each clip (or,
 *          with window_chunks = 0, spans each whole clip of at most 30 s)
 *       -> post LayerNorm, proj1 (d -> d), GELU, proj2 (d -> output_dim).
 *
 * Sources (pages on Qwen3-ASR):
 *   OneSpeech Qwen3 docs, "Front end and graph numerics" (features, chunks,
 *     PE reset, bf16 operator-boundary policy) and "Low-level recognition"
 *     (input rules: empty allowed, nonempty > 200 samples, nonfinite rejected);
 *   qwenasr.cpp ARCHITECTURE.md, "GGUF layout" (dims and tensor inventory),
 *     "Mel frontend", "Conv2d subsampling stem", "Windowed audio tower",
 *     "Public API" (status codes, thread-local last error, ABI version);
 *   M* ASR page, Qwen3-ASR "Graph" (one packed forward per batch, one attention
 *     segment per window of every request; requests up to 20 minutes).
 */
#ifndef QA_ENCODER_H
#define QA_ENCODER_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QA_ABI_VERSION 1

/* Status codes (qwenasr.cpp "Public API" numbering).  Functions returning
 * int return one of these. */
typedef enum qa_status {
    QA_STATUS_OK = 0,
    QA_STATUS_INVALID_PARAMS = -1,
    QA_STATUS_LOAD_FAILED = -2,
    QA_STATUS_ENCODE_FAILED = -3,
    QA_STATUS_OOM = -4
} qa_status;

/* Element type of the weights handed to qa_encoder_create, and the operand
 * precision of every contraction.  QA_DTYPE_BF16: bf16 operands rounded to
 * nearest-even at operator boundaries, fp32 accumulation, fp32 residual
 * stream, LayerNorm statistics and softmax (OneSpeech "Front end and graph
 * numerics").  The DFT and mel contractions are fp32 in both modes. */
typedef enum qa_dtype { QA_DTYPE_F32 = 0, QA_DTYPE_BF16 = 1 } qa_dtype;

/* Tap ids for qa_encoder_tap (stage outputs of the last qa_encode). */
typedef enum qa_tap {
    QA_TAP_LOG_MEL = 0,   /* normalised log-mel, fp32 [total_frames x 128], frame-major, clips in order */
    QA_TAP_STEM = 1,      /* conv_out output before PE, fp32 [total_tokens x d_model] */
    QA_TAP_LAYER0 = 2     /* residual stream after encoder layer 0, fp32 [total_tokens x d_model] */
} qa_tap;

/* Encoder dimensions; the field names follow the audio.* metadata keys of the
 * qwenasr.cpp "GGUF layout" section. */
typedef struct qa_dims {
    int abi_version;      /* must equal QA_ABI_VERSION */
    int n_mels;           /* num_mel_bins: must be 128 */
    int conv_channels;    /* downsample_hidden_size (480); multiple of 32, <= 1024 */
    int d_model;          /* multiple of 64, <= 2048 */
    int n_layers;         /* encoder_layers, >= 0 */
    int n_heads;          /* encoder_attention_heads; n_heads * head_dim == d_model */
    int head_dim;         /* must be 64 */
    int ffn_dim;          /* encoder_ffn_dim, multiple of 64 */
    int output_dim;       /* output_dim, multiple of 64 */
    int chunk_frames;     /* n_window * 2: must be 100 */
    int window_chunks;    /* n_window_infer / chunk_frames: 1..9 (8 -> 104-token windows, 9 -> 117), or 0 for
                             full-input attention: one segment per clip, clips of at most 30 s
                             (OneSpeech "Front end and graph numerics": the CPU graphs attend over
                             the whole bounded input; longer audio is chunked before encoding) */
    qa_dtype dtype;       /* QA_DTYPE_F32 or QA_DTYPE_BF16 (an int-sized enum) */
} qa_dims;

/* Weights: HOST pointers in PyTorch layouts, element type = dims.dtype
 * (QA_DTYPE_BF16: uint16 bfloat16 bit patterns; QA_DTYPE_F32: float).
 *   conv{1,2,3}_w  [C, C_in, 3 (mel), 3 (time)], C_in = 1 for conv1;  conv*_b [C]
 *   conv_out_w     [d_model, C * 16], input index c * 16 + f (no bias)
 *   per layer (arrays of n_layers pointers):
 *     ln1_w/b, ln2_w/b [d]; q/k/v/o_w [d, d]; q/k/v/o_b [d];
 *     fc1_w [ffn, d], fc1_b [ffn]; fc2_w [d, ffn], fc2_b [d]
 *   post_ln_w/b [d]; proj1_w [d, d], proj1_b [d]; proj2_w [out, d], proj2_b [out]
 * The library copies (and repacks) everything; the caller may free its
 * buffers as soon as qa_encoder_create returns. */
typedef struct qa_weights {
    const void *conv1_w, *conv1_b, *conv2_w, *conv2_b, *conv3_w, *conv3_b, *conv_out_w;
    const void *const *ln1_w, *const *ln1_b;
    const void *const *q_w, *const *q_b, *const *k_w, *const *k_b, *const *v_w, *const *v_b;
    const void *const *o_w, *const *o_b;
    const void *const *ln2_w, *const *ln2_b;
    const void *const *fc1_w, *const *fc1_b, *const *fc2_w, *const *fc2_b;
    const void *post_ln_w, *post_ln_b, *proj1_w, *proj1_b, *proj2_w, *proj2_b;
} qa_weights;

typedef struct qa_encoder qa_encoder;   /* opaque */

/* ABI version the library was built with. */
int qa_abi_version(void);

/* Thread-local message describing the most recent failure on this thread
 * (never NULL; "" if none). */
const char *qa_last_error(void);

/* Number of encoder tokens (output rows) of one clip of n_samples samples,
 * with 100-frame chunks: F = n_samples / 160 frames (OneSpeech "Front end and
 * graph numerics": sample_count / 160 frames, the final STFT frame dropped),
 * cut into chunks of 100 frames that each yield up to 13 tokens (same
 * section); a chunk of m frames yields the stem's output length, m halved
 * and rounded up three times (qwenasr.cpp "Conv2d subsampling stem": three
 * stride-2 convolutions and the after-cnn length), i.e. 13 for a full chunk
 * and ceil(m / 8) for a tail.  0 for an empty clip (OneSpeech "Low-level
 * recognition": empty audio gives an empty result); -1 (and qa_last_error
 * set) if 1 <= n_samples <= 200 (same section: nonempty audio must exceed
 * 200 samples), n_samples < 0 or n_samples > 19,200,000 (M* ASR page,
 * "Serving notes": a request holds at most 20 minutes).  Pure host
 * arithmetic. */
int64_t qa_encode_num_tokens(int64_t n_samples);

/* Validate dims and weights, copy and repack the weights into device memory
 * of the current HIP device.  Returns NULL on failure (qa_last_error says
 * why): invalid dims or NULL weight pointers -> INVALID_PARAMS semantics,
 * device allocation or copy failure -> LOAD_FAILED semantics. */
qa_encoder *qa_encoder_create(const qa_weights *w, const qa_dims *d);

/* Enqueue all later work of this handle on `hip_stream` (a hipStream_t;
 * NULL = the null stream).  A batch of more than 4,096 tokens also runs part
 * of its layers on one or two more streams the handle owns (created with it,
 * default priority), forked from and joined back into `hip_stream` by events
 * inside the call, so that later work on `hip_stream` sees every result.
 * Returns QA_STATUS_OK or INVALID_PARAMS. */
int qa_encoder_set_stream(qa_encoder *e, void *hip_stream);

/* The most streams a qa_encode call may run on, 1 to 4 (default 4): a batch
 * of more than 4,096 tokens runs, from conv3 on, as 3 parts (up to 8,192
 * tokens) or 2 parts (more), each on a stream of its own (see
 * qa_encoder_set_stream), capped at n; 1 keeps every launch on the handle's
 * stream.  The results are bit-identical either way (rows are independent in
 * every kernel and the splits fall between attention windows).  Returns
 * QA_STATUS_OK, or INVALID_PARAMS for a NULL handle or n outside 1 .. 4. */
int qa_encoder_set_max_lanes(qa_encoder *e, int n);

/* Encode a packed batch: every step of the tower above, one packed forward
 * over all clips with one attention segment per window of every clip (M* ASR
 * page, Qwen3-ASR "Graph"; qwenasr.cpp "Windowed audio tower").
 *   pcm      DEVICE pointer, float32, all clips concatenated in `lengths`
 *            order (sum(lengths) samples, 16 kHz mono).  Caller-owned.
 *   lengths  HOST array of n_clips int64 sample counts.  0 = empty clip (no
 *            tokens); otherwise 201 .. 19,200,000 (201 .. 480,000 with
 *            full-input attention, dims.window_chunks = 0): the bounds of
 *            qa_encode_num_tokens (OneSpeech "Low-level recognition", M*
 *            "Serving notes"; 30 s per OneSpeech "Front end and graph
 *            numerics" for full-input attention).
 *   n_clips  >= 0.
 *   out      DEVICE pointer, float32 [sum_i qa_encode_num_tokens(lengths[i])
 *            x output_dim], rows clip-major, then chunk, then token-in-chunk.
 *            Caller-owned; may be NULL when the total is 0.
 * All argument checks happen before any device work.  The work is enqueued
 * on the handle's stream (a batch of more than 4,096 tokens also on the
 * handle's second stream, joined back into it: see qa_encoder_set_stream);
 * the call then synchronises the handle's stream to read a device-side
 * validation flag.  Returns QA_STATUS_OK; INVALID_PARAMS for bad
 * arguments, a nonfinite sample (any sample of any clip) or a power or mel
 * value beyond float32 range in any STFT frame, the dropped final frame
 * included (OneSpeech "Low-level recognition": such inputs are rejected;
 * then `out` is unspecified); OOM if the workspace cannot grow;
 * ENCODE_FAILED on a launch/runtime error.  Mel energies are floored at
 * 1e-10 and not capped above (OneSpeech "Front end and graph numerics").
 * Calls on one handle must not overlap. */
int qa_encode(qa_encoder *e, const float *pcm, const int64_t *lengths, int n_clips, float *out);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): qa_encode with the same
 * arguments, kernels and results, but its workspace is a fixed device array
 * of QA_NOALLOC_SCRATCH_BYTES bytes per GPU, part of the library's device
 * image (each GPU the library runs on holds one until the process ends; its
 * address is taken once per device by qa_encoder_create).  The call makes no
 * device, pinned-host or event allocation: the small planning tables go to
 * the device from pageable host memory.  A batch whose workspace exceeds the
 * array is refused with INVALID_PARAMS before any device work (a 30 s clip of
 * the 0.6B bf16 shape needs about 47 MiB; the workspace grows with the total
 * audio: roughly 1.2 MiB per second at 480 stem channels, about 3.5 times
 * that for fp32 encoders and stems wider than 512 channels, which store
 * conv1's output).  Taps and
 * profiling events are not recorded by this call (qa_encoder_tap then fails
 * until the next qa_encode with taps).  Every call on one GPU, through any
 * handle, shares that GPU's array and overwrites it: calls that overlap on
 * one GPU (other streams, other threads, other handles) race and must be
 * serialised by the caller.  Returns as qa_encode; ENCODE_FAILED if the
 * array's device address could not be obtained. */
#define QA_NOALLOC_SCRATCH_BYTES (160u * 1024u * 1024u)
int qa_encode_noalloc(qa_encoder *e, const float *pcm, const int64_t *lengths, int n_clips, float *out);

/* Keep stage outputs of later qa_encode calls for qa_encoder_tap (costs one
 * extra conv_out GEMM and a copy per call, and runs the layers on the
 * handle's stream alone; the outputs are bit-identical).  enable: 0 or 1. */
int qa_encoder_enable_taps(qa_encoder *e, int enable);

/* Copy tap `tap` (QA_TAP_*) of the last qa_encode into the DEVICE buffer dst
 * (capacity in float elements), synchronously on the handle's stream.
 * Returns the element count copied, or -1 (taps disabled, unknown tap, or
 * capacity too small; qa_last_error set). */
int64_t qa_encoder_tap(qa_encoder *e, int tap, float *dst, int64_t capacity);

/* Per-kernel timing with HIP events recorded on the handle's stream around
 * every launch (0 disables; the default).  While it times every launch, every
 * kernel runs on the handle's stream alone, so that each time is that
 * kernel's own (see qa_encoder_set_profiling_label for one label).  qa_encoder_kernel_times fills up
 * to `cap` entries of: a static NUL-terminated label, the summed
 * milliseconds and the launch count accumulated since profiling was last
 * enabled, and returns the number of labels (which may exceed cap). */
int qa_encoder_set_profiling(qa_encoder *e, int enable);
int qa_encoder_kernel_times(qa_encoder *e, const char **labels, double *total_ms,
                            int64_t *launches, int cap);

/* Restrict the profiling events to the launches labelled `label` (a copy is
 * kept; NULL or "" = every launch, the default), so that a timed run carries
 * two events per such launch instead of two per kernel.  Restricted, a batch
 * of more than 4,096 tokens keeps its second stream (see
 * qa_encoder_set_stream): the first stem kernel ("stem12" or "conv1") runs
 * before the fork on the handle's stream, and a launch past the fork is timed
 * on the stream it runs on, beside the other stream's work.  Returns
 * QA_STATUS_OK or INVALID_PARAMS (NULL handle). */
int qa_encoder_set_profiling_label(qa_encoder *e, const char *label);

/* Release device memory and the handle.  NULL is a no-op. */
void qa_encoder_free(qa_encoder *e);

/* ------------------------------------------------------------------------
 * Audio splice + Qwen3 Thinker prefill, the step after the encoder
 * (qwenasr.cpp ARCHITECTURE.md "Qwen3 Thinker decoder": per layer RMSNorm ->
 * q/k/v projections -> per-head RMSNorm on q and k -> 1D NEOX RoPE (base 1e6)
 * -> causal grouped-query attention -> output projection + residual; RMSNorm
 * -> SwiGLU (silu(gate) * up) -> down projection + residual; final RMSNorm ->
 * output projection tied to the token embedding; no bias anywhere.
 * "Prompt assembly and audio splice": the prompt's id sequence is embedded,
 * then the placeholder span is overwritten with the encoder states.)
 * Readings where the page is silent: RMSNorm eps 1e-6; positions 0..T-1 of
 * each prompt (prefill from an empty cache); each prompt of a packed batch
 * attends only to itself.  Precision as for the encoder: bf16 operands at
 * operator boundaries (the q/k after norm and RoPE, v, the attention output
 * and the SwiGLU output included), fp32 accumulation, residual stream,
 * RMSNorm statistics and softmax.
 */
typedef struct qa_thinker_dims {
    int abi_version;   /* must equal QA_ABI_VERSION */
    int hidden;        /* embedding_length: multiple of 64, <= 4096 (1024 / 2048 on the page) */
    int n_layers;      /* block_count (28) */
    int n_q_heads;     /* attention.head_count (16), a multiple of n_kv_heads, <= 64 */
    int n_kv_heads;    /* attention.head_count_kv (8) */
    int head_dim;      /* attention.key_length: must be 128 */
    int ffn_dim;       /* feed_forward_length: multiple of 16 (3072 / 6144) */
    int vocab;         /* vocab_size (151936) */
    qa_dtype dtype;    /* QA_DTYPE_F32 or QA_DTYPE_BF16 */
} qa_thinker_dims;

/* HOST pointers in PyTorch layouts (Linear = [out, in]), element type = dtype.
 *   embed [vocab, hidden] (also the output projection);
 *   per layer (arrays of n_layers pointers): attn_norm, ffn_norm [hidden];
 *     q_w [n_q_heads 128, hidden]; k_w, v_w [n_kv_heads 128, hidden];
 *     q_norm, k_norm [128]; o_w [hidden, n_q_heads 128];
 *     gate_w, up_w [ffn, hidden]; down_w [hidden, ffn];
 *   out_norm [hidden].
 * Copied (and repacked) at create; the caller may free them afterwards. */
typedef struct qa_thinker_weights {
    const void *embed;
    const void *const *attn_norm, *const *q_w, *const *k_w, *const *v_w, *const *q_norm, *const *k_norm;
    const void *const *o_w, *const *ffn_norm, *const *gate_w, *const *up_w, *const *down_w;
    const void *out_norm;
} qa_thinker_weights;

typedef struct qa_thinker qa_thinker;   /* opaque */

/* Validate and copy the weights to the current HIP device.  NULL on failure
 * (qa_last_error says why). */
qa_thinker *qa_thinker_create(const qa_thinker_weights *w, const qa_thinker_dims *d);

/* Enqueue later work of this handle on hip_stream (NULL = null stream). */
int qa_thinker_set_stream(qa_thinker *t, void *hip_stream);

/* Prefill a packed batch of n_prompts prompts.
 *   ids            HOST int32 [sum lengths]: token ids, prompts in order (ids
 *                  inside an audio span are ignored; others must be < vocab).
 *   lengths        HOST int64 [n_prompts], each 1..65536 (context_length).
 *   audio          DEVICE float32 [sum audio_counts x hidden]: the encoder
 *                  states spliced into the prompts, in prompt order (e.g. the
 *                  output of qa_encode with output_dim == hidden).  Caller-owned.
 *   audio_offsets, audio_counts
 *                  HOST int64 [n_prompts]: the placeholder span of each prompt
 *                  (0 <= offset, offset + count <= length).
 *   hidden_out     DEVICE float32 [sum lengths x hidden] or NULL: the hidden
 *                  states after the final RMSNorm.
 *   logits_out     DEVICE float32 [n_prompts x vocab] or NULL: the logits of
 *                  each prompt's last token.
 * Argument checks happen before any device work; the call synchronises the
 * handle's stream before it returns.  Returns QA_STATUS_OK, INVALID_PARAMS,
 * OOM or ENCODE_FAILED (launch error).  Calls on one handle must not overlap. */
int qa_thinker_prefill(qa_thinker *t, const int32_t *ids, const int64_t *lengths, int n_prompts,
                       const float *audio, const int64_t *audio_offsets, const int64_t *audio_counts,
                       float *hidden_out, float *logits_out);

/* Release device memory and the handle.  NULL is a no-op. */
void qa_thinker_free(qa_thinker *t);

/* ------------------------------------------------------------------------
 * Resampling to 16 kHz, the step in front of the front end (qwenasr.cpp
 * ARCHITECTURE.md "Upstream model": any input is resampled to 16 kHz mono
 * before the frontend; "Module map": a Kaiser polyphase resampler).  The page
 * does not give the filter; this library's reading:
 *   up / down = 16000 / rate_in reduced by their gcd; a linear-phase low-pass
 *   FIR of 2 half + 1 taps, half = 10 max(up, down), cut-off 1 / max(up, down)
 *   of the upsampled Nyquist frequency, Kaiser window beta = 5, unit DC gain,
 *   scaled by up; output sample n is the filtered zero-stuffed input at
 *   upsampled index n down (no delay), zeros outside the clip.  (The same
 *   filter as scipy.signal.resample_poly(x, up, down, window=("kaiser", 5)).)
 */
typedef struct qa_resampler qa_resampler;   /* opaque: the filter table on the device */

/* Output length for n_in samples at rate_in Hz: ceil(n_in up / down).
 * -1 (qa_last_error set) if n_in < 0 or rate_in is outside 1000..768000. */
int64_t qa_resample_length(int64_t n_in, int rate_in);

/* Design the filter for rate_in (1000..768000 Hz) and copy its polyphase
 * table to the current HIP device.  NULL on failure (qa_last_error says why). */
qa_resampler *qa_resampler_create(int rate_in);

/* Resample one mono clip: in = DEVICE float32 [n_in], out = DEVICE float32
 * [qa_resample_length(n_in, rate_in)], both caller-owned, not overlapping.
 * Enqueued on hip_stream (a hipStream_t; NULL = null stream), no
 * synchronisation.  Returns QA_STATUS_OK, INVALID_PARAMS (NULL handle or
 * pointers, n_in < 0) or ENCODE_FAILED (launch error). */
int qa_resample(qa_resampler *r, void *hip_stream, const float *in, int64_t n_in, float *out);

/* Release the table and the handle.  NULL is a no-op. */
void qa_resampler_free(qa_resampler *r);

#ifdef __cplusplus
}
#endif

#endif /* QA_ENCODER_H */
