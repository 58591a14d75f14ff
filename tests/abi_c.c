/* Plain C99 consumer of the public header: exercises the early-return paths
 * of every entry point.  Needs no GPU and no weights.  Exit status 0 = pass. */
#include <stdio.h>
#include <string.h>

#include "qa_encoder.h"

static int fails = 0;
#define CHECK(cond)                                                   \
    do {                                                              \
        if (!(cond)) {                                                \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond); \
            fails++;                                                  \
        }                                                             \
    } while (0)

int main(void) {
    qa_dims d;
    qa_weights w;
    int64_t lens[2];
    const char *labels[4];
    double ms[4];
    int64_t cnt[4];

    memset(&w, 0, sizeof w);
    CHECK(qa_abi_version() == QA_ABI_VERSION);
    CHECK(qa_last_error() != NULL);

    /* token counts */
    CHECK(qa_encode_num_tokens(0) == 0);
    CHECK(qa_encode_num_tokens(32000) == 26);
    CHECK(qa_encode_num_tokens(480000) == 390);
    CHECK(qa_encode_num_tokens(19200000) == 15600);
    CHECK(qa_encode_num_tokens(201) == 1);
    CHECK(qa_encode_num_tokens(200) == -1);
    CHECK(strlen(qa_last_error()) > 0);
    CHECK(qa_encode_num_tokens(-5) == -1);
    CHECK(qa_encode_num_tokens(19200001) == -1);

    /* create: bad dims are rejected before any device work */
    memset(&d, 0, sizeof d);
    d.abi_version = QA_ABI_VERSION + 1;
    CHECK(qa_encoder_create(&w, &d) == NULL);
    CHECK(strstr(qa_last_error(), "abi_version") != NULL);
    d.abi_version = QA_ABI_VERSION;
    d.n_mels = 128; d.conv_channels = 480; d.d_model = 1024; d.n_layers = 24; d.n_heads = 16;
    d.head_dim = 64; d.ffn_dim = 4096; d.output_dim = 2048; d.chunk_frames = 100; d.window_chunks = 8;
    d.dtype = QA_DTYPE_BF16;
    CHECK(qa_encoder_create(NULL, &d) == NULL);
    CHECK(qa_encoder_create(&w, NULL) == NULL);
    CHECK(qa_encoder_create(&w, &d) == NULL);           /* NULL weight pointers */
    d.n_heads = 15;
    CHECK(qa_encoder_create(&w, &d) == NULL);
    d.n_heads = 16; d.n_mels = 80;
    CHECK(qa_encoder_create(&w, &d) == NULL);
    d.n_mels = 128; d.window_chunks = 9;
    CHECK(qa_encoder_create(&w, &d) == NULL);
    d.window_chunks = 8; d.dtype = 7;
    CHECK(qa_encoder_create(&w, &d) == NULL);

    /* handle-less calls */
    lens[0] = 32000; lens[1] = 0;
    CHECK(qa_encode(NULL, NULL, lens, 2, NULL) == QA_STATUS_INVALID_PARAMS);
    CHECK(qa_encoder_set_stream(NULL, NULL) == QA_STATUS_INVALID_PARAMS);
    CHECK(qa_encoder_set_max_lanes(NULL, 1) == QA_STATUS_INVALID_PARAMS);
    CHECK(qa_encoder_enable_taps(NULL, 1) == QA_STATUS_INVALID_PARAMS);
    CHECK(qa_encoder_set_profiling(NULL, 1) == QA_STATUS_INVALID_PARAMS);
    CHECK(qa_encoder_tap(NULL, QA_TAP_LOG_MEL, NULL, 0) == -1);
    CHECK(qa_encoder_kernel_times(NULL, labels, ms, cnt, 4) == -1);
    qa_encoder_free(NULL);

    /* resampler: argument checks only (no device work) */
    CHECK(qa_resample_length(44100, 44100) == 16000);
    CHECK(qa_resample_length(3000, 44100) == 1089);
    CHECK(qa_resample_length(0, 8000) == 0);
    CHECK(qa_resample_length(-1, 44100) == -1);
    CHECK(qa_resample_length(100, 999) == -1);
    CHECK(qa_resampler_create(999) == NULL);
    CHECK(qa_resampler_create(768001) == NULL);
    CHECK(qa_resample(NULL, NULL, NULL, 10, NULL) == QA_STATUS_INVALID_PARAMS);
    qa_resampler_free(NULL);

    /* Thinker prefill: argument checks only */
    {
        qa_thinker_dims td;
        qa_thinker_weights tw;
        int32_t tid[2] = {1, 2};
        int64_t tl[1] = {2}, to[1] = {0}, tc[1] = {0};
        memset(&td, 0, sizeof td);
        memset(&tw, 0, sizeof tw);
        td.abi_version = QA_ABI_VERSION; td.hidden = 2048; td.n_layers = 28; td.n_q_heads = 16; td.n_kv_heads = 8;
        td.head_dim = 128; td.ffn_dim = 6144; td.vocab = 151936; td.dtype = QA_DTYPE_BF16;
        CHECK(qa_thinker_create(&tw, &td) == NULL);          /* NULL weight pointers */
        CHECK(qa_thinker_create(NULL, &td) == NULL);
        td.head_dim = 64;
        CHECK(qa_thinker_create(&tw, &td) == NULL);
        CHECK(strstr(qa_last_error(), "head_dim") != NULL);
        td.head_dim = 128; td.n_kv_heads = 5;
        CHECK(qa_thinker_create(&tw, &td) == NULL);
        CHECK(qa_thinker_prefill(NULL, tid, tl, 1, NULL, to, tc, NULL, NULL) == QA_STATUS_INVALID_PARAMS);
        CHECK(qa_thinker_set_stream(NULL, NULL) == QA_STATUS_INVALID_PARAMS);
        qa_thinker_free(NULL);
    }

    if (fails) return 1;
    printf("abi_c: all checks passed\n");
    return 0;
}
