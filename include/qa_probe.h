/*
 * qa_probe.h -- ceiling probes run by the benchmark beside the encoder
 * (libqa_probe.so, gfx950).  Not part of the encoder's path: they measure,
 * in the same run, the bf16 MFMA rate a register-only loop sustains and the
 * HBM rate of plain streaming kernels, against which the encoder kernels'
 * roofline fractions are also reported.  Plain C99; every call enqueues on
 * `stream` (a hipStream_t, NULL = null stream) and returns 0, -1 for bad
 * arguments, or -3 for a launch error.
 */
#ifndef QA_PROBE_H
#define QA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* `blocks` workgroups of 4 waves, each wave running `iters` rounds of 32
 * v_mfma_f32_16x16x32_bf16 (8 independent chains) on register operands: random bf16
 * values with full mantissas (random = 1) or all 1.0 (random = 0).  scratch:
 * a DEVICE float the kernel may write (never in practice). */
int qa_probe_mfma_bf16(void *stream, int blocks, int iters, int random, float *scratch);
/* The flops one qa_probe_mfma_bf16(blocks, iters) call performs. */
double qa_probe_mfma_flops(int blocks, int iters);
/* Read `bytes` (a multiple of 16) of DEVICE memory at src once. */
int qa_probe_read(void *stream, const void *src, int64_t bytes, float *scratch);
/* Copy `bytes` (a multiple of 16) from src to dst (DEVICE, not overlapping). */
int qa_probe_copy(void *stream, const void *src, void *dst, int64_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* QA_PROBE_H */
