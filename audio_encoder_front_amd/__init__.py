"""MI355X-native AuT audio-encoder forward (Qwen3-ASR front end) behind a C ABI.

The compute runs in libqa_encoder.so (HIP kernels for gfx950); this package is
its thin Python binding.  Importing it fails loudly if the library is not
built.
"""
from ._binding import *  # noqa: F401,F403
from ._binding import (Encoder, QAError, encode, library, make_dims, qa_abi_version, qa_encode,  # noqa: F401
                       qa_encode_noalloc,
                       qa_encode_num_tokens, qa_encoder_create, qa_encoder_enable_taps, qa_encoder_free,
                       qa_encoder_kernel_times, qa_encoder_set_max_lanes, qa_encoder_set_profiling,
                       qa_encoder_set_profiling_label,
                       qa_encoder_set_stream,
                       qa_encoder_tap, qa_last_error, Resampler, qa_resample_length, qa_resampler_create,
                       qa_resample, resample, Thinker, make_thinker_dims, qa_thinker_create,
                       qa_thinker_set_stream, qa_thinker_prefill, thinker_prefill)
