"""Plain fp64 CPU oracle of the AuT audio-encoder forward (TEST INFRASTRUCTURE).

Only the test-suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product path (the HIP library and its Python
binding) never calls it, and it shares no code with that path.

It is written from four web pages on Qwen3-ASR:

* [OneSpeech]  recursiveai.org OneSpeech docs for Qwen3, section "Front end and
  graph numerics" (features, chunking, PE reset, precision policy) and the
  input rules under "Low-level recognition".
* [qwenasr]    qwenasr.cpp docs/ARCHITECTURE.md, sections "Mel frontend",
  "Conv2d subsampling stem", "Windowed audio tower", "GGUF layout",
  "Mel DFT without an FFT op", "Conv2d stem", "Attention and RoPE", "Glossary".
* [M*]         mstar.stanford.edu ASR page, "Qwen3-ASR" / "Graph" paragraph
  (one packed forward, one attention segment per window of every request;
  requests up to 20 minutes).

Every function below is the plain definition: explicit cos/sin DFT matrices
(no FFT), im2col + matmul convolution, dense softmax per window, no fusion.

`oracle.resample` is the resampler to 16 kHz that [qwenasr] "Module map" puts
in front of the front end (Kaiser polyphase; its parameters are a reading).
`oracle.thinker` is the step after the encoder: the audio splice into the
prompt embeddings and the Qwen3 Thinker prefill ([qwenasr] "Qwen3 Thinker
decoder", "Prompt assembly and audio splice").

Pins (see tests/test_oracle_*.py): every function is checked against closed
forms, invariants, brute force or an independent library routine, except the
whole-forward composition, which is pinned only through its pinned parts plus
special-case weights that reduce it to a closed form (identity layers).
"""
from .encoder import *  # noqa: F401,F403
