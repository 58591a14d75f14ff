"""The allocation-free entry point qa_encode_noalloc (for callers that cannot
allocate device memory) against qa_encode through the C ABI: the same
kernels on a fixed per-GPU scratch array, so the outputs must be identical
(every kernel on the path is deterministic), on two calls in a row, the
second with a smaller batch, interleaved with qa_encode calls on the
growable workspace; and a batch beyond the array is refused before any
device work."""
import numpy as np
import pytest

import synth
from parity_util import make_encoder

pytestmark = pytest.mark.gpu


def _pair(enc, clips):
    import torch
    import audio_encoder_front_amd as qa
    lens = [len(c) for c in clips]
    pcm = torch.from_numpy(np.concatenate(clips).astype(np.float32)).cuda()
    rows = sum(qa.qa_encode_num_tokens(n) for n in lens)
    qa.qa_encoder_set_stream(enc, torch.cuda.current_stream())
    a = torch.full((rows, enc.dims.output_dim), float("nan"), device="cuda")
    b = torch.full((rows, enc.dims.output_dim), float("nan"), device="cuda")
    qa.qa_encode_noalloc(enc, pcm, lens, a)
    qa.qa_encode(enc, pcm, lens, b)
    torch.cuda.synchronize()
    return a.cpu().numpy(), b.cpu().numpy()


@pytest.mark.parametrize("name,big,small", [
    ("tiny", [32000, 150000, 201], [16160]),
    ("b06_1", [480000], [16000 * 7 + 160 * 37 + 11, 0, 40000]),
    # 4,292 tokens: past the split-K sizes, so the layers run as three lanes
    ("tiny_bf16", [16000 * 300, 16000 * 30 + 160 * 13 + 3], [16000 * 100 + 7]),
])
def test_noalloc_matches_qa_encode(name, big, small):
    if name == "tiny_bf16":   # bf16 (fused stem): 4,292 tokens need about 62 MB of workspace
        import dataclasses
        dims, seed = dataclasses.replace(synth.DIMS_TINY, dtype="bf16"), 150
    else:
        dims, seed = synth.WORKLOADS[name].dims, synth.WORKLOADS[name].weight_seed
    enc = make_encoder(dims, synth.make_weights(dims, seed))
    for call, lens in enumerate((big, small)):
        clips = [synth.speech_like_clip(n, [300, call, i]) for i, n in enumerate(lens)]
        print(f"case: {name} call {call}, lengths {lens}", flush=True)
        a, b = _pair(enc, clips)
        assert a.shape[0] > 0 and np.all(np.isfinite(a))
        assert np.array_equal(a, b), f"call {call}: max |diff| {np.abs(a - b).max()}"
    enc.free()


def test_noalloc_refuses_batches_beyond_the_scratch():
    import torch
    import audio_encoder_front_amd as qa
    wl = synth.WORKLOADS["b06_1"]
    enc = make_encoder(wl.dims, synth.make_weights(wl.dims, wl.weight_seed))
    lens = [480000] * 8                      # eight 30 s clips: about 320 MiB of workspace
    pcm = torch.zeros(sum(lens), device="cuda")
    out = torch.empty((sum(qa.qa_encode_num_tokens(n) for n in lens), wl.dims.output_dim), device="cuda")
    with pytest.raises(qa.QAError) as ei:
        qa.qa_encode_noalloc(enc, pcm, lens, out)
    assert ei.value.status == qa._binding.QA_STATUS_INVALID_PARAMS and "at most" in str(ei.value)
    # and the call after the refusal works
    x = synth.speech_like_clip(48000, [301, 0])
    a, b = _pair(enc, [x])
    assert np.array_equal(a, b)
    enc.free()
