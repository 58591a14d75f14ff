"""GPU parity: the HIP library (through the C ABI) against the fp64 oracle on
the same seeded inputs.  Tolerances: normalised log-mel max-abs 1e-4 (fp32
encoder) / 2e-3 (bf16), per-window relative L2 of the output 1e-4 / 1e-2; the
pre-PE stem output and the layer-0 residual are checked per window too."""
import numpy as np
import pytest

import oracle as O
import synth
from parity_util import compare, make_encoder, run_gpu, tail_reading_check, workload_inputs

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module")
def tiny():
    wl, clips, w = workload_inputs("tiny")
    enc = make_encoder(wl.dims, w)
    yield wl, clips, w, enc
    enc.free()


def test_tiny_workload_full_parity(tiny):
    wl, clips, w, enc = tiny
    _print("case: tiny workload, 1 clip x 32000 samples, fp32")
    out, taps = run_gpu(enc, clips, taps=True)
    rep = compare(wl.dims, w, clips, out, taps)
    _print("tiny", rep)


def test_tiny_encoder_ragged_batch(tiny):
    # several front-end tiles, two GEMM row tiles, tail chunks of 1, 25, 75
    # and 99 frames, an empty clip, a 1-frame clip and a ragged 2-window clip
    wl, _, w, enc = tiny
    lens = [201, 16160, 0, 15999, 100000, 140000, 16000 * 3 + 160 * 99 + 37]
    clips = [synth.speech_like_clip(n, [77, i]) for i, n in enumerate(lens)]
    _print("case: tiny encoder ragged batch", lens)
    out, taps = run_gpu(enc, clips, taps=True)
    assert out.shape[0] == sum(O.clip_num_tokens(n) for n in lens)
    rep = compare(wl.dims, w, clips, out, taps)
    _print("ragged", rep)
    # tails of 1, 25 and 75 frames end in a row where the readings differ
    rows = tail_reading_check(wl.dims, w, clips, taps)
    _print("tail rows (clip, frames, vs A, vs B)", rows)
    assert {m for _, m, _, _ in rows} >= {1, 25, 75}


def test_tiny_encoder_silence_and_tone_edges(tiny):
    wl, _, w, enc = tiny
    t = np.arange(48000) / 16000.0
    clips = [np.zeros(20000, np.float32),                                   # digital silence -> -1.5
             (0.3 * np.sin(2 * np.pi * 440 * t)).astype(np.float32),         # noise-free tone
             synth.speech_like_clip(64000, [78, 0])]
    clips[2][10000:30000] = 0.0                                             # clamp active
    _print("case: silence / tone / gap")
    out, taps = run_gpu(enc, clips, taps=True)
    nf0 = 20000 // 160
    # log10 of the 1e-10 floor in fp32 is -10 to within an ulp: -1.5 +- 1e-6
    assert np.abs(taps["log_mel"][:nf0] + 1.5).max() <= 1e-6
    compare(wl.dims, w, clips, out, taps)


def test_rejects_nonfinite_and_short_clips(tiny):
    import torch
    import audio_encoder_front_amd as qa
    wl, _, w, enc = tiny
    x = synth.speech_like_clip(8000, [79, 0])
    x[1234] = np.nan
    pcm = torch.from_numpy(x).cuda()
    out = torch.empty((qa.qa_encode_num_tokens(8000), 256), device="cuda")
    with pytest.raises(qa.QAError) as ei:
        qa.qa_encode(enc, pcm, [8000], out)
    assert ei.value.status == qa._binding.QA_STATUS_INVALID_PARAMS
    x[1234] = 1e25                      # power beyond float32 range
    pcm = torch.from_numpy(x).cuda()
    with pytest.raises(qa.QAError):
        qa.qa_encode(enc, pcm, [8000], out)
    with pytest.raises(qa.QAError):
        qa.qa_encode(enc, pcm[:200], [200], out)
    # the handle still works after rejected calls
    x = synth.speech_like_clip(8000, [79, 1])
    res, _ = run_gpu(enc, [x])
    compare(wl.dims, w, [x], res, None)


def test_rejects_trailing_nan_and_power_overflow_outside_the_bands(tiny):
    """Every sample is checked, also those that only the dropped final STFT
    frame reads (L mod 160 >= 41), and every power bin, also bin 0 which no
    mel band weighs (OneSpeech "Low-level recognition": nonfinite samples and
    power beyond float32 are rejected)."""
    import torch
    import audio_encoder_front_amd as qa
    wl, _, w, enc = tiny
    L = 160 * 50 + 150
    out = torch.empty((qa.qa_encode_num_tokens(L), 256), device="cuda")
    for case in ("nan at L-1", "nan at 160F+40", "dc 1e17"):
        x = synth.speech_like_clip(L, [9, 4]).astype(np.float64)
        if case == "nan at L-1":
            x[L - 1] = np.nan
        elif case == "nan at 160F+40":
            x[160 * 50 + 40] = np.nan
        else:
            x = x + 1e17          # P_0 = 4e38 > float32 max; every mel band finite
        _print("case:", case)
        with pytest.raises(O.InvalidInput):
            O.log_mel(x)
        pcm = torch.from_numpy(x.astype(np.float32)).cuda()
        with pytest.raises(qa.QAError) as ei:
            qa.qa_encode(enc, pcm, [L], out)
        assert ei.value.status == qa._binding.QA_STATUS_INVALID_PARAMS
    # the sample just before the trailing range is read by a kept frame
    x = synth.speech_like_clip(L, [9, 4])
    x[160 * 50 + 39] = np.inf
    pcm = torch.from_numpy(x).cuda()
    with pytest.raises(qa.QAError):
        qa.qa_encode(enc, pcm, [L], out)
    # and a clean clip of that length still encodes
    x = synth.speech_like_clip(L, [9, 5])
    res, taps = run_gpu(enc, [x], taps=True)
    compare(wl.dims, w, [x], res, taps)


def test_loud_clip_keeps_mel_energies_above_1e30(tiny):
    """Only the 1e-10 floor applies (no 1e30 cap): a clip scaled by 1e15 has
    mel energies up to ~1e33, accepted and matching the oracle's log-mel."""
    wl, _, w, enc = tiny
    x = synth.speech_like_clip(16000 * 3 + 77, [9, 6]).astype(np.float64) * 1e15
    assert O.log_mel_raw(x).max() > 30.5          # mel energies past 1e30
    _print("case: loud clip x 1e15")
    res, taps = run_gpu(enc, [x.astype(np.float32)], taps=True)
    rep = compare(wl.dims, w, [x.astype(np.float32)], res, taps)
    _print("loud", rep)


def test_repeated_calls_shrink_and_grow_and_are_deterministic(tiny):
    wl, _, w, enc = tiny
    big = [synth.speech_like_clip(n, [80, i]) for i, n in enumerate((150000, 33333))]
    small = [synth.speech_like_clip(9000, [81, 0])]
    a, _ = run_gpu(enc, big)
    b, _ = run_gpu(enc, small)
    c, _ = run_gpu(enc, big)
    assert np.array_equal(a, c)
    compare(wl.dims, w, small, b, None)


def test_empty_batch(tiny):
    wl, _, w, enc = tiny
    out, _ = run_gpu(enc, [np.zeros(0, np.float32), np.zeros(0, np.float32)])
    assert out.shape == (0, 256)


@pytest.fixture(scope="module")
def b06():
    wl, clips, w = workload_inputs("b06_1")
    enc = make_encoder(wl.dims, w)
    yield wl, clips, w, enc
    enc.free()


def test_b06_single_30s_full_parity(b06):
    wl, clips, w, enc = b06
    _print("case: 0.6B bf16, one 30 s clip")
    out, taps = run_gpu(enc, clips, taps=True)
    rep = compare(wl.dims, w, clips, out, taps)
    _print("b06_1", rep)


def test_b06_packed_32_clips(b06):
    wl, _, w, enc = b06
    wl32 = synth.WORKLOADS["b06_32"]
    clips = synth.make_audio(wl32)
    _print("case: 0.6B bf16, 32 clips U(1,30) s")
    out, taps = run_gpu(enc, clips, taps=True)
    # without taps the batch (5,986 tokens) runs as three lanes by default,
    # as two with at most 2 streams, as one with 1: all bit-identical
    import audio_encoder_front_amd as qa
    out3, _ = run_gpu(enc, clips)
    assert np.array_equal(out3, out)
    for n in (2, 1):
        qa.qa_encoder_set_max_lanes(enc, n)
        outn, _ = run_gpu(enc, clips)
        assert np.array_equal(outn, out), f"max lanes {n}"
    qa.qa_encoder_set_max_lanes(enc, 4)
    for bad in (0, 5):
        with pytest.raises(qa.QAError):
            qa.qa_encoder_set_max_lanes(enc, bad)
    # the bench's timed steps: events around the fused stem only, lanes kept
    # (the stem runs once per encode, before the fork)
    qa.qa_encoder_set_profiling_label(enc, "stem12")
    qa.qa_encoder_set_profiling(enc, True)
    outp, _ = run_gpu(enc, clips)
    times = qa.qa_encoder_kernel_times(enc)
    qa.qa_encoder_set_profiling(enc, False)
    qa.qa_encoder_set_profiling_label(enc, None)
    assert np.array_equal(outp, out)
    assert set(times) == {"stem12"} and times["stem12"][1] == 1 and times["stem12"][0] > 0
    # every window of every clip (73), per window and per row, and the
    # log-mel of every clip
    rep = compare(wl.dims, w, clips, out, taps, progress="b06_32")
    assert rep["windows_checked"] == 73
    _print("b06_32", rep)
    rows = tail_reading_check(wl.dims, w, clips, taps)
    _print("b06_32 tail rows", len(rows))
    assert len(rows) >= 8


def test_b06_window_boundaries_and_tails(b06):
    wl, _, w, enc = b06
    # 104 tokens exactly (8 chunks), 105 tokens (8 chunks + 1-frame tail),
    # 9 chunks (117 tokens, a ragged 13-token second window), 1 frame
    lens = [800 * 160, 801 * 160 + 5, 900 * 160, 201]
    clips = [synth.speech_like_clip(n, [82, i]) for i, n in enumerate(lens)]
    out, taps = run_gpu(enc, clips, taps=True)
    assert out.shape[0] == 104 + 105 + 117 + 1
    compare(wl.dims, w, clips, out, taps)
    rows = tail_reading_check(wl.dims, w, clips, taps)
    assert {m for _, m, _, _ in rows} == {1}


@pytest.fixture(scope="module")
def b17():
    wl = synth.WORKLOADS["b17_20m"]
    w = synth.make_weights(wl.dims, wl.weight_seed)
    enc = make_encoder(wl.dims, w)
    yield wl, w, enc
    enc.free()


def test_b17_twenty_minutes_every_window(b17):
    wl, w, enc = b17
    clips = synth.make_audio(wl)
    _print("case: 1.7B bf16, one 20-minute clip (every window)")
    out, taps = run_gpu(enc, clips, taps=True)
    assert out.shape == (15600, 2048)
    assert np.all(np.isfinite(out))
    out2, _ = run_gpu(enc, clips)        # two lanes (no taps): bit-identical
    assert np.array_equal(out2, out)
    rep = compare(wl.dims, w, clips, out, taps, progress="b17_20m")
    assert rep["windows_checked"] == 150
    _print("b17_20m", rep)


def test_b17_packed_16_clips_every_window(b17):
    wl, w, enc = b17
    clips = synth.make_audio(synth.WORKLOADS["b17_16"])
    _print("case: 1.7B bf16, 16 clips logU(10,300) s (every window)")
    out, taps = run_gpu(enc, clips, taps=True)
    assert out.shape == (21162, 2048)
    out2, _ = run_gpu(enc, clips)        # two lanes (no taps): bit-identical
    assert np.array_equal(out2, out)
    rep = compare(wl.dims, w, clips, out, taps, progress="b17_16")
    assert rep["windows_checked"] == 213
    _print("b17_16", rep)
    rows = tail_reading_check(wl.dims, w, clips, taps)
    _print("b17_16 tail rows", rows)
    assert len(rows) >= 8


def test_lanes_fp32(tiny):
    """Batches past the split-K sizes run conv_out, the layers and the
    projection as parts on separate streams, split at the windows whose
    starts are nearest the even split points: three parts for this batch of
    4,292 tokens (at tokens 1,456 and 2,912, inside the 300 s clip), two
    when the handle allows at most 2 streams (token 2,184); with taps on
    they run as one.  All runs are bit-identical, and the windows at the
    splits, the ends and the second clip match the oracle."""
    import audio_encoder_front_amd as qa
    wl, _, w, enc = tiny
    lens = [16000 * 300, 16000 * 30 + 160 * 13 + 3]
    clips = [synth.speech_like_clip(n, [97, i]) for i, n in enumerate(lens)]
    _print("case: tiny fp32, lanes", lens)
    out3, _ = run_gpu(enc, clips)
    qa.qa_encoder_set_max_lanes(enc, 2)
    out2, _ = run_gpu(enc, clips)
    qa.qa_encoder_set_max_lanes(enc, 4)
    out, taps = run_gpu(enc, clips, taps=True)
    assert out.shape[0] == 4292
    assert np.array_equal(out3, out)
    assert np.array_equal(out2, out)
    rep = compare(wl.dims, w, clips, out, taps,
                  windows_per_clip=lambda ci, nw: [0, 12, 13, 14, 19, 20, 21, 22, 26, 27, 28, nw - 1]
                  if ci == 0 else range(nw))
    _print("lanes", rep)


@pytest.mark.parametrize("base,window_chunks", [("tiny", 9), ("tiny", 1), ("b06", 9), ("b06", 1)])
def test_other_window_sizes(base, window_chunks):
    """Attention windows of 9 chunks (117 tokens: 8 key tiles, whose last P.V
    step is a full 32-key step) and of 1 chunk (13 tokens: one query tile,
    mostly zero key rows), fp32 miniature (one head per workgroup) and 0.6B
    bf16 (14 heads: two per workgroup, direct-to-LDS K/V)."""
    import dataclasses
    dims = dataclasses.replace(synth.DIMS_TINY if base == "tiny" else synth.DIMS_06B, window_chunks=window_chunks)
    w = synth.make_weights(dims, 110 + window_chunks)
    enc = make_encoder(dims, w)
    lens = [480000, 12 * 16000 + 77, 16000 * 9 + 160 * 40]
    clips = [synth.speech_like_clip(n, [93, i]) for i, n in enumerate(lens)]
    _print(f"case: {base} {dims.dtype}, {window_chunks}-chunk windows", lens)
    out, taps = run_gpu(enc, clips, taps=True)
    rep = compare(dims, w, clips, out, taps)
    _print(f"{base} window {window_chunks}", rep)
    enc.free()


def test_bf16_wide_stem_valu_conv1():
    """bf16 with 544 stem channels (> 512): conv1 takes the VALU kernel with an
    NHWC output and conv2 runs as an implicit GEMM over it, instead of the
    fused conv1-in-conv2 kernel."""
    import dataclasses
    dims = dataclasses.replace(synth.DIMS_TINY, conv_channels=544, dtype="bf16")
    w = synth.make_weights(dims, 120)
    enc = make_encoder(dims, w)
    lens = [16000 * 10 + 160 * 37 + 11, 16000 * 2]
    clips = [synth.speech_like_clip(n, [94, i]) for i, n in enumerate(lens)]
    _print("case: tiny bf16, 544 stem channels", lens)
    out, taps = run_gpu(enc, clips, taps=True)
    rep = compare(dims, w, clips, out, taps)
    _print("wide stem", rep)
    enc.free()


@pytest.mark.parametrize("channels", [64, 288, 416, 480, 512])
def test_bf16_fused_stem_widths(channels):
    """The fused conv1-in-conv2 kernel at other stem widths: 2 slabs and one
    partly filled 256-channel tile (64); 512-channel tiles of which one
    32-channel group (288), 416 channels, or 480 (the 0.6B / 1.7B stem) are
    real and the other waves' rows padding; the widest stem it takes, every
    row real and 16 slabs (512).  Clip lengths give tail chunks and tiles at
    both ends of a chunk's 25 time columns."""
    import dataclasses
    dims = dataclasses.replace(synth.DIMS_TINY, conv_channels=channels, dtype="bf16")
    w = synth.make_weights(dims, 140 + channels)
    enc = make_encoder(dims, w)
    lens = [16000 * 4 + 160 * 61 + 7, 16000 + 160 * 3]
    clips = [synth.speech_like_clip(n, [96, i]) for i, n in enumerate(lens)]
    _print(f"case: tiny bf16, {channels} stem channels", lens)
    out, taps = run_gpu(enc, clips, taps=True)
    rep = compare(dims, w, clips, out, taps)
    _print("fused stem width", rep)
    enc.free()


@pytest.mark.parametrize("channels", [288, 480, 512])
def test_bf16_fused_stem_many_tiles_per_workgroup(channels):
    """The 512-channel fused stem over more pixel tiles than the GPU has CUs
    (83 chunks, 415 tiles): its workgroups walk several tiles, taking them
    from the tile counter, and set up each next tile inside the current one
    (B operands and first patch in the last slab, the log-mel window two tiles
    ahead), across clip boundaries and tail chunks."""
    import dataclasses
    dims = dataclasses.replace(synth.DIMS_TINY, conv_channels=channels, dtype="bf16")
    w = synth.make_weights(dims, 150 + channels)
    enc = make_encoder(dims, w)
    lens = [16000 * 47 + 160 * 29 + 3, 16000 * 30, 16000 * 4 + 160 * 51]
    clips = [synth.speech_like_clip(n, [97, i]) for i, n in enumerate(lens)]
    _print(f"case: tiny bf16, {channels} stem channels, many tiles", lens)
    out, taps = run_gpu(enc, clips, taps=True)
    rep = compare(dims, w, clips, out, taps)
    _print("fused stem many tiles", rep)
    enc.free()


@pytest.mark.parametrize("d_model,n_heads,ffn_dim", [(64, 1, 64), (128, 2, 192)])
def test_bf16_short_k_gemms(d_model, n_heads, ffn_dim):
    """bf16 encoders so narrow that the GEMMs run 1 to 3 K stages of 64
    values (q/k/v, O-proj, FC1, FC2, proj1, proj2 with K = d or FFN): the
    A-operand ring then fetches stages past the end of K (zeros) from its
    first iteration on; conv_out (K = 32 x 16 = 512, 8 stages) splits K for
    this small batch."""
    import dataclasses
    dims = dataclasses.replace(synth.DIMS_TINY, d_model=d_model, n_heads=n_heads, ffn_dim=ffn_dim,
                               output_dim=d_model, dtype="bf16")
    w = synth.make_weights(dims, 130 + d_model)
    enc = make_encoder(dims, w)
    lens = [16000 * 3 + 160 * 37 + 11, 16000]
    clips = [synth.speech_like_clip(n, [95, i]) for i, n in enumerate(lens)]
    _print(f"case: bf16 d={d_model} heads={n_heads} ffn={ffn_dim}", lens)
    out, taps = run_gpu(enc, clips, taps=True)
    rep = compare(dims, w, clips, out, taps)
    _print("short-K GEMMs", rep)
    enc.free()
