"""Pins of the oracle's front end (framing, Hann, DFT, mel, log, affine) against
closed forms, invariants, brute force and independent library routines."""
import json
import math
import os

import numpy as np
import pytest

import oracle as O
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_shapes.json")))


def test_hann_closed_form_sums():
    # periodic Hann of length N: sum w = N/2, sum w^2 = 3N/8
    w = O.hann_periodic(400)
    assert abs(w.sum() - 200.0) < 1e-12
    assert abs((w * w).sum() - 150.0) < 1e-12
    assert w[0] == 0.0 and abs(w[200] - 1.0) < 1e-15
    # periodic (not symmetric): w[n] == w[N-n]
    assert np.allclose(w[1:], w[1:][::-1], atol=1e-15)


def test_reflect_pad_mirrors_without_edge():
    x = np.arange(10.0)
    p = O.reflect_pad(x, 3)
    assert p.tolist() == [3, 2, 1, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 8, 7, 6]


@pytest.mark.parametrize("n", [8, 16])
def test_dft_matches_direct_double_loop(n):
    rng = np.random.default_rng(0)
    fr = rng.standard_normal((3, n))
    win = np.ones(n)
    p = O.power_spectrum(fr, win)
    for r in range(3):
        for k in range(n // 2 + 1):
            re = sum(fr[r, t] * math.cos(2 * math.pi * k * t / n) for t in range(n))
            im = -sum(fr[r, t] * math.sin(2 * math.pi * k * t / n) for t in range(n))
            assert abs(p[r, k] - (re * re + im * im)) < 1e-9 * max(1.0, p[r, k])


def test_dft_matches_numpy_rfft_n400():
    rng = np.random.default_rng(1)
    fr = rng.standard_normal((5, 400))
    w = O.hann_periodic()
    ref = np.abs(np.fft.rfft(fr * w, axis=1)) ** 2
    p = O.power_spectrum(fr)
    assert np.max(np.abs(p - ref) / np.maximum(ref.max(axis=1, keepdims=True), 1e-300)) < 1e-12


def test_parseval_per_frame():
    rng = np.random.default_rng(2)
    fr = rng.standard_normal((4, 400))
    w = O.hann_periodic()
    p = O.power_spectrum(fr)
    lhs = p[:, 0] + 2 * p[:, 1:200].sum(axis=1) + p[:, 200]
    rhs = 400.0 * ((fr * w) ** 2).sum(axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-12)


def test_pure_tone_lands_in_bins_10_11_12():
    # 0.3 sin(2 pi 440 t): 440 Hz = bin 11 of a 400-point DFT at 16 kHz.  The
    # Hann DFT has W(0)=N/2, W(+-1)=-N/4, so |X_11| = 0.3*200/2 = 30 and
    # |X_10| = |X_12| = 0.3*100/2 = 15 on frames that see no padding.
    t = np.arange(32000) / 16000.0
    x = 0.3 * np.sin(2 * np.pi * 440.0 * t)
    p = O.power_spectrum(O.stft_frames(x))
    for j in (2, 50, 100, 198):
        assert abs(p[j, 11] - 900.0) < 1e-9
        assert abs(p[j, 10] - 225.0) < 1e-9 and abs(p[j, 12] - 225.0) < 1e-9
        rest = np.delete(p[j], [10, 11, 12])
        assert rest.max() < 1e-15


def test_mel_scale_closed_forms():
    assert O.hz_to_mel(1000.0) == pytest.approx(15.0, abs=1e-12)
    assert O.hz_to_mel(6400.0) == pytest.approx(42.0, abs=1e-12)    # 15 + 27 * ln(6.4)/ln(6.4)
    assert O.hz_to_mel(500.0) == pytest.approx(7.5, abs=1e-12)
    assert O.hz_to_mel(8000.0) == pytest.approx(15 + 27 * math.log(8) / math.log(6.4), abs=1e-12)
    f = np.array([0.0, 123.0, 999.0, 1000.0, 2500.0, 7999.0])
    assert np.allclose(O.mel_to_hz(O.hz_to_mel(f)), f, atol=1e-9)


def test_mel_filterbank_structure():
    fb = O.mel_filterbank()
    assert fb.shape == (128, 201)
    assert np.all(fb >= 0)
    assert np.all(fb.sum(axis=1) > 0)            # no empty filter
    # centres uniform in mel between mel(0) and mel(8000): 130 edge points
    step = O.hz_to_mel(8000.0) / 129
    edges = O.mel_to_hz(step * np.arange(130))
    for m in range(128):
        nz = np.nonzero(fb[m])[0] * 40.0
        assert nz.min() > edges[m] - 1e-9 and nz.max() < edges[m + 2] + 1e-9
    # area normalisation: each triangle integrates to 1 over Hz; the 40 Hz
    # Riemann sum is close for filters spanning many bins
    wide = [m for m in range(128) if edges[m + 2] - edges[m] > 200.0]
    assert len(wide) > 20
    for m in wide:
        assert abs(fb[m].sum() * 40.0 - 1.0) < 0.025
    assert int((fb > 0).sum()) == 394


def test_tone_energy_in_expected_mel_bin():
    # mel(440 Hz) = 6.6; centres sit at step*(m+1) with step = mel(8000)/129,
    # so the nearest centre is m = round(6.6/step) - 1 = 18.
    step = O.hz_to_mel(8000.0) / 129
    expect = int(round(6.6 / step)) - 1
    assert expect == 18
    t = np.arange(32000) / 16000.0
    x = 0.3 * np.sin(2 * np.pi * 440.0 * t)
    e = O.power_spectrum(O.stft_frames(x)) @ O.mel_filterbank().T
    assert np.all(e[2:198].argmax(axis=1) == expect)
    # noisy tiny workload: the normalised log-mel peaks in the same bin
    xs = synth.make_audio(synth.WORKLOADS["tiny"])[0]
    m = O.log_mel(xs)
    assert np.all(m[:, 2:198].argmax(axis=0) == expect)


def test_frame_count_drops_last_frame():
    rng = np.random.default_rng(3)
    for n in (201, 319, 320, 321, 32000, 32159):
        m = O.log_mel(rng.standard_normal(n))
        assert m.shape == (128, n // 160)
    assert O.log_mel(np.zeros(480000) + 1e-3).shape == tuple(GOLD["mel_30s"]["shape"])


def test_silence_is_minus_one_and_a_half():
    m = O.log_mel(np.zeros(5000))
    assert np.all(m == -1.5)


def test_log_affine_bounds():
    x = synth.make_audio(synth.WORKLOADS["b06_32"])[0][:40000].copy()
    x[12000:20000] = 0.0                # digital silence: bins far below the peak
    raw = O.log_mel_raw(x)
    m = O.log_mel(x)
    M = raw.max()
    assert m.max() == pytest.approx((M + 4) / 4, abs=1e-12)
    assert m.min() >= (M - 8 + 4) / 4 - 1e-12
    assert np.allclose(m[raw > M - 8], (raw[raw > M - 8] + 4) / 4, atol=1e-12)
    assert (raw < M - 8).any()          # the clamp is active


def test_input_contract():
    with pytest.raises(O.InvalidInput):
        O.validate_clip(200)
    with pytest.raises(O.InvalidInput):
        O.validate_clip(GOLD["twenty_minutes"]["samples"] + 1)
    O.validate_clip(0)
    O.validate_clip(201)
    O.validate_clip(GOLD["twenty_minutes"]["samples"])


def test_rejects_nonfinite_and_float32_overflow():
    x = synth.speech_like_clip(8000, [79, 0]).astype(np.float64)
    x[1234] = np.nan
    with pytest.raises(O.InvalidInput):
        O.log_mel(x)
    x[1234] = 1e25                      # |X|^2 ~ 1e50 > float32 max
    with pytest.raises(O.InvalidInput):
        O.log_mel(x)
    x[1234] = 1e3                       # large but representable
    assert np.all(np.isfinite(O.log_mel(x)))


def test_tone_mel_closed_form_values():
    # The noise-free 0.3 sin(2 pi 440 t) puts P_11 = 900 on interior frames and
    # P_10 = P_12 = 225 (test above).  Band 18's triangle spans 420.89 ..
    # 467.65 Hz (below 1 kHz the Slaney scale is 3 f / 200, so its edges are
    # 18, 19, 20 steps of mel(8000)/129 mapped back linearly), so it holds
    # bin 11 (440 Hz) only: fb[18, 11] = 0.8174 * 2 / 46.77 Hz = 0.0349524 and
    # E_18 = 900 * 0.0349524 = 31.457.
    fb = O.mel_filterbank()
    assert fb[18, 11] == pytest.approx(0.0349524, abs=5e-8)
    assert fb[18, 10] == 0.0 and fb[18, 12] == 0.0
    t = np.arange(32000) / 16000.0
    x = 0.3 * np.sin(2 * np.pi * 440.0 * t)
    e = O.power_spectrum(O.stft_frames(x)) @ fb.T
    assert np.allclose(e[2:198, 18], 31.457, atol=5e-4)


def test_matches_published_whisper_feature_extractor():
    """OneSpeech "Front end and graph numerics": the features agree with the
    published float32 Whisper feature extractor to a max-abs 3e-5.  That
    extractor (transformers' WhisperFeatureExtractor, 128 bins, no padding to
    30 s) is an implementation independent of the oracle; its float32 path
    must land within the page's 3e-5 and its float64 path within float32
    rounding of the oracle."""
    tr = pytest.importorskip("transformers")
    fe = tr.WhisperFeatureExtractor(feature_size=128)
    x = synth.make_audio(synth.WORKLOADS["b06_1"])[0][:16000 * 7 + 123]
    ref = O.log_mel(x.astype(np.float64))
    f32 = fe(x, sampling_rate=16000, padding="longest", return_tensors="np")["input_features"][0]
    assert f32.shape == ref.shape
    assert np.abs(f32 - ref).max() <= 3e-5
    f64 = fe._np_extract_fbank_features(x.astype(np.float64)[None], "cpu")[0]
    assert np.abs(f64 - ref).max() <= 2e-6
    # the tiny workload (tone + noise), a 201-sample clip and a tail frame count
    for clip in (synth.make_audio(synth.WORKLOADS["tiny"])[0], synth.speech_like_clip(201, [9, 1]),
                 synth.speech_like_clip(16000 * 2 + 160 * 37 + 99, [9, 2])):
        r = O.log_mel(clip.astype(np.float64))
        f = fe._np_extract_fbank_features(clip.astype(np.float64)[None], "cpu")[0]
        assert f.shape == r.shape and np.abs(f - r).max() <= 2e-6


def test_no_upper_clamp_on_mel_energy():
    """Reading of the pages' clamp: only the 1e-10 floor.  Scaling a clip by s
    scales every power and mel energy by s^2, so the raw log-mel shifts by
    exactly 2 log10(s) wherever the floor is inactive; at s = 1e15 the mel
    energies reach ~1e31, past the 1e30 cap of qwenasr "Mel frontend", and
    the shift still holds (a cap would pin them at 30).  The published
    extractor agrees at that scale."""
    x = synth.make_audio(synth.WORKLOADS["b06_1"])[0][:16000 * 3 + 77].astype(np.float64)
    raw = O.log_mel_raw(x)
    assert raw.min() > -10.0                         # the floor is not reached
    big = O.log_mel_raw(x * 1e15)
    assert big.max() > 31.0
    assert np.abs(big - (raw + 30.0)).max() < 1e-9
    tr = pytest.importorskip("transformers")
    fe = tr.WhisperFeatureExtractor(feature_size=128)
    f = fe._np_extract_fbank_features((x * 1e15)[None], "cpu")[0]
    assert np.abs(f - O.log_mel(x * 1e15)).max() <= 2e-6


def test_rejects_power_overflow_in_a_bin_outside_every_band():
    # DC of 1e17: X_0 = 200e17 gives P_0 = 4e38 > float32 max, while the bins
    # a mel band weighs stay finite (P_1 = 1e38): bin 0 lies outside every
    # Slaney band, so the rejection must come from the power check itself.
    x = np.full(5000, 1e17) + synth.speech_like_clip(5000, [9, 3]).astype(np.float64)
    fr = O.stft_frames(x)
    p = O.power_spectrum(fr)
    assert p[:, 0].max() > O.F32_MAX
    assert (p @ O.mel_filterbank().T).max() < O.F32_MAX
    assert np.all(O.mel_filterbank()[:, 0] == 0.0)
    with pytest.raises(O.InvalidInput):
        O.log_mel(x)


def test_rejects_nonfinite_trailing_sample():
    # L = 160 F + r with r >= 41: samples 160 F + 40 .. L - 1 are read only by
    # the final (dropped) STFT frame; they are still part of the input
    L = 160 * 50 + 150
    x = synth.speech_like_clip(L, [9, 4]).astype(np.float64)
    x[L - 1] = np.nan
    with pytest.raises(O.InvalidInput):
        O.log_mel(x)
