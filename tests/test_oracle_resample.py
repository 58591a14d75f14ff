"""Pins of the resampler oracle (reading R1 of [qwenasr] "Module map": Kaiser
polyphase resampling to 16 kHz): an independent library routine
(scipy.signal.resample_poly with the same window, cut-off and length), the
window and Bessel function against numpy / scipy, and closed forms (a tone
keeps its frequency and amplitude, DC gain 1, 16 kHz input is returned
unchanged, the length formula, shift covariance)."""
import math

import numpy as np
import pytest
import scipy.signal as ss
import scipy.special as sp

import oracle.resample as R

RATES = [44100, 48000, 22050, 8000, 11025, 32000, 96000, 24000, 12000, 44056]


def test_bessel_and_window_match_library_routines():
    z = np.linspace(0, 12, 97)
    assert np.allclose(R.bessel_i0(z), sp.i0(z), rtol=1e-14)
    for n in (21, 101, 8821):
        assert np.abs(R.kaiser(n, 5.0) - np.kaiser(n, 5.0)).max() < 1e-13


@pytest.mark.parametrize("rate", RATES)
def test_matches_scipy_resample_poly(rate):
    rng = np.random.default_rng(rate)
    up, down = R.ratio(rate)
    for n in (1, 7, 333, 2500):
        x = rng.standard_normal(n)
        ref = ss.resample_poly(x, up, down, window=("kaiser", 5.0))
        y = R.resample(x, rate)
        assert y.shape == ref.shape == (R.output_length(n, rate),)
        assert np.abs(y - ref).max() < 1e-12


def test_ratio_and_length_closed_forms():
    assert R.ratio(44100) == (160, 441)
    assert R.ratio(48000) == (1, 3)
    assert R.ratio(8000) == (2, 1)
    assert R.ratio(16000) == (1, 1)
    for rate in RATES:
        for n in (0, 1, 441, 44100, 123457):
            assert R.output_length(n, rate) == math.ceil(n * 16000 / rate)
    with pytest.raises(ValueError):
        R.ratio(999)


def test_filter_is_linear_phase_with_gain_up():
    for rate in (44100, 8000, 48000):
        up, down, half, h = R.design(rate)
        assert h.shape == (2 * half + 1,) and half == 10 * max(up, down)
        assert np.allclose(h, h[::-1], atol=1e-15)
        assert h.sum() == pytest.approx(up, rel=1e-13)


def test_16k_input_is_returned_unchanged():
    x = np.random.default_rng(1).standard_normal(1000)
    assert np.abs(R.resample(x, 16000) - x).max() < 1e-14


@pytest.mark.parametrize("rate", [44100, 48000, 8000, 22050])
def test_tone_and_dc_pass_through(rate):
    # A 1 kHz tone (well inside every passband) keeps frequency, amplitude and
    # phase away from the clip edges; a constant keeps its value.
    n = rate // 2
    t = np.arange(n) / rate
    y = R.resample(np.sin(2 * np.pi * 1000.0 * t) + 0.25, rate)
    m = np.arange(y.shape[0])
    edge = 60                                # output samples affected by the zero padding
    ref = np.sin(2 * np.pi * 1000.0 * m / 16000.0) + 0.25
    assert np.abs(y[edge:-edge] - ref[edge:-edge]).max() < 2e-3


def test_stopband_rejects_aliases():
    # 44.1 kHz -> 16 kHz: an 11 kHz tone lies above the new Nyquist (8 kHz)
    # and must be removed, not folded to 5 kHz.
    rate = 44100
    t = np.arange(rate // 2) / rate
    y = R.resample(np.sin(2 * np.pi * 11000.0 * t), rate)
    assert np.abs(y[100:-100]).max() < 1e-2


def test_shift_covariance():
    # delaying the input by `down` samples delays the output by exactly `up`
    rate = 44100
    up, down = R.ratio(rate)
    x = np.random.default_rng(3).standard_normal(3000)
    y0 = R.resample(x, rate)
    y1 = R.resample(np.concatenate([np.zeros(down), x]), rate)
    assert np.abs(y1[up:up + y0.shape[0]] - y0).max() < 1e-13
