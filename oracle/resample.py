"""fp64 oracle of the resampler to 16 kHz (test infrastructure only).

[qwenasr] "Module map" names the step in front of the log-mel front end: a
Kaiser polyphase resampler to 16 kHz mono ("Any input is resampled to 16 kHz
mono before the frontend", "Upstream model").  The page gives neither the
window parameter nor the filter length, so this module fixes a reading
(reading R1, also stated where the library designs its filter):

* the rate ratio is reduced, up / down = 16000 / g : rate / g with
  g = gcd(16000, rate);
* the anti-alias / anti-image filter is a linear-phase FIR low-pass of
  2 * half + 1 taps, half = 10 * max(up, down), cut-off at 1 / max(up, down)
  of the upsampled signal's Nyquist frequency, windowed by a Kaiser window of
  beta = 5, scaled to unit gain at DC and then by `up` (the zero-insertion
  loss);
* output sample n is the filtered, zero-stuffed input at upsampled index
  n * down, the filter centred there (no delay), samples outside the clip
  being zero; a clip of n samples gives ceil(n * up / down) output samples.

The output sample is written as the direct sum over the taps that meet a
nonzero (original) input sample -- the definition of the polyphase form, with
no blocking or reordering.
"""
from __future__ import annotations

import math
from typing import Tuple

import numpy as np

TARGET_RATE = 16000
KAISER_BETA = 5.0
HALF_FACTOR = 10
MIN_RATE = 1000
MAX_RATE = 768000


def bessel_i0(z: np.ndarray) -> np.ndarray:
    """Modified Bessel function of the first kind, order 0, by its power
    series I0(z) = sum_k ((z / 2)^k / k!)^2, summed until the terms vanish."""
    z = np.asarray(z, dtype=np.float64)
    term = np.ones_like(z)
    total = np.ones_like(z)
    k = 0
    while True:
        k += 1
        term = term * (z / (2.0 * k)) ** 2
        total = total + term
        if np.all(term <= 1e-17 * total):
            return total


def kaiser(n: int, beta: float) -> np.ndarray:
    """Kaiser window w[i] = I0(beta sqrt(1 - (2 i / (n - 1) - 1)^2)) / I0(beta)."""
    i = np.arange(n, dtype=np.float64)
    r = 2.0 * i / (n - 1) - 1.0
    return bessel_i0(beta * np.sqrt(np.maximum(0.0, 1.0 - r * r))) / bessel_i0(np.array(beta))


def ratio(rate: int) -> Tuple[int, int]:
    """(up, down) = (16000, rate) divided by their gcd (reading R1)."""
    if not (MIN_RATE <= rate <= MAX_RATE):
        raise ValueError(f"rate {rate} outside {MIN_RATE}..{MAX_RATE}")
    g = math.gcd(TARGET_RATE, rate)
    return TARGET_RATE // g, rate // g


def design(rate: int) -> Tuple[int, int, int, np.ndarray]:
    """(up, down, half, h): the Kaiser-windowed sinc low-pass of reading R1,
    h[k] = fc sinc(fc (k - half)) w[k], normalised to sum 1, times up."""
    up, down = ratio(rate)
    half = HALF_FACTOR * max(up, down)
    taps = 2 * half + 1
    fc = 1.0 / max(up, down)
    k = np.arange(taps, dtype=np.float64) - half
    arg = np.pi * fc * k
    sinc = np.where(k == 0, 1.0, np.sin(arg) / np.where(k == 0, 1.0, arg))
    h = fc * sinc * kaiser(taps, KAISER_BETA)
    h = h / h.sum()
    return up, down, half, h * up


def output_length(n: int, rate: int) -> int:
    """ceil(n up / down)."""
    up, down = ratio(rate)
    return -(-n * up // down)


def resample(x: np.ndarray, rate: int, outputs=None) -> np.ndarray:
    """y[n] = sum_k h[k] u[n down + half - k], u the input zero-stuffed by up
    (u[i up] = x[i], zero elsewhere); only the terms with i = (n down + half -
    k) / up an integer in [0, len(x)) contribute.  `outputs`: evaluate only
    these output indices (default: all)."""
    x = np.asarray(x, dtype=np.float64)
    up, down, half, h = design(rate)
    n_out = output_length(x.shape[0], rate)
    ns = range(n_out) if outputs is None else list(outputs)
    y = np.zeros(len(ns))
    for o, n in enumerate(ns):
        t = n * down + half                 # upsampled index seen by tap k = 0
        k0 = t % up                          # first tap landing on an input sample
        ks = np.arange(k0, h.shape[0], up)
        idx = (t - ks) // up
        ok = (idx >= 0) & (idx < x.shape[0])
        y[o] = np.dot(h[ks[ok]], x[idx[ok]])
    return y
