"""Coefficients of the device GELU (run: python -m audio_encoder_front_amd.gelu_coeffs
or python audio_encoder_front_amd/gelu_coeffs.py).

The kernels evaluate the erf form of GELU, gelu(z) = z (1 + erf(z / sqrt 2)) / 2,
as relu(z) - a erfc(a / sqrt 2) / 2 with a = |z| clamped to [0, A], and
erfc(a / sqrt 2) / 2 = exp2(P(a)) for a polynomial P: degree 6 with A = 6
(gelu_erf, max abs error 2.6e-7) where the result stays fp32, and degree 4
with A = 5 (gelu_erf_bf16, max abs error 6.4e-6, two fused multiply-adds
fewer) where the result is rounded to bf16 at once.  P is a
weighted least-squares fit of log2(erfc(a / sqrt 2)) - 1 on Chebyshev points,
the weight being the GELU error that an error in P causes (a erfc(...) ln2 / 2),
refined by Lawson reweighting toward the minimax solution.  Past A the tail
term is below 1e-8 (A = 6) or 1.5e-6 (A = 5) and the clamp keeps it so.

This script prints the float32 coefficients and checks the float32 evaluation
(Horner, exp2) against scipy's erf on a dense grid.
"""
from __future__ import annotations

import numpy as np
import scipy.special as sp

VARIANTS = {"gelu_erf": (6, 6.0), "gelu_erf_bf16": (4, 5.0)}   # name: (degree, A)


def fit(deg: int, clamp: float) -> np.ndarray:
    a = np.cos(np.linspace(0.0, np.pi, 4000)) * clamp / 2 + clamp / 2
    y = np.log2(sp.erfc(a / np.sqrt(2.0))) - 1.0
    w = np.maximum(np.maximum(a, 1e-3) * sp.erfc(a / np.sqrt(2.0)) * np.log(2.0) / 2, 1e-12)
    x = 2 * a / clamp - 1
    V = np.polynomial.chebyshev.chebvander(x, deg)
    c, *_ = np.linalg.lstsq(V * w[:, None], y * w, rcond=None)
    for _ in range(30):
        r = np.abs(V @ c - y) * w
        ww = w * (r / r.max() + 1e-3) ** 0.5
        c, *_ = np.linalg.lstsq(V * ww[:, None], y * ww, rcond=None)
    p = np.polynomial.Polynomial(np.polynomial.chebyshev.cheb2poly(c))
    return p(np.polynomial.Polynomial([-1.0, 2.0 / clamp])).coef.astype(np.float32)


def gelu_f32(z: np.ndarray, coef: np.ndarray, clamp: float) -> np.ndarray:
    f = np.float32
    z = z.astype(f)
    a = np.minimum(np.abs(z), f(clamp))
    y = coef[-1]
    for c in coef[-2::-1]:
        y = (y * a + c).astype(f)
    e = np.exp2(y).astype(f)
    return (np.maximum(z, f(0)) - a * e).astype(f)


def main() -> None:
    z = np.linspace(-60, 60, 6_000_001).astype(np.float32)
    zd = z.astype(np.float64)
    ref = 0.5 * zd * (1 + sp.erf(zd / np.sqrt(2.0)))
    for name, (deg, clamp) in VARIANTS.items():
        coef = fit(deg, clamp)
        err = np.abs(gelu_f32(z, coef, clamp) - ref)
        print("// %s: P(a), a = min(|z|, %g), highest degree first" % (name, clamp))
        for c in coef[::-1]:
            print("    %.9ef," % c)
        print("// max abs error %.3e (at z = %.4f)" % (err.max(), z[err.argmax()]))


if __name__ == "__main__":
    main()
