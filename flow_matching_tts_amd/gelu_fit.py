"""Coefficients of the bf16-output GELU used by the GEMM epilogue (``gelu_bf16`` in csrc/common.h).

GELU is the exact form x * Phi(x) = x * (1 + erf(x / sqrt 2)) / 2. It is rewritten as

    GELU(x) = (x + |x| - y * erfc(y / sqrt 2)) / 2,    y = min(|x|, Y),

which equals x * Phi(x) for |x| <= Y (erf is odd). For |x| > Y the dropped term is below
Y * erfc(Y / sqrt 2) / 2 (6e-9 for Y = 6). erfc(y / sqrt 2) is evaluated as exp2(P(y)). P is
a degree-8 polynomial fitted to log2 erfc(y / sqrt 2) on [0, Y]: a least-squares fit in the
Chebyshev basis on a dense uniform grid, converted to the power basis in y and rounded to
float32. A fit in the log domain bounds the relative error of erfc uniformly, so the relative
error of GELU stays small in the negative tail, where the values are tiny. The device
evaluates P by Horner's rule with fused multiply-adds, then one v_exp_f32: one transcendental
and no division.

Run ``python -m flow_matching_tts_amd.gelu_fit`` to print the coefficients and the error over
a dense grid in float64 (against math.erf) and in float32 (as the device evaluates them).
"""
from __future__ import annotations

import math

import numpy as np

Y_MAX = 6.0
DEGREE = 8
GRID = 200001


def fit(degree: int = DEGREE, y_max: float = Y_MAX, n: int = GRID) -> np.ndarray:
    """float32 power-basis coefficients c[0..degree] of P(y) ~ log2 erfc(y / sqrt 2)."""
    from numpy.polynomial import chebyshev as ch
    ys = np.linspace(0.0, y_max, n)
    target = np.log2([math.erfc(y / math.sqrt(2.0)) for y in ys])
    u = 2.0 * ys / y_max - 1.0
    cc, *_ = np.linalg.lstsq(ch.chebvander(u, degree), target, rcond=None)
    in_u = np.polynomial.Polynomial(ch.cheb2poly(cc))
    in_y = in_u(np.polynomial.Polynomial([-1.0, 2.0 / y_max]))
    return in_y.coef.astype(np.float32)


def gelu_approx(x: np.ndarray, c: np.ndarray, y_max: float = Y_MAX, f32: bool = False) -> np.ndarray:
    """The device formula; with f32=True every step is rounded to float32 as on the GPU."""
    t = np.float32 if f32 else np.float64
    x = np.asarray(x, t)
    ax = np.abs(x)
    y = np.minimum(ax, t(y_max))
    p = np.full_like(y, t(c[-1]))
    for a in c[-2::-1]:
        p = (p * y + t(a)).astype(t)
    e = np.exp2(p).astype(t)
    return (t(0.5) * ((x + ax).astype(t) - (y * e).astype(t))).astype(t)


def gelu_exact(x: np.ndarray) -> np.ndarray:
    return np.array([0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0))) for v in np.asarray(x, np.float64)])


def max_errors(c: np.ndarray, lo: float = -12.0, hi: float = 12.0, n: int = 48001, f32: bool = False):
    """(max absolute error, max relative error over x != 0) of the approximation on [lo, hi]."""
    xs = np.linspace(lo, hi, n)
    want = gelu_exact(xs)
    got = gelu_approx(xs, c, f32=f32).astype(np.float64)
    err = np.abs(got - want)
    nz = np.abs(want) > 1e-30
    return float(err.max()), float((err[nz] / np.abs(want[nz])).max())


if __name__ == "__main__":
    c = fit()
    print("coefficients c0..c%d:" % DEGREE)
    for i, v in enumerate(c):
        print(f"  c{i} = {float(v):.9e}f")
    for f32 in (False, True):
        a, r = max_errors(c, -6.0, 6.0, f32=f32)
        print(f"{'float32' if f32 else 'float64'} evaluation on [-6, 6]: max abs {a:.2e}, max rel {r:.2e}")
