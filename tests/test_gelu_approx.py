"""The bf16-output GELU of the GEMM epilogue against the exact x * Phi(x) (CPU).

The device constants in csrc/common.h must be the ones flow_matching_tts_amd/gelu_fit.py
derives, and the formula, evaluated here in float64 and in float32 with those constants,
must stay within its stated bounds of math.erf's GELU: relative error below 1e-5 on
[-6, 6] (a bf16 rounding is 2^-9), absolute error below 6e-9 past it.
"""
import math
import os
import re

import numpy as np
import pytest

from flow_matching_tts_amd import gelu_fit as G

COMMON_H = os.path.join(os.path.dirname(__file__), "..", "flow_matching_tts_amd", "csrc", "common.h")


def device_coefficients():
    src = open(COMMON_H).read()
    body = src[src.index("float gelu_bf16(float x)"):]
    body = body[:body.index("\n}\n")]
    vals = [float(v) for v in re.findall(r"([-+]?\d\.\d+e[-+]\d+)f", body)]
    # Horner from the top: c8, c7, ..., c0
    return np.array(vals[::-1], np.float32)


def test_device_constants_are_the_fitted_ones():
    c = device_coefficients()
    assert len(c) == G.DEGREE + 1
    np.testing.assert_array_equal(c, G.fit())


@pytest.mark.parametrize("f32", [False, True])
def test_relative_error_inside_the_fit_range(f32):
    a, r = G.max_errors(device_coefficients(), -6.0, 6.0, n=60001, f32=f32)
    assert r < 1e-5, r
    assert a < 6e-7, a


def test_absolute_error_past_the_fit_range():
    c = device_coefficients()
    xs = np.concatenate([np.linspace(-40.0, -6.0, 2001), np.linspace(6.0, 40.0, 2001)])
    err = np.abs(G.gelu_approx(xs, c) - G.gelu_exact(xs))
    assert err.max() < 6e-9, err.max()


def test_special_values():
    c = device_coefficients()
    x = np.array([0.0, -0.0, 1e-30, -1e-30, np.inf, np.nan], np.float32)
    got = G.gelu_approx(x, c, f32=True)
    assert got[0] == 0.0 and got[1] == 0.0
    assert abs(got[2] - 5e-31) < 1e-5 * 5e-31 and abs(got[3] + 5e-31) < 1e-5 * 5e-31   # erfc(0) = 1 to 1e-5
    assert got[4] == np.inf and np.isnan(got[5])
    # the exact function at a few points of the textbook table of Phi
    for v, phi in [(1.0, 0.8413447460685429), (-1.0, 0.15865525393145707), (2.5, 0.9937903346742238)]:
        assert abs(G.gelu_approx(np.array([v]), c)[0] - v * phi) < 1e-5 * abs(v * phi)
        assert abs(0.5 * (1 + math.erf(v / math.sqrt(2))) - phi) < 1e-15
