"""The ALU-only GELU of JA_GELU_POLY (ja_gelu_poly.h) against exact gelu_tanh.

The polynomial's coefficients are read from the generated header and
evaluated in float32 with the header's Horner order; the reference is the
tanh form in float64.  Also checks that the committed generator reproduces
the header."""
import importlib.util
import math
import os
import re

import numpy as np

CSRC = os.path.join(os.path.dirname(__file__), "..", "recsys_jagged_attention_amd", "csrc")


def header_poly():
    text = open(os.path.join(CSRC, "ja_gelu_poly.h")).read()
    a = float(re.search(r"kGeluPolyA = ([0-9.eE+-]+)f", text).group(1))
    body = text[text.index("kGeluPolyE[kGeluPolyDeg] = {"):]
    body = body[:body.index("};")]
    coef = [float(c) for c in re.findall(r"([-+0-9.eE]+)f,", body)]
    return a, np.array(coef, dtype=np.float32)


def gelu_exact(x):
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def gelu_poly32(x):
    a, c = header_poly()
    x = np.asarray(x, dtype=np.float32)
    xc = np.clip(x, np.float32(-a), np.float32(a))
    t = xc * xc
    e = np.full_like(t, c[-1])
    for k in range(len(c) - 2, -1, -1):
        e = e * t + c[k]
    g = e * t + np.float32(0.5) * xc
    return np.where(x >= a, x, np.where(x <= -a, np.float32(0.0), g)).astype(np.float64)


def test_polynomial_error_bound():
    x = np.linspace(-12.0, 12.0, 400001)
    err = np.abs(gelu_poly32(x) - gelu_exact(x))
    assert err.max() < 5e-4, err.max()


def test_polynomial_limits_and_origin():
    a, _ = header_poly()
    assert gelu_poly32([0.0])[0] == 0.0
    big = np.array([a, a + 1, 20.0, 1e4])
    np.testing.assert_array_equal(gelu_poly32(big), big)
    np.testing.assert_array_equal(gelu_poly32(-big), 0.0)
    # no jump larger than the error bound where the clamp takes over
    for s in (a, -a):
        lo, hi = gelu_poly32([np.nextafter(np.float32(s), np.float32(0))])[0], gelu_poly32([s])[0]
        assert abs(hi - lo) < 5e-4


def test_generator_reproduces_header():
    spec = importlib.util.spec_from_file_location("gen_gelu_poly", os.path.join(CSRC, "gen_gelu_poly.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    a, c = header_poly()
    assert gen.A == a and gen.DEG == len(c)
    np.testing.assert_allclose(gen.fit(), c, rtol=1e-6, atol=0)
