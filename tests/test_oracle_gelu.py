"""Pins of the oracle's FFN activation (R13: GELU, erf form, on the BF16 up
projection output, rounded once to BF16) against routes other than itself.

* f64_to_bf16 against exact rational rounding (tests/exact.py), including
  values on and one fp64 step either side of BF16 midpoints, the cases a
  double rounding through fp32 gets wrong;
* GELU at points where the standard normal CDF is tabulated (textbook
  values of Phi), and over every finite BF16 input against y * Phi(y) from
  scipy's normal distribution (ndtr, a different routine from erfc);
* the identity GELU(y) - GELU(-y) = y, the limits y -> +-inf, signed zeros;
* torch's float64 GELU where its 1 + erf form loses few digits (y > -3).

test_planted_mistakes plants plausible mistakes (the tanh approximation, the
1 + erf form, a double rounding) and shows these checks reject them.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch
from scipy.stats import norm

import oracle as O
from tests import exact as E

# Standard normal CDF, textbook table values (to 16 significant digits)
PHI = {0.5: 0.6914624612740131, 1.0: 0.8413447460685429, 2.0: 0.9772498680518208,
       3.0: 0.9986501019683699, -1.0: 0.1586552539314571, -2.0: 0.02275013194817921,
       -3.0: 0.001349898031630095}


def bf16_of_value(v: float) -> int:
    """Exact nearest-even BF16 of an fp64 value (sign kept for zeros)."""
    if v == 0.0:
        return 0x8000 if np.signbit(v) else 0
    b = E.bf16_bits(E.bf16(Fraction(v)))
    if E.bf16(Fraction(v)) == 0:                 # underflow to zero keeps the sign
        return 0x8000 if v < 0 else 0
    return b


def finite_bf16() -> np.ndarray:
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return bits[np.isfinite(O.bf16_to_f32(bits))]


# ---------------------------------------------------------------------------
# f64 -> BF16 rounding
# ---------------------------------------------------------------------------

def midpoint_cases(rng, n=400):
    """fp64 values on BF16 midpoints and one fp64 step to either side."""
    out = []
    lo = rng.integers(0x0080, 0x7F00, size=n).astype(np.uint16)   # normal BF16, positive
    a = O.bf16_to_f32(lo).astype(np.float64)
    b = O.bf16_to_f32(lo + 1).astype(np.float64)
    m = (a + b) / 2                                               # exact in fp64
    for v in (m, np.nextafter(m, np.inf), np.nextafter(m, -np.inf)):
        out.append(v)
        out.append(-v)
    return np.concatenate(out)


def check_f64_to_bf16(fn, values):
    got = fn(values)
    want = np.array([bf16_of_value(float(v)) for v in values], dtype=np.uint16)
    return np.array_equal(got, want)


def test_f64_to_bf16_exact_rounding():
    rng = np.random.default_rng(20)
    vals = np.concatenate([
        midpoint_cases(rng),
        rng.standard_normal(500) * 10.0 ** rng.integers(-30, 30, size=500),
        np.array([0.0, -0.0, 1.0, -1.0, 3.3895313892515355e38, 1e-40, -1e-40, 9.2e-41]),
    ])
    assert check_f64_to_bf16(O.f64_to_bf16, vals)


# ---------------------------------------------------------------------------
# GELU
# ---------------------------------------------------------------------------

def check_gelu_table(gelu_f64, gelu_bf16):
    ys = np.array(sorted(PHI), dtype=np.float32)
    yb = O.f32_to_bf16(ys)
    g = gelu_f64(yb)
    want = np.array([float(y) * PHI[float(y)] for y in ys], dtype=np.float64)
    if not np.allclose(g, want, rtol=1e-14, atol=0):
        return False
    return np.array_equal(gelu_bf16(yb),
                          np.array([bf16_of_value(float(v)) for v in want], dtype=np.uint16))


def check_gelu_vs_ndtr(gelu_f64, gelu_bf16):
    bits = finite_bf16()
    y = O.bf16_to_f32(bits).astype(np.float64)
    ref = y * norm.cdf(y)
    g = gelu_f64(bits)
    big = np.abs(ref) > 1e-290
    if not np.all(np.abs(g - ref)[big] <= 1e-12 * np.abs(ref)[big]):
        return False
    return np.array_equal(gelu_bf16(bits), O.f64_to_bf16(ref))


def test_gelu_textbook_values():
    assert check_gelu_table(O.gelu_f64, O.gelu_bf16)


def test_gelu_every_bf16_input_against_normal_cdf():
    assert check_gelu_vs_ndtr(O.gelu_f64, O.gelu_bf16)


def test_gelu_reflection_identity():
    bits = finite_bf16()
    y = O.bf16_to_f32(bits).astype(np.float64)
    keep = np.abs(y) < 1e300
    y = y[keep]
    g = O.gelu_f64(bits[keep])
    gm = O.gelu_f64(O.f32_to_bf16(-y.astype(np.float32)))
    scale = np.maximum(np.abs(y), np.abs(g))
    assert np.all(np.abs(g - gm - y) <= 4 * np.finfo(np.float64).eps * scale)


def test_gelu_limits_and_zeros():
    big = O.f32_to_bf16(np.array([6.0, 10.0, 1e4, 3e38], np.float32))
    assert np.array_equal(O.gelu_bf16(big), big)              # y * Phi(y) rounds to y
    neg = O.f32_to_bf16(np.array([-40.0, -1e4, -3e38], np.float32))
    assert np.all(O.gelu_bf16(neg) == 0x8000)                 # underflows to -0
    assert O.gelu_bf16(np.array([0x0000], np.uint16))[0] == 0x0000
    assert O.gelu_bf16(np.array([0x8000], np.uint16))[0] == 0x8000
    # small negative outputs keep their digits (no 1 + erf cancellation)
    v = O.bf16_to_f32(O.gelu_bf16(O.f32_to_bf16(np.array([-10.0], np.float32))))[0]
    assert v < 0 and abs(v / (-10.0 * norm.cdf(-10.0)) - 1) < 2.0 ** -8


def test_gelu_agrees_with_torch_without_cancellation():
    bits = finite_bf16()
    y = O.bf16_to_f32(bits).astype(np.float64)
    keep = (y > -3.0) & (np.abs(y) < 1e300)
    t = torch.nn.functional.gelu(torch.from_numpy(y[keep])).numpy()
    g = O.gelu_f64(bits[keep])
    big = np.abs(t) > 1e-290
    assert np.all(np.abs(g - t)[big] <= 1e-12 * np.abs(t)[big])


def test_postscale_gelu_chain():
    rng = np.random.default_rng(21)
    acc = rng.integers(-200000, 200000, size=(5, 7)).astype(np.int32)
    sa = rng.uniform(1e-3, 1e-1, size=5).astype(np.float32)
    sw = rng.uniform(1e-5, 1e-3, size=7).astype(np.float32)
    b = O.f32_to_bf16(rng.standard_normal(7).astype(np.float32))
    assert np.array_equal(O.postscale_gelu_bf16(acc, sa, sw),
                          O.gelu_bf16(O.postscale_bf16(acc, sa, sw)))
    assert np.array_equal(O.postscale_gelu_bf16(acc, sa, sw, b),
                          O.gelu_bf16(O.postscale_bias_bf16(acc, sa, sw, b)))


# ---------------------------------------------------------------------------
# planted mistakes
# ---------------------------------------------------------------------------

def _gelu_tanh_f64(bits):
    y = O.bf16_to_f32(bits).astype(np.float64)
    return 0.5 * y * (1 + np.tanh(np.sqrt(2 / np.pi) * (y + 0.044715 * y ** 3)))


def _gelu_one_plus_erf_f64(bits):
    from scipy.special import erf
    y = O.bf16_to_f32(bits).astype(np.float64)
    return 0.5 * y * (1 + erf(y / np.sqrt(2.0)))


def _f64_to_bf16_double_rounding(x):
    return O.f32_to_bf16(np.asarray(x, np.float64).astype(np.float32))


def test_planted_mistakes():
    tanh_bf16 = lambda b: O.f64_to_bf16(_gelu_tanh_f64(b))
    assert not check_gelu_table(_gelu_tanh_f64, tanh_bf16)
    erf_bf16 = lambda b: O.f64_to_bf16(_gelu_one_plus_erf_f64(b))
    assert not check_gelu_vs_ndtr(_gelu_one_plus_erf_f64, erf_bf16)
    rng = np.random.default_rng(20)
    assert not check_f64_to_bf16(_f64_to_bf16_double_rounding, midpoint_cases(rng))
