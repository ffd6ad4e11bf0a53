"""Pins for the oracle's Gaussian Lloyd-Max codebooks (TQ-MSE base quantizer).

Page: "RoPE-Aware Bit Allocation for KV-Cache Quantization", abstract -- the base
quantizer is TurboQuant-MSE; read as the MSE-optimal scalar quantizer of N(0,1)
with 2^w levels.  Pinned against textbook values (Max, 1960), the closed form at
one bit, the Panter-Dite high-rate constant, and quadrature computed here with
scipy (a different route from the oracle's closed forms).
"""
import math

import numpy as np
import pytest
from scipy import integrate, stats

import oracle

# Max (1960), "Quantizing for minimum distortion", Table I (N(0,1)): positive levels and MSE.
TEXTBOOK = {
    1: ([0.7980], 0.3634),
    2: ([0.4528, 1.510], 0.1175),
    3: ([0.2451, 0.7560, 1.344, 2.152], 0.03454),
    4: ([0.1284, 0.3881, 0.6568, 0.9423, 1.256, 1.618, 2.069, 2.733], 0.009497),
}


@pytest.mark.parametrize("w", [1, 2, 3, 4])
def test_textbook_levels(w):
    lv, D = TEXTBOOK[w]
    cb = oracle.codebook(w)
    pos = cb["levels"][(1 << w) // 2:]
    np.testing.assert_allclose(pos, lv, atol=6e-4)
    assert abs(cb["D"] - D) / D < 2e-3


def test_one_bit_closed_form():
    cb = oracle.codebook(1)
    assert abs(cb["levels"][1] - math.sqrt(2 / math.pi)) < 1e-15
    assert abs(cb["D"] - (1 - 2 / math.pi)) < 1e-15


@pytest.mark.parametrize("w", range(1, 9))
def test_symmetry_and_residual(w):
    cb = oracle.codebook(w)
    c = cb["levels"]
    np.testing.assert_array_equal(c, -c[::-1])
    assert np.all(np.diff(c) > 0)
    assert cb["resid"] < 1e-13


@pytest.mark.parametrize("w", [2, 5, 8])
def test_centroid_condition_by_quadrature(w):
    """Each level is the conditional mean of its cell; D is the integrated squared error."""
    c = oracle.codebook(w)["levels"]
    t = np.concatenate([[-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]])
    D = 0.0
    for j in range(len(c)):
        a, b = t[j], t[j + 1]
        P = stats.norm.cdf(b) - stats.norm.cdf(a) if a < 0 else stats.norm.sf(a) - stats.norm.sf(b)
        m1 = integrate.quad(lambda x: x * stats.norm.pdf(x), a, b, epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(m1 / P - c[j]) < 1e-9 * max(1.0, abs(c[j]))
        D += integrate.quad(lambda x: (x - c[j]) ** 2 * stats.norm.pdf(x), a, b, epsabs=1e-17, epsrel=1e-12)[0]
    assert abs(D - oracle.codebook(w)["D"]) / D < 1e-8


def test_high_rate_limit_and_decreasing_gains():
    T = oracle.tables()
    D = T["D"]
    # Panter-Dite: D_w * 4^w -> sqrt(3) * pi / 2 ~ 2.7207 as w grows
    assert abs(D[8] * 4 ** 8 - math.sqrt(3) * math.pi / 2) < 0.03
    # ... approached from below, monotonically
    assert D[6] * 4 ** 6 < D[7] * 4 ** 7 < D[8] * 4 ** 8 < math.sqrt(3) * math.pi / 2
    dD = T["dD64"]
    assert np.all(dD > 0)
    # strictly decreasing marginal gains (separable convexity -> greedy is optimal)
    assert np.all(dD[:-1] > dD[1:])
    assert np.all(T["dD"][:-1] > T["dD"][1:])


def _fp16_margin(x: float) -> float:
    """Relative distance of x from the nearest binary16 rounding midpoint."""
    ax = abs(x)
    e = math.floor(math.log2(ax))
    ulp = 2.0 ** (max(e, -14) - 10)
    frac = ax / ulp - math.floor(ax / ulp)
    return abs(frac - 0.5) * ulp / ax


@pytest.mark.parametrize("w", range(1, 9))
def test_fp16_rounding_is_robust(w):
    """Every level lies far (relative 1e-9) from a binary16 tie, so its rounding is
    insensitive to solver noise (~1e-11 relative)."""
    cb = oracle.codebook(w)
    for x, h in zip(cb["levels"], cb["levels_h"]):
        assert _fp16_margin(x) > 1e-9
        assert abs(h - x) <= 2.0 ** (math.floor(math.log2(abs(x))) - 11) + 1e-18
        assert np.float16(x) == np.float16(h)


def test_fp32_gain_table_is_robust():
    """The binary32 distortion drops used by the greedy allocator are not near ties."""
    T = oracle.tables()
    for x in T["dD64"]:
        f = np.float32(x)
        up = np.nextafter(f, np.float32(np.inf))
        dn = np.nextafter(f, np.float32(0))
        mid_hi = (float(f) + float(up)) / 2
        mid_lo = (float(f) + float(dn)) / 2
        assert min(abs(x - mid_hi), abs(x - mid_lo)) / x > 1e-10


@pytest.mark.parametrize("w", range(1, 9))
def test_thresholds_are_exact_midpoints(w):
    cb = oracle.codebook(w)
    lv = cb["levels_h"]
    thr = cb["thresholds"]
    for j in range(1, 1 << w):
        assert float(thr[j]) == 0.5 * (lv[j - 1] + lv[j])
    assert thr[(1 << w) // 2] == 0.0
