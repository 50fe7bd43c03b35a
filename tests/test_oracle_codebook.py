"""Pins for the oracle's Lloyd-Max codebook (CPU only).

What fixes the codebook independently of the oracle's own code:
* the closed form of the 1-bit Lloyd-Max quantizer of N(0,1): +-sqrt(2/pi),
  mean squared error 1 - 2/pi;
* J. Max's 1960 table of Gaussian Lloyd-Max quantizers (tests/golden);
* the TQ4 page's 72.5% error reduction from 8 to 16 centroids (tests/golden);
* numerical integration (scipy.integrate.quad) of the distortion and centroid
  conditions, an evaluation route that shares nothing with the closed forms.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy import integrate

from oracle import codebook as cb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _phi(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def test_one_bit_closed_form():
    c = cb.lloyd_max_normal(2)
    assert c[1] == pytest.approx(math.sqrt(2 / math.pi), abs=1e-15)
    assert c[0] == -c[1]
    assert cb.distortion(c) == pytest.approx(1 - 2 / math.pi, abs=1e-15)


def test_one_bit_reached_in_one_step_from_any_symmetric_start():
    for a in (0.1, 0.5, 3.0):
        c = cb.lloyd_step([-a, a])
        assert c[1] == pytest.approx(math.sqrt(2 / math.pi), abs=1e-15)


@pytest.mark.parametrize("levels", ["2", "4", "8", "16"])
def test_matches_max_1960_table(levels):
    ref = _load("max1960_gaussian.json")[levels]
    c = np.array(cb.lloyd_max_normal(int(levels)))
    pos = c[c > 0]
    np.testing.assert_allclose(pos, ref["levels"], atol=6e-4)
    mids = (c[:-1] + c[1:]) / 2
    np.testing.assert_allclose(mids[mids >= 0], ref["decisions"], atol=6e-4)
    assert cb.distortion(c) == pytest.approx(ref["mse"], rel=6e-4)


def test_pages_72_5_percent():
    fig = _load("pages_figures.json")["error_reduction_16_vs_8_centroids"]
    d16 = cb.distortion(cb.lloyd_max_normal(16))
    d8 = cb.distortion(cb.lloyd_max_normal(8))
    assert 1 - d16 / d8 == pytest.approx(fig["value"], abs=5e-4)


@pytest.mark.parametrize("levels", [4, 8, 16])
def test_symmetry_and_monotone_distortion(levels):
    c, hist = cb.lloyd_max_normal(levels, history=True)
    c = np.array(c)
    assert np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(c, -c[::-1])
    # Lloyd never increases the distortion (up to fp64 evaluation noise)
    assert max(np.diff(hist)) <= 1e-15
    assert hist[-1] < hist[0]


def test_unique_fixed_point_from_other_starts():
    ref = np.array(cb.lloyd_max_normal(16))
    starts = [np.linspace(-3.5, 3.5, 16), np.sort(np.random.default_rng(3).normal(size=16) * 2)]
    for s in starts:
        c = np.array(cb.lloyd_max_normal(16, start=s))
        np.testing.assert_allclose(c, ref, atol=1e-12)


def test_closed_form_distortion_matches_quadrature():
    c = cb.lloyd_max_normal(16)
    bnd = cb.boundaries(c)
    total = 0.0
    for k, ck in enumerate(c):
        a, b = bnd[k], bnd[k + 1]
        val, _ = integrate.quad(lambda x: (x - ck) ** 2 * _phi(x), a, b, epsabs=1e-14, epsrel=1e-12)
        assert cb.cell_distortion(a, b, ck) == pytest.approx(val, abs=1e-13)
        total += val
    assert cb.distortion(c) == pytest.approx(total, abs=1e-12)


def test_centroid_condition_by_quadrature():
    c = cb.lloyd_max_normal(16)
    bnd = cb.boundaries(c)
    for k, ck in enumerate(c):
        a, b = bnd[k], bnd[k + 1]
        m0, _ = integrate.quad(_phi, a, b, epsabs=1e-15, epsrel=1e-13)
        m1, _ = integrate.quad(lambda x: x * _phi(x), a, b, epsabs=1e-15, epsrel=1e-13)
        assert ck == pytest.approx(m1 / m0, abs=1e-10)


def test_float32_table_is_robust_to_rounding():
    """Every fp64 centroid sits well away from a float32 rounding boundary."""
    c64 = np.array(cb.lloyd_max_normal(16))
    c32 = c64.astype(np.float32)
    ulp = np.spacing(np.abs(c32)).astype(np.float64)
    frac = np.abs(c64 - c32.astype(np.float64)) / ulp
    assert np.all(frac < 0.45)
    m = cb.tq4_midpoints_f32(c32)
    assert m[7] == 0.0
    np.testing.assert_array_equal(m, -m[::-1])
