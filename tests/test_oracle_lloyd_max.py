"""Pins for the oracle's codebook design (Lloyd-Max for a Gaussian coordinate)."""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.integrate import quad

from oracle import freeze_tables
from oracle.lloyd_max import decision_boundaries, frozen_codebook, lloyd_max_normal, mse_normal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "max1960_gaussian_levels.txt")


def _pdf(x):
    return math.exp(-0.5 * x * x) / math.sqrt(2 * math.pi)


def _golden_levels():
    out = {}
    for line in open(GOLDEN):
        line = line.split("#")[0].strip()
        if line:
            n, *vals = line.split()
            out[int(n)] = [float(v) for v in vals]
    return out


@pytest.mark.parametrize("levels", [2, 8, 16])
def test_textbook_levels(levels):
    # Max (1960) prints 4 significant figures, computed with 1960 numerics: his 16-level
    # table is off by about half a unit in places (0.3881 for 0.38805; his 16-level distortion
    # 0.009497 against 0.009501 by quadrature), so agreement is asked to one unit of the last digit.
    c, _, _ = lloyd_max_normal(levels)
    ref = _golden_levels()[levels]
    for got, want in zip(c[levels // 2:], ref):
        digits = len(str(want).split(".")[1])
        assert abs(got - want) <= 10 ** -digits, (got, want)


def test_two_level_closed_form():
    c, b, _ = lloyd_max_normal(2)
    assert c[1] == pytest.approx(math.sqrt(2 / math.pi), abs=1e-15)
    assert c[0] == -c[1]
    assert mse_normal(c) == pytest.approx(1 - 2 / math.pi, abs=1e-14)


@pytest.mark.parametrize("levels", [8, 16])
def test_fixed_point_conditions_by_quadrature(levels):
    """Each centroid is its cell's conditional mean; each boundary the midpoint of its neighbours.
    Conditional means are recomputed by numerical quadrature, independent of the closed form."""
    c, b, _ = lloyd_max_normal(levels)
    edges = [-math.inf] + list(b) + [math.inf]
    for k in range(levels):
        mass = quad(_pdf, edges[k], edges[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
        first = quad(lambda x: x * _pdf(x), edges[k], edges[k + 1], epsabs=1e-15, epsrel=1e-13)[0]
        assert first / mass == pytest.approx(c[k], abs=1e-11)
    np.testing.assert_allclose(b, 0.5 * (c[:-1] + c[1:]), atol=1e-15, rtol=0)


@pytest.mark.parametrize("levels", [2, 8, 16])
def test_mse_by_quadrature(levels):
    c, b, _ = lloyd_max_normal(levels)
    edges = [-math.inf] + list(b) + [math.inf]
    tot = sum(quad(lambda x, ck=ck: (x - ck) ** 2 * _pdf(x), edges[k], edges[k + 1],
                   epsabs=1e-15, epsrel=1e-13)[0] for k, ck in enumerate(c))
    assert mse_normal(c) == pytest.approx(tot, rel=1e-10)
    # Max (1960) prints the 8-level distortion as 0.03455
    if levels == 8:
        assert abs(mse_normal(c) - 0.03455) < 5e-6


def test_lloyd_max_is_a_local_minimum():
    """Perturbing any level raises the MSE (the fixed point is a minimum, not a saddle)."""
    c, _, _ = lloyd_max_normal(8)
    base = mse_normal(c)
    for k in range(4, 8):
        for d in (-1e-3, 1e-3):
            p = c.copy()
            p[k] += d
            p[7 - k] -= d
            assert mse_normal(p) > base


@pytest.mark.parametrize("bits", [3, 4])
def test_frozen_codebook_symmetry_and_order(bits):
    cb = frozen_codebook(bits)
    u = cb.view(np.uint16)
    n = 2 ** bits
    for k in range(n):
        assert u[k] == (u[n - 1 - k] ^ 0x8000)       # bitwise mirror: only the sign bit differs
    assert np.all(np.diff(cb.astype(np.float64)) > 0)
    # every entry is the RNE fp16 of the scaled level: within half an fp16 ulp
    c, _, _ = lloyd_max_normal(n)
    target = c / math.sqrt(128)
    ulp = np.spacing(np.abs(cb)).astype(np.float64)
    assert np.all(np.abs(cb.astype(np.float64) - target) <= 0.5 * ulp)


@pytest.mark.parametrize("bits", [3, 4])
def test_thresholds_are_exact_midpoints(bits):
    cb = frozen_codebook(bits)
    beta = decision_boundaries(cb)
    for j in range(len(beta)):
        exact = (Fraction(float(cb[j])) + Fraction(float(cb[j + 1]))) / 2
        assert Fraction(float(beta[j])) == exact
    assert beta[len(beta) // 2] == 0.0


def test_table_file_matches_oracle(codebooks):
    t = freeze_tables.table()
    for fmt in ("turbo3", "turbo4"):
        want = np.array([int(h, 16) for h in t[fmt]["codebook_fp16_hex"]], dtype=np.uint16)
        np.testing.assert_array_equal(codebooks[fmt].view(np.uint16), want)
