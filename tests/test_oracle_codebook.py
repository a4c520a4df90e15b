"""Pins for the oracle's Lloyd-Max codebook (CPU only).

The pages fix the method (Lloyd-Max on the fixed marginal, one codebook per
d) but print no codebook.  Pins: the textbook Gaussian table (Max 1960, in
tests/golden/), the K = 2 closed form, the centroid and midpoint conditions
checked by independent numerical integration, and the high-resolution
(Panter-Dite) distortion asymptote.
"""
import os

import numpy as np
import pytest
from scipy import integrate
from scipy.stats import norm

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lloyd_max_gaussian.txt")


def _textbook():
    rows = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        k, c, t, dist = [f.strip() for f in line.split("|")]
        rows.append((int(k), [float(v) for v in c.split()],
                     [] if t == "-" else [float(v) for v in t.split()], float(dist)))
    return rows


@pytest.mark.parametrize("row", _textbook(), ids=lambda r: f"K{r[0]}")
def test_matches_max_1960_table(row):
    K, cpos, tpos, dist = row
    cb = oracle.lloyd_max_gaussian(K)
    np.testing.assert_allclose(cb["centroids"][K // 2:], cpos, atol=1.5e-3)
    np.testing.assert_allclose(cb["thresholds"][K // 2:], tpos, atol=1.5e-3)
    assert abs(cb["distortion"] - dist) < 1e-3 * dist + 1e-5


def test_two_levels_closed_form():
    cb = oracle.lloyd_max_gaussian(2)
    assert abs(cb["centroids"][1] - np.sqrt(2 / np.pi)) < 1e-15
    assert abs(cb["distortion"] - (1 - 2 / np.pi)) < 1e-15


@pytest.mark.parametrize("K", [4, 8, 16, 64])
def test_centroid_and_midpoint_conditions_by_quadrature(K):
    cb = oracle.lloyd_max_gaussian(K)
    c, t = cb["centroids"], cb["thresholds"]
    assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)
    # exact symmetry and a zero middle threshold
    assert np.array_equal(c, -c[::-1]) and t[K // 2 - 1] == 0.0
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    D = 0.0
    for j in range(K):
        a, b = edges[j], edges[j + 1]
        mass = integrate.quad(norm.pdf, a, b, epsabs=1e-15, epsrel=1e-14)[0]
        first = integrate.quad(lambda x: x * norm.pdf(x), a, b, epsabs=1e-15, epsrel=1e-14)[0]
        assert abs(first / mass - c[j]) < 1e-9
        assert abs(mass - cb["cell_prob"][j]) < 1e-12
        D += integrate.quad(lambda x: (x - c[j]) ** 2 * norm.pdf(x), a, b,
                            epsabs=1e-15, epsrel=1e-13)[0]
    assert abs(D - cb["distortion"]) < 1e-10


def test_high_resolution_distortion():
    # Panter-Dite: D ~ (pi sqrt(3) / 2) / K^2 for a unit Gaussian as K grows
    cb = oracle.lloyd_max_gaussian(64)
    ratio = cb["distortion"] * 64 ** 2 / (np.pi * np.sqrt(3) / 2)
    assert 0.9 < ratio < 1.0
    assert abs(cb["distortion"] - 6.4424e-4) < 1e-7


def test_codebook_bits():
    for bits in (1, 2, 3, 4, 6):
        assert len(oracle.codebook(bits)["centroids"]) == 2 ** bits
