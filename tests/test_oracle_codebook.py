"""Pins for the oracle's Lloyd-Max codebook (CPU only).

The pages fix the method (Lloyd-Max on the fixed marginal, one codebook per
d) but print no codebook.  Pins: the textbook Gaussian table (Max 1960, in
tests/golden/), the K = 2 closed form, the centroid and midpoint conditions
checked by independent numerical integration, and the high-resolution
(Panter-Dite) distortion asymptote.  For the exact sphere marginal f_d: the
d = 3 uniform quantizer, the K = 2 closed form E|U|, the conditions by
quadrature of the density itself, optimality against the Gaussian codebook,
and the O(1/d) approach to the Gaussian codebook.
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


# --- the exact sphere marginal f_d (one coordinate of a uniform direction) ---

def _sphere_pdf(d):
    """Density of U = sqrt(d) T written out from f_d(t) = C_d (1 - t^2)^((d-3)/2)."""
    from scipy.special import gamma
    c = gamma(d / 2) / (np.sqrt(np.pi) * gamma((d - 1) / 2))   # moderate d only
    return lambda u: c / np.sqrt(d) * max(0.0, 1 - u * u / d) ** ((d - 3) / 2)


@pytest.mark.parametrize("L", [2, 4, 8, 16, 64])
def test_sphere_d3_is_the_uniform_quantizer(L):
    # d = 3: f_3 is uniform on [-1, 1] (Archimedes), so Lloyd-Max gives the
    # uniform quantizer of [-sqrt 3, sqrt 3]: step 2 sqrt(3)/L, D = step^2/12
    cb = oracle.lloyd_max_sphere(L, 3)
    want = np.sqrt(3) * (-1 + (2 * np.arange(L) + 1) / L)
    np.testing.assert_allclose(cb["centroids"], want, rtol=0, atol=1e-12)
    assert abs(cb["distortion"] - 1.0 / L ** 2) < 1e-14


@pytest.mark.parametrize("d", [3, 4, 7, 100, 3072])
def test_sphere_one_bit_closed_form(d):
    # two levels: c = E|U| = sqrt(d) Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    from scipy.special import gammaln
    c = np.sqrt(d) * np.exp(gammaln(d / 2) - gammaln((d + 1) / 2)) / np.sqrt(np.pi)
    cb = oracle.lloyd_max_sphere(2, d)
    assert abs(cb["centroids"][1] - c) < 1e-12 * c
    assert abs(cb["distortion"] - (1 - c * c)) < 1e-12


@pytest.mark.parametrize("d,L", [(5, 4), (16, 16), (64, 8)])
def test_sphere_conditions_by_quadrature(d, L):
    cb = oracle.lloyd_max_sphere(L, d)
    c, t = cb["centroids"], cb["thresholds"]
    assert np.array_equal(c, -c[::-1]) and t[L // 2 - 1] == 0.0
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)
    pdf = _sphere_pdf(d)
    rd = np.sqrt(d)
    edges = np.concatenate([[-rd], t, [rd]])
    D = 0.0
    for j in range(L):
        a, b = edges[j], edges[j + 1]
        mass = integrate.quad(pdf, a, b, epsabs=1e-15, epsrel=1e-13)[0]
        first = integrate.quad(lambda x: x * pdf(x), a, b, epsabs=1e-15, epsrel=1e-13)[0]
        assert abs(first / mass - c[j]) < 1e-9
        assert abs(mass - cb["cell_prob"][j]) < 1e-11
        D += integrate.quad(lambda x: (x - c[j]) ** 2 * pdf(x), a, b,
                            epsabs=1e-15, epsrel=1e-12)[0]
    assert abs(D - cb["distortion"]) < 1e-10
    # the general distortion formula agrees, and the Gaussian codebook does
    # worse than the sphere codebook under the sphere marginal (optimality)
    assert abs(oracle.sphere_distortion(c, t, d) - cb["distortion"]) < 1e-12
    g = oracle.lloyd_max_gaussian(L)
    Dg = sum(integrate.quad(lambda x: (x - g["centroids"][j]) ** 2 * pdf(x),
                            *np.concatenate([[-rd], g["thresholds"], [rd]])[j:j + 2],
                            epsabs=1e-15, epsrel=1e-12)[0] for j in range(L))
    assert abs(oracle.sphere_distortion(g["centroids"], g["thresholds"], d) - Dg) < 1e-10
    assert Dg > cb["distortion"]


def test_sphere_tends_to_gaussian_at_rate_one_over_d():
    g = oracle.lloyd_max_gaussian(16)["centroids"]
    k = [d * np.max(np.abs(oracle.lloyd_max_sphere(16, d)["centroids"] - g))
         for d in (1000, 4000, 16000)]
    assert 1.0 < k[0] < 20.0
    assert abs(k[1] / k[0] - 1) < 0.01 and abs(k[2] / k[1] - 1) < 0.005


@pytest.mark.parametrize("d", [3, 64, 3072, 12288])
def test_sphere_many_levels_converge(d):
    for bits in (6, 8):
        cb = oracle.codebook_sphere(bits, d)
        c = cb["centroids"]
        assert np.all(np.diff(c) > 0) and c[-1] < np.sqrt(d)
        assert abs(np.sum(cb["cell_prob"]) - 1) < 1e-12
