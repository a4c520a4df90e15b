"""Pins for the oracle's RPBH rotation (CPU only).

What the pages fix: Pi_d = blkdiag(H_h D_1, ...) P_pi is a rotation (an
orthogonal matrix); weights take Pi^T and activations Pi, so they cancel in
the product; the leading permutation makes every rotated coordinate of a
unit vector have variance ~1/d.
"""
import numpy as np
import pytest
import scipy.linalg

import oracle
import synth


@pytest.mark.parametrize("h", [1, 2, 4, 8, 16, 64, 256, 1024])
def test_sylvester_matches_scipy(h):
    np.testing.assert_array_equal(oracle.sylvester(h), scipy.linalg.hadamard(h))


@pytest.mark.parametrize("n", [1, 2, 8, 128, 512])
def test_fwht_matches_dense_product(n):
    y = np.random.default_rng(n).standard_normal((5, n))
    ref = y @ scipy.linalg.hadamard(n).T.astype(np.float64)
    np.testing.assert_allclose(oracle.fwht(y), ref, rtol=0, atol=1e-12 * n)


def test_h1_is_a_signed_gather():
    # h = 1 leaves only D P_pi: (Pi x)_k = D_k x[pi(k)], the gather convention
    perm, signs = synth.rotation_params(40, 7)
    x = np.random.default_rng(1).standard_normal(40)
    got = oracle.rpbh_rotate(x[None], perm, signs, 1)[0]
    for k in range(40):
        assert got[k] == signs[k] * x[perm[k]]


def test_identity_perm_unit_signs_is_block_hadamard():
    d, h = 64, 16
    Pi = oracle.rpbh_matrix(np.arange(d), np.ones(d, np.int8), h)
    ref = scipy.linalg.block_diag(*[scipy.linalg.hadamard(h)] * (d // h)) / np.sqrt(h)
    np.testing.assert_allclose(Pi, ref, rtol=0, atol=1e-15)
    Pi = oracle.rpbh_matrix(np.arange(d), np.ones(d, np.int8), d)
    np.testing.assert_allclose(Pi, scipy.linalg.hadamard(d) / np.sqrt(d), rtol=0, atol=1e-15)


def test_signs_act_after_the_permutation():
    # with h = 2 and a swap permutation the sign of permuted slot 0 multiplies x[1]
    perm = np.array([1, 0], np.int32)
    signs = np.array([-1, 1], np.int8)
    Pi = oracle.rpbh_matrix(perm, signs, 2)
    H = np.array([[1.0, 1.0], [1.0, -1.0]]) / np.sqrt(2)
    P = np.array([[0.0, 1.0], [1.0, 0.0]])
    np.testing.assert_allclose(Pi, H @ np.diag([-1.0, 1.0]) @ P, atol=1e-15)


@pytest.mark.parametrize("d,h", [(256, 64), (256, 256), (3072, 128)])
def test_pi_is_orthogonal(d, h):
    perm, signs = synth.rotation_params(d, d + h)
    Pi = oracle.rpbh_matrix(perm, signs, h)
    np.testing.assert_allclose(Pi @ Pi.T, np.eye(d), rtol=0, atol=1e-12)


@pytest.mark.parametrize("d,h", [(256, 64), (256, 16), (512, 512)])
def test_fast_rotation_equals_dense(d, h):
    perm, signs = synth.rotation_params(d, 3)
    X = np.random.default_rng(2).standard_normal((7, d))
    Pi = oracle.rpbh_matrix(perm, signs, h)
    np.testing.assert_allclose(oracle.rpbh_rotate(X, perm, signs, h), X @ Pi.T,
                               rtol=0, atol=1e-12)
    Xr = oracle.rpbh_rotate(X, perm, signs, h)
    np.testing.assert_allclose(oracle.rpbh_inverse_rotate(Xr, perm, signs, h), X,
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(oracle.rpbh_inverse_rotate(Xr, perm, signs, h), Xr @ Pi,
                               rtol=0, atol=1e-12)


def test_rotation_cancels_in_the_product():
    inp = synth.make(1)
    W, X = inp["W"].astype(np.float64), inp["X"].astype(np.float64)
    perm, signs, h = inp["perm"], inp["signs"], inp["h"]
    Wp = oracle.rpbh_rotate(W, perm, signs, h)           # W Pi^T
    Xp = oracle.rpbh_rotate(X, perm, signs, h)           # (Pi x) per token
    ref = X @ W.T
    got = Xp @ Wp.T
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-12


def test_norm_is_invariant():
    inp = synth.make(2, M=16, N=8)
    X = synth.bf16_bits_to_f32(inp["X"]).astype(np.float64)
    Xp = oracle.rpbh_rotate(X, inp["perm"], inp["signs"], inp["h"])
    np.testing.assert_allclose(np.linalg.norm(Xp, axis=1), np.linalg.norm(X, axis=1),
                               rtol=1e-13)


def _mc_second_moment(x, h, S, with_perm, seed):
    """d * E[(Pi x)_k^2] per coordinate over S random draws of (pi, D)."""
    d = x.shape[0]
    g = np.random.default_rng(seed)
    perms = np.argsort(g.random((S, d)), axis=1) if with_perm else np.tile(np.arange(d), (S, 1))
    signs = np.where(g.random((S, d)) < 0.5, -1.0, 1.0)
    y = x[perms] * signs
    z = oracle.fwht(y.reshape(S, d // h, h)).reshape(S, d) / np.sqrt(h)
    return d * np.mean(z * z, axis=0)


def test_permutation_gives_variance_one_over_d():
    # E_{pi,D}[(Pi x~)_k^2] = 1/d exactly for any unit x~ and any k: the signs
    # cancel cross terms, leaving (energy routed to k's block)/h, and a uniform
    # permutation routes h/d of the energy there on average.
    d, h, S = 256, 64, 20000
    x = np.zeros(d)
    x[3] = x[5] = 1 / np.sqrt(2)                           # a 2-spike direction
    v = _mc_second_moment(x, h, S, True, 11)
    assert 0.93 < v.min() and v.max() < 1.07               # CLT band ~6 sigma
    assert abs(v.mean() - 1.0) < 1e-12                     # sum_k z_k^2 = ||x||^2
    # Block-RHT (no permutation): the spikes stay in block 0, variance there
    # is d/h = 4 times too large and zero elsewhere.
    vb = _mc_second_moment(x, h, 2000, False, 12)
    assert np.all(np.abs(vb[:h] - d / h) < 0.5)
    np.testing.assert_allclose(vb[h:], 0.0, atol=1e-12)


def test_haar_is_orthogonal():
    Q = oracle.haar_matrix(96, 5)
    np.testing.assert_allclose(Q @ Q.T, np.eye(96), atol=1e-12)


def test_haar_distribution_moments():
    """Haar measure on O(d): every entry has mean 0 and variance 1/d, and the
    trace has mean 0 and second moment 1 (Diaconis & Shahshahani 1994, the
    moments of tr Q for Q uniform on O(d), d >= 2).  A QR without the sign
    correction of R's diagonal fails this: Householder QR gives
    Q[0, 0] = -|A[0, 0]| / ||A[:, 0]|| <= 0, so the mean of Q[0, 0] would be
    about -sqrt(2 / (pi d))."""
    d, n = 6, 4000
    Qs = np.stack([oracle.haar_matrix(d, 1000 + i) for i in range(n)])
    q00 = Qs[:, 0, 0]
    tr = np.trace(Qs, axis1=1, axis2=2)
    se = np.sqrt(1.0 / d / n)                        # standard error of a mean entry
    assert abs(q00.mean()) < 5 * se
    assert np.all(np.abs(Qs.mean(axis=0)) < 5 * se)
    assert abs((Qs ** 2).mean(axis=0).mean() - 1.0 / d) < 1e-12   # rows are unit vectors
    assert abs(tr.mean()) < 5 * np.sqrt(1.0 / n)                   # Var(tr Q) = 1
    assert abs((tr ** 2).mean() - 1.0) < 5 * np.sqrt(2.0 / n)      # E[tr^4] = 3


def test_down_permutation_folds_into_up_rows():
    """Pi_down GELU(z) with pi applied to z's rows first is the block
    rotation alone: blkdiag(H D) GELU(P_pi z) = Pi_down GELU(z) (GELU acts
    elementwise, so it commutes with the permutation)."""
    g = np.random.default_rng(11)
    d, h = 512, 128
    perm = g.permutation(d)
    signs = g.choice([-1.0, 1.0], size=d)
    Z = g.standard_normal((6, d)) * 2.0
    full = oracle.rpbh_rotate(oracle.gelu_erf(Z), perm, signs, h)
    folded = oracle.block_rht_rotate(oracle.gelu_erf(Z[:, perm]), signs, h)
    assert np.allclose(full, folded, rtol=0, atol=1e-12)
