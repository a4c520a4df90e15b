"""The random rotations of the method, in fp64.

OrbitQuant page, Method: the randomized permuted block-Hadamard (RPBH)
rotation is Pi_d = blkdiag(H_h D_1, ..., H_h D_{d/h}) P_pi with H_h the
Walsh-Hadamard matrix, D_i Rademacher sign diagonals and P_pi a uniform
random permutation; the permutation spreads coordinates across blocks.

Readings taken: (P_pi x)_k = x[pi(k)] (gather); D_i acts on the permuted
coordinates of block i; H_h / sqrt(h) so Pi_d is orthogonal.  Hence
(Pi_d x) = for each block b: H_h/sqrt(h) (signs * x[perm])[b*h:(b+1)*h].

The ablation in the Experiments section also names Block-RHT (RPBH without
the permutation), Full RHT (one randomized Hadamard over all of d) and a
dense Haar rotation; they are here as special cases for comparison.
"""
import numpy as np

from .hadamard import sylvester, fwht


def _check(perm, signs, h):
    perm = np.asarray(perm)
    signs = np.asarray(signs)
    d = perm.shape[0]
    if signs.shape != (d,) or d % h:
        raise ValueError("need len(signs) == len(perm) == d and d % h == 0")
    if not np.array_equal(np.sort(perm), np.arange(d)):
        raise ValueError("perm is not a permutation of 0..d-1")
    return perm.astype(np.int64), signs.astype(np.float64), d


def rpbh_matrix(perm, signs, h) -> np.ndarray:
    """Dense Pi_d = B P, B = blkdiag(H_h D_1, ...)/sqrt(h), P[k, perm[k]] = 1."""
    perm, signs, d = _check(perm, signs, h)
    P = np.zeros((d, d))
    P[np.arange(d), perm] = 1.0
    Hh = sylvester(h) / np.sqrt(h)
    B = np.zeros((d, d))
    for b in range(d // h):
        sl = slice(b * h, (b + 1) * h)
        B[sl, sl] = Hh @ np.diag(signs[sl])
    return B @ P


def rpbh_rotate(X, perm, signs, h) -> np.ndarray:
    """x' = Pi_d x for every row x of X (the activation side; the weight side
    W' = W Pi_d^T is the same map on the rows of W)."""
    perm, signs, d = _check(perm, signs, h)
    X = np.asarray(X, dtype=np.float64)
    y = X[..., perm] * signs                     # D (P_pi x)
    lead = y.shape[:-1]
    z = fwht(y.reshape(*lead, d // h, h))        # H_h per block
    return z.reshape(*lead, d) / np.sqrt(h)


def rpbh_inverse_rotate(Xp, perm, signs, h) -> np.ndarray:
    """x = Pi_d^T x' for every row (undoes rpbh_rotate).

    Pi^T = P^T blkdiag(D_i H_h)/sqrt(h): Hadamard per block (H_h symmetric),
    then the signs, then scatter back through the permutation.
    """
    perm, signs, d = _check(perm, signs, h)
    Xp = np.asarray(Xp, dtype=np.float64)
    lead = Xp.shape[:-1]
    y = fwht(Xp.reshape(*lead, d // h, h)).reshape(*lead, d) / np.sqrt(h)
    y = y * signs
    x = np.empty_like(y)
    x[..., perm] = y
    return x


def block_rht_rotate(X, signs, h) -> np.ndarray:
    """Block-RHT: RPBH with the identity permutation."""
    d = np.asarray(signs).shape[0]
    return rpbh_rotate(X, np.arange(d), signs, h)


def full_rht_rotate(X, perm, signs) -> np.ndarray:
    """Full RHT: one randomized Hadamard over all of d (h = d)."""
    d = np.asarray(signs).shape[0]
    return rpbh_rotate(X, perm, signs, d)


def haar_matrix(d: int, seed: int) -> np.ndarray:
    """A Haar-distributed random orthogonal d x d matrix (QR of a Gaussian
    matrix with the signs of R's diagonal moved into Q)."""
    g = np.random.Generator(np.random.PCG64(seed))
    A = g.standard_normal((d, d))
    Q, R = np.linalg.qr(A)
    return Q * np.sign(np.diag(R))
