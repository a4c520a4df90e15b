"""Walsh-Hadamard matrices for the RPBH rotation (fp64).

OrbitQuant page, Method: each diagonal block of Pi_d is H_h D_i with H_h the
Walsh-Hadamard matrix.  Reading taken: H_h in Sylvester (natural) order,
H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]; entries are +-1 here and the
1/sqrt(h) that makes the block orthonormal is applied by the caller.
"""
import numpy as np


def sylvester(h: int) -> np.ndarray:
    """Dense +-1 Hadamard matrix of order h (a power of two), Sylvester order."""
    if h < 1 or h & (h - 1):
        raise ValueError("h must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < h:
        H = np.block([[H, H], [H, -H]])
    return H


def fwht(y: np.ndarray) -> np.ndarray:
    """Unnormalised fast Walsh-Hadamard transform over the last axis: H_n y.

    Plain radix-2 butterflies in float64, one stage per bit of the index;
    the result equals sylvester(n) @ y.
    """
    y = np.array(y, dtype=np.float64, copy=True)
    n = y.shape[-1]
    if n & (n - 1):
        raise ValueError("length must be a power of two")
    lead = y.shape[:-1]
    span = 1
    while span < n:
        v = y.reshape(*lead, n // (2 * span), 2, span)
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        span *= 2
    return y
