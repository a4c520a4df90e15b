"""Lloyd-Max codebook for the fixed marginal of rotated coordinates (fp64).

OrbitQuant page, Method: after the RPBH rotation a unit vector's coordinates
follow a fixed marginal f_d close to N(0, 1/d); Lloyd-Max is run offline on
f_d to get a single codebook C_d per input dimension d, shared by weights
and activations of that dimension.

Reading taken: f_d = N(0, 1/d).  A Lloyd-Max quantizer is scale-equivariant,
so C_d is the N(0,1) codebook divided by sqrt(d); this module returns the
N(0,1) codebook ("N(0,1) units") and callers scale by 1/sqrt(d).

Lloyd-Max conditions for a density f with K levels (Lloyd 1957 / Max 1960):
  thresholds  t_j = (c_j + c_{j+1}) / 2                (nearest neighbour)
  centroids   c_j = E[X | t_{j-1} < X <= t_j]           (centroid)
For N(0,1): E[X | a < X <= b] = (phi(a) - phi(b)) / (Q(a) - Q(b)) with phi the
density and Q(x) = erfc(x / sqrt 2) / 2 the upper tail (erfc keeps the tail
masses accurate).  The density is symmetric, so only the positive half is
iterated and the negative half is its mirror image: the codebook is exactly
symmetric and the middle threshold is exactly 0.

Iteration: plain Lloyd alternation from a quantile start until the centroid
step is below 1e-11, then the same fixed-point equations c = F(c) are solved
to machine precision with scipy.optimize.fsolve (MINPACK).  For a
log-concave density the fixed point is unique (Fleischer 1964), so any
correct solver lands on the same codebook.
"""
import numpy as np
from scipy.optimize import fsolve
from scipy.special import erfc
from scipy.stats import norm

_SQRT2 = np.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


def _phi(x):
    return np.exp(-0.5 * x * x) * _INV_SQRT_2PI


def _upper_tail(x):
    return 0.5 * erfc(x / _SQRT2)


def _cell_edges(cpos):
    """Positive-half cell edges 0 = tau_0 < tau_1 < ... < tau_{h-1} < tau_h = inf."""
    return np.concatenate([[0.0], 0.5 * (cpos[:-1] + cpos[1:]), [np.inf]])


def _centroids(tau):
    a, b = tau[:-1], tau[1:]
    return (_phi(a) - _phi(b)) / (_upper_tail(a) - _upper_tail(b))


def lloyd_max_gaussian(levels: int, max_iter: int = 200000):
    """Lloyd-Max quantizer of N(0,1) with `levels` (even) output levels.

    Returns dict(centroids[levels] ascending, thresholds[levels-1] ascending,
    distortion D = E[(X - Q(X))^2], cell_prob[levels], iterations).
    """
    if levels < 2 or levels % 2:
        raise ValueError("levels must be an even number >= 2")
    half = levels // 2
    # start: the conditional means' positions at equal-probability quantiles
    c = norm.ppf(0.5 + (np.arange(half) + 0.5) / (2 * half))
    it = 0
    for it in range(1, max_iter + 1):
        c_new = _centroids(_cell_edges(c))
        step = np.max(np.abs(c_new - c))
        c = c_new
        if step < 1e-11:
            break
    if half > 1:
        fixed_point = lambda v: _centroids(_cell_edges(v)) - v
        c, info, ier, msg = fsolve(fixed_point, c, xtol=1e-15, full_output=True)
        # ier != 1 only reports that no further progress was possible; the
        # residual decides whether the fixed point was reached
        if np.max(np.abs(fixed_point(c))) > 1e-13:
            raise RuntimeError(f"Lloyd-Max fixed point not reached: {msg}")
    tau = _cell_edges(c)
    pos_prob = _upper_tail(tau[:-1]) - _upper_tail(tau[1:])
    centroids = np.concatenate([-c[::-1], c])
    thresholds = np.concatenate([-tau[1:-1][::-1], [0.0], tau[1:-1]])
    cell_prob = np.concatenate([pos_prob[::-1], pos_prob])
    # at the centroid fixed point E[X Q(X)] = E[Q(X)^2], so D = 1 - sum p c^2
    distortion = 1.0 - np.sum(cell_prob * centroids ** 2)
    return dict(centroids=centroids, thresholds=thresholds, distortion=distortion,
                cell_prob=cell_prob, iterations=it)


def codebook(bits: int):
    """The 2^bits-level codebook in N(0,1) units (see the module note)."""
    return lloyd_max_gaussian(2 ** bits)
