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

The exact marginal (``lloyd_max_sphere``): one coordinate T of a direction
drawn uniformly from the unit sphere S^{d-1} has density
f_d(t) = C_d (1 - t^2)^((d-3)/2) on [-1, 1], C_d = Gamma(d/2) /
(sqrt(pi) Gamma((d-1)/2)), and T^2 ~ Beta(1/2, (d-1)/2).  In N(0,1) units
U = sqrt(d) T, so for 0 <= u < sqrt(d), with t = u / sqrt(d):
  upper tail     P(U > u) = (1 - I_{t^2}(1/2, (d-1)/2)) / 2  (regularized beta)
  first moment   int_u^sqrt(d) v g(v) dv = sqrt(d) C_d (1 - t^2)^((d-1)/2) / (d-1)
(the second from d/dt (1-t^2)^((d-1)/2) = -(d-1) t (1-t^2)^((d-3)/2)); the
centroid of (a, b] is the difference of first moments over the difference of
tails, as for the Gaussian, whose first-moment tail is phi(u).  f_d is
log-concave for d >= 3, so the fixed point is again unique.  As d grows f_d
in these units tends to N(0,1).
"""
import functools

import numpy as np
from scipy.optimize import fsolve
from scipy.special import betainc, betaincc, erfc, gammaln
from scipy.stats import norm

_SQRT2 = np.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / np.sqrt(2.0 * np.pi)


def _phi(x):
    return np.exp(-0.5 * x * x) * _INV_SQRT_2PI


def _upper_tail(x):
    return 0.5 * erfc(x / _SQRT2)


def _cell_edges(cpos, top=np.inf):
    """Positive-half cell edges 0 = tau_0 < tau_1 < ... < tau_{h-1} < tau_h = top."""
    return np.concatenate([[0.0], 0.5 * (cpos[:-1] + cpos[1:]), [top]])


def _gauss_moment(x):
    return _phi(x)  # int_x^inf v phi(v) dv


def _sphere_fns(d):
    """Upper tail and first-moment tail of U = sqrt(d) T (see the module note)."""
    if d < 3:
        raise ValueError("the sphere marginal needs d >= 3")
    rd = np.sqrt(float(d))
    log_c = gammaln(d / 2.0) - gammaln((d - 1) / 2.0) - 0.5 * np.log(np.pi)

    def tail(u):
        # I_{1-t^2}((d-1)/2, 1/2) = 1 - I_{t^2}(1/2, (d-1)/2), evaluated as the
        # complement from t^2 itself: forming 1 - t^2 first would amplify its
        # rounding by about (d-1)/2
        t2 = np.minimum(np.asarray(u, dtype=np.float64) / rd, 1.0) ** 2
        return 0.5 * betaincc(0.5, (d - 1) / 2.0, t2)

    def moment(u):
        t2 = np.minimum(np.asarray(u, dtype=np.float64) / rd, 1.0) ** 2
        with np.errstate(divide="ignore"):
            return rd * np.exp(log_c + 0.5 * (d - 1) * np.log1p(-t2)) / (d - 1)

    return tail, moment, rd


def _lloyd_max(levels, tail, moment, top, start, max_iter):
    """Lloyd-Max for a symmetric density given its upper tail P(X > x) and
    first-moment tail E[X; X > x] on the positive half (support up to top)."""
    if levels < 2 or levels % 2:
        raise ValueError("levels must be an even number >= 2")
    half = levels // 2

    def centroids(tau):
        a, b = tau[:-1], tau[1:]
        return (moment(a) - moment(b)) / (tail(a) - tail(b))

    c = start(half)
    it = 0
    for it in range(1, max_iter + 1):
        c_new = centroids(_cell_edges(c, top))
        step = np.max(np.abs(c_new - c))
        c = c_new
        if step < 1e-11:
            break
    if half > 1:
        fixed_point = lambda v: centroids(_cell_edges(v, top)) - v  # noqa: E731
        c, info, ier, msg = fsolve(fixed_point, c, xtol=1e-15, full_output=True)
        # ier != 1 only reports that no further progress was possible; the
        # residual decides whether the fixed point was reached
        if np.max(np.abs(fixed_point(c))) > 1e-13:
            raise RuntimeError(f"Lloyd-Max fixed point not reached: {msg}")
    tau = _cell_edges(c, top)
    pos_prob = tail(tau[:-1]) - tail(tau[1:])
    centroids_all = np.concatenate([-c[::-1], c])
    thresholds = np.concatenate([-tau[1:-1][::-1], [0.0], tau[1:-1]])
    cell_prob = np.concatenate([pos_prob[::-1], pos_prob])
    # at the centroid fixed point E[X Q(X)] = E[Q(X)^2]; E[X^2] = 1 for both
    # marginals in N(0,1) units, so D = 1 - sum p c^2
    distortion = 1.0 - np.sum(cell_prob * centroids_all ** 2)
    return dict(centroids=centroids_all, thresholds=thresholds, distortion=distortion,
                cell_prob=cell_prob, iterations=it)


def lloyd_max_gaussian(levels: int, max_iter: int = 200000):
    """Lloyd-Max quantizer of N(0,1) with `levels` (even) output levels.

    Returns dict(centroids[levels] ascending, thresholds[levels-1] ascending,
    distortion D = E[(X - Q(X))^2], cell_prob[levels], iterations).
    """
    # start: the conditional means' positions at equal-probability quantiles
    start = lambda half: norm.ppf(0.5 + (np.arange(half) + 0.5) / (2 * half))  # noqa: E731
    return _lloyd_max(levels, _upper_tail, _gauss_moment, np.inf, start, max_iter)


@functools.lru_cache(maxsize=None)
def _gaussian_positive_centroids(half):
    c = lloyd_max_gaussian(2 * half)["centroids"][half:]
    c.setflags(write=False)
    return c


def lloyd_max_sphere(levels: int, d: int, max_iter: int = 200):
    """Lloyd-Max quantizer of the exact marginal f_d of one coordinate of a
    uniform direction on S^{d-1}, in N(0,1) units (U = sqrt(d) T, |U| <=
    sqrt(d), E[U^2] = 1).  Same return value as lloyd_max_gaussian.

    The fixed point is unique (f_d is log-concave for d >= 3), so the start
    only affects the work: the N(0,1) codebook, shrunk into the support when
    its outer level lies beyond 0.9 sqrt(d); at most max_iter Lloyd steps,
    then the fixed-point polish."""
    tail, moment, rd = _sphere_fns(d)

    def start(half):
        c = _gaussian_positive_centroids(half)
        return c * min(1.0, 0.9 * rd / c[-1])
    return _lloyd_max(levels, tail, moment, rd, start, max_iter)


def sphere_distortion(centroids, thresholds, d):
    """E[(U - Q(U))^2] of any quantizer (sorted centroids, thresholds) under
    the sphere marginal: E[U^2] - 2 sum_j c_j E[U; cell j] + sum_j c_j^2 P(cell j).
    By symmetry E[U; U > x] = moment(|x|) and P(U > x) = 1 - tail(-x) for
    x < 0, so both sums come from the positive-half functions."""
    tail, moment, rd = _sphere_fns(d)
    c = np.asarray(centroids, dtype=np.float64)
    edges = np.concatenate([[-rd], np.asarray(thresholds, dtype=np.float64), [rd]])
    up = np.where(edges >= 0, tail(np.abs(edges)), 1.0 - tail(np.abs(edges)))  # P(U > x)
    first_up = moment(np.abs(edges))                                           # E[U; U > x]
    mass = up[:-1] - up[1:]
    first = first_up[:-1] - first_up[1:]
    return 1.0 - 2.0 * np.sum(c * first) + np.sum(c * c * mass)


def codebook_sphere(bits: int, d: int):
    """The 2^bits-level codebook of the exact marginal f_d, N(0,1) units."""
    return lloyd_max_sphere(2 ** bits, d)


def codebook(bits: int):
    """The 2^bits-level codebook in N(0,1) units (see the module note)."""
    return lloyd_max_gaussian(2 ** bits)
