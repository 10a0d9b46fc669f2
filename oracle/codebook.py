"""Lloyd-Max codebook for one rotated coordinate.

"TurboQuant QJL投影深度剖析" §二 step 1: after the random rotation every
coordinate of the unit vector follows a scaled Beta law (close to N(0, 1/d) in
high dimension).  §二 step 2: the codebook is the optimal scalar quantiser for
that law, found by solving a continuous 1-D k-means (Lloyd-Max) problem, and
each coordinate is quantised by looking up its decision interval.  The MLX
write-up (背景) calls this the PolarQuant stage, with b-1 bits for K and all b
bits for V.

Readings:
  * The law used is the exact one, not the Gaussian approximation: one
    coordinate t of a uniform unit vector in R^d has density
        f_d(t) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) * (1 - t^2)^((d-3)/2)
    on [-1, 1], i.e. (t + 1)/2 ~ Beta((d-1)/2, (d-1)/2).
  * Lloyd's two conditions are iterated in the usual order: boundaries are
    midpoints of neighbouring centroids; each centroid is the conditional mean
    of its cell.  Cell masses use the regularised incomplete beta function and
    the cell first moment its closed form
        int_a^b t f_d(t) dt = C/(d-1) * ((1-a^2)^((d-1)/2) - (1-b^2)^((d-1)/2)).
  * Start: centroids at the (k + 1/2)/n quantiles of f_d.  Stop when no
    centroid moves by 1e-15 or more.
  * The law is symmetric, so the optimum is (the quantiser's fixed point is
    unique because f_d is log-concave for d >= 3).  The final centroids are
    projected onto exact antisymmetry, c_k = -c_{n-1-k}, which only removes
    rounding noise and makes the middle boundary exactly 0 for every even n.
  * Storage precision (the pages store the codebook as a precomputed table
    but do not say at what precision): the table is fp32, the precision in
    which the pages keep the rotation (QJL deep-dive §二: Pi is a 64 KB table,
    128 x 128 four-byte values).  Dequantisation and the key residual apply the
    Lloyd-Max centroids rounded to the nearest fp32; decisions compare fp32
    rotated coordinates with the fp32 roundings of the exact midpoints.
"""
import math

import numpy as np
from scipy import special


def density_const(d: int) -> float:
    return math.exp(math.lgamma(d / 2.0) - math.lgamma((d - 1) / 2.0)) / math.sqrt(math.pi)


def density(t, d: int):
    t = np.asarray(t, dtype=np.float64)
    return density_const(d) * np.power(np.clip(1.0 - t * t, 0.0, None), (d - 3) / 2.0)


def cdf(t, d: int):
    a = (d - 1) / 2.0
    return special.betainc(a, a, (np.asarray(t, np.float64) + 1.0) / 2.0)


def first_moment(a, b, d: int):
    e = (d - 1) / 2.0
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return density_const(d) / (d - 1) * (np.power(np.clip(1 - a * a, 0, None), e)
                                         - np.power(np.clip(1 - b * b, 0, None), e))


def lloyd_max(d: int, bits: int, tol: float = 1e-15, max_iter: int = 200000):
    """Return (centroids, boundaries, iterations) as float64 arrays; 2**bits
    ascending centroids and 2**bits - 1 boundaries."""
    if d < 3:
        raise ValueError("the coordinate law needs d >= 3")
    n = 1 << bits
    a = (d - 1) / 2.0
    probs = (np.arange(n) + 0.5) / n
    c = 2.0 * special.betaincinv(a, a, probs) - 1.0
    it = 0
    for it in range(1, max_iter + 1):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        mass = cdf(edges[1:], d) - cdf(edges[:-1], d)
        c_new = first_moment(edges[:-1], edges[1:], d) / mass
        step = np.max(np.abs(c_new - c))
        c = c_new
        if step < tol:
            break
    c = 0.5 * (c - c[::-1])
    t = 0.5 * (c[:-1] + c[1:])
    return c, t, it


def coordinate_mse(c, t, d: int) -> float:
    """E[(y - Q(y))^2] for one coordinate, using the centroid condition:
    E[y^2] - sum_k c_k^2 P(cell k), with E[y^2] = 1/d."""
    edges = np.concatenate(([-1.0], t, [1.0]))
    mass = cdf(edges[1:], d) - cdf(edges[:-1], d)
    return 1.0 / d - float(np.sum(c * c * mass))


_CACHE = {}


def codebook(d: int, bits: int):
    """Cached exact (centroids, boundaries) for (d, bits)."""
    key = (d, bits)
    if key not in _CACHE:
        c, t, _ = lloyd_max(d, bits)
        _CACHE[key] = (c, t)
    return _CACHE[key]


def table_centroids(c) -> np.ndarray:
    """Reconstruction values as held in the fp32 codebook table: each centroid
    rounded to the nearest fp32, returned as float64."""
    return np.asarray(c, np.float64).astype(np.float32).astype(np.float64)


def table_codebook(d: int, bits: int):
    """(fp32-table centroids, exact boundaries): the codebook that compression
    and dequantisation apply (decide() rounds the boundaries to fp32)."""
    c, t = codebook(d, bits)
    return table_centroids(c), t
