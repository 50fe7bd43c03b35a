"""Lloyd-Max scalar quantizer for the standard normal law, in float64.

TQ4 page, "格式原理" item 2: after the rotation every coordinate is mapped
on its own to the nearest of the optimal centroids for N(0,1).  The paragraph
after the list says the codebook is built with Lloyd's algorithm on the
distribution of the rotated coordinates (with a closed form for 1 and 2 bits),
and that going from 8 to 16 centroids cut the quantization error by 72.5%.

Lloyd's algorithm for a density p with L levels alternates two conditions
until it reaches a fixed point:

* nearest-neighbour: the decision boundaries are the midpoints of adjacent
  centroids;
* centroid: each centroid is the conditional mean of X over its cell,
  E[X | a < X < b] = (phi(a) - phi(b)) / (Phi(b) - Phi(a)) for N(0,1).

The mean squared error of a codebook with boundaries a_k, b_k and
representatives c_k is sum_k E[(X - c_k)^2 ; a_k < X < b_k], which for the
normal law integrates in closed form (see :func:`cell_distortion`).

Only the standard library's ``erfc``/``exp`` are used; numbers are float64.
Test infrastructure only (see the package docstring).
"""

import math

import numpy as np

_INV_SQRT2 = 1.0 / math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def pdf(x: float) -> float:
    """Standard normal density phi(x); 0 at +-inf."""
    if math.isinf(x):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * x * x)


def cell_mass(a: float, b: float) -> float:
    """P(a < X < b) for X ~ N(0,1), a <= b (either may be infinite).

    Uses erfc on the side away from the origin so that tail cells keep full
    relative precision (Phi(x) = erfc(-x/sqrt(2))/2).
    """
    if a >= 0.0:
        return 0.5 * (math.erfc(a * _INV_SQRT2) - math.erfc(b * _INV_SQRT2))
    if b <= 0.0:
        return 0.5 * (math.erfc(-b * _INV_SQRT2) - math.erfc(-a * _INV_SQRT2))
    return 1.0 - 0.5 * math.erfc(-a * _INV_SQRT2) - 0.5 * math.erfc(b * _INV_SQRT2)


def _x_pdf(x: float) -> float:
    """x*phi(x), with the limit 0 at +-inf."""
    if math.isinf(x):
        return 0.0
    return x * pdf(x)


def cell_centroid(a: float, b: float) -> float:
    """E[X | a < X < b] for X ~ N(0,1)."""
    return (pdf(a) - pdf(b)) / cell_mass(a, b)


def cell_distortion(a: float, b: float, c: float) -> float:
    """Integral over (a, b) of (x - c)^2 phi(x) dx.

    With  int x^2 phi = Phi - x phi,  int x phi = -phi,  int phi = Phi:
      = [P - (b phi(b) - a phi(a))] - 2c [phi(a) - phi(b)] + c^2 P,
    where P = Phi(b) - Phi(a).
    """
    p = cell_mass(a, b)
    return (p - (_x_pdf(b) - _x_pdf(a))) - 2.0 * c * (pdf(a) - pdf(b)) + c * c * p


def boundaries(centroids) -> list:
    """Decision boundaries of the nearest-neighbour rule: -inf, midpoints, +inf."""
    c = list(centroids)
    mids = [(c[k] + c[k + 1]) / 2.0 for k in range(len(c) - 1)]
    return [-math.inf] + mids + [math.inf]


def distortion(centroids) -> float:
    """Mean squared error of nearest-neighbour quantization of N(0,1) to ``centroids``."""
    bnd = boundaries(centroids)
    return sum(cell_distortion(bnd[k], bnd[k + 1], c) for k, c in enumerate(centroids))


def lloyd_step(centroids) -> list:
    """One Lloyd iteration: midpoint boundaries, then conditional means."""
    bnd = boundaries(centroids)
    return [cell_centroid(bnd[k], bnd[k + 1]) for k in range(len(centroids))]


def lloyd_max_normal(levels: int, tol: float = 1e-15, max_iter: int = 200000,
                     start=None, history: bool = False):
    """Lloyd-Max codebook of ``levels`` ascending centroids for N(0,1), float64.

    Starts from ``start`` (default: ``levels`` evenly spaced points on
    [-2, 2], a symmetric start) and iterates :func:`lloyd_step` until the
    largest centroid change is below ``tol``.  Returns the centroids (and, if
    ``history``, the list of distortions after every step, starting with the
    start codebook's).  Raises if it does not converge.
    """
    if start is None:
        c = [-2.0 + 4.0 * (k + 0.5) / levels for k in range(levels)]
    else:
        c = [float(v) for v in start]
    hist = [distortion(c)]
    for _ in range(max_iter):
        nc = lloyd_step(c)
        delta = max(abs(u - v) for u, v in zip(nc, c))
        c = nc
        if history:
            hist.append(distortion(c))
        if delta < tol:
            return (c, hist) if history else c
    raise RuntimeError(f"Lloyd iteration for {levels} levels did not converge")


def tq4_codebook_f32():
    """The 16 TQ4_1S centroids as float32 (ascending; index 0 is the most negative).

    Reading taken: the fp64 Lloyd-Max fixed point rounded to float32 (the pages
    print no values).  Index order is ascending so that index k is the k-th
    smallest centroid.
    """
    return np.asarray(lloyd_max_normal(16), dtype=np.float64).astype(np.float32)


def tq4_midpoints_f32(c32=None):
    """The 15 decision thresholds m_k = float32((c_k + c_{k+1}) / 2), sum in fp64."""
    if c32 is None:
        c32 = tq4_codebook_f32()
    c = np.asarray(c32, dtype=np.float64)
    return ((c[:-1] + c[1:]) / 2.0).astype(np.float32)
