"""Lloyd-Max scalar codebook for one rotated coordinate (oracle side).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

noze.it "TurboQuant-MLX: quantizzare pesi e KV cache...":
* section "Il metodo TurboQuant, in breve": after the random rotation every
  coordinate follows a known distribution and gets its own optimal scalar
  quantizer; no calibration data is used (data-oblivious);
* section "Cosa aggiunge turboquant-mlx": the optimal scalar quantizer is a
  Lloyd-Max codebook.

Reading taken (the page does not name the law): the rotated vector is a
uniform point on the unit sphere of R^d, whose single coordinate has density

    f_d(x) = K_d (1 - x^2)^((d - 3) / 2) on [-1, 1],
    K_d = Gamma(d/2) / (sqrt(pi) Gamma((d - 1)/2)),

equivalently (1 + x)/2 ~ Beta((d-1)/2, (d-1)/2).  The codebook is the
Lloyd-Max fixed point for f_d:

    boundaries t_j = (c_j + c_{j+1}) / 2        (nearest-neighbour condition)
    centroids  c_j = E[X | t_{j-1} < X < t_j]   (centroid condition)

iterated from the equal-mass quantile start until the centroids stop moving.
f_d is log-concave for d >= 3, so the fixed point is unique (Fleischer 1964)
and does not depend on the start.
"""
from __future__ import annotations

from dataclasses import dataclass
from functools import lru_cache

import numpy as np
from scipy import special


def density_const(d: int) -> float:
    """K_d, the normaliser of f_d."""
    return float(np.exp(special.gammaln(d / 2.0) - special.gammaln((d - 1) / 2.0)) / np.sqrt(np.pi))


def density(x, d: int):
    """f_d(x) for x in [-1, 1]."""
    x = np.asarray(x, dtype=np.float64)
    return density_const(d) * np.clip(1.0 - x * x, 0.0, None) ** ((d - 3) / 2.0)


def cdf(x, d: int):
    """P(X <= x) = I_{(1+x)/2}((d-1)/2, (d-1)/2) (regularised incomplete beta)."""
    a = (d - 1) / 2.0
    z = np.clip((1.0 + np.asarray(x, dtype=np.float64)) / 2.0, 0.0, 1.0)
    return special.betainc(a, a, z)


def first_moment(lo, hi, d: int):
    """Integral of x f_d(x) over [lo, hi] in closed form.

    The antiderivative of x (1 - x^2)^((d-3)/2) is -(1 - x^2)^((d-1)/2) / (d - 1).
    """
    p = (d - 1) / 2.0
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    g = lambda x: np.clip(1.0 - x * x, 0.0, None) ** p
    return density_const(d) / (d - 1) * (g(lo) - g(hi))


def cell_mass(lo, hi, d: int):
    """P(lo < X < hi), the difference of the two cdf values."""
    return cdf(hi, d) - cdf(lo, d)


@dataclass(frozen=True)
class Codebook:
    d: int
    bits: int
    centroids: np.ndarray   # 2**bits levels, ascending, symmetric about 0
    boundaries: np.ndarray  # 2**bits - 1 decision thresholds, ascending
    iterations: int

    @property
    def levels(self) -> int:
        return 1 << self.bits


def _lloyd_max(d: int, bits: int, tol: float, max_iter: int) -> Codebook:
    L = 1 << bits
    # Quantile start: centroids at the conditional means of L equal-mass cells.
    # Cell edges are the (j/L)-quantiles, found by bisection on the cdf.
    qs = np.arange(1, L) / L
    lo = np.full(L - 1, -1.0)
    hi = np.full(L - 1, 1.0)
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        below = cdf(mid, d) < qs
        lo = np.where(below, mid, lo)
        hi = np.where(below, hi, mid)
    t = 0.5 * (lo + hi)
    edges = np.concatenate(([-1.0], t, [1.0]))
    c = first_moment(edges[:-1], edges[1:], d) / cell_mass(edges[:-1], edges[1:], d)
    it = 0
    best_step = np.inf
    stall = 0
    while it < max_iter:
        it += 1
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate(([-1.0], t, [1.0]))
        c_new = first_moment(edges[:-1], edges[1:], d) / cell_mass(edges[:-1], edges[1:], d)
        c_new = 0.5 * (c_new - c_new[::-1])  # the law is symmetric: keep the codebook so
        step = float(np.max(np.abs(c_new - c)))
        c = c_new
        if step < tol:
            break
        # Linear convergence can stall at the rounding floor above tol; stop then.
        if step < best_step:
            best_step, stall = step, 0
        else:
            stall += 1
            if stall > 50 and step < 1e-13:
                break
    t = 0.5 * (c[:-1] + c[1:])
    if L % 2 == 0:
        t[L // 2 - 1] = 0.0  # middle threshold of a symmetric codebook is exactly 0
    return Codebook(d=d, bits=bits, centroids=c, boundaries=t, iterations=it)


@lru_cache(maxsize=None)
def lloyd_max(d: int, bits: int, tol: float = 1e-15, max_iter: int = 200000) -> Codebook:
    """Lloyd-Max codebook (float64) for one coordinate of a uniform unit vector in R^d."""
    if d < 3 or not (1 <= bits <= 8):
        raise ValueError("need d >= 3 and 1 <= bits <= 8")
    return _lloyd_max(d, bits, tol, max_iter)


def mse(cb: Codebook) -> float:
    """Per-coordinate mean squared error E[(X - Q(X))^2] of the codebook under f_d.

    The integrand (x - c_j)^2 f_d(x) is integrated cell by cell with 200-point
    Gauss-Legendre quadrature, so this does not reuse the closed-form mass or
    first moment that the iteration itself relies on.
    """
    d = cb.d
    edges = np.concatenate(([-1.0], cb.boundaries, [1.0]))
    xg, wg = np.polynomial.legendre.leggauss(200)
    total = 0.0
    for j in range(cb.levels):
        a, b = edges[j], edges[j + 1]
        x = 0.5 * (b - a) * xg + 0.5 * (a + b)
        w = 0.5 * (b - a) * wg
        total += float(np.sum(w * (x - cb.centroids[j]) ** 2 * density(x, d)))
    return total


def distortion(cb: Codebook) -> float:
    """d * MSE: expected squared reconstruction error of a unit vector."""
    return cb.d * mse(cb)
