"""The data-free scale objective behind Universal Optimal Scaling (CPU oracle; test infrastructure).

Sources (page titles and sections):
  * Pith review of MXAttention, Referee summary and major comment 1 (sec. 4.1,
    Eqs. 21-23): J(q) = E[D(X_q)], with D(x) = E(x)/x**3 and
    E(x) = integral_0^x (v - Pi(v))**2 dv, Pi the projection onto the
    non-negative E2M1 grid, X_q the normalised block maximum under the ceiling
    rule with boundary q.
  * Same review, What carries the argument and Axiom ledger (Lemma 1, Eqs.
    31-32): with power-of-two scaling, log2 X_q has the 1-periodic wrapped
    density h of log2 M, and the sign of J'(q) is the sign of D(q) - D(q/2).
  * Same review, Figure 2 caption: J(q) under a log-uniform density and
    under non-uniform wrapped densities ("first harmonic", "two harmonics",
    "concentrated") all share the minimum q = 7.25; the first branch of the
    difference is negative and in the second the factor 4q - 27 vanishes
    outside the interval.  Referee summary: the closed-form boundary is
    29/4 = 7.25.

Readings: Pi(v) is the nearest grid point, saturating at 6 for v > 6.  The
four wrapped densities used for the sweep are this repository's choice (the
pages do not print their coefficients): h = 1; 1 + 0.8 cos(2 pi u);
1 + 0.5 cos(2 pi u) + 0.4 sin(4 pi u + 0.3); a wrapped normal with sigma 0.08
centred at u = 0.8.  Integrals are numerical (scipy quad with the grid's
breakpoints), not closed forms.
"""
from __future__ import annotations

import math

import numpy as np
from scipy import integrate

GRID_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
# points where the integrand (v - Pi(v))**2 changes its formula: grid points and midpoints
_BREAKS = np.unique(np.concatenate([GRID_POS, (GRID_POS[1:] + GRID_POS[:-1]) / 2]))


def project(v):
    """Pi(v): the nearest non-negative E2M1 grid point (6 for everything above 6)."""
    v = np.asarray(v, dtype=np.float64)
    return GRID_POS[np.argmin(np.abs(v[..., None] - GRID_POS), axis=-1)]


def _sq_err(v):
    return (v - project(v)) ** 2


def E(x):
    """E(x) = integral_0^x (v - Pi(v))**2 dv.

    Summed piece by piece between consecutive breakpoints, where the integrand
    is a single quadratic, with 3-point Gauss-Legendre (exact for quadratics).
    Vectorised over x."""
    x = np.atleast_1d(np.asarray(x, dtype=np.float64))
    t, w = np.polynomial.legendre.leggauss(3)
    edges = np.concatenate([_BREAKS, [np.inf]])
    total = np.zeros_like(x)
    for a, b in zip(edges[:-1], edges[1:]):
        hi = np.minimum(b, x)
        m = hi > a
        if not m.any():
            continue
        lo_, hi_ = a, hi[m]
        half = (hi_ - lo_) / 2
        mid = (hi_ + lo_) / 2
        nodes = mid[:, None] + half[:, None] * t
        total[m] += half * (_sq_err(nodes) * w).sum(axis=1)
    return total


def E_quad(x: float) -> float:
    """E(x) by scipy's adaptive quadrature (an independent cross-check of E)."""
    if x <= 0:
        return 0.0
    pts = [p for p in _BREAKS if 0 < p < x]
    val, _ = integrate.quad(lambda v: float(_sq_err(v)), 0.0, x, points=pts or None,
                            limit=200, epsabs=1e-15, epsrel=1e-13)
    return val


def D(x):
    x = np.asarray(x, dtype=np.float64)
    return E(x) / np.atleast_1d(x) ** 3


def delta(q):
    """Delta(q) = D(q) - D(q/2): the factor that decides the sign of J'(q)."""
    q = np.asarray(q, dtype=np.float64)
    return D(q) - D(q / 2.0)


def density_log_uniform(u):
    return np.ones_like(np.asarray(u, dtype=np.float64))


def density_first_harmonic(u):
    return 1.0 + 0.8 * np.cos(2 * np.pi * np.asarray(u))


def density_two_harmonics(u):
    u = np.asarray(u)
    return 1.0 + 0.5 * np.cos(2 * np.pi * u) + 0.4 * np.sin(4 * np.pi * u + 0.3)


def density_concentrated(u, centre: float = 0.8, sigma: float = 0.08):
    u = np.asarray(u, dtype=np.float64)
    k = np.arange(-4, 5)
    z = (u[..., None] - centre - k) / sigma
    return np.exp(-0.5 * z ** 2).sum(axis=-1) / (sigma * math.sqrt(2 * math.pi))


DENSITIES = {
    "log-uniform": density_log_uniform,
    "first-harmonic": density_first_harmonic,
    "two-harmonics": density_two_harmonics,
    "concentrated": density_concentrated,
}


def J(q: float, h=density_log_uniform, nodes: int = 48) -> float:
    """J(q) = integral over one period of D(2**u) h(u) du, u in (log2 q - 1, log2 q].

    (X_q = M / 2**e lies in (q/2, q]; its log2 has the wrapped density h.)
    Gauss-Legendre with `nodes` points on each piece between breakpoints."""
    lo, hi = math.log2(q) - 1.0, math.log2(q)
    cuts = [lo] + [math.log2(p) for p in _BREAKS if q / 2 < p < q] + [hi]
    t, w = np.polynomial.legendre.leggauss(nodes)
    total = 0.0
    for a, b in zip(cuts[:-1], cuts[1:]):
        u = (a + b) / 2 + (b - a) / 2 * t
        total += (b - a) / 2 * float((D(2.0 ** u) * h(u) * w).sum())
    return total


def J_quad(q: float, h=density_log_uniform) -> float:
    """J(q) by nested adaptive quadrature (slow; cross-checks J at a few points)."""
    lo, hi = math.log2(q) - 1.0, math.log2(q)
    pts = [math.log2(p) for p in _BREAKS if q / 2 < p < q]
    val, _ = integrate.quad(lambda u: E_quad(2.0 ** u) / 2.0 ** (3 * u) * float(h(u)), lo, hi,
                            points=pts or None, limit=200, epsabs=1e-14, epsrel=1e-12)
    return val
