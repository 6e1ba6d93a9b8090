"""Lloyd-Max scalar codebook for the standard normal law.

Test infrastructure only (see ``oracle/__init__.py``).

The turboquant-plus-rs README ("Architecture" step 1; "Modules" ``codebook``)
states that each rotated coordinate is quantized by the MSE-optimal scalar
quantizer of the post-rotation Gaussian, found by Lloyd's algorithm (closed
form at 1 bit).  Reading: the rotated, norm-divided coordinate
z = H(D x)/|x| is treated as N(0, 1) (the "post-rotation Gaussian").

Lloyd's two optimality conditions for a density with L = 2**k cells:
  * each threshold is the midpoint of its two neighbouring centroids;
  * each centroid is the conditional mean of its cell,
      c_i = (phi(t_{i-1}) - phi(t_i)) / (Phi(t_i) - Phi(t_{i-1}))
    for the normal density phi and CDF Phi, with t_{-1} = -inf, t_{L-1} = +inf.
The codebook is the fixed point of the map c -> (conditional means of the
midpoint cells).  It is reached by plain Lloyd iterations from the quantile
start c_i = Phi^{-1}((i + 1/2)/L) until the largest move is below 1e-6, then
by Newton steps on the same fixed-point equations (the map's Jacobian is
tridiagonal), which take it to the limit of float64 evaluation.  The normal
law is log-concave, so the fixed point is unique and the start does not
matter; it is also symmetric, c_i = -c_{L-1-i}, and every iterate is made
exactly antisymmetric so that the middle threshold is exactly 0.

Stored form (what both sides of the codec use): centroids rounded to float32
and thresholds = float32 of the float64 midpoints.

Pins (tests/test_oracle_lloyd.py): the 1-bit closed form +-sqrt(2/pi) and its
distortion 1 - 2/pi; the fixed-point conditions; symmetry; the published
Max (1960) table for 2 and 3 bits; an independent k-means solve on dense
normal quantiles; the high-resolution distortion law.
"""
from __future__ import annotations

import math
from functools import lru_cache
from statistics import NormalDist

import numpy as np
from scipy.special import erfc

SQRT2 = math.sqrt(2.0)
INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _phi(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        r = INV_SQRT_2PI * np.exp(-0.5 * x * x)
    return np.where(np.isinf(x), 0.0, r)


def _upper_tail(x: np.ndarray) -> np.ndarray:
    """1 - Phi(x), accurate in the upper tail."""
    return 0.5 * erfc(np.asarray(x, dtype=np.float64) / SQRT2)


def _cell_mass(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Phi(b) - Phi(a) for a < b, without cancellation in either tail."""
    return np.where(a >= 0.0, _upper_tail(a) - _upper_tail(b),
                    np.where(b <= 0.0, _upper_tail(-b) - _upper_tail(-a),
                             1.0 - _upper_tail(b) - _upper_tail(-a)))


def _lloyd_step(c: np.ndarray):
    """One Lloyd update: midpoints, then conditional means.  Returns (new c, a, b, mass)."""
    t = 0.5 * (c[:-1] + c[1:])
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    a, b = edges[:-1], edges[1:]
    mass = _cell_mass(a, b)
    return (_phi(a) - _phi(b)) / mass, a, b, mass


def _antisym(c: np.ndarray) -> np.ndarray:
    return 0.5 * (c - c[::-1])


@lru_cache(maxsize=None)
def lloyd_max_normal(k: int) -> tuple[tuple[float, ...], tuple[float, ...]]:
    """(centroids, thresholds) in float64 for 2**k levels of N(0, 1), ascending."""
    if k < 0:
        raise ValueError("k must be >= 0")
    L = 1 << k
    if L == 1:
        return (0.0,), ()
    nd = NormalDist()
    c = np.array([nd.inv_cdf((i + 0.5) / L) for i in range(L)], dtype=np.float64)
    c = _antisym(c)
    for _ in range(1_000_000):
        new = _antisym(_lloyd_step(c)[0])
        move = float(np.max(np.abs(new - c)))
        c = new
        if move < 1e-6:
            break
    best = c
    best_res = math.inf
    for _ in range(40):
        g, a, b, mass = _lloyd_step(c)
        res = float(np.max(np.abs(g - c)))
        if res < best_res:
            best, best_res = c, res
        if res == 0.0:
            break
        fa = np.where(np.isinf(a), 0.0, a)
        fb = np.where(np.isinf(b), 0.0, b)
        d_lo = _phi(a) * (g - fa) / mass      # d(mean)/d(left edge)
        d_hi = _phi(b) * (fb - g) / mass      # d(mean)/d(right edge)
        jac = np.diag(0.5 * (d_lo + d_hi) - 1.0)
        jac += np.diag(0.5 * d_lo[1:], -1) + np.diag(0.5 * d_hi[:-1], 1)
        c = _antisym(c + np.linalg.solve(jac, -(g - c)))
    c = best
    t = 0.5 * (c[:-1] + c[1:])
    return tuple(float(v) for v in c), tuple(float(v) for v in t)


def distortion(k: int) -> float:
    """E[(z - Q(z))^2] for z ~ N(0,1) under the k-bit Lloyd-Max quantizer (float64)."""
    c, t = lloyd_max_normal(k)
    edges = np.concatenate([[-np.inf], np.array(t), [np.inf]])
    a, b = edges[:-1], edges[1:]
    c = np.array(c)
    mass = _cell_mass(a, b)
    ea = np.where(np.isinf(a), 0.0, a) * _phi(a)
    eb = np.where(np.isinf(b), 0.0, b) * _phi(b)
    second = mass + ea - eb                 # E[z^2 ; a < z < b]
    first = _phi(a) - _phi(b)               # E[z ; a < z < b]
    return float(np.sum(second - 2.0 * c * first + c * c * mass))


def stored_codebook(k: int) -> tuple[np.ndarray, np.ndarray]:
    """(c32, t32): float32 centroids and float32 thresholds, as float64 arrays."""
    c, t = lloyd_max_normal(k)
    c32 = np.array(c, dtype=np.float32).astype(np.float64)
    t32 = np.array(t, dtype=np.float32).astype(np.float64)
    return c32, t32
