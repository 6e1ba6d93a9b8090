"""Pins for oracle/lloyd.py: Lloyd-Max codebook of N(0,1)."""
import json
import math
import os

import numpy as np
import pytest
from scipy.stats import norm

from oracle import lloyd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_one_bit_closed_form():
    # 1-bit optimum: +-E|z| = +-sqrt(2/pi), distortion 1 - 2/pi (closed form)
    c, t = lloyd.lloyd_max_normal(1)
    r = math.sqrt(2.0 / math.pi)
    assert c == pytest.approx((-r, r), abs=1e-15)
    assert t == (0.0,)
    assert lloyd.distortion(1) == pytest.approx(1.0 - 2.0 / math.pi, abs=1e-14)


@pytest.mark.parametrize("k", range(1, 9))
def test_fixed_point_conditions_and_symmetry(k):
    c, t = (np.array(v) for v in lloyd.lloyd_max_normal(k))
    assert np.all(np.diff(c) > 0)
    assert np.array_equal(t, 0.5 * (c[:-1] + c[1:]))
    assert np.array_equal(c, -c[::-1])
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    # conditional means computed with scipy's normal law, independent of the
    # solver's helpers; each cell mass is taken from the tail it lies in (sf in
    # the upper tail, cdf in the lower), so that no tail cell loses digits to
    # cancellation and the fixed point is checked to float64 evaluation
    a, b = edges[:-1], edges[1:]
    mass = np.where(a >= 0.0, norm.sf(a) - norm.sf(b),
                    np.where(b <= 0.0, norm.cdf(b) - norm.cdf(a), 1.0 - norm.sf(b) - norm.cdf(a)))
    means = (norm.pdf(a) - norm.pdf(b)) / mass
    assert np.max(np.abs(means - c)) < 1e-12
    if k >= 1:
        assert t[len(t) // 2] == 0.0


def test_max_1960_table():
    g = json.load(open(os.path.join(GOLDEN, "max1960_gaussian.json")))
    for L, row in g["levels"].items():
        k = int(L).bit_length() - 1
        c, t = lloyd.lloyd_max_normal(k)
        pos_c = c[len(c) // 2:]
        pos_t = t[len(t) // 2:]
        assert np.allclose(pos_c, row["outputs_pos"], atol=6e-4)
        assert np.allclose(pos_t, row["thresholds_pos"], atol=6e-4)
        assert lloyd.distortion(k) == pytest.approx(row["mse"], abs=2e-5)


@pytest.mark.parametrize("k", [2, 3, 4])
def test_independent_kmeans_on_quantile_grid(k):
    # 1-D k-means on a dense equal-mass grid of normal quantiles approximates the
    # continuous Lloyd problem by a different route (sample means of grid points,
    # no closed-form integrals).  The grid is sorted, so each cell is an index
    # range and its mean comes from prefix sums.
    n = 2_000_000
    z = norm.ppf((np.arange(n) + 0.5) / n)
    prefix = np.concatenate([[0.0], np.cumsum(z)])
    L = 1 << k
    c = np.linspace(-2.0, 2.0, L)
    for _ in range(100_000):
        t = 0.5 * (c[:-1] + c[1:])
        edges = np.concatenate([[0], np.searchsorted(z, t), [n]])
        new = (prefix[edges[1:]] - prefix[edges[:-1]]) / np.diff(edges)
        if np.max(np.abs(new - c)) < 1e-13:
            c = new
            break
        c = new
    ref, _ = lloyd.lloyd_max_normal(k)
    assert np.max(np.abs(c - np.array(ref))) < 2e-4   # grid discretisation ~1e-4 in the tails


def test_high_resolution_distortion_law():
    # Panter-Dite: 4**k * D_k -> sqrt(3) pi / 2 as k grows
    lim = math.sqrt(3.0) * math.pi / 2.0
    vals = [4.0 ** k * lloyd.distortion(k) for k in range(4, 9)]
    assert all(v < lim for v in vals)
    assert all(b > a for a, b in zip(vals, vals[1:]))
    assert abs(vals[-1] - lim) / lim < 0.01


def test_stored_codebook_rounding():
    for k in range(1, 9):
        c32, t32 = lloyd.stored_codebook(k)
        c, t = lloyd.lloyd_max_normal(k)
        assert np.array_equal(c32, np.array(c, dtype=np.float32).astype(np.float64))
        assert np.array_equal(t32, np.array(t, dtype=np.float32).astype(np.float64))
        assert np.array_equal(c32, -c32[::-1]) and np.array_equal(t32, -t32[::-1])
