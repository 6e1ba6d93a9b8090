"""Pins for oracle/prng.py: SplitMix64, binary16 rounding, Box-Muller, D."""
import math

import numpy as np
import pytest
from scipy import stats

from oracle import prng


def test_splitmix64_published_outputs_seed0():
    # SplitMix64 started at state 0 (Steele/Lea/Flood 2014; Vigna's splitmix64.c):
    # the first four outputs are widely published.
    expect = [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F, 0xF88BB8A8724C81EC]
    assert [prng.splitmix64(0, i) for i in range(4)] == expect


def test_splitmix64_is_counter_based():
    # output i of seed s equals output 0 of seed s + i*GAMMA (mod 2**64)
    for s in (0, 1, 42, 2**63 + 5):
        for i in (1, 7, 1 << 32):
            assert prng.splitmix64(s, i) == prng.splitmix64((s + i * prng.GAMMA) & prng.MASK64, 0)


@pytest.mark.parametrize("x,expect", [
    (1.0 + 2.0 ** -11, 1.0),                       # tie -> even (mantissa 0)
    (1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -9),       # tie -> even (mantissa 2)
    (1.0 + 2.0 ** -11 + 2.0 ** -30, 1.0 + 2.0 ** -10),
    (2.0 ** -25, 0.0),                             # subnormal tie -> 0
    (3 * 2.0 ** -25, 2.0 ** -23),                  # subnormal tie -> even
    (-(2.0 ** -14) * (1 + 2.0 ** -12), -(2.0 ** -14)),
    (65504.0, 65504.0),
    (65519.9, 65504.0),
    (65520.0, math.inf),                           # tie at the top rounds to overflow
    (-3.14159265358979, -3.140625),
])
def test_round_to_half_hand_cases(x, expect):
    assert prng.round_to_half(x) == expect


def test_round_to_half_matches_numpy_converter():
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-8, 5, 20000),
                         rng.standard_normal(2000)])
    mine = np.array([prng.round_to_half(float(v)) for v in xs])
    ref = xs.astype(np.float16).astype(np.float64)
    assert np.array_equal(mine, ref)


def test_box_muller_invariant_and_distribution():
    seed = 1234
    for p in range(200):
        g0, g1 = prng.gaussian_pair(seed, prng.STREAM_S + 2 * p)
        x1 = prng.splitmix64(seed, prng.STREAM_S + 2 * p)
        u1 = ((x1 >> 11) + 1) * 2.0 ** -53
        assert math.isclose(g0 * g0 + g1 * g1, -2.0 * math.log(u1), rel_tol=1e-12, abs_tol=1e-300)
    g = prng.gaussians(7, 100_000, prng.STREAM_S)
    assert abs(g.mean()) < 4.0 / math.sqrt(g.size)
    assert abs(g.var() - 1.0) < 4.0 * math.sqrt(2.0 / g.size)
    assert stats.kstest(g, "norm").pvalue > 1e-3


def test_qjl_matrix_is_binary16_gaussian_row_major():
    S = prng.qjl_matrix(3, 16, 8)
    g = prng.gaussians(3, 16 * 8, prng.STREAM_S)
    assert np.array_equal(S.ravel(), np.array([prng.round_to_half(v) for v in g]))
    assert np.array_equal(S, S.astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("seed,m,d", [(0, 16, 8), (42, 128, 128), (2**64 - 1, 33, 32)])
def test_fast_variants_agree(seed, m, d):
    assert np.array_equal(prng.qjl_matrix(seed, m, d), prng.qjl_matrix_fast(seed, m, d))
    assert np.array_equal(prng.sign_diagonal(seed, d), prng.sign_diagonal_fast(seed, d))


def test_sign_diagonal_balance_and_bit_mapping():
    D = prng.sign_diagonal(99, 256)
    for j in range(256):
        bit = (prng.splitmix64(99, j // 64) >> (j % 64)) & 1
        assert D[j] == (-1.0 if bit else 1.0)
    allD = np.concatenate([prng.sign_diagonal_fast(s, 512) for s in range(200)])
    assert abs((allD < 0).mean() - 0.5) < 0.01
