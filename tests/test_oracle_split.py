"""Pins for the Haar rotation and the outlier/normal split of the oracle
(oracle/turboquant.py haar_rotation, oracle/split.py)."""
import math

import numpy as np
import pytest

from oracle import lloyd, prng, split
from oracle import turboquant as tq


# ---- channel selection -------------------------------------------------------
def test_outlier_channels_hand_example():
    # variances: channel 0 -> 0, channel 1 -> 100, channel 2 -> 1
    X = np.array([[0.0, 10.0, 1.0], [0.0, -10.0, -1.0]])
    assert split.channel_variance(X).tolist() == [0.0, 100.0, 1.0]
    assert split.outlier_channels(X, 1).tolist() == [1, 0, 2]
    assert split.outlier_channels(X, 2).tolist() == [1, 2, 0]


def test_outlier_channels_planted():
    rng = np.random.default_rng(7)
    d, n_out = 64, 8
    planted = np.sort(rng.choice(d, n_out, replace=False))
    sig = rng.uniform(0.5, 1.0, d)
    sig[planted] = 8.0
    X = rng.standard_normal((2000, d)) * sig[None, :]
    chan = split.outlier_channels(X, n_out)
    assert chan[:n_out].tolist() == planted.tolist()
    assert chan[n_out:].tolist() == sorted(set(range(d)) - set(planted.tolist()))


def test_outlier_channels_ties_take_lower_index():
    X = np.tile(np.array([[1.0], [-1.0]]), (3, 6))      # six identical channels
    assert split.outlier_channels(X, 2).tolist() == [0, 1, 2, 3, 4, 5]
    X[:, 4] *= 2.0                                        # one larger channel
    assert split.outlier_channels(X, 2).tolist() == [0, 4, 1, 2, 3, 5]


def test_channel_variance_closed_forms():
    X = np.zeros((10, 3))
    X[:, 0] = 5.0                                         # constant: 0
    X[:, 1] = np.where(np.arange(10) % 2 == 0, 3.0, -3.0)  # +-a: a^2
    X[:, 2] = np.arange(10)                               # 0..n-1: (n^2-1)/12
    assert np.allclose(split.channel_variance(X), [0.0, 9.0, 99.0 / 12.0], rtol=1e-15, atol=0)


# ---- Haar rotation ------------------------------------------------------------
def _gram_schmidt(G):
    """Classical Gram-Schmidt on the columns (the QR with positive diagonal), pure Python."""
    n = len(G)
    cols = [[G[i][j] for i in range(n)] for j in range(n)]
    qs = []
    for v in cols:
        w = list(v)
        for q in qs:
            r = sum(a * b for a, b in zip(q, v))
            w = [a - r * b for a, b in zip(w, q)]
        nrm = math.sqrt(sum(a * a for a in w))
        qs.append([a / nrm for a in w])
    return [[qs[j][i] for j in range(n)] for i in range(n)]   # Q[i][j] = column j


def test_haar_2x2_closed_form():
    g = prng.haar_gaussian(123, 2)
    R = tq.haar_rotation(123, 2)
    c0 = g[:, 0] / math.hypot(g[0, 0], g[1, 0])              # first column of Q: g0/|g0|
    assert np.allclose(R[:, 0] / math.sqrt(2), c0, atol=1e-7)
    # second column: unit, orthogonal, positive component along g1
    c1 = R[:, 1] / math.sqrt(2)
    assert abs(c0 @ c1) < 1e-7 and abs(np.linalg.norm(c1) - 1) < 1e-7 and c1 @ g[:, 1] > 0


@pytest.mark.parametrize("d,seed", [(5, 1), (12, 99), (24, 5)])
def test_haar_matches_gram_schmidt(d, seed):
    Q = np.array(_gram_schmidt(prng.haar_gaussian(seed, d).tolist()))
    R = tq.haar_rotation(seed, d)
    assert np.allclose(R / math.sqrt(d), Q, atol=2e-7 * math.sqrt(d) + 1e-10)


def test_haar_orthogonal_and_stored_in_float32():
    R = tq.haar_rotation(5, 224)
    assert np.array_equal(R, R.astype(np.float32).astype(np.float64))
    assert np.abs(R.T @ R / 224 - np.eye(224)).max() < 1e-6
    x = np.random.default_rng(3).standard_normal((20, 224))
    u = x @ R.T
    assert np.allclose(np.linalg.norm(u, axis=1), math.sqrt(224) * np.linalg.norm(x, axis=1), rtol=1e-6)


def test_haar_rotated_coordinates_are_standard_normal():
    x = np.random.default_rng(11).standard_normal(24)
    zs = np.concatenate([tq.haar_rotation(s, 24) @ x / np.linalg.norm(x) for s in range(400)])
    assert abs(zs.mean()) < 4 / math.sqrt(zs.size)
    assert abs(zs.var() - 1.0) < 0.05


def test_haar_quantizer_accepts_any_width_and_rejects_bad():
    assert tq.record_words(224, 3, 224, tq.ROLE_KEY, tq.ROT_HAAR) == 2 * 7 + 7 + 2
    assert tq.record_words(224, 3, 0, tq.ROLE_VALUE, tq.ROT_HAAR) == 3 * 7 + 1
    with pytest.raises(tq.OracleError):
        tq.record_words(224, 3, 224, tq.ROLE_KEY)                  # Hadamard needs a power of two
    with pytest.raises(tq.OracleError):
        tq.record_words(513, 3, 16, tq.ROLE_KEY, tq.ROT_HAAR)


def test_haar_lattice_round_trip():
    qz = tq.Quantizer(40, 3, 40, 9, tq.ROLE_KEY, rotation=tq.ROT_HAAR)
    rng = np.random.default_rng(4)
    idx0 = rng.integers(0, 4, (30, 40))
    n = rng.uniform(0.5, 20.0, 30)
    # x = (n/d) R^T c[idx0] has z = R x / |x| ~ c[idx0] sqrt(d)/|c[idx0]|, so choose
    # the norm consistently: |x| = n |c[idx0]| / sqrt(d) up to the float32 rounding of R
    X = (n[:, None] / 40) * (qz.c32[idx0] @ qz.R)
    enc = tq.encode(qz, X)
    # the lattice point has z_j = sqrt(d) c_j / |c| which lands in the cell of c_j only
    # when |c| ~ sqrt(d) (true on average); compare against the brute-force nearest cell
    brute = np.array([[int(np.sum(qz.t32 < v)) for v in row] for row in enc.z])
    assert np.array_equal(enc.idx, brute)
    assert np.allclose(enc.n, np.linalg.norm(X, axis=1), rtol=1e-15)


def test_haar_distortion_law():
    qz = tq.Quantizer(224, 2, 0, 17, tq.ROLE_VALUE, rotation=tq.ROT_HAAR)
    X = np.random.default_rng(5).standard_normal((1500, 224))
    xh = tq.decode_values(qz, tq.encode(qz, X).records)
    ratio = np.mean(np.sum((X - xh) ** 2, axis=1) / np.sum(X * X, axis=1))
    assert abs(ratio / lloyd.distortion(2) - 1.0) < 0.05


def test_haar_qjl_unbiased_over_seeds():
    d = 12
    rng = np.random.default_rng(8)
    x, q = rng.standard_normal(d), rng.standard_normal(d)
    est = []
    for s in range(3000):
        qz = tq.Quantizer(d, 2, d, 1000 + s, tq.ROLE_KEY, rotation=tq.ROT_HAAR)
        rec = tq.encode(qz, x[None, :]).records
        est.append(float(tq.dequantize_keys(qz, rec)[0] @ q))
    est = np.array(est)
    se = est.std() / math.sqrt(est.size)
    assert abs(est.mean() - x @ q) < 4 * se


# ---- the split codec ----------------------------------------------------------
def test_split_layout_and_bits():
    sq = split.split_quantizer(256, 32, 3, 5, tq.ROLE_KEY)
    assert (sq.normal.d, sq.normal.bits, sq.normal.m, sq.normal.rotation) == (224, 3, 224, tq.ROT_HAAR)
    assert (sq.outlier.d, sq.outlier.bits, sq.outlier.m, sq.outlier.rotation) == (32, 4, 32, tq.ROT_HADAMARD)
    assert sq.outlier.seed == 5 ^ split.OUTLIER_SEED_XOR
    assert 4 * sq.normal.words == 92 and 4 * sq.outlier.words == 24
    assert split.split_bits_per_value(256, 32, 3, tq.ROLE_KEY) == (92 + 24) * 8 / 256
    sv = split.split_quantizer(256, 32, 3, 5, tq.ROLE_VALUE)
    assert 4 * sv.normal.words == 88 and 4 * sv.outlier.words == 20


def test_split_scores_equal_sum_of_compressed_parts():
    d, n_out = 48, 16
    sqs = split.split_quantizers(2, d, n_out, 3, 21, tq.ROLE_KEY)
    rng = np.random.default_rng(2)
    X = rng.standard_normal((2, 7, d)) * np.exp(rng.uniform(-0.7, 2.0, (2, 1, d)))
    q = rng.standard_normal((1, 4, d))
    chans = np.stack([split.outlier_channels(X[g], n_out) for g in range(2)])
    encs = [split.encode_split(sqs[g], X[g], chans[g]) for g in range(2)]
    rn = np.stack([e[0].records for e in encs])[None]
    ro = np.stack([e[1].records for e in encs])[None]
    s = split.scores_split(sqs, chans, rn, ro, q)
    for hq in range(4):
        g = hq * 2 // 4
        ch = chans[g]
        ref = (tq.compressed_score_terms(sqs[g].normal, rn[0, g], q[0, hq, ch[n_out:]])
               + tq.compressed_score_terms(sqs[g].outlier, ro[0, g], q[0, hq, ch[:n_out]])) / math.sqrt(d)
        assert np.allclose(s[0, hq], ref, rtol=1e-12, atol=1e-12)


def test_split_values_lattice_points_and_scatter():
    d, n_out = 64, 16
    sq = split.split_quantizer(d, n_out, 3, 3, tq.ROLE_VALUE)
    rng = np.random.default_rng(6)
    out = np.sort(rng.choice(d, n_out, replace=False))
    chan = np.array(out.tolist() + sorted(set(range(d)) - set(out.tolist())))
    i_o = rng.integers(0, 16, (5, n_out))
    i_n = rng.integers(0, 8, (5, d - n_out))
    n_o, n_n = rng.uniform(1, 3, 5), rng.uniform(1, 3, 5)
    # lattice points x = (n/d') Pi'^T c[idx] of each part: then z = sqrt(d') c / |c| exactly
    # (Hadamard) or up to the float32 rounding of R (Haar)
    xo = (n_o[:, None] / n_out) * ((sq.outlier.c32[i_o] @ tq.hadamard(n_out).T) * sq.outlier.D[None, :])
    xn = (n_n[:, None] / (d - n_out)) * (sq.normal.c32[i_n] @ sq.normal.R)
    X = np.zeros((5, d))
    X[:, chan[:n_out]] = xo
    X[:, chan[n_out:]] = xn
    en, eo = split.encode_split(sq, X, chan)
    co, cn = sq.outlier.c32[i_o], sq.normal.c32[i_n]
    zo = math.sqrt(n_out) * co / np.linalg.norm(co, axis=1, keepdims=True)
    zn = math.sqrt(d - n_out) * cn / np.linalg.norm(cn, axis=1, keepdims=True)
    assert np.allclose(eo.z, zo, rtol=0, atol=1e-12)
    assert np.allclose(en.z, zn, rtol=0, atol=2e-6)
    cells = lambda z, t: np.searchsorted(t, z.astype(np.float32).astype(np.float64).ravel(), "left").reshape(z.shape)
    assert np.array_equal(eo.idx, cells(zo, sq.outlier.t32))
    xd = split.decode_values_split(sq, chan, en.records, eo.records)
    assert np.array_equal(xd[:, chan[:n_out]], tq.decode_values(sq.outlier, eo.records))
    assert np.array_equal(xd[:, chan[n_out:]], tq.decode_values(sq.normal, en.records))
