"""Pins of the Gram-table oracle (oracle/gram.py) against facts that do not
come from the oracle itself: the polarization identity, inner products of
decoded vectors through the orthogonal rotation, exact codeword round trips,
brute-force nearest codewords, a hand-packed record and the zero vector
(page "fib-quant 0.1.0-beta.4 README", "New modules", Scoring; "What's in the
box", Codec and Rotation)."""
import math

import numpy as np
import pytest

from kv_cache_vector_diag_amd import inputs
from oracle import gram
from oracle.turboquant import OracleError


def test_table_polarization_identity():
    """G[i, j] = (|c_i + c_j|^2 - |c_i - c_j|^2) / 4, symmetric, diagonal |c_i|^2;
    4 KB of float32 at N = 32 as the page states."""
    C = inputs.block_codebook(3, 32, 4, 128).astype(np.float64)
    G = gram.gram_table(C)
    for i in range(32):
        for j in range(32):
            s = C[i] + C[j]
            dlt = C[i] - C[j]
            pol = (math.fsum(s * s) - math.fsum(dlt * dlt)) / 4.0
            assert abs(G[i, j] - pol) < 1e-15
        assert abs(G[i, i] - math.fsum(C[i] * C[i])) < 1e-15
    assert G.astype(np.float32).nbytes == 4096


def test_rotation_is_orthogonal_with_hadamard_entries():
    for d in (2, 8, 128):
        s = inputs.sign_bits(d, d)
        P = gram.rotation_matrix(s, d)
        assert np.allclose(P @ P.T, np.eye(d), atol=1e-12)
        assert np.allclose(np.abs(P), 1.0 / math.sqrt(d))
        # column j carries the sign of D: the first row of H is all ones
        dv = gram.sign_vector(s, d)
        assert np.allclose(P[0] * math.sqrt(d), dv)


@pytest.mark.parametrize("d,k,N,B,Hkv,Hq,T", [(128, 4, 32, 2, 2, 4, 9), (16, 2, 4, 1, 1, 3, 5), (64, 8, 256, 1, 2, 2, 3),
                                              (8, 1, 2, 2, 1, 1, 4)])
def test_scores_equal_inner_product_of_decoded_vectors(d, k, N, B, Hkv, Hq, T):
    """The Gram-table score is scale <q^, x^_t> for the decoded vectors (the
    table skips the inverse rotation and the norm scaling, nothing else);
    query head hq reads kv head hq * H_kv // H_q."""
    C = inputs.block_codebook(5, N, k, d)
    s = inputs.sign_bits(5, d)
    nb = d // k
    qi, qn = inputs.block_codes(5, B * Hq, nb, N, d, stream=11)
    ki, kn = inputs.block_codes(5, B * Hkv * T, nb, N, d, stream=12)
    qrec = gram.pack_record(qi, qn, d, k, N).reshape(B, Hq, -1)
    krec = gram.pack_record(ki, kn, d, k, N).reshape(B, Hkv, T, -1)
    got = gram.scores(C, qrec, krec, d, k, scale=0.37)
    qd = gram.decode(C, s, qrec.reshape(B * Hq, -1), d, k).reshape(B, Hq, d)
    kd = gram.decode(C, s, krec.reshape(-1, krec.shape[-1]), d, k).reshape(B, Hkv, T, d)
    for b in range(B):
        for hq in range(Hq):
            h = hq * Hkv // Hq
            for t in range(T):
                want = 0.37 * math.fsum(qd[b, hq] * kd[b, h, t])
                assert abs(got[b, hq, t] - want) <= 1e-12 * max(1.0, abs(want)) + 1e-12
    # default scale is 1/sqrt(d)
    dflt = gram.scores(C, qrec, krec, d, k)
    assert np.allclose(dflt, got / 0.37 / math.sqrt(d), rtol=1e-14, atol=1e-14)


def test_encode_recovers_exact_codewords():
    """A vector whose rotated, normalised blocks are codewords encodes to those
    codewords, with its norm.  Codewords e_j / sqrt(2) in R^4, two blocks: every
    code concatenates to a unit vector."""
    d, k, N = 8, 4, 4
    C = np.eye(4) / math.sqrt(2.0)
    s = inputs.sign_bits(9, d)
    P = gram.rotation_matrix(s, d)
    for i0 in range(4):
        for i1 in range(4):
            c = np.concatenate([C[i0], C[i1]])
            x = 3.5 * (P.T @ c)
            rec, flags, _ = gram.encode(C, s, x[None, :], d, k)
            idx, n = gram.unpack_record(rec, d, k, N)
            assert not flags[0]
            assert list(idx[0]) == [i0, i1]
            assert n[0] == np.float32(3.5)


def test_decode_inverts_the_rotation():
    """decode(encode(x)) = x for x = n D H c / sqrt(d) whose blocks are codewords,
    with D and H written out here by loops, not taken from the oracle: the
    decoder applies the inverse rotation Pi^T = D H / sqrt(d).  Applying Pi =
    H D / sqrt(d) instead gives a different vector whenever D is not the
    identity (checked), so the direction is pinned, not only inner products."""
    d, k, N = 8, 4, 4
    C = np.eye(4) / math.sqrt(2.0)
    s = inputs.sign_bits(9, d)
    dv = [-1.0 if (int(s[j // 32]) >> (j % 32)) & 1 else 1.0 for j in range(d)]
    assert min(dv) < 0 < max(dv)
    H = [[(-1.0) ** bin(i & j).count("1") for j in range(d)] for i in range(d)]
    for i0, i1, nrm in ((0, 3, 3.5), (2, 2, 0.75), (1, 0, 12.0)):
        c = list(C[i0]) + list(C[i1])
        x = np.array([nrm * dv[i] * math.fsum(H[i][j] * c[j] for j in range(d)) / math.sqrt(d) for i in range(d)])
        rec, flags, _ = gram.encode(C, s, x[None, :], d, k)
        assert not flags[0]
        back = gram.decode(C, s, rec, d, k)[0]
        assert np.max(np.abs(back - x)) < 1e-12 * nrm
        wrong = np.array([nrm * math.fsum(H[i][j] * dv[j] * c[j] for j in range(d)) / math.sqrt(d) for i in range(d)])
        assert np.max(np.abs(wrong - x)) > 0.1 * nrm


def test_encode_picks_the_nearest_codeword_brute_force():
    """Each block's index minimises the squared distance over all codewords
    (plain loops on the exact rotated coordinates), the lowest index on
    ties."""
    d, k, N = 16, 4, 8
    C = inputs.block_codebook(2, N, k, d).astype(np.float64)
    s = inputs.sign_bits(2, d)
    X = inputs.kv_normal(2, 1, 20, d)[0].astype(np.float64)
    rec, _, _ = gram.encode(C, s, X, d, k)
    idx, n = gram.unpack_record(rec, d, k, N)
    H = np.array([[(-1.0) ** bin(i & j).count("1") for j in range(d)] for i in range(d)])
    dv = gram.sign_vector(s, d)
    for r in range(X.shape[0]):
        nrm = math.sqrt(math.fsum(X[r] * X[r]))
        assert n[r] == np.float32(nrm)
        n32 = float(np.float32(nrm))
        u = [math.fsum(H[i, j] * dv[j] * X[r, j] for j in range(d)) / (math.sqrt(d) * n32) for i in range(d)]
        for b in range(d // k):
            dist = [math.fsum((u[b * k + e] - C[i, e]) ** 2 for e in range(k)) for i in range(N)]
            best = min(range(N), key=lambda i: (dist[i], i))
            assert idx[r, b] == best


def test_record_packing_hand_example():
    """d=16, k=2, N=32: eight 5-bit indices, LSB first, index b at bit 5b; the
    seventh (7 = 0b111) straddles words 0 and 1."""
    idx = np.array([[1, 2, 3, 4, 5, 6, 7, 31]])
    rec = gram.pack_record(idx, np.array([2.0], dtype=np.float32), 16, 2, 32)
    w0 = 1 + (2 << 5) + (3 << 10) + (4 << 15) + (5 << 20) + (6 << 25) + ((7 & 3) << 30)
    w1 = (7 >> 2) + (31 << 3)
    assert rec.shape == (1, 3)
    assert [int(v) for v in rec[0]] == [w0, w1, 0x40000000]
    assert w0 == 3427929153 and w1 == 249
    back, n = gram.unpack_record(rec, 16, 2, 32)
    assert list(back[0]) == [1, 2, 3, 4, 5, 6, 7, 31] and n[0] == 2.0
    assert gram.record_words(128, 4, 32) == 6        # 32 indices x 5 bits = 5 words, + norm


def test_zero_and_non_finite_vectors():
    d, k, N = 32, 4, 16
    C = inputs.block_codebook(4, N, k, d).astype(np.float64)
    s = inputs.sign_bits(4, d)
    X = np.zeros((3, d))
    X[1, 5] = np.inf
    X[2, 0] = 1e30      # squared norm past the float32 range
    rec, flags, _ = gram.encode(C, s, X, d, k)
    idx, n = gram.unpack_record(rec, d, k, N)
    assert list(flags) == [False, True, True]
    assert n[0] == 0.0
    smallest = int(np.argmin(np.sum(C * C, axis=1)))
    assert all(i == smallest for i in idx[0])
    q = gram.pack_record(idx[:1], np.array([1.0], dtype=np.float32), d, k, N).reshape(1, 1, -1)
    assert np.all(gram.scores(C, q, rec[:1].reshape(1, 1, 1, -1), d, k) == 0.0)


def test_argument_checks():
    with pytest.raises(OracleError, match="ZERO_DIMENSION"):
        gram.check_args(0, 4, 32)
    for d, k, N in ((96, 4, 32), (1024, 4, 32), (128, 3, 32), (4, 8, 32)):
        with pytest.raises(OracleError, match="BAD_DIMENSION"):
            gram.check_args(d, k, N)
    for N in (1, 3, 512):
        with pytest.raises(OracleError, match="INVALID_CODEBOOK"):
            gram.check_args(128, 4, N)
    assert gram.check_args(128, 4, 32) == 5
