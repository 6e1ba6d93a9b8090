"""Pins for oracle/turboquant.py against what the pages and mathematics fix."""
import json
import math
import os

import numpy as np
import pytest
import scipy.linalg
from scipy.special import softmax as sp_softmax

from oracle import turboquant as tq

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("d", [2, 4, 8, 16, 64, 128, 256, 512])
def test_hadamard_sylvester(d):
    H = tq.hadamard(d)
    assert np.array_equal(H @ H, d * np.eye(d))                      # H.H = d.I exactly
    assert np.array_equal(H, scipy.linalg.hadamard(d).astype(float))  # library routine, Sylvester order


def test_rotation_orthogonal_and_norm_preserving():
    qz = tq.Quantizer(128, 3, 128, 11, tq.ROLE_KEY)
    Pi = tq.hadamard(128) * qz.D[None, :] / math.sqrt(128)
    assert np.allclose(Pi.T @ Pi, np.eye(128), atol=1e-13)
    x = np.random.default_rng(1).standard_normal((50, 128))
    u, n = tq.rotate(qz, x)
    assert np.allclose(np.linalg.norm(u, axis=1), math.sqrt(128) * np.linalg.norm(x, axis=1), rtol=1e-13)
    assert np.allclose(n, np.linalg.norm(x, axis=1), rtol=1e-15)


def test_pack_bit_order_hand_example():
    bits = np.zeros((1, 40), dtype=np.uint8)
    bits[0, [0, 2, 31, 32, 39]] = 1
    w = tq.pack_bits(bits)
    assert w.shape == (1, 2)
    assert int(w[0, 0]) == (1 | 4 | (1 << 31))
    assert int(w[0, 1]) == (1 | (1 << 7))
    assert np.array_equal(tq.unpack_bits(w, 40), bits)


@pytest.mark.parametrize("d,bits,m,role,words", [
    (128, 3, 128, tq.ROLE_KEY, 2 * 4 + 4 + 2),
    (128, 2, 128, tq.ROLE_KEY, 1 * 4 + 4 + 2),
    (128, 4, 128, tq.ROLE_KEY, 3 * 4 + 4 + 2),
    (128, 4, 0, tq.ROLE_VALUE, 4 * 4 + 1),
    (8, 4, 16, tq.ROLE_KEY, 3 * 1 + 1 + 2),
    (256, 8, 256, tq.ROLE_KEY, 7 * 8 + 8 + 2),
    (2, 2, 1, tq.ROLE_KEY, 1 + 1 + 2),
])
def test_record_words(d, bits, m, role, words):
    assert tq.record_words(d, bits, m, role) == words


def test_argument_errors_mirror_bitpolar():
    cases = [((0, 3, 8, tq.ROLE_KEY), "ZERO_DIMENSION"), ((6, 3, 8, tq.ROLE_KEY), "BAD_DIMENSION"),
             ((1024, 3, 8, tq.ROLE_KEY), "BAD_DIMENSION"), ((8, 1, 8, tq.ROLE_KEY), "INVALID_BIT_WIDTH"),
             ((8, 10, 8, tq.ROLE_KEY), "INVALID_BIT_WIDTH"), ((8, 0, 0, tq.ROLE_VALUE), "INVALID_BIT_WIDTH"),
             ((8, 9, 0, tq.ROLE_VALUE), "INVALID_BIT_WIDTH"), ((8, 3, 0, tq.ROLE_KEY), "ZERO_PROJECTIONS")]
    for args, code in cases:
        with pytest.raises(tq.OracleError) as e:
            tq.check_args(*args)
        assert e.value.code == code


@pytest.mark.parametrize("bits,role", [(3, tq.ROLE_KEY), (4, tq.ROLE_VALUE), (2, tq.ROLE_VALUE), (9, tq.ROLE_KEY)])
def test_index_is_nearest_centroid(bits, role):
    # Midpoint thresholds <=> nearest centroid: brute force argmin |z - c| away from ties.
    qz = tq.Quantizer(64, bits, 64, 5, role)
    x = np.random.default_rng(2).standard_normal((300, 64))
    enc = tq.encode(qz, x)
    dist = np.abs(enc.z[..., None] - qz.c32[None, None, :])
    brute = np.argmin(dist, axis=-1)
    srt = np.sort(dist, axis=-1)
    clear = (srt[..., 1] - srt[..., 0]) > 1e-9
    assert clear.mean() > 0.999
    assert np.array_equal(enc.idx[clear], brute[clear])


@pytest.mark.parametrize("bits,role", [(3, tq.ROLE_KEY), (4, tq.ROLE_KEY), (4, tq.ROLE_VALUE), (8, tq.ROLE_VALUE)])
def test_code_word_round_trip(bits, role):
    # x = a D H c0 (c0 = c[idx0]) has H D x = a d c0, |x| = a sqrt(d) |c0|, hence
    # z = sqrt(d) c0/|c0| in closed form.  Where that z stays in idx0's cells the
    # code word comes back, decoding gives (n32/(a d)) x (no renormalisation), and
    # the key residual is (a d - n32) c0 / sqrt(d).
    d = 128
    qz = tq.Quantizer(d, bits, d, 9, role)
    rng = np.random.default_rng(3)
    idx0 = np.searchsorted(qz.t32, rng.standard_normal((20, d)))   # typical code words
    c0 = qz.c32[idx0]
    cn0 = np.linalg.norm(c0, axis=1)
    a = 0.25
    x = a * (c0 @ tq.hadamard(d).T) * qz.D[None, :]
    enc = tq.encode(qz, x)
    assert np.allclose(enc.z, (math.sqrt(d) / cn0)[:, None] * c0, rtol=1e-12, atol=1e-13)
    n32 = np.float32(a * math.sqrt(d) * cn0).astype(np.float64)
    f = tq.unpack_record(qz, enc.records)
    assert np.array_equal(f.n32, n32)
    same = np.all(enc.idx == idx0, axis=1)
    if qz.k <= 3:                                   # wide cells: every code word comes back
        assert same.all()
    assert same.sum() >= 1
    if role == tq.ROLE_KEY:
        assert np.allclose(enc.gamma[same], np.abs(a * d - n32[same]) * cn0[same] / math.sqrt(d), rtol=1e-9)
    else:
        xh = tq.decode_values(qz, enc.records)
        assert np.allclose(xh[same], (n32[same] / (a * d))[:, None] * x[same], rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_mse_distortion_matches_lloyd(bits):
    # E|x - x^|^2 / |x|^2 ~ D_k for Gaussian inputs (the post-rotation coordinate law).
    from oracle.lloyd import distortion
    qz = tq.Quantizer(128, bits, 0, 21, tq.ROLE_VALUE)
    x = np.random.default_rng(4).standard_normal((3000, 128))
    xh = tq.decode_values(qz, tq.encode(qz, x).records)
    rel = np.mean(np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1))
    assert rel == pytest.approx(distortion(bits), rel=0.05)


@pytest.mark.slow
@pytest.mark.parametrize("bits", [2, 3])
def test_qjl_inner_product_unbiased_over_seeds(bits):
    # Over many quantizer seeds the TurboQuant estimate of <q, x> is unbiased
    # ("eliminate inner-product bias"), while the MSE-only estimate is shrunk by
    # about (1 - D_k) (2/pi at 1 bit).  Variance obeys the QJL bound pi/(2m)|q|^2|r|^2.
    from oracle.lloyd import distortion
    d = m = 64
    rng = np.random.default_rng(5)
    x = rng.standard_normal(d)
    q = rng.standard_normal(d)
    truth = float(q @ x)
    est, mse_only, bound = [], [], []
    nseeds = 20000
    for s in range(nseeds):
        qz = tq.Quantizer(d, bits, m, 1000 + s, tq.ROLE_KEY, fast_prng=True)
        enc = tq.encode(qz, x[None])
        est.append(tq.compressed_score_terms(qz, enc.records, q)[0])
        f = tq.unpack_record(qz, enc.records)
        qt = tq.hadamard(d) @ (qz.D * q)
        mse_only.append(float(f.n32[0] / d * (qz.c32[f.idx[0]] @ qt)))
        bound.append(math.pi / (2 * m) * float(q @ q) * float(enc.gamma[0]) ** 2)
    est = np.array(est)
    se = est.std(ddof=1) / math.sqrt(nseeds)
    assert abs(est.mean() - truth) < 4.0 * se
    shrink = np.mean(mse_only) / truth
    assert shrink == pytest.approx(1.0 - distortion(bits - 1), abs=0.03)
    # est - <q,x> has conditional mean 0 given D and conditional variance at most
    # pi/(2m)|q|^2|r|^2, so its variance over seeds is below the mean bound
    assert np.var(est - truth) <= 1.05 * np.mean(bound)


def test_compressed_score_identity():
    # The no-decode formula equals dequantize-then-dot (linearity), to 1e-12.
    for bits, m in [(3, 128), (2, 128), (4, 64), (9, 200)]:
        qz = tq.Quantizer(128, bits, m, 77, tq.ROLE_KEY)
        rng = np.random.default_rng(bits)
        x = rng.standard_normal((40, 128))
        q = rng.standard_normal(128)
        rec = tq.encode(qz, x).records
        full = tq.dequantize_keys(qz, rec) @ q
        comp = tq.compressed_score_terms(qz, rec, q)
        assert np.allclose(comp, full, rtol=1e-12, atol=1e-12)


def test_zero_vector_and_flags():
    qz = tq.Quantizer(16, 4, 20, 1, tq.ROLE_KEY)
    x = np.zeros((4, 16))
    x[1, 3] = np.nan
    x[2, 0] = np.inf
    x[3, :] = 1e20                                  # squared norm beyond binary32
    enc = tq.encode(qz, x)
    assert enc.flags.tolist() == [False, True, True, True]
    assert np.all(enc.idx[0] == (1 << (qz.k - 1)) - 1)
    f = tq.unpack_record(qz, enc.records[:1])
    assert f.n32[0] == 0.0 and f.gamma32[0] == 0.0 and np.all(f.signs == 1.0)
    assert np.all(tq.dequantize_keys(qz, enc.records[:1]) == 0.0)
    # m = 20 signs, all 1; the 12 unused high bits of the sign word are 0
    assert int(enc.records[0, qz.k]) == (1 << 20) - 1


def test_scores_gqa_mapping_and_scale():
    qzs = tq.quantizers(2, 32, 3, 32, 100, tq.ROLE_KEY)
    rng = np.random.default_rng(8)
    B, Hkv, Hq, T = 2, 2, 6, 9
    krec = np.stack([np.stack([tq.encode(qzs[(b * Hkv + h) % 2], rng.standard_normal((T, 32))).records
                               for h in range(Hkv)]) for b in range(B)])
    q = rng.standard_normal((B, Hq, 32))
    s = tq.scores(qzs, krec, q)
    for b in range(B):
        for hq in range(Hq):
            h = hq * Hkv // Hq
            ref = tq.dequantize_keys(qzs[(b * Hkv + h) % 2], krec[b, h]) @ q[b, hq] / math.sqrt(32)
            assert np.allclose(s[b, hq], ref, rtol=1e-14)
    assert np.allclose(tq.scores(qzs, krec, q, scale=0.5), s * math.sqrt(32) * 0.5)


def test_attend_special_cases():
    qk = tq.quantizers(1, 16, 3, 16, 4, tq.ROLE_KEY)
    qv = tq.quantizers(1, 16, 2, 16, 4, tq.ROLE_VALUE)
    rng = np.random.default_rng(9)
    k = rng.standard_normal((7, 16))
    v = rng.standard_normal((7, 16))
    kr = tq.encode(qk[0], k).records[None, None]
    vr = tq.encode(qv[0], v).records[None, None]
    q = rng.standard_normal((1, 1, 16))
    o = tq.attend(qk, kr, qv, vr, q)[0, 0]
    w = sp_softmax(tq.scores(qk, kr, q)[0, 0])
    assert np.allclose(o, w @ tq.decode_values(qv[0], vr[0, 0]), rtol=1e-13)
    o1 = tq.attend(qk, kr[:, :, :1], qv, vr[:, :, :1], q)[0, 0]          # one token: weight 1
    assert np.allclose(o1, tq.decode_values(qv[0], vr[0, 0, :1])[0], rtol=1e-13)


def test_formats_table_bits_per_value_and_ratio():
    g = json.load(open(os.path.join(GOLDEN, "formats_table.json")))
    d = g["head_dim_assumed"]
    rows = {r["format"]: r for r in g["rows"]}
    for name in ("turbo3", "turbo2"):                   # TurboQuant key records reproduce the table
        r = rows[name]
        bpv = tq.bits_per_value(d, r["bits"], d, tq.ROLE_KEY)
        assert bpv == r["bits_per_value"]
        assert round(16.0 / bpv, 1) == r["compression"]
    r = rows["turbo4"]
    # 4.25 b/value is reproduced by the 4-bit MSE record (one float32 side scalar);
    # the 4-bit TurboQuant key record carries one more scalar and 128 sign bits: 4.50.
    assert tq.bits_per_value(d, 4, d, tq.ROLE_VALUE) == r["bits_per_value"]
    assert round(16.0 / r["bits_per_value"], 1) == r["compression"]
    assert tq.bits_per_value(d, 4, d, tq.ROLE_KEY) == 4.5


def test_memory_stats():
    st = tq.memory_stats(128, 3, 3, 128, 1024, 32, 32)
    vecs = 1024 * 32 * 32
    assert st["orig_fp16_bytes"] == 2 * vecs * 128 * 2
    assert st["compressed_bytes"] == vecs * (56 + 52)
    assert st["ratio_vs_fp16"] == pytest.approx(2 * 256 / 108)
    assert tq.memory_stats(128, 3, 3, 128, 0, 32, 32)["ratio_vs_fp16"] == 1.0


def test_bitpolar_contract_shapes():
    g = json.load(open(os.path.join(GOLDEN, "bitpolar_contract.json")))
    c = g["sample_config"]
    qk = tq.Quantizer(c["head_dim"], c["bits"], c["projections"], c["seed"], tq.ROLE_KEY)
    qv = tq.Quantizer(c["head_dim"], c["bits"], c["projections"], c["seed"], tq.ROLE_VALUE)
    n = g["pushes_for_scores"]
    kr = tq.encode(qk, np.full((n, 8), g["key_fill"])).records
    vr = tq.encode(qv, np.full((n, 8), g["value_fill"])).records
    s = tq.scores([qk], kr[None, None], np.full((1, 1, 8), g["query_fill"]))
    assert s.shape == (1, 1, n) and np.all(np.isfinite(s))
    dec = tq.decode_values(qv, vr[:1])
    assert dec.shape == (1, 8)
    assert tq.memory_stats(8, 4, 4, 16, 1, 1, 1)["ratio_vs_fp16"] > 0
    mh = tq.quantizers(g["multi_head"]["heads_push"], 8, 4, 16, 42, tq.ROLE_KEY)
    assert [q.seed for q in mh] == [42, 43, 44, 45]
