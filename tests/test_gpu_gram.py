"""GPU parity of Gram-table scoring of block-codebook codes (tq_gram_table,
tq_gram_encode, tq_gram_scores) against oracle/gram.py (page "fib-quant
0.1.0-beta.4 README", "New modules", Scoring; "What's in the box", Codec and
Rotation).

Tolerances come from the float32 arithmetic of the kernels:
  * table: k products summed by fma, |G32 - G| <= k u sum_e |c_ie c_je|;
  * scores: the table entry times scale n_q (2 roundings), nb additions and
    the product by n_t, so |s32 - s| <= (nb + k + 4) u scale n_q n_t nb max|G|;
  * encode: the oracle takes the nearest codeword of the exact (float64)
    rotated block; the kernel decides on the block rounded to float32.  An
    index may differ only where the exact block lies within 1e-6 of the
    boundary between the two codewords (the bisecting hyperplane), in units of
    the coordinate scale 1/sqrt(d) of the normalised rotated vector (the same
    band as the scalar quantizer's 1e-6 on z ~ N(0, 1)), and such blocks stay
    below 1e-5 of all; norms are the float32 rounding of a float64 sum and
    agree bit for bit.
with u = 2^-24.
"""
import math

import numpy as np
import pytest

from kv_cache_vector_diag_amd import inputs
from oracle import gram

from .parity import rec_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = 2.0 ** -24


def _t(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    return (t if dtype is None else t.to(dtype)).to(DEV)


@pytest.mark.parametrize("N,k", [(2, 1), (32, 4), (256, 8), (16, 2), (64, 4)])
def test_gram_table(gpu_lib, N, k):
    C = inputs.block_codebook(1, N, k, 128)
    G = gpu_lib.tq_gram_table(_t(C)).cpu().numpy().astype(np.float64)
    Cd = C.astype(np.float64)
    want = gram.gram_table(Cd)
    bound = k * U * (np.abs(Cd) @ np.abs(Cd).T) + 1e-30
    assert np.all(np.abs(G - want) <= bound)


def _check_codes(gpu_rec, ref_rec, dist, d, k, N, what, C):
    gi, gn = gram.unpack_record(gpu_rec, d, k, N)
    oi, on = gram.unpack_record(ref_rec, d, k, N)
    assert np.array_equal(gn.astype(np.float32), on.astype(np.float32)), f"{what}: norms"
    bad = np.argwhere(gi != oi)
    band = 1e-6 / math.sqrt(d)
    Cd = np.asarray(C, dtype=np.float64)
    for r, blk in bad:
        a, o = gi[r, blk], oi[r, blk]
        # distance of the exact block to the hyperplane equidistant from codewords a and o
        gap = (dist[r, blk, a] - dist[r, blk, o]) / (2.0 * np.linalg.norm(Cd[a] - Cd[o]))
        assert 0.0 <= gap <= band, (what, int(r), int(blk), gap, band)
    assert len(bad) <= max(1, gi.size // 100000), (what, len(bad), gi.size)


@pytest.mark.parametrize("d,k,N,dtype,G,Nv", [
    (128, 4, 32, "bf16", 3, 700), (128, 4, 32, "f16", 2, 300), (64, 4, 32, "f32", 2, 200),
    (256, 4, 32, "bf16", 2, 130), (512, 1, 256, "f32", 1, 40), (32, 8, 16, "bf16", 2, 100),
    (8, 2, 4, "f32", 3, 50), (2, 1, 2, "f32", 1, 33), (128, 2, 64, "bf16", 1, 129),
])
def test_gram_encode(gpu_lib, d, k, N, dtype, G, Nv):
    import torch
    b = gpu_lib
    seed = 17 + d + k
    C = inputs.block_codebook(seed, N, k, d)
    s = inputs.sign_bits(seed, d)
    x = inputs.to_torch(inputs.kv_normal(seed, G, Nv, d), dtype, DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rec = b.tq_gram_encode(_t(C), _t(s.view(np.int32)), x, d, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ref, flags, dist = gram.encode(C, s, inputs.exact_values(x).reshape(-1, d), d, k)
    assert not flags.any()
    _check_codes(rec_np(rec).reshape(G * Nv, -1), ref, dist, d, k, N, f"encode d={d} k={k} N={N}", C)


def test_gram_encode_zero_and_non_finite(gpu_lib):
    """A zero vector has norm 0 and, block by block, the codeword of least norm;
    non-finite input sets the status bit."""
    import torch
    b = gpu_lib
    d, k, N = 128, 4, 32
    C = inputs.block_codebook(5, N, k, d)
    s = inputs.sign_bits(5, d)
    x = torch.zeros((1, 3, d), dtype=torch.float32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rec = b.tq_gram_encode(_t(C), _t(s.view(np.int32)), x, d, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    idx, n = gram.unpack_record(rec_np(rec).reshape(3, -1), d, k, N)
    assert np.all(n == 0.0)
    assert np.all(idx == int(np.argmin(np.sum(C.astype(np.float64) ** 2, axis=1))))
    x[0, 1, 7] = float("nan")
    b.tq_gram_encode(_t(C), _t(s.view(np.int32)), x, d, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & b.STATUS_NON_FINITE


def _score_case(b, d, k, N, B, Hkv, Hq, T, seed, scale=0.0):
    nb = d // k
    C = inputs.block_codebook(seed, N, k, d)
    qi, qn = inputs.block_codes(seed, B * Hq, nb, N, d, stream=11)
    ki, kn = inputs.block_codes(seed, B * Hkv * T, nb, N, d, stream=12)
    qrec = gram.pack_record(qi, qn, d, k, N).reshape(B, Hq, -1)
    krec = gram.pack_record(ki, kn, d, k, N).reshape(B, Hkv, T, -1)
    table = b.tq_gram_table(_t(C))
    sc = b.tq_gram_scores(table, _t(qrec.view(np.int32)), _t(krec.view(np.int32)), d, k, scale=scale)
    ref = gram.scores(C, qrec, krec, d, k, scale=scale if scale > 0 else None)
    Gmax = float(np.max(np.abs(gram.gram_table(C))))
    sv = scale if scale > 0 else 1.0 / math.sqrt(d)
    nq = qn.astype(np.float64).reshape(B, Hq, 1)
    kv = kn.astype(np.float64).reshape(B, Hkv, T)[:, np.arange(Hq) * Hkv // Hq, :]
    bound = (nb + k + 4) * U * sv * nq * kv * nb * Gmax + 1e-30
    return sc.cpu().numpy().astype(np.float64), ref, bound


@pytest.mark.parametrize("d,k,N,B,Hkv,Hq,T", [
    (128, 4, 32, 2, 2, 8, 3000),    # fast kernel, 4 query heads per kv head, ragged last chunk
    (128, 4, 32, 1, 4, 4, 1025),    # one query head per kv head, one key past a chunk
    (128, 4, 32, 2, 2, 4, 77),      # two per kv head, less than a chunk
    (64, 4, 32, 1, 2, 4, 500),      # d/k = 16
    (256, 4, 32, 1, 1, 2, 1100),    # d/k = 64, indices straddle words
    (128, 4, 16, 1, 2, 2, 300),     # N = 16
    (128, 4, 64, 1, 1, 4, 300),     # N = 64
    (128, 2, 32, 1, 2, 6, 200),     # generic kernel: 3 query heads per kv head, d/k = 64
    (16, 1, 256, 1, 1, 1, 50),      # generic kernel, 8-bit indices
    (8, 8, 2, 2, 1, 1, 10),         # one block per vector
])
def test_gram_scores(gpu_lib, d, k, N, B, Hkv, Hq, T):
    got, ref, bound = _score_case(gpu_lib, d, k, N, B, Hkv, Hq, T, seed=29)
    err = np.abs(got - ref)
    assert np.all(err <= bound), (float(err.max()), float(np.max(err / bound)))


def test_gram_scores_explicit_scale_and_empty(gpu_lib):
    import torch
    got, ref, bound = _score_case(gpu_lib, 128, 4, 32, 1, 2, 4, 40, seed=3, scale=0.25)
    assert np.all(np.abs(got - ref) <= bound)
    b = gpu_lib
    C = inputs.block_codebook(3, 32, 4, 128)
    table = b.tq_gram_table(_t(C))
    q = torch.zeros((1, 4, 6), dtype=torch.int32, device=DEV)
    k = torch.zeros((1, 2, 0, 6), dtype=torch.int32, device=DEV)
    out = b.tq_gram_scores(table, q, k, 128, 4)
    assert out.shape == (1, 4, 0)


def test_gram_end_to_end_encode_then_score(gpu_lib):
    """Queries and keys encoded on the GPU and scored there, against the
    oracle's encode and score of the same vectors: where every index agrees
    the scores agree to the score bound."""
    import torch
    b = gpu_lib
    d, k, N, B, Hkv, Hq, T, seed = 128, 4, 32, 2, 2, 8, 1500, 41
    C = inputs.block_codebook(seed, N, k, d)
    s = inputs.sign_bits(seed, d)
    K = inputs.to_torch(inputs.kv_normal(seed, B * Hkv, T, d), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    Ct, st = _t(C), _t(s.view(np.int32))
    krec = b.tq_gram_encode(Ct, st, K, d).view(B, Hkv, T, -1)
    qrec = b.tq_gram_encode(Ct, st, q, d)
    sc = b.tq_gram_scores(b.tq_gram_table(Ct), qrec, krec, d, k)
    torch.cuda.synchronize()
    kref, _, kdist = gram.encode(C, s, inputs.exact_values(K).reshape(-1, d), d, k)
    qref, _, qdist = gram.encode(C, s, inputs.exact_values(q).reshape(-1, d), d, k)
    _check_codes(rec_np(krec).reshape(-1, krec.shape[-1]), kref, kdist, d, k, N, "keys", C)
    _check_codes(rec_np(qrec).reshape(-1, qrec.shape[-1]), qref, qdist, d, k, N, "queries", C)
    ref = gram.scores(C, qref.reshape(B, Hq, -1), kref.reshape(B, Hkv, T, -1), d, k)
    same_k = np.all(rec_np(krec).reshape(-1, krec.shape[-1]) == kref, axis=1).reshape(B, Hkv, T)
    same_q = np.all(rec_np(qrec).reshape(-1, qrec.shape[-1]) == qref, axis=1).reshape(B, Hq)
    got = sc.cpu().numpy().astype(np.float64)
    Gmax = float(np.max(np.abs(gram.gram_table(C))))
    nb = d // k
    checked = 0
    for bb in range(B):
        for hq in range(Hq):
            if not same_q[bb, hq]:
                continue
            h = hq * Hkv // Hq
            m = same_k[bb, h]
            _, qn = gram.unpack_record(qref.reshape(B, Hq, -1)[bb, hq][None, :], d, k, N)
            _, kn = gram.unpack_record(kref.reshape(B, Hkv, T, -1)[bb, h], d, k, N)
            bound = (nb + k + 4) * U / math.sqrt(d) * qn[0] * kn * nb * Gmax
            assert np.all(np.abs(got[bb, hq] - ref[bb, hq])[m] <= bound[m])
            checked += int(m.sum())
    assert checked >= 0.99 * B * Hq * T


def test_gram_step_in_a_graph_equals_eager(gpu_lib):
    """Query encode + Gram scores captured in a HIP graph: every replay, with
    eager work between the replays, equals the eager step."""
    import torch
    b = gpu_lib
    d, k, N, B, Hkv, Hq, T, seed = 128, 4, 32, 2, 2, 8, 2100, 91
    C = _t(inputs.block_codebook(seed, N, k, d))
    sg = _t(inputs.sign_bits(seed, d).view(np.int32))
    K = inputs.to_torch(inputs.kv_normal(seed, B * Hkv, T, d), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    krec = b.tq_gram_encode(C, sg, K, d).view(B, Hkv, T, -1)
    table = b.tq_gram_table(C)
    qrec = torch.empty((B, Hq, krec.shape[-1]), dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, T), dtype=torch.float32, device=DEV)

    def step():
        b.tq_gram_encode(C, sg, q, d, rec=qrec)
        b.tq_gram_scores(table, qrec, krec, d, k, out=out)

    step()
    torch.cuda.synchronize()
    ref_q, ref_s = qrec.clone(), out.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        qrec.zero_()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(qrec, ref_q) and torch.equal(out, ref_s), f"replay {r}"
        _ = (out.sum() + 1.0).item()


def _gram_cases(n=12, seed=77):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        d = int(r.choice([2, 8, 32, 64, 128, 128, 256, 512]))
        k = int(r.choice([x for x in (1, 2, 4, 8) if x <= d]))
        N = int(r.choice([2, 4, 16, 32, 32, 64, 256]))
        Hkv = int(r.choice([1, 2, 4]))
        gq = int(r.choice([1, 2, 3, 4]))
        out.append((i, d, k, N, str(r.choice(["bf16", "f16", "f32"])), int(r.integers(1, 3)), Hkv, Hkv * gq,
                    int(r.integers(1, 2500))))
    return out


@pytest.mark.parametrize("i,d,k,N,dtype,B,Hkv,Hq,T", _gram_cases())
def test_gram_sweep(gpu_lib, i, d, k, N, dtype, B, Hkv, Hq, T):
    """Seeded shapes across both score kernels: GPU encode of keys and queries
    against the oracle's codes, then the GPU scores of the oracle's records
    against the oracle's scores."""
    import torch
    b = gpu_lib
    seed = 500 + i
    C = inputs.block_codebook(seed, N, k, d)
    s = inputs.sign_bits(seed, d)
    K = inputs.to_torch(inputs.kv_normal(seed, B * Hkv, T, d), dtype, DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), dtype, DEV)
    Ct, st = _t(C), _t(s.view(np.int32))
    krec = b.tq_gram_encode(Ct, st, K, d)
    qrec = b.tq_gram_encode(Ct, st, q, d)
    torch.cuda.synchronize()
    kref, _, kdist = gram.encode(C, s, inputs.exact_values(K).reshape(-1, d), d, k)
    qref, _, qdist = gram.encode(C, s, inputs.exact_values(q).reshape(-1, d), d, k)
    _check_codes(rec_np(krec).reshape(-1, krec.shape[-1]), kref, kdist, d, k, N, f"keys case {i}", C)
    _check_codes(rec_np(qrec).reshape(-1, qrec.shape[-1]), qref, qdist, d, k, N, f"queries case {i}", C)
    w = kref.shape[-1]
    sc = b.tq_gram_scores(b.tq_gram_table(Ct), _t(qref.reshape(B, Hq, w).view(np.int32)),
                          _t(kref.reshape(B, Hkv, T, w).view(np.int32)), d, k)
    ref = gram.scores(C, qref.reshape(B, Hq, w), kref.reshape(B, Hkv, T, w), d, k)
    _, qn = gram.unpack_record(qref, d, k, N)
    _, kn = gram.unpack_record(kref, d, k, N)
    nb = d // k
    Gmax = float(np.max(np.abs(gram.gram_table(C))))
    kv = kn.reshape(B, Hkv, T)[:, np.arange(Hq) * Hkv // Hq, :]
    bound = (nb + k + 4) * U / math.sqrt(d) * qn.reshape(B, Hq, 1) * kv * nb * Gmax + 1e-30
    assert np.all(np.abs(sc.cpu().numpy().astype(np.float64) - ref) <= bound), f"scores case {i}"
