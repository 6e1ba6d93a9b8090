"""Seeded sweep of shapes across every dispatch route of the compressed-cache
calls (MFMA kernels at head_dim 128, tiled wide-codebook kernels, the generic
per-vector kernels, both rotations): records, scores, decoded values and the
attention output against the oracle, each case drawn from a fixed generator so
that the list is the same on every run.  The bounds are those of the other
parity tests (tests/parity.py)."""
import numpy as np
import pytest

from kv_cache_vector_diag_amd import inputs
from oracle import turboquant as tq

from .parity import assert_close, check_mismatch_fraction, compare_records, rec_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _cases(n=24, seed=2026):
    r = np.random.default_rng(seed)
    out = []
    for i in range(n):
        rot = tq.ROT_HAAR if i % 4 == 3 else tq.ROT_HADAMARD
        if rot == tq.ROT_HAAR:
            d = int(r.choice([5, 24, 64, 100, 128, 200]))
        else:
            d = int(r.choice([2, 8, 32, 64, 128, 128, 128, 256, 512]))
        kb = int(r.integers(2, 10))
        vb = int(r.integers(1, 9))
        m = int(r.choice([d, d, 1, 7, 128, 300]))
        dtype = str(r.choice(["bf16", "f16", "f32"]))
        Hkv = int(r.choice([1, 2, 4]))
        gq = int(r.choice([1, 2, 3, 4]))
        B = int(r.integers(1, 3))
        T = int(r.integers(1, 1400))
        n_cb = int(r.choice([1, Hkv]))
        out.append((i, d, kb, vb, m, dtype, B, Hkv, Hkv * gq, T, n_cb, rot))
    # draws inside the head_dim-128 MFMA routes (encode, scores, fused attention)
    for i in range(n, n + 8):
        kb, vb = int(r.integers(2, 5)), int(r.integers(1, 5))
        dtype = str(r.choice(["bf16", "f16", "f32"]))
        Hkv, gq = int(r.choice([1, 2, 4])), int(r.choice([1, 2, 4]))
        rot = tq.ROT_HAAR if i % 4 == 3 and dtype != "f32" else tq.ROT_HADAMARD
        out.append((i, 128, kb, vb, 128, dtype, int(r.integers(1, 3)), Hkv, Hkv * gq, int(r.integers(1, 2600)),
                    int(r.choice([1, Hkv])), rot))
    return out


@pytest.mark.parametrize("i,d,kb,vb,m,dtype,B,Hkv,Hq,T,n_cb,rot", _cases())
def test_sweep(gpu_lib, i, d, kb, vb, m, dtype, B, Hkv, Hq, T, n_cb, rot):
    import torch
    b = gpu_lib
    seed = 1000 + i
    G = B * Hkv
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_K), dtype, DEV)
    V = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_V), dtype, DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), dtype, DEV)
    kcb = b.make_codebooks(n_cb, d, kb, m, seed, b.ROLE_KEY, device=DEV, rotation=rot)
    vcb = b.make_codebooks(n_cb, d, vb, 0, seed + 77, b.ROLE_VALUE, device=DEV, rotation=rot)
    kq = [tq.Quantizer(d, kb, m, seed + c, tq.ROLE_KEY, rotation=rot) for c in range(n_cb)]
    vq = [tq.Quantizer(d, vb, 0, seed + 77 + c, tq.ROLE_VALUE, rotation=rot) for c in range(n_cb)]
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    krec = b.tq_encode_keys(kcb, n_cb, K, d, kb, m, status=st, rotation=rot)
    vrec = b.tq_encode_values(vcb, n_cb, V, d, vb, status=st, rotation=rot)
    krec4, vrec4 = krec.view(B, Hkv, T, -1), vrec.view(B, Hkv, T, -1)
    s = b.tq_scores(kcb, n_cb, krec4, q, d, kb, m, status=st, rotation=rot)
    dec = b.tq_decode_values(vcb, n_cb, vrec, d, vb, status=st, rotation=rot)
    o = b.tq_attend(kcb, n_cb, vcb, n_cb, krec4, vrec4, q, d, kb, vb, m, status=st, rotation=rot)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    kx, vx, qv = inputs.exact_values(K), inputs.exact_values(V), inputs.exact_values(q)
    kr, vr = rec_np(krec), rec_np(vrec)
    reps = []
    for g in range(G):
        reps.append(compare_records(kq[g % n_cb], kr[g], tq.encode(kq[g % n_cb], kx[g]), fraction=False))
        reps.append(compare_records(vq[g % n_cb], vr[g], tq.encode(vq[g % n_cb], vx[g]), fraction=False))
    check_mismatch_fraction(reps)
    # scores, decode and attention on the GPU's own records (stage-wise parity);
    # the oracle's group g of (b, h) uses quantizer (b * Hkv + h) mod n_cb
    kq_g = [kq[g % n_cb] for g in range(G)]
    vq_g = [vq[g % n_cb] for g in range(G)]
    ref_s = np.stack([tq.scores(kq_g[bb * Hkv:(bb + 1) * Hkv], rec_np(krec4)[bb:bb + 1], qv[bb:bb + 1])[0]
                      for bb in range(B)])
    assert_close(s.cpu().numpy(), ref_s, f"scores case {i}")
    for g in range(G):
        assert_close(dec[g].cpu().numpy(), tq.decode_values(vq_g[g], vr[g]), f"decode case {i} g={g}")
    ref_o = np.stack([tq.attend(kq_g[bb * Hkv:(bb + 1) * Hkv], rec_np(krec4)[bb:bb + 1],
                                vq_g[bb * Hkv:(bb + 1) * Hkv], rec_np(vrec4)[bb:bb + 1], qv[bb:bb + 1])[0]
                      for bb in range(B)])
    assert_close(o.cpu().numpy(), ref_o, f"attend case {i}")
