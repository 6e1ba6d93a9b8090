"""GPU parity of Haar-rotation codebooks through the rotation-named entry points
(tq_encode_keys_ex, tq_encode_values_ex, tq_scores_ex, tq_decode_values_ex,
tq_attend_ex): records, scores, decoded values and attention outputs against
the oracle (oracle/turboquant.py with rotation ROT_HAAR), for head dims that
take each attention path: MFMA value partials (multiple of 32), LUT partials
(multiple of 8), and the per-(b, hq) kernel (any other)."""
import pytest

from kv_cache_vector_diag_amd import inputs
from oracle import turboquant as tq

from .parity import assert_close, check_mismatch_fraction, compare_records, rec_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _haar(b, n_cb, d, bits, m, seed, role):
    cbs = b.make_codebooks(n_cb, d, bits, m, seed, role, device=DEV, rotation=b.ROT_HAAR)
    qzs = [tq.Quantizer(d, bits, m, (seed + i) & ((1 << 64) - 1), role, rotation=tq.ROT_HAAR) for i in range(n_cb)]
    return cbs, qzs


@pytest.mark.parametrize("d,m,kb,vb,B,Hkv,Hq,T", [
    (128, 128, 3, 2, 1, 2, 4, 700),     # value partials on MFMA
    (224, 224, 4, 3, 1, 1, 2, 1100),    # the split layers' normal-part width, two chunks
    (200, 64, 2, 2, 1, 2, 2, 300),      # LUT value partials
    (100, 100, 3, 4, 1, 1, 1, 257),     # per-(b, hq) attention kernel
    (17, 5, 2, 1, 1, 1, 1, 65),         # odd head_dim
])
def test_haar_encode_scores_decode_attend(gpu_lib, d, m, kb, vb, B, Hkv, Hq, T):
    import torch
    b = gpu_lib
    seed = 21
    G = B * Hkv
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_K), "bf16", DEV)
    V = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_V), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    kcb, kq = _haar(b, Hkv, d, kb, m, seed, tq.ROLE_KEY)
    vcb, vq = _haar(b, Hkv, d, vb, 0, seed + 50, tq.ROLE_VALUE)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    krec = b.tq_encode_keys(kcb, Hkv, K, d, kb, m, status=st, rotation=b.ROT_HAAR)
    vrec = b.tq_encode_values(vcb, Hkv, V, d, vb, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    kx, vx = inputs.exact_values(K), inputs.exact_values(V)
    kr, vr = rec_np(krec), rec_np(vrec)
    reps = []
    for g in range(G):
        reps.append(compare_records(kq[g % Hkv], kr[g], tq.encode(kq[g % Hkv], kx[g]), fraction=False))
        reps.append(compare_records(vq[g % Hkv], vr[g], tq.encode(vq[g % Hkv], vx[g]), fraction=False))
    check_mismatch_fraction(reps)

    krec4, vrec4 = krec.view(B, Hkv, T, -1), vrec.view(B, Hkv, T, -1)
    qv = inputs.exact_values(q)
    s = b.tq_scores(kcb, Hkv, krec4, q, d, kb, m, status=st, rotation=b.ROT_HAAR)
    dec = b.tq_decode_values(vcb, Hkv, vrec, d, vb, status=st, rotation=b.ROT_HAAR)
    o = b.tq_attend(kcb, Hkv, vcb, Hkv, krec4, vrec4, q, d, kb, vb, m, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert_close(s.cpu().numpy(), tq.scores(kq, rec_np(krec4), qv), "scores")
    for g in range(G):
        assert_close(dec[g].cpu().numpy(), tq.decode_values(vq[g % Hkv], vr[g]), f"decode g={g}")
    assert_close(o.cpu().numpy(), tq.attend(kq, rec_np(krec4), vq, rec_np(vrec4), qv), "attend")


def test_haar_blob_through_hadamard_call_is_flagged(gpu_lib):
    """A Haar blob handed to a call that names the Walsh-Hadamard rotation is a
    header mismatch: the status word says so (the sizes differ as well, so only
    the first blob is read)."""
    import torch
    b = gpu_lib
    d = 128
    cb, _ = _haar(b, 1, d, 3, 128, 5, tq.ROLE_KEY)
    x = inputs.to_torch(inputs.kv_normal(5, 1, 40, d, inputs.STREAM_K), "bf16", DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rec = torch.empty((1, 40, b.tq_record_bytes(d, 3, 128, b.ROLE_KEY) // 4), dtype=torch.int32, device=DEV)
    b.tq_encode_keys(cb, 1, x, d, 3, 128, rec=rec, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 2
