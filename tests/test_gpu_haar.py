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


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("kb,vb", [(2, 1), (3, 2), (4, 3), (4, 4)])
def test_haar_mfma_encode_d128(gpu_lib, dtype, kb, vb):
    """At head_dim 128 with 16-bit inputs the Haar rotation runs on the matrix
    cores (R in three exact 16-bit terms): records against the oracle, for every
    key and value width, with groups that span several blocks and a ragged tail."""
    import torch
    b = gpu_lib
    d, m, G, N, seed = 128, 128, 3, 2 * 1024 + 77, 61
    K = inputs.to_torch(inputs.kv_normal(seed, G, N, d, inputs.STREAM_K), dtype, DEV)
    V = inputs.to_torch(inputs.kv_normal(seed, G, N, d, inputs.STREAM_V), dtype, DEV)
    kcb, kq = _haar(b, 2, d, kb, m, seed, tq.ROLE_KEY)
    vcb, vq = _haar(b, 2, d, vb, 0, seed + 9, tq.ROLE_VALUE)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    krec = b.tq_encode_keys(kcb, 2, K, d, kb, m, status=st, rotation=b.ROT_HAAR)
    vrec = b.tq_encode_values(vcb, 2, V, d, vb, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    kx, vx = inputs.exact_values(K), inputs.exact_values(V)
    kr, vr = rec_np(krec), rec_np(vrec)
    reps = []
    for g in range(G):
        reps.append(compare_records(kq[g % 2], kr[g], tq.encode(kq[g % 2], kx[g]), fraction=False))
        reps.append(compare_records(vq[g % 2], vr[g], tq.encode(vq[g % 2], vx[g]), fraction=False))
    check_mismatch_fraction(reps)


@pytest.mark.parametrize("kb,Hkv,Hq,T", [(2, 2, 2, 300), (3, 2, 4, 1100), (4, 1, 4, 2049), (3, 4, 16, 77)])
def test_haar_scores_d128(gpu_lib, kb, Hkv, Hq, T):
    """At head_dim 128 (128 projections) the compressed-key score kernel takes
    Haar codebooks: the query is rotated by the dense R, the rest of the score
    is rotation-agnostic.  Scores against the oracle for every key width and
    query-group size, over several tiles with a ragged tail."""
    import torch
    b = gpu_lib
    d, m, B, seed = 128, 128, 2, 71
    G = B * Hkv
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_K), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    kcb, kq = _haar(b, Hkv, d, kb, m, seed, tq.ROLE_KEY)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    krec = b.tq_encode_keys(kcb, Hkv, K, d, kb, m, status=st, rotation=b.ROT_HAAR).view(B, Hkv, T, -1)
    s = b.tq_scores(kcb, Hkv, krec, q, d, kb, m, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert_close(s.cpu().numpy(), tq.scores(kq, rec_np(krec), inputs.exact_values(q)), "scores")


@pytest.mark.parametrize("kb,vb,B,Hkv,Hq,T", [(2, 1, 2, 2, 2, 1500), (4, 3, 1, 2, 8, 1030), (3, 3, 1, 1, 4, 40)])
def test_haar_fused_attend_d128(gpu_lib, kb, vb, B, Hkv, Hq, T):
    """At head_dim 128 the fused attention path takes Haar codebooks (query
    rotated by R in the query preparation, R^T applied once in the merge):
    outputs against the oracle over several chunks with a ragged tail."""
    import torch
    b = gpu_lib
    d, m, seed = 128, 128, 83
    G = B * Hkv
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_K), "bf16", DEV)
    V = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_V), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    kcb, kq = _haar(b, Hkv, d, kb, m, seed, tq.ROLE_KEY)
    vcb, vq = _haar(b, Hkv, d, vb, 0, seed + 50, tq.ROLE_VALUE)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    krec = b.tq_encode_keys(kcb, Hkv, K, d, kb, m, status=st, rotation=b.ROT_HAAR).view(B, Hkv, T, -1)
    vrec = b.tq_encode_values(vcb, Hkv, V, d, vb, status=st, rotation=b.ROT_HAAR).view(B, Hkv, T, -1)
    o = b.tq_attend(kcb, Hkv, vcb, Hkv, krec, vrec, q, d, kb, vb, m, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert_close(o.cpu().numpy(), tq.attend(kq, rec_np(krec), vq, rec_np(vrec), inputs.exact_values(q)), "attend")


@pytest.mark.parametrize("d,vb,N", [(256, 8, 300), (224, 6, 130), (128, 8, 129), (33, 7, 64), (9, 5, 200)])
def test_haar_decode_wide_codebooks(gpu_lib, d, vb, N):
    """Decode of Haar values with 5-8-bit codebooks (up to 256 centroids) on the
    matrix-core route, head dims across its K-chunk counts (2, 4, 8, 16), groups
    that end mid-tile, two codebooks: decoded vectors against the oracle's."""
    import torch
    b = gpu_lib
    seed, G = 41, 2
    V = inputs.to_torch(inputs.kv_normal(seed, G, N, d, inputs.STREAM_V), "bf16", DEV)
    vcb, vq = _haar(b, G, d, vb, 0, seed, tq.ROLE_VALUE)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    vrec = b.tq_encode_values(vcb, G, V, d, vb, status=st, rotation=b.ROT_HAAR)
    dec = b.tq_decode_values(vcb, G, vrec, d, vb, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    vr = rec_np(vrec)
    for g in range(G):
        assert_close(dec[g].cpu().numpy(), tq.decode_values(vq[g], vr[g]), f"decode d={d} bits={vb} g={g}")


@pytest.mark.parametrize("d,m,kb,Hkv,Hq,T", [(96, 96, 2, 2, 6, 700), (96, 40, 3, 1, 8, 513), (160, 160, 4, 1, 12, 300),
                                             (48, 64, 3, 2, 10, 1100)])
def test_haar_scores_head_batches(gpu_lib, d, m, kb, Hkv, Hq, T):
    """Scores at head dims off the MFMA score kernel with 3 to 12 query heads per
    kv head: the table-driven kernel prepares the query side four heads at a
    time, so these cover partial and several batches, chunks of 512 tokens
    and a ragged last chunk; scores of the GPU's records against the oracle."""
    import torch
    b = gpu_lib
    seed, B = 77, 1
    G = B * Hkv
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_K), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    kcb, kq = _haar(b, Hkv, d, kb, m, seed, tq.ROLE_KEY)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    krec = b.tq_encode_keys(kcb, Hkv, K, d, kb, m, status=st, rotation=b.ROT_HAAR)
    krec4 = krec.view(B, Hkv, T, -1)
    s = b.tq_scores(kcb, Hkv, krec4, q, d, kb, m, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert_close(s.cpu().numpy(), tq.scores(kq, rec_np(krec4), inputs.exact_values(q)), f"scores d={d} Hq={Hq}")
