"""GPU parity of the Haar-rotation encodes on the matrix cores off head_dim
128 (multiples of 8): below 128 with 16-bit inputs, padded to 128 (zero rows
and columns of R and S, zero input coordinates, padded coordinates and
projections masked out of the record); in (128, 256] with bf16 inputs, R
streamed through LDS in 16-column chunks; and edge rows (zero, tiny, huge,
one-hot) on every MFMA encode; Walsh-Hadamard head dims below 128 (powers
of two, 16-bit inputs) padded the same way.  Records against the oracle for key
widths 2-4 with up to 128 projections, value widths 1-4, bf16 and f16, ragged
and strided token ranges, shared and per-head codebooks; then scores and
decoded values of those records against the oracle."""
import numpy as np
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


@pytest.mark.parametrize("d,kb,m,vb,dtype,G,N,n_cb,stride", [
    (64, 3, 64, 3, "bf16", 3, 700, 3, 1),
    (64, 4, 128, 4, "f16", 2, 333, 1, 2),      # more projections than coordinates
    (96, 2, 96, 2, "bf16", 2, 257, 2, 1),      # three plane words
    (32, 4, 32, 1, "bf16", 2, 129, 1, 1),      # one plane word
    (112, 3, 100, 3, "f16", 1, 65, 1, 3),      # partial sign word
    (40, 2, 7, 4, "bf16", 2, 31, 2, 1),        # half a 16-coordinate slice padded; one short tile
    (16, 3, 1, 2, "bf16", 1, 1, 1, 1),         # a single vector, a single projection
    (120, 4, 128, 4, "bf16", 1, 1000, 1, 1),
])
def test_haar_padded_encode(gpu_lib, d, kb, m, vb, dtype, G, N, n_cb, stride):
    import torch
    b = gpu_lib
    seed = 300 + d + kb
    K = inputs.to_torch(inputs.kv_normal(seed, G, N * stride, d, inputs.STREAM_K), dtype, DEV)[:, ::stride, :]
    V = inputs.to_torch(inputs.kv_normal(seed, G, N * stride, d, inputs.STREAM_V), dtype, DEV)[:, ::stride, :]
    kcb, kq = _haar(b, n_cb, d, kb, m, seed, tq.ROLE_KEY)
    vcb, vq = _haar(b, n_cb, d, vb, 0, seed + 50, tq.ROLE_VALUE)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    krec = b.tq_encode_keys(kcb, n_cb, K, d, kb, m, status=st, rotation=b.ROT_HAAR)
    vrec = b.tq_encode_values(vcb, n_cb, V, d, vb, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    kx, vx = inputs.exact_values(K), inputs.exact_values(V)
    kr, vr = rec_np(krec), rec_np(vrec)
    reps = []
    for g in range(G):
        reps.append(compare_records(kq[g % n_cb], kr[g], tq.encode(kq[g % n_cb], kx[g]), fraction=False))
        reps.append(compare_records(vq[g % n_cb], vr[g], tq.encode(vq[g % n_cb], vx[g]), fraction=False))
    check_mismatch_fraction(reps)
    # the records feed the score and decode calls like any other
    q = inputs.to_torch(inputs.queries(seed, G, 1, d), dtype, DEV)
    s = b.tq_scores(kcb, n_cb, krec.view(G, 1, N, -1), q, d, kb, m, status=st, rotation=b.ROT_HAAR)
    dec = b.tq_decode_values(vcb, n_cb, vrec, d, vb, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert_close(s.cpu().numpy(), tq.scores(kq, rec_np(krec.view(G, 1, N, -1)), inputs.exact_values(q)), "scores")
    for g in range(G):
        assert_close(dec[g].cpu().numpy(), tq.decode_values(vq[g % n_cb], vr[g]), f"decode g={g}")


def test_haar_padded_blob_check(gpu_lib):
    """A d=64 Haar blob of other bits handed to a d=64 call is a header mismatch on
    the padded kernel too (the blob is the larger one, so the call reads only
    bytes it holds)."""
    import torch
    b = gpu_lib
    d = 64
    cb4, _ = _haar(b, 1, d, 4, 64, 5, tq.ROLE_KEY)
    assert cb4.numel() >= b.tq_codebook_bytes_ex(d, 3, 64, b.ROLE_KEY, b.ROT_HAAR)
    x = inputs.to_torch(inputs.kv_normal(5, 1, 40, d, inputs.STREAM_K), "bf16", DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    b.tq_encode_keys(cb4, 1, x, d, 3, 64, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) & 2


@pytest.mark.parametrize("d,kb,m,vb,G,N,n_cb,stride", [
    (256, 3, 256, 3, 2, 700, 2, 1),           # d = 256: R streamed through LDS in K-chunks
    (256, 4, 256, 4, 1, 333, 1, 2),
    (200, 2, 100, 1, 2, 257, 1, 1),           # padded to 256; a partial sign word
    (224, 3, 224, 2, 1, 65, 1, 3),            # the split layers' normal-part width
    (136, 4, 7, 4, 2, 31, 2, 1),              # just past 128; one short tile
    (256, 2, 1, 3, 1, 1, 1, 1),               # a single vector, a single projection
])
def test_haar_wide_head_encode(gpu_lib, d, kb, m, vb, G, N, n_cb, stride):
    """Head dims in (128, 256], multiples of 8, bf16: the streamed-R MFMA encode."""
    import torch
    b = gpu_lib
    seed = 500 + d + kb
    K = inputs.to_torch(inputs.kv_normal(seed, G, N * stride, d, inputs.STREAM_K), "bf16", DEV)[:, ::stride, :]
    V = inputs.to_torch(inputs.kv_normal(seed, G, N * stride, d, inputs.STREAM_V), "bf16", DEV)[:, ::stride, :]
    kcb, kq = _haar(b, n_cb, d, kb, m, seed, tq.ROLE_KEY)
    vcb, vq = _haar(b, n_cb, d, vb, 0, seed + 50, tq.ROLE_VALUE)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    krec = b.tq_encode_keys(kcb, n_cb, K, d, kb, m, status=st, rotation=b.ROT_HAAR)
    vrec = b.tq_encode_values(vcb, n_cb, V, d, vb, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    kx, vx = inputs.exact_values(K), inputs.exact_values(V)
    kr, vr = rec_np(krec), rec_np(vrec)
    reps = []
    for g in range(G):
        reps.append(compare_records(kq[g % n_cb], kr[g], tq.encode(kq[g % n_cb], kx[g]), fraction=False))
        reps.append(compare_records(vq[g % n_cb], vr[g], tq.encode(vq[g % n_cb], vx[g]), fraction=False))
    check_mismatch_fraction(reps)


@pytest.mark.parametrize("d,rot", [(128, "wh"), (64, "wh"), (128, "haar"), (64, "haar"), (256, "haar")])
def test_encode_edge_rows_bf16(gpu_lib, d, rot):
    """Zero, tiny (1e-30 and 1e-20: squares below the float32 range), huge (1e10)
    and one-hot bf16 rows on the MFMA encodes (keys b=4, values 4 bits)."""
    import torch
    b = gpu_lib
    seed = 17
    rng = np.random.default_rng(4)
    rows = [np.zeros(d), rng.standard_normal(d) * 1e-30, rng.standard_normal(d) * 1e-20,
            rng.standard_normal(d) * 1e10, np.where(np.arange(d) == 77 % d, 3.0, 0.0)]
    Xc, _ = inputs.kv_channel_std(seed, 1, 60, d)
    X = inputs.to_torch(np.concatenate([np.stack(rows)[None], Xc], axis=1).astype(np.float32), "bf16", DEV)
    rotation = b.ROT_HAAR if rot == "haar" else b.ROT_HADAMARD
    for role, bits, m in ((tq.ROLE_KEY, 4, d), (tq.ROLE_VALUE, 4, 0)):
        if rot == "haar":
            cb, qz = _haar(b, 1, d, bits, m, seed, role)
        else:
            cb = b.make_codebooks(1, d, bits, m, seed, role, device=DEV)
            qz = tq.quantizers(1, d, bits, m, seed, role)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        rec = (b.tq_encode_keys(cb, 1, X, d, bits, m, status=st, rotation=rotation) if role == tq.ROLE_KEY
               else b.tq_encode_values(cb, 1, X, d, bits, status=st, rotation=rotation))
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        xv = inputs.exact_values(X)
        check_mismatch_fraction([compare_records(qz[0], rec_np(rec)[0], tq.encode(qz[0], xv[0]), fraction=False)])


@pytest.mark.parametrize("d,kb,m,vb,dtype,G,N,n_cb", [
    (64, 3, 64, 3, "bf16", 3, 700, 3),
    (64, 4, 128, 4, "f16", 2, 333, 1),
    (32, 2, 32, 2, "bf16", 2, 257, 2),
    (16, 4, 16, 1, "bf16", 2, 129, 1),
    (8, 3, 5, 4, "f16", 1, 65, 1),
])
def test_hadamard_padded_encode(gpu_lib, d, kb, m, vb, dtype, G, N, n_cb):
    """Walsh-Hadamard head dims below 128 (powers of two, 16-bit inputs) on the
    MFMA encode: with zero inputs past d, the first d rows of H_128 D x are H_d D x."""
    import torch
    b = gpu_lib
    seed = 700 + d + kb
    K = inputs.to_torch(inputs.kv_normal(seed, G, N, d, inputs.STREAM_K), dtype, DEV)
    V = inputs.to_torch(inputs.kv_normal(seed, G, N, d, inputs.STREAM_V), dtype, DEV)
    kcb = b.make_codebooks(n_cb, d, kb, m, seed, b.ROLE_KEY, device=DEV)
    vcb = b.make_codebooks(n_cb, d, vb, 0, seed + 50, b.ROLE_VALUE, device=DEV)
    kq = tq.quantizers(n_cb, d, kb, m, seed, tq.ROLE_KEY)
    vq = tq.quantizers(n_cb, d, vb, 0, seed + 50, tq.ROLE_VALUE)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    krec = b.tq_encode_keys(kcb, n_cb, K, d, kb, m, status=st)
    vrec = b.tq_encode_values(vcb, n_cb, V, d, vb, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    kx, vx = inputs.exact_values(K), inputs.exact_values(V)
    kr, vr = rec_np(krec), rec_np(vrec)
    reps = []
    for g in range(G):
        reps.append(compare_records(kq[g % n_cb], kr[g], tq.encode(kq[g % n_cb], kx[g]), fraction=False))
        reps.append(compare_records(vq[g % n_cb], vr[g], tq.encode(vq[g % n_cb], vx[g]), fraction=False))
    check_mismatch_fraction(reps)
