"""GPU parity of the mixed-precision layer path: outlier channel selection,
split encode (Haar normal part + Walsh-Hadamard outlier part), split scores and
split value decode, against the oracle (oracle/split.py) on the same seeded
inputs: bf16 head vectors with per-channel std log-uniform in [0.5, 8]."""
import math

import numpy as np
import pytest

from kv_cache_vector_diag_amd import inputs
from oracle import split
from oracle import turboquant as tq

from .parity import assert_close, check_mismatch_fraction, compare_records, rec_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _status():
    import torch
    return torch.zeros(1, dtype=torch.int32, device=DEV)


def _chan_ok(X, chan_gpu, n_out):
    """The GPU map equals the oracle's; where the oracle's variance gap at the
    cut is below float64 noise both choices are valid, so only the rest is compared."""
    ref = split.outlier_channels(X, n_out)
    var = np.sort(split.channel_variance(X))[::-1]
    if var[n_out - 1] - var[n_out] <= 1e-9 * var[n_out - 1]:
        return
    assert chan_gpu.tolist() == ref.tolist()


# 4-channel loads (head_dim % 4 == 0, aligned rows) and the one-channel kernel
# (head_dim 50, odd token stride)
@pytest.mark.parametrize("G,N,d,n_out,dtype,stride", [(4, 3000, 256, 32, "bf16", 1), (3, 1, 64, 16, "bf16", 1),
                                                      (2, 700, 48, 16, "bf16", 1), (2, 900, 128, 16, "f32", 1),
                                                      (2, 600, 64, 8, "f16", 1), (2, 500, 50, 8, "bf16", 1),
                                                      (2, 400, 64, 8, "bf16", 3)])
def test_outlier_channels(gpu_lib, G, N, d, n_out, dtype, stride):
    import torch
    b = gpu_lib
    Xf, _ = inputs.kv_channel_std(5, G, N, d)
    if stride > 1:
        # rows of d + 1 elements: every row start is misaligned for the wide loads
        Xp = np.zeros((G, N, d + 1), dtype=Xf.dtype)
        Xp[..., :d] = Xf
        X = inputs.to_torch(Xp, dtype, DEV)[..., :d]
    else:
        X = inputs.to_torch(Xf, dtype, DEV)
    chan = b.tq_outlier_channels(X, d, n_out)
    torch.cuda.synchronize()
    xv = inputs.exact_values(X)
    c = chan.cpu().numpy()
    for g in range(G):
        _chan_ok(xv[g], c[g], n_out)


def test_outlier_channels_empty_sequence(gpu_lib):
    import torch
    b = gpu_lib
    X = torch.zeros((2, 0, 64), dtype=torch.bfloat16, device=DEV)
    chan = b.tq_outlier_channels(X, 64, 8)
    torch.cuda.synchronize()
    ref = split.outlier_channels(np.zeros((0, 64)), 8)
    assert all(chan.cpu().numpy()[g].tolist() == ref.tolist() for g in range(2))


def _split_setup(b, role, G, N, d, n_out, bits, seed, n_cb=None, use_workspace=True):
    import torch
    n_cb = n_cb or G
    Xf, _ = inputs.kv_channel_std(seed, G, N, d, stream=inputs.STREAM_K if role == tq.ROLE_KEY else inputs.STREAM_V)
    X = inputs.to_torch(Xf, "bf16", DEV)
    chan = b.tq_outlier_channels(X, d, n_out)
    cbn, cbo = b.split_codebooks(n_cb, d, n_out, bits, seed, role, device=DEV)
    sqs = split.split_quantizers(n_cb, d, n_out, bits, seed, role)
    st = _status()
    rn, ro = b.tq_encode_split(role, cbn, cbo, n_cb, X, d, n_out, bits, chan, status=st, use_workspace=use_workspace)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    return X, chan, sqs, (cbn, cbo), rn, ro


# head_dim 256 / 32 outliers / bits 2-3 with scratch runs the MFMA split kernel;
# without scratch (or other shapes) the generic kernels
@pytest.mark.parametrize("role", [tq.ROLE_KEY, tq.ROLE_VALUE])
@pytest.mark.parametrize("G,N,d,n_out,bits,ws", [(3, 333, 256, 32, 3, True), (3, 333, 256, 32, 3, False),
                                                 (2, 300, 256, 32, 2, True), (1, 1, 256, 32, 3, True),
                                                 (2, 65, 64, 16, 2, True),
                                                 (40, 70, 256, 32, 3, True)])   # many groups: XCD-major
def test_split_encode_parity(gpu_lib, role, G, N, d, n_out, bits, ws):
    b = gpu_lib
    X, chan, sqs, _, rn, ro = _split_setup(b, role, G, N, d, n_out, bits, 5, use_workspace=ws)
    xv = inputs.exact_values(X)
    c = chan.cpu().numpy()
    reps = []
    for g in range(G):
        _chan_ok(xv[g], c[g], n_out)
        en, eo = split.encode_split(sqs[g], xv[g], c[g])      # the oracle on the GPU's channel map
        reps.append(compare_records(sqs[g].normal, rec_np(rn)[g], en, fraction=False))
        reps.append(compare_records(sqs[g].outlier, rec_np(ro)[g], eo, fraction=False))
    check_mismatch_fraction(reps)


def test_split_scores_parity(gpu_lib):
    """B=2 sequences x 2 kv heads x 300 tokens, 4 query heads (GQA 2:1), d=256."""
    import torch
    b = gpu_lib
    B, Hkv, Hq, T, d, n_out, bits = 2, 2, 4, 300, 256, 32, 3
    G = B * Hkv
    X, chan, sqs, (cbn, cbo), rn, ro = _split_setup(b, tq.ROLE_KEY, G, T, d, n_out, bits, 5, n_cb=Hkv)
    q = inputs.to_torch(inputs.queries(5, B, Hq, d), "bf16", DEV)
    s = b.tq_scores_split(cbn, cbo, Hkv, chan, rn.view(B, Hkv, T, -1), ro.view(B, Hkv, T, -1), q, d, n_out, bits)
    torch.cuda.synchronize()
    ref = split.scores_split(sqs, chan.cpu().numpy(), rec_np(rn).reshape(B, Hkv, T, -1),
                             rec_np(ro).reshape(B, Hkv, T, -1), inputs.exact_values(q))
    assert_close(s.cpu().numpy(), ref, "split scores")
    assert abs(ref).max() > 0.1


def test_split_decode_parity(gpu_lib):
    import torch
    b = gpu_lib
    G, N, d, n_out, bits = 3, 200, 256, 32, 3
    X, chan, sqs, (cbn, cbo), rn, ro = _split_setup(b, tq.ROLE_VALUE, G, N, d, n_out, bits, 6)
    out = b.tq_decode_values_split(cbn, cbo, G, chan, rn, ro, d, n_out, bits)
    torch.cuda.synchronize()
    c = chan.cpu().numpy()
    for g in range(G):
        ref = split.decode_values_split(sqs[g], c[g], rec_np(rn)[g], rec_np(ro)[g])
        assert_close(out.cpu().numpy()[g], ref, f"split decode g={g}")


def test_split_bad_channel_flagged(gpu_lib):
    import torch
    b = gpu_lib
    G, N, d, n_out, bits = 1, 8, 64, 16, 3
    Xf, _ = inputs.kv_channel_std(7, G, N, d)
    X = inputs.to_torch(Xf, "bf16", DEV)
    chan = torch.arange(d, dtype=torch.int32, device=DEV).reshape(1, d).clone()
    chan[0, 3] = d + 5                                   # out of range: flagged, read as channel 0
    cbn, cbo = b.split_codebooks(1, d, n_out, bits, 7, tq.ROLE_KEY, device=DEV)
    st = _status()
    b.tq_encode_split(tq.ROLE_KEY, cbn, cbo, 1, X, d, n_out, bits, chan, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & b.STATUS_BAD_CHANNEL


def test_split_mfma_path_bad_channel_flagged(gpu_lib):
    import torch
    b = gpu_lib
    G, N, d, n_out, bits = 1, 40, 256, 32, 3
    Xf, _ = inputs.kv_channel_std(7, G, N, d)
    X = inputs.to_torch(Xf, "bf16", DEV)
    chan = torch.arange(d, dtype=torch.int32, device=DEV).reshape(1, d).clone()
    chan[0, 100] = -3                                    # out of range: flagged by the fragment builder
    cbn, cbo = b.split_codebooks(1, d, n_out, bits, 7, tq.ROLE_KEY, device=DEV)
    st = _status()
    b.tq_encode_split(tq.ROLE_KEY, cbn, cbo, 1, X, d, n_out, bits, chan, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & b.STATUS_BAD_CHANNEL


@pytest.mark.parametrize("role", [tq.ROLE_KEY, tq.ROLE_VALUE])
def test_split_encode_tiny_rows(gpu_lib, role):
    """Rows scaled by 1e-30 and 1e-20 (squares below the float32 range) and a zero
    row among ordinary ones, on the MFMA split kernel."""
    import torch
    b = gpu_lib
    G, N, d, n_out, bits, seed = 2, 90, 256, 32, 3, 8
    Xf, _ = inputs.kv_channel_std(seed, G, N, d)
    Xf[:, 3] *= np.float32(1e-30)
    Xf[:, 4] *= np.float32(1e-20)
    Xf[:, 5] = 0.0
    X = inputs.to_torch(Xf, "bf16", DEV)
    chan = b.tq_outlier_channels(X, d, n_out)
    cbn, cbo = b.split_codebooks(G, d, n_out, bits, seed, role, device=DEV)
    sqs = split.split_quantizers(G, d, n_out, bits, seed, role)
    st = _status()
    rn, ro = b.tq_encode_split(role, cbn, cbo, G, X, d, n_out, bits, chan, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    xv = inputs.exact_values(X)
    c = chan.cpu().numpy()
    reps = []
    for g in range(G):
        en, eo = split.encode_split(sqs[g], xv[g], c[g])
        reps.append(compare_records(sqs[g].normal, rec_np(rn)[g], en, fraction=False))
        reps.append(compare_records(sqs[g].outlier, rec_np(ro)[g], eo, fraction=False))
    check_mismatch_fraction(reps)
