"""tq_encode_kv: keys and values of the same tokens in one call (turboquant-
plus-rs 0.1.0 README, Architecture: keys take the MSE stage and the QJL
residual, values the MSE stage).  Its records must be bit for bit those of
tq_encode_keys and tq_encode_values, on the shapes that share one launch and
on those that fall back to two; one paired case is also checked against the
oracle."""
import numpy as np
import pytest

from kv_cache_vector_diag_amd import inputs
from oracle import turboquant as tq

from .parity import check_mismatch_fraction, compare_records, rec_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

# (d, k_bits, v_bits, dtype, G, N, row stride): one launch for d=128, turbo3
# keys, 2- or 3-bit values, f32 or bf16; the rest run the two encodes
CASES = [
    (128, 3, 3, "f32", 1, 1024, 128),
    (128, 3, 2, "bf16", 5, 1000, 128),
    (128, 3, 3, "bf16", 3, 33, 192),
    (128, 3, 2, "f32", 2, 1, 128),
    (128, 4, 4, "bf16", 2, 300, 128),
    (128, 3, 3, "f16", 2, 257, 128),
    (64, 3, 3, "bf16", 2, 129, 64),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_encode_kv_equals_separate_encodes(gpu_lib, case):
    import torch
    b = gpu_lib
    d, kb, vb, dt, G, N, stride = CASES[case]
    m = d
    seed = 300 + case
    print(f"case {case}: d={d} k_bits={kb} v_bits={vb} {dt} G={G} N={N} stride={stride}", flush=True)
    kcb = b.make_codebooks(G, d, kb, m, seed, b.ROLE_KEY, device=DEV)
    vcb = b.make_codebooks(G, d, vb, 0, seed, b.ROLE_VALUE, device=DEV)
    Kf = inputs.kv_normal(seed, G, N, d, inputs.STREAM_K)
    Vf = inputs.kv_normal(seed, G, N, d, inputs.STREAM_V)
    if stride != d:        # rows inside a wider buffer: same strides for k and v
        pad = np.zeros((G, N, stride), dtype=np.float32)
        Kb, Vb = pad.copy(), pad.copy()
        Kb[..., :d], Vb[..., :d] = Kf, Vf
        K = inputs.to_torch(Kb, dt, DEV)[..., :d]
        V = inputs.to_torch(Vb, dt, DEV)[..., :d]
    else:
        K, V = inputs.to_torch(Kf, dt, DEV), inputs.to_torch(Vf, dt, DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    kref = b.tq_encode_keys(kcb, G, K, d, kb, m)
    vref = b.tq_encode_values(vcb, G, V, d, vb)
    krec, vrec = b.tq_encode_kv(kcb, G, vcb, G, K, V, d, kb, vb, m, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(krec, kref), "key records differ from tq_encode_keys"
    assert torch.equal(vrec, vref), "value records differ from tq_encode_values"
    if case == 1:
        xk, xv = inputs.exact_values(K), inputs.exact_values(V)
        reps = []
        for g in (0, G - 1):
            kq = tq.Quantizer(d, kb, m, seed + g, tq.ROLE_KEY)
            vq = tq.Quantizer(d, vb, 0, seed + g, tq.ROLE_VALUE)
            reps.append(compare_records(kq, rec_np(krec)[g], tq.encode(kq, xk[g]), fraction=False))
            reps.append(compare_records(vq, rec_np(vrec)[g], tq.encode(vq, xv[g]), fraction=False))
        check_mismatch_fraction(reps)
