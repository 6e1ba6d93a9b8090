"""tq_attend_static (the allocation-free form of tq_attend, its scratch a
library-owned device array) against tq_attend with a caller workspace, through
the C ABI: two calls in a row, the second on a smaller input, on the fused
chunk path and on the scores + partials path.  The two entry points run the
same kernels on the same inputs, so their outputs must agree bit for bit; the
first call is also held to the oracle's softmax-weighted decoded values
(bitpolar attention_scores, then softmax and the value sum) within the
float tolerance |gpu - oracle| <= 1e-4 + 1e-3 |oracle|."""
import numpy as np
import pytest

from kv_cache_vector_diag_amd import inputs
from oracle import turboquant as tq

from .parity import assert_close, rec_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(b, d, kb, vb, B, Hkv, Hq, T, seed):
    import torch
    G = B * Hkv
    kcb = b.make_codebooks(Hkv, d, kb, 128, seed, b.ROLE_KEY, device=DEV)
    vcb = b.make_codebooks(Hkv, d, vb, 0, seed, b.ROLE_VALUE, device=DEV)
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_K), "bf16", DEV)
    V = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_V), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    krec = b.tq_encode_keys(kcb, Hkv, K, d, kb, 128).view(B, Hkv, T, -1)
    vrec = b.tq_encode_values(vcb, Hkv, V, d, vb).view(B, Hkv, T, -1)
    torch.cuda.synchronize()
    return kcb, vcb, krec, vrec, q


@pytest.mark.parametrize("kb,vb,shapes", [
    (3, 2, [(2, 2, 8, 3000), (1, 2, 8, 1100)]),     # fused chunk pass (<= 3 planes each, 4 heads per kv head)
    (5, 4, [(2, 2, 4, 2500), (1, 1, 2, 700)]),      # scores, then chunk partials and the merge
])
def test_attend_static_equals_attend(gpu_lib, kb, vb, shapes):
    import torch
    b = gpu_lib
    d = 128
    assert b.load().tq_attend_static_scratch_bytes() == 32 << 20
    for call, (B, Hkv, Hq, T) in enumerate(shapes):
        seed = 61 + 7 * call + kb
        print(f"tq_attend_static call {call}: B={B} Hkv={Hkv} Hq={Hq} T={T} kb={kb} vb={vb}", flush=True)
        kcb, vcb, krec, vrec, q = _case(b, d, kb, vb, B, Hkv, Hq, T, seed)
        assert b.tq_attend_workspace_bytes(d, B, Hq, T) <= b.load().tq_attend_static_scratch_bytes()
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        got = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
        b.tq_attend_static(kcb, Hkv, vcb, Hkv, krec, vrec, q, d, kb, vb, 128, out=got, status=st)
        want = b.tq_attend(kcb, Hkv, vcb, Hkv, krec, vrec, q, d, kb, vb, 128)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert torch.equal(got, want), f"call {call}: static scratch and workspace results differ"
        if call == 0:
            kq = tq.quantizers(Hkv, d, kb, 128, seed, tq.ROLE_KEY)
            vq = tq.quantizers(Hkv, d, vb, 0, seed, tq.ROLE_VALUE)
            ref = tq.attend(kq, rec_np(krec), vq, rec_np(vrec), inputs.exact_values(q))
            assert_close(got.cpu().numpy(), ref, f"attend_static vs oracle, kb={kb} vb={vb}")


def test_attend_static_refuses_past_its_scratch(gpu_lib):
    """A call needing more than the 32 MiB array returns TQ_ERR_SCRATCH_LIMIT
    before touching any pointer (nothing enqueued)."""
    b = gpu_lib
    lib = b.load()
    B, Hq, T = 16, 32, 32768     # 64 MiB of scores on the unfused path
    assert b.tq_attend_workspace_bytes(128, B, Hq, T) > lib.tq_attend_static_scratch_bytes()
    rc = lib.tq_attend_static(128, 5, 4, 128, 0, None, 8, None, 8, None, None, B, 8, T, None, 1, Hq, 0.0, None, None,
                              None)
    assert rc == -16
    assert "ScratchLimit" in lib.tq_status_string(rc).decode()
