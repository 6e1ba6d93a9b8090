"""Streaming append into a paged compressed cache (tq_append_kv): one token per
sequence and step, all kv heads, records written to shuffled pool pages.  The
gathered pages must equal the batch encode of the same vectors bit for bit
(page "fib-quant 0.1.0-beta.4 README", "Streaming KV encoder": the streamed
tensor is identical to the batch one), and the records match the oracle
within the sign band."""
import numpy as np
import pytest

from kv_cache_vector_diag_amd import inputs
from oracle import turboquant as tq

from .parity import assert_close, check_mismatch_fraction, compare_records

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _stream(b, d, kb, vb, m, B, Hkv, T, P, n_kcb, n_vcb, dtype, seed, extra_pages=3):
    import torch
    G = B * Hkv
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_K), dtype, DEV).view(B, Hkv, T, d)
    V = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_V), dtype, DEV).view(B, Hkv, T, d)
    kcb = b.make_codebooks(n_kcb, d, kb, m, seed, b.ROLE_KEY, device=DEV)
    vcb = b.make_codebooks(n_vcb, d, vb, 0, seed + 7, b.ROLE_VALUE, device=DEV)
    kw = b.tq_record_bytes(d, kb, m, b.ROLE_KEY) // 4
    vw = b.tq_record_bytes(d, vb, 0, b.ROLE_VALUE) // 4
    max_pages = (T + P - 1) // P
    num_pages = B * max_pages + extra_pages
    perm = np.random.default_rng(seed).permutation(num_pages)[: B * max_pages].astype(np.int32)
    table = torch.from_numpy(perm.reshape(B, max_pages)).to(DEV)
    kpool = torch.full((num_pages, Hkv, P, kw), -1, dtype=torch.int32, device=DEV)
    vpool = torch.full((num_pages, Hkv, P, vw), -1, dtype=torch.int32, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    for t in range(T):
        pos = torch.full((B,), t, dtype=torch.int32, device=DEV)
        b.tq_append_kv(kcb, n_kcb, vcb, n_vcb, K[:, :, t].contiguous(), V[:, :, t].contiguous(), d, kb, vb, m, pos,
                       table, P, kpool, vpool, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    # gather each (b, h) back into token order
    kp, vp, tab = kpool.cpu().numpy(), vpool.cpu().numpy(), table.cpu().numpy()
    tk = np.arange(T)
    kg = np.stack([np.stack([kp[tab[bb, tk // P], h, tk % P] for h in range(Hkv)]) for bb in range(B)])
    vg = np.stack([np.stack([vp[tab[bb, tk // P], h, tk % P] for h in range(Hkv)]) for bb in range(B)])
    kbatch = b.tq_encode_keys(kcb, n_kcb, K.reshape(G, T, d), d, kb, m).view(B, Hkv, T, kw)
    vbatch = b.tq_encode_values(vcb, n_vcb, V.reshape(G, T, d), d, vb).view(B, Hkv, T, vw)
    torch.cuda.synchronize()
    return K, V, kg, vg, kbatch.cpu().numpy(), vbatch.cpu().numpy(), kpool, table


@pytest.mark.parametrize("d,kb,vb,m,B,Hkv,T,P,n_kcb,n_vcb,dtype", [
    (128, 3, 2, 128, 3, 4, 300, 64, 4, 4, "bf16"),   # MFMA encode, heads as groups of the batch
    (128, 4, 4, 128, 2, 4, 130, 32, 3, 2, "bf16"),   # a codebook count not dividing H_kv: one group per vector
    (64, 3, 3, 64, 5, 2, 100, 96, 2, 1, "f32"),      # wide-codebook kernel, fp32 input, one partial page
])
def test_stream_append_equals_batch_encode(gpu_lib, d, kb, vb, m, B, Hkv, T, P, n_kcb, n_vcb, dtype):
    b = gpu_lib
    K, V, kg, vg, kbatch, vbatch, _, _ = _stream(b, d, kb, vb, m, B, Hkv, T, P, n_kcb, n_vcb, dtype, seed=31)
    assert np.array_equal(kg.view(np.uint32), kbatch.view(np.uint32))
    assert np.array_equal(vg.view(np.uint32), vbatch.view(np.uint32))
    # and the oracle, for two groups
    reps = []
    kx = inputs.exact_values(K.reshape(B * Hkv, T, d))
    vx = inputs.exact_values(V.reshape(B * Hkv, T, d))
    for g in (0, B * Hkv - 1):
        kq = tq.Quantizer(d, kb, m, 31 + g % n_kcb, tq.ROLE_KEY)
        vq = tq.Quantizer(d, vb, 0, 38 + g % n_vcb, tq.ROLE_VALUE)
        reps.append(compare_records(kq, kg.reshape(B * Hkv, T, -1)[g].view(np.uint32), tq.encode(kq, kx[g]),
                                    fraction=False))
        reps.append(compare_records(vq, vg.reshape(B * Hkv, T, -1)[g].view(np.uint32), tq.encode(vq, vx[g]),
                                    fraction=False))
    check_mismatch_fraction(reps)


def test_append_bad_position_or_page_is_flagged(gpu_lib):
    """A position past the page table, a negative one, or a page outside the
    pool sets TQ_STATUS_BAD_PAGE and writes nothing for that sequence."""
    import torch
    b = gpu_lib
    d, B, Hkv, P = 128, 3, 2, 32
    kcb = b.make_codebooks(Hkv, d, 3, 128, 1, b.ROLE_KEY, device=DEV)
    vcb = b.make_codebooks(Hkv, d, 2, 0, 2, b.ROLE_VALUE, device=DEV)
    kw = b.tq_record_bytes(d, 3, 128, b.ROLE_KEY) // 4
    vw = b.tq_record_bytes(d, 2, 0, b.ROLE_VALUE) // 4
    k = inputs.to_torch(inputs.kv_normal(1, B * Hkv, 1, d), "bf16", DEV).view(B, Hkv, d)
    table = torch.tensor([[0, 1], [2, 9], [3, 4]], dtype=torch.int32, device=DEV)   # page 9: outside 5 pages
    kpool = torch.full((5, Hkv, P, kw), -1, dtype=torch.int32, device=DEV)
    vpool = torch.full((5, Hkv, P, vw), -1, dtype=torch.int32, device=DEV)
    for pos_list, bad in (([0, 0, 0], False), ([64, 5, 6], True), ([3, 40, 7], True), ([-1, 8, 9], True)):
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        before = kpool.clone()
        pos = torch.tensor(pos_list, dtype=torch.int32, device=DEV)
        b.tq_append_kv(kcb, Hkv, vcb, Hkv, k, k, d, 3, 2, 128, pos, table, P, kpool, vpool, status=st)
        torch.cuda.synchronize()
        assert bool(int(st.item()) & 8) == bad
        for bb in range(B):
            p = pos_list[bb]
            ok = 0 <= p < 2 * P and 0 <= int(table[bb, p // P]) < 5
            if not ok:
                continue
            page = int(table[bb, p // P])
            assert not torch.equal(kpool[page, :, p % P], before[page, :, p % P])
        changed = (kpool != before).any(dim=(1, 2, 3)).nonzero().flatten().tolist()
        allowed = {int(table[bb, pos_list[bb] // P]) for bb in range(B)
                   if 0 <= pos_list[bb] < 2 * P and 0 <= int(table[bb, pos_list[bb] // P]) < 5}
        assert set(changed) <= allowed


@pytest.mark.parametrize("kb,B,Hkv,Hq,T,P", [(3, 3, 4, 8, 300, 64), (2, 2, 2, 2, 97, 32), (4, 1, 2, 8, 1100, 256)])
def test_scores_from_paged_pool_equal_contiguous(gpu_lib, kb, B, Hkv, Hq, T, P):
    """tq_scores_paged over the streamed pool gives the scores of tq_scores over
    the batch-encoded records (the same kernel, addressed through the pages)."""
    import torch
    b = gpu_lib
    d = 128
    K, V, kg, vg, kbatch, vbatch, kpool, table = _stream(b, d, kb, 2, 128, B, Hkv, T, P, Hkv, Hkv, "bf16", seed=41)
    assert np.array_equal(kg.view(np.uint32), kbatch.view(np.uint32))
    kcb = b.make_codebooks(Hkv, d, kb, 128, 41, b.ROLE_KEY, device=DEV)
    q = inputs.to_torch(inputs.queries(41, B, Hq, d), "bf16", DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    sp = b.tq_scores_paged(kcb, Hkv, kpool, table, P, T, q, d, kb, 128, status=st)
    sc = b.tq_scores(kcb, Hkv, torch.from_numpy(kbatch).to(DEV), q, d, kb, 128)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(sp, sc)
    ref = tq.scores([tq.Quantizer(d, kb, 128, 41 + h, tq.ROLE_KEY) for h in range(Hkv)], kbatch.view(np.uint32),
                    inputs.exact_values(q))
    assert_close(sp.cpu().numpy(), ref, "paged scores")
    # a page outside the pool: flagged, its tokens read as zero records
    bad = table.clone()
    bad[0, 0] = kpool.shape[0] + 5
    st.zero_()
    b.tq_scores_paged(kcb, Hkv, kpool, bad, P, T, q, d, kb, 128, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & 8


def test_paged_step_in_a_graph_equals_eager(gpu_lib):
    """The decode step (append + paged scores) captured in a HIP graph: every
    replay, with eager work and synchronisations between the replays, gives the
    eager step's pools and scores (the calls enqueue kernels only: no
    allocation, copy or memset on the stream)."""
    import torch
    b = gpu_lib
    d, kb, vb, m, B, Hkv, Hq, T, P = 128, 3, 3, 128, 3, 4, 8, 300, 64
    K, V, kg, vg, kbatch, vbatch, kpool, table = _stream(b, d, kb, vb, m, B, Hkv, T, P, Hkv, Hkv, "bf16", seed=53)
    kcb = b.make_codebooks(Hkv, d, kb, m, 53, b.ROLE_KEY, device=DEV)
    vcb = b.make_codebooks(Hkv, d, vb, 0, 60, b.ROLE_VALUE, device=DEV)
    vpool = torch.zeros((kpool.shape[0], Hkv, P, b.tq_record_bytes(d, vb, 0, b.ROLE_VALUE) // 4), dtype=torch.int32,
                        device=DEV)
    kn = inputs.to_torch(inputs.kv_normal(54, B, Hkv, d), "bf16", DEV).contiguous()
    vn = inputs.to_torch(inputs.kv_normal(55, B, Hkv, d), "bf16", DEV).contiguous()
    q = inputs.to_torch(inputs.queries(53, B, Hq, d), "bf16", DEV)
    pos = torch.full((B,), T, dtype=torch.int32, device=DEV)
    work = torch.empty(b.load().tq_append_workspace_bytes(d, kb, vb, m, B, Hkv), dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty((B, Hq, T + 1), dtype=torch.float32, device=DEV)

    def step():
        b.tq_append_kv(kcb, Hkv, vcb, Hkv, kn, vn, d, kb, vb, m, pos, table, P, kpool, vpool, work=work, status=st)
        b.tq_scores_paged(kcb, Hkv, kpool, table, P, T + 1, q, d, kb, m, out=out, status=st)

    step()
    torch.cuda.synchronize()
    ref_s, ref_k, ref_v = out.clone(), kpool.clone(), vpool.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()                       # warm-up on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(3):
        out.fill_(float("nan"))
        kpool[table[:, T // P].long(), :, T % P] = -1
        vpool[table[:, T // P].long(), :, T % P] = -1
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_s), f"replay {r}: scores"
        assert torch.equal(kpool, ref_k) and torch.equal(vpool, ref_v), f"replay {r}: pools"
        _ = (out.sum() + 1.0).item()   # eager work between the replays
    assert int(st.item()) == 0
