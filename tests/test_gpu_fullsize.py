"""Parity at the full workload sizes, in the launch configuration bench.py times:
the GPU encodes / scores / attends the whole workload; the oracle checks
sampled groups and tokens, regenerating exactly those inputs on the CPU.

  * 32K-context decode step: 16 x 8 kv heads x 32768 tokens, d=128, bf16 keys
    (seed 3) -> turbo3 records; 32 bf16 query heads (GQA 4:1) scored.
  * prefill encode: 32 layers x 8 kv heads x 4096 tokens, d=128, bf16 with 4
    outlier channels x8 (seed 1); K b=4, V 4-bit.
  * long-context step: 4 x 8 kv heads x 131072 tokens, d=128, turbo2 K + 2-bit V
    (seed 4); attention output of sampled (sequence, head) pairs.
  * mixed-precision layers: 32 layers x 8 kv heads x 16384 tokens, d=256, per-
    channel std log-uniform in [0.5, 8] (seed 5); boundary layers b=8, others
    split (32 outliers at 4 bits, 224 channels at 3 bits, Haar).
  * Gram-table scoring, the paged decode step and the Haar-rotation step at
    their bench shapes (below)."""
import numpy as np
import pytest

from kv_cache_vector_diag_amd import inputs
from oracle import split
from oracle import turboquant as tq

from .parity import assert_close, check_mismatch_fraction, compare_records, rec_np

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _sample_tokens(rng, N, n):
    t = np.unique(np.concatenate([[0, N - 1], rng.choice(N, n, replace=False)]))
    return t


def _bf16_exact(a):
    return inputs.exact_values(inputs.to_torch(a, "bf16"))


def test_decode_step_32k_encode_and_scores(gpu_lib):
    import torch
    b = gpu_lib
    B, Hkv, Hq, T, d, bits, m, seed = 16, 8, 32, 32768, 128, 3, 128, 3
    G = B * Hkv
    kcb = b.make_codebooks(Hkv, d, bits, m, seed, b.ROLE_KEY, device=DEV)
    qzs = tq.quantizers(Hkv, d, bits, m, seed, tq.ROLE_KEY)
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rec = b.tq_encode_keys(kcb, Hkv, K, d, bits, m, status=st)
    scores = b.tq_scores(kcb, Hkv, rec.view(B, Hkv, T, -1), q, d, bits, m)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    del K
    rng = np.random.default_rng(0)
    qv = inputs.exact_values(q)
    reps = []
    for g in (0, 77, G - 1):
        toks = _sample_tokens(rng, T, 1500)
        X = _bf16_exact(inputs.kv_normal(seed, G, T, d, groups=[g]))[0][toks]
        grec = rec_np(rec[g])[toks]
        reps.append(compare_records(qzs[g % Hkv], grec, tq.encode(qzs[g % Hkv], X), fraction=False))
        bb, h = divmod(g, Hkv)
        ref = tq.scores([qzs[h]], grec[None, None], qv[bb:bb + 1, 4 * h:4 * h + 4])
        got = scores[bb, 4 * h:4 * h + 4][:, torch.from_numpy(toks).to(DEV)].cpu().numpy()[None]
        assert_close(got, ref, f"scores g={g}")
    check_mismatch_fraction(reps)


def test_prefill_encode_full(gpu_lib):
    import torch
    b = gpu_lib
    L, Hkv, T, d, seed = 32, 8, 4096, 128, 1
    G = L * Hkv
    Kf, Vf, _ = inputs.kv_outliers(seed, G, T, d)
    K, V = inputs.to_torch(Kf, "bf16", DEV), inputs.to_torch(Vf, "bf16", DEV)
    kcb = b.make_codebooks(G, d, 4, 128, seed, b.ROLE_KEY, device=DEV)
    vcb = b.make_codebooks(G, d, 4, 0, seed, b.ROLE_VALUE, device=DEV)
    krec = b.tq_encode_keys(kcb, G, K, d, 4, 128)
    vrec = b.tq_encode_values(vcb, G, V, d, 4)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    reps = []
    for g in (0, 131, G - 1):
        toks = _sample_tokens(rng, T, 800)
        kq = tq.Quantizer(d, 4, 128, seed + g, tq.ROLE_KEY)
        vq = tq.Quantizer(d, 4, 0, seed + g, tq.ROLE_VALUE)
        kx = inputs.exact_values(K[g])[toks]
        vx = inputs.exact_values(V[g])[toks]
        reps.append(compare_records(kq, rec_np(krec[g])[toks], tq.encode(kq, kx), fraction=False))
        reps.append(compare_records(vq, rec_np(vrec[g])[toks], tq.encode(vq, vx), fraction=False))
    check_mismatch_fraction(reps)
    # the inputs the GPU encoded are the generator's, regenerated alone on the CPU
    assert np.array_equal(inputs.exact_values(K[5]), _bf16_exact(inputs.kv_outliers(seed, G, T, d, groups=[5])[0])[0])


def test_long_context_attend_full(gpu_lib):
    import torch
    b = gpu_lib
    B, Hkv, Hq, T, d, seed = 4, 8, 8, 131072, 128, 4
    G = B * Hkv
    kcb = b.make_codebooks(Hkv, d, 2, 128, seed, b.ROLE_KEY, device=DEV)
    vcb = b.make_codebooks(Hkv, d, 2, 0, seed, b.ROLE_VALUE, device=DEV)
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_K), "bf16", DEV)
    V = inputs.to_torch(inputs.kv_normal(seed, G, T, d, inputs.STREAM_V), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    krec = b.tq_encode_keys(kcb, Hkv, K, d, 2, 128).view(B, Hkv, T, -1)
    vrec = b.tq_encode_values(vcb, Hkv, V, d, 2).view(B, Hkv, T, -1)
    del K, V
    out = b.tq_attend(kcb, Hkv, vcb, Hkv, krec, vrec, q, d, 2, 2, 128)
    torch.cuda.synchronize()
    kq = tq.quantizers(Hkv, d, 2, 128, seed, tq.ROLE_KEY)
    vq = tq.quantizers(Hkv, d, 2, 0, seed, tq.ROLE_VALUE)
    qv = inputs.exact_values(q)
    for bb, h in ((0, 0), (3, 5)):
        ref = tq.attend([kq[h]], rec_np(krec[bb, h])[None, None], [vq[h]], rec_np(vrec[bb, h])[None, None],
                        qv[bb:bb + 1, h:h + 1])
        assert_close(out[bb, h].cpu().numpy()[None, None], ref, f"attend b={bb} h={h}")


def test_mixed_precision_layers_full(gpu_lib):
    import torch
    b = gpu_lib
    L, Hkv, T, d, n_out, seed = 32, 8, 16384, 256, 32, 5
    G = L * Hkv
    s0, s1 = 2 * Hkv, (L - 2) * Hkv
    GS = s1 - s0
    rng = np.random.default_rng(2)
    reps = []
    for role, stream in ((b.ROLE_KEY, inputs.STREAM_K), (b.ROLE_VALUE, inputs.STREAM_V)):
        X = torch.empty((G, T, d), dtype=torch.bfloat16, device=DEV)
        for l in range(L):
            gl = list(range(l * Hkv, (l + 1) * Hkv))
            X[gl[0]:gl[-1] + 1] = inputs.to_torch(inputs.kv_channel_std(seed, G, T, d, stream=stream, groups=gl)[0],
                                                  "bf16", DEV)
        # split layers: channel maps, split encode (MFMA path), sampled parity
        chan = b.tq_outlier_channels(X[s0:s1], d, n_out)
        cbn, cbo = b.split_codebooks(GS, d, n_out, 3, seed + s0, role, device=DEV)
        st = torch.zeros(1, dtype=torch.int32, device=DEV)
        rn, ro = b.tq_encode_split(role, cbn, cbo, GS, X[s0:s1], d, n_out, 3, chan, status=st)
        # boundary layers 0, 1: b=8, no split
        key = role == b.ROLE_KEY
        cb8 = b.make_codebooks(s0, d, 8, d if key else 0, seed, role, device=DEV)
        r8 = (b.tq_encode_keys(cb8, s0, X[:s0], d, 8, d, status=st) if key
              else b.tq_encode_values(cb8, s0, X[:s0], d, 8, status=st))
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        for gs in (0, GS - 1):
            g = s0 + gs
            Xg = inputs.exact_values(X[g])
            ch = chan[gs].cpu().numpy()
            assert ch.tolist() == split.outlier_channels(Xg, n_out).tolist()
            sq = split.split_quantizer(d, n_out, 3, seed + g, role)
            toks = _sample_tokens(rng, T, 600)
            en, eo = split.encode_split(sq, Xg[toks], ch)
            reps.append(compare_records(sq.normal, rec_np(rn[gs])[toks], en, fraction=False))
            reps.append(compare_records(sq.outlier, rec_np(ro[gs])[toks], eo, fraction=False))
        # the first split layer's records through the split score / decode calls
        # (all 16384 tokens of its 8 heads), sampled tokens against the oracle
        toks = _sample_tokens(rng, T, 200)
        sqs = [split.split_quantizer(d, n_out, 3, seed + s0 + h, role) for h in range(Hkv)]
        ch8 = chan[:Hkv].cpu().numpy()
        rn8, ro8 = rec_np(rn[:Hkv]), rec_np(ro[:Hkv])
        if key:
            q = inputs.to_torch(inputs.queries(seed, 1, 4 * Hkv, d), "bf16", DEV)
            sc = b.tq_scores_split(cbn, cbo, GS, chan[:Hkv], rn[:Hkv].reshape(1, Hkv, T, -1),
                                   ro[:Hkv].reshape(1, Hkv, T, -1), q, d, n_out, 3, status=st)
            torch.cuda.synchronize()
            ref = split.scores_split(sqs, ch8, rn8[:, toks][None], ro8[:, toks][None], inputs.exact_values(q))
            assert_close(sc.cpu().numpy()[:, :, toks], ref, "split scores (full layer)")
        else:
            dec = b.tq_decode_values_split(cbn, cbo, GS, chan[:Hkv], rn[:Hkv], ro[:Hkv], d, n_out, 3, status=st)
            torch.cuda.synchronize()
            for h in (0, Hkv - 1):
                ref = split.decode_values_split(sqs[h], ch8[h], rn8[h][toks], ro8[h][toks])
                assert_close(dec[h].cpu().numpy()[toks], ref, f"split decode (full layer) h={h}")
        assert int(st.item()) == 0
        toks = _sample_tokens(rng, T, 300)
        q8 = tq.Quantizer(d, 8, d if key else 0, seed + 3, role)
        reps.append(compare_records(q8, rec_np(r8[3])[toks], tq.encode(q8, inputs.exact_values(X[3])[toks]),
                                    fraction=False))
        del X
    check_mismatch_fraction(reps)


def test_gram_scoring_32k_full_size(gpu_lib):
    """Gram-table scoring at the decode-step shape (16 x 8 kv heads x 32768
    tokens, d=128, blocks of 4, 32 codewords, 32 query heads), the keys and
    queries encoded on the GPU: sampled tokens of three groups against the
    oracle's encode, and their scores where the codes agree."""
    import math

    import torch
    from oracle import gram

    from .test_gpu_gram import U, _check_codes
    b = gpu_lib
    B, Hkv, Hq, T, d, k, N, seed = 16, 8, 32, 32768, 128, 4, 32, 3
    G = B * Hkv
    C = inputs.block_codebook(seed, N, k, d)
    s = inputs.sign_bits(seed, d)
    Ct = torch.from_numpy(C).to(DEV)
    st = torch.from_numpy(s.view(np.int32)).to(DEV)
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    krec = b.tq_gram_encode(Ct, st, K, d, status=status)
    qrec = b.tq_gram_encode(Ct, st, q, d, status=status)
    sc = b.tq_gram_scores(b.tq_gram_table(Ct), qrec, krec.view(B, Hkv, T, -1), d, k)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    del K
    qref, _, qdist = gram.encode(C, s, inputs.exact_values(q).reshape(-1, d), d, k)
    _check_codes(rec_np(qrec).reshape(B * Hq, -1), qref, qdist, d, k, N, "queries", C)
    qref = qref.reshape(B, Hq, -1)
    same_q = np.all(rec_np(qrec) == qref, axis=2)
    Gmax = float(np.max(np.abs(gram.gram_table(C))))
    rng = np.random.default_rng(1)
    for g in (0, 77, G - 1):
        toks = _sample_tokens(rng, T, 1500)
        X = _bf16_exact(inputs.kv_normal(seed, G, T, d, groups=[g]))[0][toks]
        kref, _, kdist = gram.encode(C, s, X, d, k)
        grec = rec_np(krec[g])[toks]
        _check_codes(grec, kref, kdist, d, k, N, f"keys g={g}", C)
        bb, h = divmod(g, Hkv)
        rows = list(range(4 * h, 4 * h + 4))
        ref = gram.scores(C, qref[bb:bb + 1, rows], kref[None, None], d, k)[0]
        got = sc[bb, 4 * h:4 * h + 4].cpu().numpy().astype(np.float64)[:, toks]
        same_k = np.all(grec == kref, axis=1)
        _, kn = gram.unpack_record(kref, d, k, N)
        for i, hq in enumerate(rows):
            if not same_q[bb, hq]:
                continue
            _, qn = gram.unpack_record(qref[bb, hq][None, :], d, k, N)
            bound = (d // k + k + 4) * U / math.sqrt(d) * qn[0] * kn * (d // k) * Gmax
            assert np.all(np.abs(got[i] - ref[i])[same_k] <= bound[same_k])


def test_paged_decode_step_full_size(gpu_lib):
    """The paged decode step at its bench shape (16 x 8 kv heads x 32768 cached
    tokens in shuffled pages of 256, turbo3 keys and 3-bit values, 32 query
    heads): one token appended per sequence, then the 32769 paged keys scored.
    The appended slots equal the batch encode of the new vectors, the paged
    scores equal tq_scores over the contiguous records bit for bit, and sampled
    rows match the oracle's scores of those records."""
    import torch
    b = gpu_lib
    B, Hkv, Hq, T, d, kb, vb, m, P, seed = 16, 8, 32, 32768, 128, 3, 3, 128, 256, 3
    G = B * Hkv
    kw = b.tq_record_bytes(d, kb, m, b.ROLE_KEY) // 4
    vw = b.tq_record_bytes(d, vb, 0, b.ROLE_VALUE) // 4
    kcb = b.make_codebooks(Hkv, d, kb, m, seed, b.ROLE_KEY, device=DEV)
    vcb = b.make_codebooks(Hkv, d, vb, 0, seed + 1, b.ROLE_VALUE, device=DEV)
    max_pages = T // P + 1
    num_pages = B * max_pages
    perm = torch.randperm(num_pages, generator=torch.Generator().manual_seed(seed)).to(torch.int32)
    table = perm.view(B, max_pages).to(DEV)
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d), "bf16", DEV)
    krec = b.tq_encode_keys(kcb, Hkv, K, d, kb, m).view(B, Hkv, T, kw)
    del K
    kpool = torch.full((num_pages, Hkv, P, kw), -1, dtype=torch.int32, device=DEV)
    vpool = torch.full((num_pages, Hkv, P, vw), -1, dtype=torch.int32, device=DEV)
    kpool[table[:, : T // P].reshape(-1).long()] = krec.view(B, Hkv, T // P, P, kw).permute(0, 2, 1, 3, 4).reshape(
        -1, Hkv, P, kw)
    kn = inputs.to_torch(inputs.kv_normal(seed + 5, B, Hkv, d), "bf16", DEV).contiguous()
    vn = inputs.to_torch(inputs.kv_normal(seed + 6, B, Hkv, d), "bf16", DEV).contiguous()
    pos = torch.full((B,), T, dtype=torch.int32, device=DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    b.tq_append_kv(kcb, Hkv, vcb, Hkv, kn, vn, d, kb, vb, m, pos, table, P, kpool, vpool, status=st)
    sp = b.tq_scores_paged(kcb, Hkv, kpool, table, P, T + 1, q, d, kb, m, status=st)
    knew = b.tq_encode_keys(kcb, Hkv, kn.transpose(0, 1).contiguous(), d, kb, m)      # [H_kv][B] records
    vnew = b.tq_encode_values(vcb, Hkv, vn.transpose(0, 1).contiguous(), d, vb)
    full = torch.cat([krec, knew.transpose(0, 1).unsqueeze(2)], dim=2).contiguous()
    sc = b.tq_scores(kcb, Hkv, full, q, d, kb, m)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    last = table[:, T // P].long()
    assert torch.equal(kpool[last, :, 0], knew.transpose(0, 1))
    assert torch.equal(vpool[last, :, 0], vnew.transpose(0, 1))
    assert torch.equal(sp, sc)
    qzs = tq.quantizers(Hkv, d, kb, m, seed, tq.ROLE_KEY)
    qv = inputs.exact_values(q)
    rng = np.random.default_rng(2)
    for bb, h in ((0, 0), (7, 3), (B - 1, Hkv - 1)):
        toks = _sample_tokens(rng, T + 1, 1500)
        grec = rec_np(full[bb, h])[toks]
        ref = tq.scores([qzs[h]], grec[None, None], qv[bb:bb + 1, 4 * h:4 * h + 4])
        assert_close(sp[bb:bb + 1, 4 * h:4 * h + 4].cpu().numpy()[:, :, toks], ref, f"paged scores b={bb} h={h}")


def test_haar_encode_and_scores_full_size(gpu_lib):
    """Haar-rotation codebooks at their bench shape (16 x 8 kv heads x 4096
    tokens, d=128, bf16 keys b=3 with 128 projections, 32 query heads), on the
    matrix-core encode and the score kernel: sampled tokens of three groups
    against the oracle, records and scores."""
    import torch
    b = gpu_lib
    B, Hkv, Hq, T, d, bits, m, seed = 16, 8, 32, 4096, 128, 3, 128, 3
    G = B * Hkv
    kcb = b.make_codebooks(Hkv, d, bits, m, seed, b.ROLE_KEY, device=DEV, rotation=b.ROT_HAAR)
    qzs = [tq.Quantizer(d, bits, m, seed + h, tq.ROLE_KEY, rotation=tq.ROT_HAAR) for h in range(Hkv)]
    K = inputs.to_torch(inputs.kv_normal(seed, G, T, d), "bf16", DEV)
    q = inputs.to_torch(inputs.queries(seed, B, Hq, d), "bf16", DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    rec = b.tq_encode_keys(kcb, Hkv, K, d, bits, m, status=st, rotation=b.ROT_HAAR)
    scores = b.tq_scores(kcb, Hkv, rec.view(B, Hkv, T, -1), q, d, bits, m, status=st, rotation=b.ROT_HAAR)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    del K
    rng = np.random.default_rng(3)
    qv = inputs.exact_values(q)
    reps = []
    for g in (0, 45, G - 1):
        toks = _sample_tokens(rng, T, 1000)
        X = _bf16_exact(inputs.kv_normal(seed, G, T, d, groups=[g]))[0][toks]
        grec = rec_np(rec[g])[toks]
        reps.append(compare_records(qzs[g % Hkv], grec, tq.encode(qzs[g % Hkv], X), fraction=False))
        bb, h = divmod(g, Hkv)
        ref = tq.scores([qzs[h]], grec[None, None], qv[bb:bb + 1, 4 * h:4 * h + 4])
        got = scores[bb, 4 * h:4 * h + 4][:, torch.from_numpy(toks).to(DEV)].cpu().numpy()[None]
        assert_close(got, ref, f"Haar scores g={g}")
    check_mismatch_fraction(reps)
