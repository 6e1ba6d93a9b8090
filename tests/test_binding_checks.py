"""The Python binding refuses mismatched tensors before anything is enqueued.

The kernels take raw pointers and sizes, so the binding checks every
caller-supplied tensor (device, dtype, contiguity, shape or byte size) first.
These tests run on the CPU: the library is replaced by a guard that lets the
host-only size queries through and fails the test if any device entry point
is reached.  Every call below must raise ValueError from the binding itself;
a call that is right in every respect but holds CPU tensors is refused last,
as not on a GPU."""
import numpy as np
import pytest
import torch

from kv_cache_vector_diag_amd import binding as b

DEVICE_CALLS = {"tq_encode_keys", "tq_encode_values", "tq_encode_kv", "tq_decode_values", "tq_scores", "tq_attend", "tq_rotate",
                "tq_outlier_channels", "tq_encode_split", "tq_scores_split", "tq_decode_values_split",
                "tq_encode_keys_ex", "tq_encode_values_ex", "tq_decode_values_ex", "tq_scores_ex", "tq_attend_ex",
                "tq_append_kv", "tq_scores_paged", "tq_gram_table", "tq_gram_encode", "tq_gram_scores"}


class _Guard:
    def __init__(self, real):
        self.real = real

    def __getattr__(self, name):
        if name in DEVICE_CALLS:
            raise AssertionError(f"{name} was reached with unchecked arguments")
        return getattr(self.real, name)


@pytest.fixture
def lib(monkeypatch):
    real = b.load()
    guard = _Guard(real)
    monkeypatch.setattr(b, "load", lambda: guard)
    return b


D, BITS, M = 128, 3, 128
KW = 14   # turbo3 key record words at head_dim 128
VW = 13   # 3-bit value record words


def _cbs(n, role=b.ROLE_KEY, bits=BITS, m=M):
    return torch.zeros(n * b.tq_codebook_bytes(D, bits, m, role), dtype=torch.uint8)


def test_encode_checks(lib):
    x = torch.zeros((2, 5, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="rec has shape"):
        lib.tq_encode_keys(_cbs(2), 2, x, D, BITS, M, rec=torch.zeros((2, 4, KW), dtype=torch.int32))
    with pytest.raises(ValueError, match="rec has dtype"):
        lib.tq_encode_keys(_cbs(2), 2, x, D, BITS, M, rec=torch.zeros((2, 5, KW), dtype=torch.float32))
    with pytest.raises(ValueError, match="cbs holds"):
        lib.tq_encode_keys(_cbs(1), 2, x, D, BITS, M)
    with pytest.raises(ValueError, match="status"):
        lib.tq_encode_keys(_cbs(2), 2, x, D, BITS, M, status=torch.zeros(1, dtype=torch.int64))
    with pytest.raises(ValueError, match="is on meta"):
        lib.tq_encode_keys(_cbs(2), 2, x, D, BITS, M, rec=torch.empty((2, 5, KW), dtype=torch.int32, device="meta"))
    with pytest.raises(ValueError, match="unsupported dtype"):
        lib.tq_encode_values(_cbs(2, b.ROLE_VALUE, 3, 0), 2, x.to(torch.int16), D, 3)
    with pytest.raises(ValueError, match="expected \\[G\\]\\[N\\]"):
        lib.tq_encode_values(_cbs(2, b.ROLE_VALUE, 3, 0), 2, x[:, :, :64], D, 3)
    with pytest.raises(ValueError, match="on the GPU"):
        lib.tq_encode_keys(_cbs(2), 2, x, D, BITS, M, rec=torch.zeros((2, 5, KW), dtype=torch.int32),
                           status=torch.zeros(1, dtype=torch.int32))


def test_encode_kv_checks(lib):
    k = torch.zeros((2, 5, D), dtype=torch.bfloat16)
    vcb = _cbs(2, b.ROLE_VALUE, 3, 0)
    with pytest.raises(ValueError, match="v must match k"):
        lib.tq_encode_kv(_cbs(2), 2, vcb, 2, k, torch.zeros((2, 4, D), dtype=torch.bfloat16), D, BITS, 3, M)
    with pytest.raises(ValueError, match="v must match k"):
        lib.tq_encode_kv(_cbs(2), 2, vcb, 2, k, torch.zeros((2, 5, D), dtype=torch.float32), D, BITS, 3, M)
    with pytest.raises(ValueError, match="krec has shape"):
        lib.tq_encode_kv(_cbs(2), 2, vcb, 2, k, k.clone(), D, BITS, 3, M, krec=torch.zeros((2, 5, KW + 1), dtype=torch.int32))
    with pytest.raises(ValueError, match="vrec has shape"):
        lib.tq_encode_kv(_cbs(2), 2, vcb, 2, k, k.clone(), D, BITS, 3, M, vrec=torch.zeros((2, 5, VW - 1), dtype=torch.int32))
    with pytest.raises(ValueError, match="vcbs holds"):
        lib.tq_encode_kv(_cbs(2), 2, _cbs(1, b.ROLE_VALUE, 3, 0), 2, k, k.clone(), D, BITS, 3, M)
    with pytest.raises(ValueError, match="on the GPU"):
        lib.tq_encode_kv(_cbs(2), 2, vcb, 2, k, k.clone(), D, BITS, 3, M)


def test_decode_and_score_checks(lib):
    vrec = torch.zeros((2, 5, VW), dtype=torch.int32)
    with pytest.raises(ValueError, match="rec has shape"):
        lib.tq_decode_values(_cbs(2, b.ROLE_VALUE, 3, 0), 2, torch.zeros((2, 5, VW + 1), dtype=torch.int32), D, 3)
    with pytest.raises(ValueError, match="out has shape"):
        lib.tq_decode_values(_cbs(2, b.ROLE_VALUE, 3, 0), 2, vrec, D, 3, out=torch.zeros((2, 5, 64)))
    krec = torch.zeros((2, 2, 7, KW), dtype=torch.int32)
    q = torch.zeros((2, 8, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="krec has shape"):
        lib.tq_scores(_cbs(2), 2, torch.zeros((2, 2, 7, KW - 1), dtype=torch.int32), q, D, BITS, M)
    with pytest.raises(ValueError, match="krec must be contiguous"):
        lib.tq_scores(_cbs(2), 2, torch.zeros((2, 2, KW, 7), dtype=torch.int32).transpose(2, 3), q, D, BITS, M)
    with pytest.raises(ValueError, match="q must be contiguous"):
        lib.tq_scores(_cbs(2), 2, krec, q[:1], D, BITS, M)
    with pytest.raises(ValueError, match="out has shape"):
        lib.tq_scores(_cbs(2), 2, krec, q, D, BITS, M, out=torch.zeros((2, 8, 6)))
    with pytest.raises(ValueError, match="cbs holds"):
        lib.tq_scores(_cbs(1), 2, krec, q, D, BITS, M)
    with pytest.raises(ValueError, match="on the GPU"):
        lib.tq_scores(_cbs(2), 2, krec, q, D, BITS, M, out=torch.zeros((2, 8, 7)))


def test_attend_checks(lib):
    krec = torch.zeros((1, 2, 9, KW), dtype=torch.int32)
    vrec = torch.zeros((1, 2, 9, VW), dtype=torch.int32)
    q = torch.zeros((1, 4, D), dtype=torch.bfloat16)
    vcb = _cbs(2, b.ROLE_VALUE, 3, 0)
    with pytest.raises(ValueError, match="vrec has shape"):
        lib.tq_attend(_cbs(2), 2, vcb, 2, krec, vrec[:, :, :8], q, D, BITS, 3, M)
    with pytest.raises(ValueError, match="work holds"):
        lib.tq_attend(_cbs(2), 2, vcb, 2, krec, vrec, q, D, BITS, 3, M, work=torch.zeros(16, dtype=torch.uint8))
    with pytest.raises(ValueError, match="vcbs holds"):
        lib.tq_attend(_cbs(2), 2, vcb[:10], 2, krec, vrec, q, D, BITS, 3, M)
    need = lib.tq_attend_workspace_bytes(D, 1, 4, 9)
    with pytest.raises(ValueError, match="on the GPU"):
        lib.tq_attend(_cbs(2), 2, vcb, 2, krec, vrec, q, D, BITS, 3, M, work=torch.zeros(need, dtype=torch.uint8))


def test_paged_checks(lib):
    B, Hkv, P, pages = 3, 2, 32, 4
    kn = torch.zeros((B, Hkv, D), dtype=torch.bfloat16)
    kpool = torch.zeros((pages, Hkv, P, KW), dtype=torch.int32)
    vpool = torch.zeros((pages, Hkv, P, VW), dtype=torch.int32)
    table = torch.zeros((B, 2), dtype=torch.int32)
    pos = torch.zeros(B, dtype=torch.int32)
    vcb = _cbs(Hkv, b.ROLE_VALUE, 3, 0)
    with pytest.raises(ValueError, match="pos holds"):
        lib.tq_append_kv(_cbs(Hkv), Hkv, vcb, Hkv, kn, kn, D, BITS, 3, M, pos[:2], table, P, kpool, vpool)
    with pytest.raises(ValueError, match="page_table must be"):
        lib.tq_append_kv(_cbs(Hkv), Hkv, vcb, Hkv, kn, kn, D, BITS, 3, M, pos, table[:2], P, kpool, vpool)
    with pytest.raises(ValueError, match="vpool has shape"):
        lib.tq_append_kv(_cbs(Hkv), Hkv, vcb, Hkv, kn, kn, D, BITS, 3, M, pos, table, P, kpool, vpool[:3])
    with pytest.raises(ValueError, match="kpool has shape"):
        lib.tq_append_kv(_cbs(Hkv), Hkv, vcb, Hkv, kn, kn, D, BITS, 3, M, pos, table, 64, kpool, vpool)
    with pytest.raises(ValueError, match="v_new has shape"):
        lib.tq_append_kv(_cbs(Hkv), Hkv, vcb, Hkv, kn, kn[:2], D, BITS, 3, M, pos, table, P, kpool, vpool)
    with pytest.raises(ValueError, match="on the GPU"):
        lib.tq_append_kv(_cbs(Hkv), Hkv, vcb, Hkv, kn, kn, D, BITS, 3, M, pos, table, P, kpool, vpool,
                         work=torch.zeros(1 << 20, dtype=torch.uint8))
    q = torch.zeros((B, 4, D), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="page_table must be"):
        lib.tq_scores_paged(_cbs(Hkv), Hkv, kpool, table[:1], P, 40, q, D, BITS, M)
    with pytest.raises(ValueError, match="exceeds the page table"):
        lib.tq_scores_paged(_cbs(Hkv), Hkv, kpool, table, P, 65, q, D, BITS, M)
    with pytest.raises(ValueError, match="on the GPU"):
        lib.tq_scores_paged(_cbs(Hkv), Hkv, kpool, table, P, 40, q, D, BITS, M)


def test_split_checks(lib):
    d, n_out, bits, G, N = 256, 32, 3, 2, 6
    cbn, cbo = b.split_codebooks(G, d, n_out, bits, 5, b.ROLE_KEY, device="cpu")
    x = torch.zeros((G, N, d), dtype=torch.bfloat16)
    chan = torch.zeros((G, d), dtype=torch.int32)
    with pytest.raises(ValueError, match="chan has shape"):
        lib.tq_encode_split(b.ROLE_KEY, cbn, cbo, G, x, d, n_out, bits, chan[:1])
    with pytest.raises(ValueError, match="cbs_outlier holds"):
        lib.tq_encode_split(b.ROLE_KEY, cbn, cbo[:100], G, x, d, n_out, bits, chan)
    wn, wo = b.split_record_words(d, n_out, bits, b.ROLE_KEY)
    with pytest.raises(ValueError, match="rec_outlier has shape"):
        lib.tq_encode_split(b.ROLE_KEY, cbn, cbo, G, x, d, n_out, bits, chan,
                            rec_outlier=torch.zeros((G, N, wo + 1), dtype=torch.int32))
    kn = torch.zeros((1, G, N, wn), dtype=torch.int32)
    ko = torch.zeros((1, G, N, wo), dtype=torch.int32)
    q = torch.zeros((1, 4, d), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="krec_outlier has shape"):
        lib.tq_scores_split(cbn, cbo, G, chan, kn, ko[:, :1], q, d, n_out, bits)
    with pytest.raises(ValueError, match="on the GPU"):
        lib.tq_scores_split(cbn, cbo, G, chan, kn, ko, q, d, n_out, bits)


def test_gram_checks(lib):
    d, k, N = 128, 4, 32
    C = torch.zeros((N, k), dtype=torch.float32)
    x = torch.zeros((2, 3, d), dtype=torch.float32)
    with pytest.raises(ValueError, match="signs holds"):
        lib.tq_gram_encode(C, torch.zeros(3, dtype=torch.int32), x, d)
    with pytest.raises(ValueError, match="codebook must be contiguous"):
        lib.tq_gram_encode(C.double(), torch.zeros(4, dtype=torch.int32), x, d)
    words = b.tq_gram_record_bytes(d, k, N) // 4
    krec = torch.zeros((1, 2, 5, words), dtype=torch.int32)
    table = torch.zeros((N, N), dtype=torch.float32)
    with pytest.raises(ValueError, match="qrec has shape"):
        lib.tq_gram_scores(table, torch.zeros((1, 4, words - 1), dtype=torch.int32), krec, d, k)
    with pytest.raises(ValueError, match="table has shape"):
        lib.tq_gram_scores(table[:, :16], torch.zeros((1, 4, words), dtype=torch.int32), krec, d, k)
    with pytest.raises(ValueError, match="on the GPU"):
        lib.tq_gram_scores(table, torch.zeros((1, 4, words), dtype=torch.int32), krec, d, k)


def test_split_codebooks_carry_the_part_seed_rule():
    """tq_make_split_codebooks seeds the outlier part with the head seed XOR the
    golden-ratio constant: its blobs equal tq_make_codebook_ex at that seed."""
    d, n_out, bits, seed = 256, 32, 3, 11
    cbn, cbo = b.split_codebooks(2, d, n_out, bits, seed, b.ROLE_KEY)
    nb = b.tq_split_codebook_bytes(b.ROLE_KEY, d, n_out, bits, 0)
    ob = b.tq_split_codebook_bytes(b.ROLE_KEY, d, n_out, bits, 1)
    for i in range(2):
        want_n = b.tq_make_codebook_ex(d - n_out, bits, d - n_out, seed + i, b.ROLE_KEY, b.ROT_HAAR)
        want_o = b.tq_make_codebook_ex(n_out, bits + 1, n_out, (seed + i) ^ 0x9E3779B97F4A7C15, b.ROLE_KEY,
                                       b.ROT_HADAMARD)
        assert np.array_equal(cbn[i * nb:(i + 1) * nb], want_n)
        assert np.array_equal(cbo[i * ob:(i + 1) * ob], want_o)
    assert b.tq_split_codebook_bytes(b.ROLE_KEY, d, 0, bits, 0) == 0
    assert b.tq_split_codebook_bytes(b.ROLE_KEY, d, n_out, bits, 2) == 0
