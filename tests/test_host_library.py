"""Host-side checks of libtq (no GPU): exports, sizes, errors, and the codebook
blob against the oracle's independent regeneration of c, t, D and S."""
import ctypes
import math
import os
import re
import struct

import numpy as np
import pytest

from kv_cache_vector_diag_amd import binding as b
from oracle import turboquant as tq
from oracle.lloyd import stored_codebook
from oracle.prng import qjl_matrix, sign_diagonal

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    hdr = open(os.path.join(ROOT, "include", "tq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:size_t|int|const char\*)\s+(tq_\w+)\s*\(", hdr, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = b.load()
    names = _declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(b.EXPORTS) == names


def _parse_blob(blob):
    (magic, ver, d, bits, m, role, k, levels, seed, oc, ot, od, os_, total, rot) = struct.unpack_from(
        "<IIiiiiiiQIIIIII", blob.tobytes(), 0)
    return dict(magic=magic, ver=ver, d=d, bits=bits, m=m, role=role, k=k, levels=levels, seed=seed,
                off_c=oc, off_t=ot, off_d=od, off_s=os_, total=total, rotation=rot)


@pytest.mark.parametrize("d,bits,m,role,seed", [
    (128, 3, 128, 0, 42), (128, 4, 128, 0, 1), (128, 2, 128, 0, 4), (128, 4, 0, 1, 1), (128, 2, 0, 1, 4),
    (8, 4, 16, 0, 42), (8, 4, 16, 1, 42), (256, 8, 256, 0, 5), (256, 8, 0, 1, 5), (32, 4, 32, 0, 2**64 - 3),
    (2, 2, 1, 0, 7), (512, 9, 1024, 0, 3), (64, 1, 0, 1, 9), (256, 4, 32, 0, 5 ^ 0x9E3779B97F4A7C15),
])
def test_blob_matches_oracle(d, bits, m, role, seed):
    blob = b.tq_make_codebook(d, bits, m, seed, role)
    assert blob.nbytes == b.tq_codebook_bytes(d, bits, m, role) and blob.nbytes % 256 == 0
    h = _parse_blob(blob)
    qz = tq.Quantizer(d, bits, m, seed, role)
    assert h["magic"] == 0x42435154 and h["ver"] == 1 and h["rotation"] == 0
    assert (h["d"], h["bits"], h["role"], h["k"], h["levels"], h["seed"]) == (d, bits, role, qz.k, 1 << qz.k, seed)
    assert h["m"] == (m if role == 0 else 0)
    L = 1 << qz.k
    c = np.frombuffer(blob[h["off_c"]:h["off_c"] + 4 * L].tobytes(), dtype="<f4").astype(np.float64)
    t = np.frombuffer(blob[h["off_t"]:h["off_t"] + 4 * L].tobytes(), dtype="<f4").astype(np.float64)
    c32, t32 = stored_codebook(qz.k)
    assert np.array_equal(c, c32)
    assert np.array_equal(t[:L - 1], t32) and t[L - 1] == math.inf
    W = (d + 31) // 32
    dw = np.frombuffer(blob[h["off_d"]:h["off_d"] + 4 * W].tobytes(), dtype="<u4")
    dbits = tq.unpack_bits(dw[None, :], d)[0]
    assert np.array_equal(np.where(dbits == 1, -1.0, 1.0), sign_diagonal(seed, d))
    if role == 0:
        S = np.frombuffer(blob[h["off_s"]:h["off_s"] + 2 * m * d].tobytes(), dtype="<f2").astype(np.float64)
        assert np.array_equal(S.reshape(m, d), qjl_matrix(seed, m, d))
    else:
        assert h["off_s"] == 0


@pytest.mark.parametrize("d,bits,m,role,seed", [
    (224, 3, 224, 0, 5), (224, 3, 0, 1, 5), (224, 8, 0, 1, 77), (12, 4, 12, 0, 99), (3, 2, 1, 0, 1), (2, 1, 0, 1, 8),
])
def test_haar_blob_matches_oracle(d, bits, m, role, seed):
    blob = b.tq_make_codebook_ex(d, bits, m, seed, role, b.ROT_HAAR)
    assert blob.nbytes == b.tq_codebook_bytes_ex(d, bits, m, role, b.ROT_HAAR) and blob.nbytes % 256 == 0
    h = _parse_blob(blob)
    qz = tq.Quantizer(d, bits, m, seed, role, rotation=tq.ROT_HAAR)
    assert h["rotation"] == 1 and (h["d"], h["bits"], h["k"], h["seed"]) == (d, bits, qz.k, seed)
    L = 1 << qz.k
    c = np.frombuffer(blob[h["off_c"]:h["off_c"] + 4 * L].tobytes(), dtype="<f4").astype(np.float64)
    assert np.array_equal(c, qz.c32)
    R = np.frombuffer(blob[h["off_d"]:h["off_d"] + 4 * d * d].tobytes(), dtype="<f4").astype(np.float64)
    R = R.reshape(d, d)
    # two independent float64 QR factorisations (Householder here, LAPACK in the
    # oracle) agree to ~1e-14; after rounding to float32 an entry may sit on the
    # other side of a rounding boundary: allow a handful of one-ulp differences
    diff = R != qz.R
    ulp = np.spacing(np.abs(qz.R).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(R - qz.R)[diff] <= ulp[diff])
    assert diff.sum() <= max(2, d * d // 5000)
    if role == 0:
        S = np.frombuffer(blob[h["off_s"]:h["off_s"] + 2 * m * d].tobytes(), dtype="<f2").astype(np.float64)
        assert np.array_equal(S.reshape(m, d), qz.S)
    assert b.tq_record_bytes_ex(d, bits, m, role, b.ROT_HAAR) == 4 * qz.words


def test_split_host_validation():
    lib = b.load()
    # normal part Haar 224 at bits, outlier part Hadamard 32 at bits + 1
    assert b.split_record_words(256, 32, 3, b.ROLE_KEY) == (23, 6)
    assert b.split_record_words(256, 32, 3, b.ROLE_VALUE) == (22, 5)
    assert lib.tq_encode_split(0, 256, 24, 3, None, None, 1, None, 1, 1, 1, 256, 256, None, None, None, None, 0,
                               None, None) == -2                                  # outlier width not a power of two
    assert lib.tq_encode_split(0, 256, 32, 9, None, None, 1, None, 1, 1, 1, 256, 256, None, None, None, None, 0,
                               None, None) == -3                                  # outlier part would need 10 bits
    assert lib.tq_encode_split(0, 256, 0, 3, None, None, 1, None, 1, 1, 1, 256, 256, None, None, None, None, 0,
                               None, None) == -5
    assert lib.tq_encode_split(0, 256, 32, 3, None, None, 1, None, 1, 0, 1, 256, 256, None, None, None, None, 0,
                               None, None) == 0
    assert lib.tq_encode_split(0, 256, 32, 3, None, None, 1, None, 1, 2, 1, 256, 256, None, None, None, None, 0,
                               None, None) == -8
    assert lib.tq_outlier_channels(256, 256, None, 1, 1, 1, 256, 256, None, None, 0, None) == -5
    assert lib.tq_outlier_channels(600, 8, None, 1, 1, 1, 600, 600, None, None, 0, None) == -2
    assert lib.tq_outlier_workspace_bytes(256, 256, 16384) == 256 * 32 * 256 * 16 + 256
    # MFMA split path scratch: per-group fragments (keys 454, values 354 of 1 KiB)
    assert b.tq_encode_split_workspace_bytes(0, 256, 32, 3, 224) == 224 * 454 * 1024
    assert b.tq_encode_split_workspace_bytes(1, 256, 32, 3, 224) == 224 * 354 * 1024
    assert b.tq_encode_split_workspace_bytes(0, 256, 32, 5, 224) == 0      # shape without the MFMA path
    assert b.tq_encode_split_workspace_bytes(0, 128, 32, 3, 224) == 0
    assert b.tq_codebook_bytes_ex(224, 3, 224, 0, 2) == 0
    with pytest.raises(b.TQError) as e:
        b.tq_make_codebook_ex(224, 3, 224, 1, 0, 2)
    assert e.value.code == -14
    with pytest.raises(b.TQError) as e:
        b.tq_make_codebook_ex(224, 3, 224, 1, 0, b.ROT_HADAMARD)
    assert e.value.code == -2


def test_record_and_codebook_sizes_match_oracle():
    for d in (2, 8, 32, 64, 128, 256, 512):
        for bits in range(2, 10):
            for m in (1, 16, 31, 32, 33, 128, 1024):
                assert b.tq_record_bytes(d, bits, m, 0) == 4 * tq.record_words(d, bits, m, 0)
        for bits in range(1, 9):
            assert b.tq_record_bytes(d, bits, 0, 1) == 4 * tq.record_words(d, bits, 0, 1)


@pytest.mark.parametrize("args,code", [
    ((0, 3, 8, 0), -1), ((6, 3, 8, 0), -2), ((1024, 3, 8, 0), -2), ((8, 1, 8, 0), -3), ((8, 10, 8, 0), -3),
    ((8, 0, 0, 1), -3), ((8, 9, 0, 1), -3), ((8, 3, 0, 0), -4), ((8, 3, 2000, 0), -12), ((8, 3, 8, 2), -11),
])
def test_argument_errors(args, code):
    assert b.tq_codebook_bytes(*args) == 0 and b.tq_record_bytes(*args) == 0
    with pytest.raises(b.TQError) as e:
        b.tq_make_codebook(args[0], args[1], args[2], 1, args[3])
    assert e.value.code == code


def test_blob_too_small_and_null():
    lib = b.load()
    buf = np.zeros(64, dtype=np.uint8)
    assert lib.tq_make_codebook(128, 3, 128, 1, 0, buf.ctypes.data, buf.nbytes) == -9
    assert lib.tq_make_codebook(128, 3, 128, 1, 0, None, 1 << 20) == -8


def test_memory_stats_matches_oracle_and_table():
    for args in [(128, 3, 3, 128, 1024, 32, 32), (128, 4, 4, 128, 4096, 32, 8), (256, 8, 8, 256, 16384, 4, 8),
                 (8, 4, 4, 16, 0, 1, 1)]:
        mine = b.tq_memory_stats(*args)
        ref = tq.memory_stats(*args)
        for key in ref:
            assert mine[key] == pytest.approx(ref[key], rel=1e-15)


def test_device_calls_validate_before_touching_the_gpu():
    lib = b.load()
    # invalid parameters and empty inputs return before any HIP call
    assert lib.tq_encode_keys(6, 3, 8, None, 1, None, 0, 1, 1, 6, 6, None, None, None) == -2
    assert lib.tq_encode_keys(128, 3, 128, None, 0, None, 0, 1, 1, 128, 128, None, None, None) == -7
    assert lib.tq_encode_keys(128, 3, 128, None, 1, None, 0, 0, 5, 128, 128, None, None, None) == 0
    assert lib.tq_encode_keys(128, 3, 128, None, 1, None, 0, 2, 5, 128, 128, None, None, None) == -8
    assert lib.tq_encode_values(128, 9, None, 1, None, 0, 1, 1, 128, 128, None, None, None) == -3
    assert lib.tq_scores(128, 3, 128, None, 1, None, 1, 3, 10, None, 0, 4, 0.0, None, None, None) == -5
    assert lib.tq_decode_values(128, 3, None, 1, None, 0, 10, None, None, None) == 0
    # tq_encode_kv: both sides' parameters and inputs are checked before any launch
    assert lib.tq_encode_kv(128, 3, 9, 128, None, 1, None, 1, None, None, 0, 1, 1, 128, 128, None, None, None,
                            None) == -3
    assert lib.tq_encode_kv(96, 3, 3, 128, None, 1, None, 1, None, None, 0, 1, 1, 96, 96, None, None, None,
                            None) == -2
    assert lib.tq_encode_kv(128, 3, 3, 128, None, 1, None, 1, None, None, 0, 0, 5, 128, 128, None, None, None,
                            None) == 0
    assert lib.tq_encode_kv(128, 3, 3, 128, None, 1, None, 1, None, None, 0, 2, 5, 128, 128, None, None, None,
                            None) == -8
    one = ctypes.c_void_p(16)
    assert lib.tq_encode_kv(128, 3, 3, 128, one, 1, one, 0, one, one, 0, 2, 5, 128, 128, one, one, None,
                            None) == -7
    assert lib.tq_encode_kv(128, 3, 3, 128, one, 1, one, 1, one, one, 0, 2, 5, 128, 128, one, None, None,
                            None) == -8


def test_gram_calls_validate_before_touching_the_gpu():
    """Gram-table codec: sizes agree with the oracle, bad shapes are refused on
    the host before any HIP call."""
    from oracle import gram
    lib = b.load()
    for d, k, N in ((128, 4, 32), (64, 4, 32), (512, 1, 256), (2, 1, 2), (16, 8, 4), (256, 2, 64)):
        assert b.tq_gram_record_bytes(d, k, N) == 4 * gram.record_words(d, k, N)
    for d, k, N, code in ((96, 4, 32, -2), (0, 4, 32, -1), (128, 3, 32, -2), (4, 8, 32, -2), (128, 4, 24, -15),
                          (128, 4, 512, -15), (128, 4, 1, -15)):
        assert lib.tq_gram_record_bytes(d, k, N) == 0
        assert lib.tq_gram_encode(d, k, N, None, None, None, 0, 1, 1, 128, 128, None, None, None) == code
        assert lib.tq_gram_scores(d, k, N, None, None, None, 1, 1, 1, 1, 0.0, None, None) == code
    assert lib.tq_gram_table(3, 32, None, None, None) == -2
    assert lib.tq_gram_table(4, 32, None, None, None) == -8
    assert lib.tq_gram_encode(128, 4, 32, None, None, None, 0, 0, 5, 128, 128, None, None, None) == 0
    assert lib.tq_gram_encode(128, 4, 32, None, None, None, 0, 2, 5, 128, 128, None, None, None) == -8
    assert lib.tq_gram_encode(128, 4, 32, None, None, None, 0, -1, 5, 128, 128, None, None, None) == -7
    assert lib.tq_gram_scores(128, 4, 32, None, None, None, 1, 3, 10, 4, 0.0, None, None) == -5
    assert lib.tq_gram_scores(128, 4, 32, None, None, None, 0, 2, 10, 4, 0.0, None, None) == 0
    assert lib.tq_gram_scores(128, 4, 32, None, None, None, 1, 2, 10, 4, 0.0, None, None) == -8
    assert "InvalidCodebook" in lib.tq_status_string(-15).decode()


def test_build_refuses_undefined_own_symbols(tmp_path):
    """The build's last check: a shared library that leaves one of the
    library's own (tq::) symbols undefined is refused and removed, as when the
    host pass drops a kernel's launch stub; one without such a symbol passes."""
    import shutil
    import subprocess
    from kv_cache_vector_diag_amd import build_lib
    if shutil.which("g++") is None or shutil.which("nm") is None:
        pytest.skip("needs g++ and nm")
    bad_src = tmp_path / "bad.cpp"
    bad_src.write_text("namespace tq { void missing_stub(); }\nextern \"C\" void entry() { tq::missing_stub(); }\n")
    good_src = tmp_path / "good.cpp"
    good_src.write_text("namespace tq { void stub() {} }\nextern \"C\" void entry() { tq::stub(); }\n")
    bad, good = tmp_path / "libbad.so", tmp_path / "libgood.so"
    for src, lib in ((bad_src, bad), (good_src, good)):
        subprocess.run(["g++", "-shared", "-fPIC", "-o", str(lib), str(src)], check=True)
    build_lib._check_symbols(str(good))
    assert good.exists()
    with pytest.raises(RuntimeError, match="_ZN2tq12missing_stubEv"):
        build_lib._check_symbols(str(bad))
    assert not bad.exists()
