"""The GPU parity helper (tests/parity.py) catches what it is meant to catch.

Mistakes are planted in oracle records on the CPU: a record that differs from
the canonical one only in an unused high bit of a plane word (head_dim below
32) or of the last sign word (projections not a multiple of 32) must fail the
comparison, as must a flipped index or sign far from any decision boundary;
the unchanged records pass.  The canonical record is bit-planar with unused
bits zero (page "turboquant-plus-rs 0.1.0 README", "Modules" utils, bit
packing)."""
import numpy as np
import pytest

from oracle import turboquant as tq

from .parity import compare_records


def _encoded(d, bits, m, role, n=40, seed=3):
    qz = tq.Quantizer(d, bits, m, seed, role)
    x = np.random.default_rng(seed).standard_normal((n, d))
    return qz, tq.encode(qz, x)


@pytest.mark.parametrize("d,bits,m,role", [(8, 3, 7, tq.ROLE_KEY), (2, 2, 1, tq.ROLE_KEY), (16, 4, 0, tq.ROLE_VALUE),
                                           (64, 3, 33, tq.ROLE_KEY)])
def test_unchanged_records_pass(d, bits, m, role):
    qz, enc = _encoded(d, bits, m, role)
    rep = compare_records(qz, enc.records.copy(), enc)
    assert rep.idx_mismatch_in_band == 0 and rep.sign_mismatch_in_band == 0


@pytest.mark.parametrize("d,bits,role", [(8, 3, tq.ROLE_KEY), (2, 2, tq.ROLE_KEY), (16, 4, tq.ROLE_VALUE)])
def test_stray_high_plane_bit_fails(d, bits, role):
    qz, enc = _encoded(d, bits, 7 if role == tq.ROLE_KEY else 0, role)
    rec = enc.records.copy()
    rec[5, 0] |= np.uint32(1 << 31)          # bit 31 of plane 0 lies past coordinate d-1
    # the unpacked fields are unchanged, only the raw word differs
    assert np.array_equal(tq.unpack_record(qz, rec).idx, enc.idx)
    with pytest.raises(AssertionError, match="unused bits"):
        compare_records(qz, rec, enc)


@pytest.mark.parametrize("m", [1, 7, 33, 100])
def test_stray_high_sign_bit_fails(m):
    qz, enc = _encoded(32, 3, m, tq.ROLE_KEY)
    rec = enc.records.copy()
    last = qz.k * 1 + (m + 31) // 32 - 1    # the last sign word
    rec[9, last] |= np.uint32(1 << 31)       # bit 31 of it lies past projection m-1 (m mod 32 != 0)
    assert np.array_equal(tq.unpack_record(qz, rec).signs, tq.unpack_record(qz, enc.records).signs)
    with pytest.raises(AssertionError, match="unused bits"):
        compare_records(qz, rec, enc)


def test_out_of_band_index_and_sign_flips_fail():
    qz, enc = _encoded(32, 3, 32, tq.ROLE_KEY)
    rec = enc.records.copy()
    rec[3, 0] ^= np.uint32(1)                # bit 0 of coordinate 0's index
    with pytest.raises(AssertionError, match="index mismatches outside"):
        compare_records(qz, rec, enc)
    rec = enc.records.copy()
    i = int(np.argmax(np.abs(enc.proj[4])))  # the sign farthest from its boundary
    rec[4, qz.k + i // 32] ^= np.uint32(1 << (i % 32))
    with pytest.raises(AssertionError, match="sign mismatches outside"):
        compare_records(qz, rec, enc)
