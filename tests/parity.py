"""Comparison helpers for GPU-vs-oracle parity (used by the gpu tests).

Tolerances: codes and signs bit-exact except coordinates within
1e-6 of a decision boundary (z within 1e-6 of a threshold; |(S rho)_i| within
1e-6 gamma of 0); the number of such mismatches must stay below 1e-5 of all
coordinates -- a rate, so it is checked over all the coordinates a test encodes
(check_mismatch_fraction over the reports of its groups), not per group, where
a single in-band flip among fewer than 1e5 coordinates would already exceed
it; a vector with an excepted index mismatch is left out of the sign, norm and
score checks.  Rotated vectors and norms: 1e-5 relative.  Scores and
decoded values: |gpu - oracle| <= 1e-4 + 1e-3 |oracle|.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from oracle import turboquant as tq

BAND = 1e-6
MISMATCH_FRACTION = 1e-5
ATOL, RTOL = 1e-4, 1e-3


@dataclass
class RecordReport:
    vectors: int
    coords: int
    idx_mismatch_in_band: int
    sign_mismatch_in_band: int
    excluded_vectors: int
    max_rel_n: float
    max_rel_gamma: float
    sign_coords: int = 0


def check_mismatch_fraction(reports) -> None:
    """In-band mismatches over all the reports' coordinates stay below 1e-5 of them."""
    idx = sum(r.idx_mismatch_in_band for r in reports)
    coords = sum(r.coords for r in reports)
    sgn = sum(r.sign_mismatch_in_band for r in reports)
    sign_coords = sum(r.sign_coords for r in reports)
    assert idx <= MISMATCH_FRACTION * coords, f"{idx} in-band index mismatches of {coords}"
    assert sgn <= MISMATCH_FRACTION * max(sign_coords, 1), f"{sgn} in-band sign mismatches of {sign_coords}"


def compare_records(qz: tq.Quantizer, gpu_rec: np.ndarray, enc: tq.Encoded, fraction: bool = True) -> RecordReport:
    """Band-rule comparison of one group's records; `fraction=False` leaves the
    mismatch-rate check to check_mismatch_fraction over several groups."""
    gpu_rec = np.ascontiguousarray(gpu_rec).view(np.uint32).reshape(-1, qz.words)
    ok = ~enc.flags
    g = tq.unpack_record(qz, gpu_rec)
    o = tq.unpack_record(qz, enc.records)
    mism = (g.idx != o.idx) & ok[:, None]
    z = enc.z
    dist = np.min(np.abs(z[..., None] - qz.t32[None, None, :]), axis=-1) if qz.k > 0 else np.full(z.shape, np.inf)
    bad = mism & ~(dist < BAND)
    assert not bad.any(), f"{int(bad.sum())} index mismatches outside the 1e-6 band, first at {np.argwhere(bad)[:5]}"
    n_idx = int(mism.sum())
    keep = ok & ~mism.any(axis=1)
    rel_n = np.abs(g.n32 - o.n32)[keep] / np.maximum(np.abs(o.n32[keep]), 1e-30)
    assert np.all(rel_n <= 1e-5), f"norm rel err {rel_n.max()}"
    n_sign = 0
    rel_g = np.zeros(0)
    # raw plane and sign words of kept vectors, bit for bit: this also holds
    # the unused high bits of each plane word (d < 32) and of the last sign
    # word at zero, as the canonical record fixes them
    nraw = qz.k * ((qz.d + 31) // 32)
    allowed = np.zeros((gpu_rec.shape[0], nraw), dtype=np.uint32)
    if qz.role == tq.ROLE_KEY:
        smis = (g.signs != o.signs) & keep[:, None]
        ratio = np.abs(enc.proj) / (math.sqrt(qz.d) * np.maximum(enc.gamma, 1e-300))[:, None]
        bad = smis & ~(ratio < BAND)
        assert not bad.any(), f"{int(bad.sum())} sign mismatches outside the band, first at {np.argwhere(bad)[:5]}"
        n_sign = int(smis.sum())
        nsw = (qz.m + 31) // 32
        allowed = np.concatenate([allowed, tq.pack_bits(smis)], axis=1)   # in-band sign flips only
        nraw += nsw
    diff = (gpu_rec[:, :nraw] ^ np.asarray(enc.records, dtype=np.uint32)[:, :nraw]) & ~allowed
    stray = diff[keep]
    assert not stray.any(), (f"record words differ beyond the band (unused bits included) in "
                             f"{int(np.count_nonzero(stray.any(axis=1)))} vectors, first "
                             f"{np.argwhere(diff & keep[:, None])[:3].tolist()}")
    if qz.role == tq.ROLE_KEY:
        rel_g = np.abs(g.gamma32 - o.gamma32)[keep] / np.maximum(np.abs(o.gamma32[keep]), 1e-30)
        small = o.gamma32[keep] < 1e-30
        assert np.all((rel_g <= 1e-5) | small), f"gamma rel err {rel_g.max()}"
    rep = RecordReport(gpu_rec.shape[0], int(mism.size), n_idx, n_sign, int((~keep).sum()),
                       float(rel_n.max(initial=0.0)), float(rel_g.max(initial=0.0)),
                       int(gpu_rec.shape[0] * qz.m) if qz.role == tq.ROLE_KEY else 0)
    if fraction:
        check_mismatch_fraction([rep])
    return rep


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str, atol=ATOL, rtol=RTOL):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    err = np.abs(gpu - ref)
    lim = atol + rtol * np.abs(ref)
    bad = ~(err <= lim)
    assert not bad.any(), (f"{what}: {int(bad.sum())}/{bad.size} outside tolerance, worst err "
                           f"{err.max():.3e} at {np.unravel_index(np.argmax(err - lim), err.shape)}")


def rec_np(t) -> np.ndarray:
    """int32 torch records -> uint32 numpy."""
    return t.detach().cpu().numpy().view(np.uint32)
