"""Mixed-precision layers: outlier/normal channel split (test infrastructure only).

Page "turboquant-plus-rs 0.1.0 README":
  * "Modules" ``outlier``: non-integer bit rates by splitting the channels of
    a head vector into outlier and normal channels, each part quantized on its
    own;
  * "Key ideas" item 3: the first and last two layers are kept at higher
    precision;
  * "Architecture" step 1 and "Modules" ``rotation``: the rotation may be
    Haar-distributed (via QR) instead of Walsh-Hadamard.  The normal part has a
    non-power-of-two width (head_dim minus the outliers), so it uses the Haar
    rotation of ``turboquant.haar_rotation``.

Readings (the pages name the split but not its parameters):
  S1  the outliers of a (layer, kv-head) are the ``n_out`` channels with the
      largest population variance over the tokens of that head (keys and
      values chosen separately); ties go to the lower channel index.  Both
      lists are kept in ascending channel order: part j of a sub-vector is the
      j-th listed channel.
  S2  the outlier part (n_out channels, a power of two) uses the Walsh-Hadamard
      rotation at bits + 1; the normal part (d - n_out channels) uses the Haar
      rotation at bits.  Keys: projections = width of the part.
  S3  seeds: the normal part uses the head seed, the outlier part the head
      seed XOR 0x9E3779B97F4A7C15.
  S4  a key score is the sum of the two parts' estimates, times 1/sqrt(d) of
      the full head_dim; decoded values are the two parts scattered back.

Pins: tests/test_oracle_split.py (hand-worked and planted variance orders,
tie rule, QR sign convention and orthogonality, lattice round trip, score
identity against the compressed form of each part).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

from . import turboquant as tq

OUTLIER_SEED_XOR = 0x9E3779B97F4A7C15


def channel_variance(X) -> np.ndarray:
    """Population variance of every channel over the rows of X (float64, two-pass)."""
    X = np.asarray(X, dtype=np.float64)
    mu = X.mean(axis=0)
    return ((X - mu[None, :]) ** 2).mean(axis=0)


def outlier_channels(X, n_out: int) -> np.ndarray:
    """Channel map of one head: [outliers ascending (n_out), normal channels ascending]."""
    X = np.asarray(X, dtype=np.float64)
    d = X.shape[1]
    if not 0 < n_out < d:
        raise tq.OracleError("DIMENSION_MISMATCH", f"n_out {n_out} not in (0, {d})")
    var = channel_variance(X) if X.shape[0] else np.zeros(d)
    order = sorted(range(d), key=lambda c: (-var[c], c))   # larger variance first, then lower index
    out = sorted(order[:n_out])
    normal = sorted(order[n_out:])
    return np.array(out + normal, dtype=np.int64)


@dataclass
class SplitQuantizer:
    d: int
    n_out: int
    bits: int
    role: int
    normal: tq.Quantizer
    outlier: tq.Quantizer


def split_quantizer(d: int, n_out: int, bits: int, seed: int, role: int) -> SplitQuantizer:
    dn = d - n_out
    key = role == tq.ROLE_KEY
    normal = tq.Quantizer(dn, bits, dn if key else 0, seed, role, rotation=tq.ROT_HAAR)
    outlier = tq.Quantizer(n_out, bits + 1, n_out if key else 0, (seed ^ OUTLIER_SEED_XOR) & ((1 << 64) - 1), role)
    return SplitQuantizer(d, n_out, bits, role, normal, outlier)


def split_quantizers(n_cb: int, d: int, n_out: int, bits: int, seed: int, role: int) -> list[SplitQuantizer]:
    return [split_quantizer(d, n_out, bits, (seed + i) & ((1 << 64) - 1), role) for i in range(n_cb)]


def encode_split(sq: SplitQuantizer, X, chan) -> tuple[tq.Encoded, tq.Encoded]:
    """(normal-part encoding, outlier-part encoding) of the rows of X [N][d]."""
    X = np.asarray(X, dtype=np.float64)
    chan = np.asarray(chan, dtype=np.int64)
    return tq.encode(sq.normal, X[:, chan[sq.n_out:]]), tq.encode(sq.outlier, X[:, chan[:sq.n_out]])


def _scatter(sq: SplitQuantizer, chan, normal_part, outlier_part) -> np.ndarray:
    chan = np.asarray(chan, dtype=np.int64)
    out = np.zeros((normal_part.shape[0], sq.d))
    out[:, chan[sq.n_out:]] = normal_part
    out[:, chan[:sq.n_out]] = outlier_part
    return out


def decode_values_split(sq: SplitQuantizer, chan, rec_normal, rec_outlier) -> np.ndarray:
    return _scatter(sq, chan, tq.decode_values(sq.normal, rec_normal), tq.decode_values(sq.outlier, rec_outlier))


def dequantize_keys_split(sq: SplitQuantizer, chan, rec_normal, rec_outlier) -> np.ndarray:
    return _scatter(sq, chan, tq.dequantize_keys(sq.normal, rec_normal),
                    tq.dequantize_keys(sq.outlier, rec_outlier))


def scores_split(sqs: list[SplitQuantizer], chans, krec_normal, krec_outlier, q, scale: float | None = None):
    """Pre-softmax scores [B][H_q][T] = scale * <q, x~_t>, x~ the scattered
    dequantized key.  chans: [B*H_kv][d]; records [B][H_kv][T][words]; group
    (b, h) uses quantizer (b*H_kv + h) mod len(sqs); scale defaults to 1/sqrt(d)."""
    krec_normal = np.asarray(krec_normal, dtype=np.uint32)
    krec_outlier = np.asarray(krec_outlier, dtype=np.uint32)
    q = np.asarray(q, dtype=np.float64)
    B, Hkv, T, _ = krec_normal.shape
    Hq = q.shape[1]
    d = sqs[0].d
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hkv):
            g = b * Hkv + h
            sq = sqs[g % len(sqs)]
            xt = dequantize_keys_split(sq, chans[g], krec_normal[b, h], krec_outlier[b, h])
            for hq in range(Hq):
                if (hq * Hkv) // Hq == h:
                    out[b, hq] = scale * (xt @ q[b, hq])
    return out


def split_bits_per_value(d: int, n_out: int, bits: int, role: int) -> float:
    """Stored bits per channel of a split record pair (planes, signs and side scalars)."""
    dn = d - n_out
    key = role == tq.ROLE_KEY
    wn = tq.record_words(dn, bits, dn if key else 0, role, tq.ROT_HAAR)
    wo = tq.record_words(n_out, bits + 1, n_out if key else 0, role)
    return 32.0 * (wn + wo) / d
