"""TurboQuant KV-cache codec, written out plainly in float64.

Test infrastructure only (see ``oracle/__init__.py``).  Dense matrices
throughout: an explicit Sylvester-Hadamard matrix instead of a fast
transform, an explicit Gaussian QJL matrix, and scores computed by fully
dequantizing each key and taking a dot product.

What it follows (page: "turboquant-plus-rs 0.1.0 README"):
  * "Architecture" step 1 (PolarQuant, b-1 bits for keys): random rotation
    (sign diagonal then Walsh-Hadamard), then the Lloyd-Max scalar quantizer
    of the post-rotation Gaussian on every coordinate; "Modules"
    ``polar_quant``: the vector norm is extracted and stored.
  * "Architecture" step 2 (QJL, 1 bit): sign of a Gaussian projection of the
    residual left by step 1, with the residual norm, used to remove the
    inner-product bias.
  * "Architecture", last paragraph: values take step 1 only, at b bits.
  * "Modules" ``utils``: bit packing and the memory-footprint calculation.
Page "bitpolar 0.3.3 src/kv_cache.rs": ``KvCacheConfig`` (head_dim, bits,
projections, seed); ``attention_scores`` returns, per stored key, the inner
product estimate times 1/sqrt(head_dim), before softmax; ``decode_values``;
``MultiHeadKvCache::new`` gives head h the seed ``seed + h`` (wrapping).

Readings where the pages are silent:
  R1  rotation Pi = H D / sqrt(d), D applied first, Sylvester order; z =
      H(D x)/|x| so that z ~ N(0, 1) per coordinate.
  R2  quantizer index idx_j = #{i : t_i < z_j} (ties go to the lower cell),
      the plain definition: the exact (float64) z against the stored float32
      thresholds.  The pages fix no working precision; a kernel that decides
      on a rounded z may differ only where z lies within its rounding of a
      threshold, which the parity band absorbs.
  R3  the stored norm is n32 = float32(|x|); reconstruction and the
      residual both use n32 (the residual is exactly what a decoder holding
      the record cannot rebuild).
  R4  the QJL stage acts on the residual of step 1 in the rotated
      coordinates, rho = Pi x - (n32/sqrt d) c[idx], with S (m x d) i.i.d.
      N(0,1) stored at binary16 precision; signs s_i = [(S rho)_i >= 0];
      gamma = |rho| stored as float32.  (S Pi is again i.i.d. Gaussian, so
      this is the same estimator as projecting the unrotated residual with a
      fresh Gaussian matrix.)
  R5  dequantized key  x~ = Pi^T [ (n32/sqrt d) c[idx]
                                   + sqrt(pi/2)/m * gamma32 * S^T (2s - 1) ];
      sqrt(pi/2)/m is the constant that makes E_S[<q, x~>] = <q, x>.
  R6  zero vector: z := 0; hence x^ = 0, rho = 0, gamma = 0, all s = 1.
  R7  a vector with a non-finite element, or whose squared norm exceeds the
      binary32 range, is flagged; its record is unspecified.
  R8  Haar alternative ("Architecture" step 1, "Modules" rotation): Pi = Q,
      the orthogonal QR factor of a seeded d x d Gaussian matrix with the
      columns signed so that the triangular factor has a positive diagonal.
      The stored matrix R = float32(sqrt(d) Q) takes the place of H D in
      every formula (u = R x, x^ = (n32/d) R^T c[idx], qt = R q), so head_dim
      need not be a power of two.

Pins: tests/test_oracle_codec.py (lattice round trip, nearest-centroid brute
force, distortion law, QJL unbiasedness over seeds, compressed-score
identity, norm preservation, bit order, footprint table of the README).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .lloyd import stored_codebook
from .prng import haar_gaussian, qjl_matrix, qjl_matrix_fast, sign_diagonal, sign_diagonal_fast

ROLE_KEY = 0
ROLE_VALUE = 1
ROT_HADAMARD = 0     # Pi = H D / sqrt(d)
ROT_HAAR = 1         # Pi = Q, Q Haar-distributed (QR of a Gaussian matrix)
FLT_MAX = float(np.finfo(np.float32).max)
QJL_CONST = math.sqrt(math.pi / 2.0)


class OracleError(ValueError):
    """Argument error, mirroring the library's status codes by name."""

    def __init__(self, code: str, msg: str = ""):
        super().__init__(f"{code}: {msg}")
        self.code = code


def hadamard(d: int) -> np.ndarray:
    """Unnormalised Sylvester-Hadamard matrix, H[i, j] = (-1)**popcount(i & j)."""
    i = np.arange(d, dtype=np.int64)
    a = i[:, None] & i[None, :]
    pc = np.zeros_like(a)
    while np.any(a):
        pc += a & 1
        a >>= 1
    return np.where(pc % 2 == 0, 1.0, -1.0)


def haar_rotation(seed: int, d: int) -> np.ndarray:
    """R = float32(sqrt(d) Q) as float64, with Q the orthogonal factor of the QR
    decomposition of the seeded Gaussian matrix, columns signed so that the
    triangular factor has a positive diagonal (this makes Q Haar-distributed).

    Page "turboquant-plus-rs 0.1.0 README", "Architecture" step 1 and "Modules"
    ``rotation`` (Haar-distributed rotation via QR, the alternative to the
    Walsh-Hadamard transform).  sqrt(d) Q plays the part of H D: u = R x has
    |u| = sqrt(d) |x| (up to the float32 rounding of R), so z = u/|x| ~ N(0,1)."""
    G = haar_gaussian(seed, d)
    Q, Rt = np.linalg.qr(G)
    Q = Q * np.sign(np.diag(Rt))[None, :]
    return (math.sqrt(d) * Q).astype(np.float32).astype(np.float64)


def check_args(d: int, bits: int, m: int, role: int, rotation: int = ROT_HADAMARD) -> int:
    """Validate (head_dim, bits, projections, role) and return k = Lloyd bits."""
    if role not in (ROLE_KEY, ROLE_VALUE):
        raise OracleError("INVALID_ROLE", str(role))
    if rotation not in (ROT_HADAMARD, ROT_HAAR):
        raise OracleError("INVALID_ROTATION", str(rotation))
    if d == 0:
        raise OracleError("ZERO_DIMENSION")
    if rotation == ROT_HAAR:
        if d < 2 or d > 512:
            raise OracleError("BAD_DIMENSION", f"head_dim {d} not in [2, 512]")
    elif d < 2 or d > 512 or (d & (d - 1)) != 0:
        raise OracleError("BAD_DIMENSION", f"head_dim {d} must be a power of two in [2, 512]")
    if role == ROLE_KEY:
        if not 2 <= bits <= 9:
            raise OracleError("INVALID_BIT_WIDTH", f"key bits {bits} not in [2, 9]")
        if m <= 0:
            raise OracleError("ZERO_PROJECTIONS")
        if m > 1024:
            raise OracleError("INVALID_PROJECTIONS", f"{m} > 1024")
        return bits - 1
    if not 1 <= bits <= 8:
        raise OracleError("INVALID_BIT_WIDTH", f"value bits {bits} not in [1, 8]")
    return bits


def record_words(d: int, bits: int, m: int, role: int, rotation: int = ROT_HADAMARD) -> int:
    k = check_args(d, bits, m, role, rotation)
    w = (d + 31) // 32
    if role == ROLE_KEY:
        return k * w + (m + 31) // 32 + 2
    return k * w + 1


@dataclass
class Quantizer:
    """State of one (layer, kv-head) quantizer, built from (d, bits, m, seed, role)."""
    d: int
    bits: int
    m: int
    seed: int
    role: int
    fast_prng: bool = False      # vectorised generator: only for many-seed statistics
    rotation: int = ROT_HADAMARD
    k: int = field(init=False)
    c32: np.ndarray = field(init=False, repr=False)
    t32: np.ndarray = field(init=False, repr=False)
    D: np.ndarray | None = field(init=False, repr=False)
    R: np.ndarray | None = field(init=False, repr=False)   # Haar: float32(sqrt(d) Q)
    S: np.ndarray | None = field(init=False, repr=False)

    def __post_init__(self):
        self.k = check_args(self.d, self.bits, self.m, self.role, self.rotation)
        self.seed &= (1 << 64) - 1
        self.c32, self.t32 = stored_codebook(self.k)
        self.R = None
        if self.rotation == ROT_HAAR:
            self.D = None
            self.R = haar_rotation(self.seed, self.d)
            self.S = qjl_matrix(self.seed, self.m, self.d) if self.role == ROLE_KEY else None
        elif self.fast_prng:
            self.D = sign_diagonal_fast(self.seed, self.d)
            self.S = qjl_matrix_fast(self.seed, self.m, self.d) if self.role == ROLE_KEY else None
        else:
            self.D = sign_diagonal(self.seed, self.d)
            self.S = qjl_matrix(self.seed, self.m, self.d) if self.role == ROLE_KEY else None

    @property
    def words(self) -> int:
        return record_words(self.d, self.bits, self.m, self.role, self.rotation)


def quantizers(n_cb: int, d: int, bits: int, m: int, seed: int, role: int) -> list[Quantizer]:
    """Quantizer i uses seed + i (wrapping), as MultiHeadKvCache does per head."""
    return [Quantizer(d, bits, m, (seed + i) & ((1 << 64) - 1), role) for i in range(n_cb)]


# ---------------------------------------------------------------------------
# Bit packing ("Modules" utils).  Plane p of idx occupies words
# [p*W, (p+1)*W); bit (j mod 32) of word p*W + j//32 is bit p of idx_j.
# Then ceil(m/32) sign words (bit i = s_i, unused high bits 0), then float32 n,
# then (keys) float32 gamma.  Little-endian 32-bit words.
# ---------------------------------------------------------------------------
def pack_bits(bits: np.ndarray) -> np.ndarray:
    """(N, L) array of 0/1 -> (N, ceil(L/32)) uint32, bit j of the row in word j//32, position j%32."""
    bits = np.asarray(bits, dtype=np.uint8)
    n, length = bits.shape
    nw = (length + 31) // 32
    padded = np.zeros((n, nw * 32), dtype=np.uint8)
    padded[:, :length] = bits
    by = np.packbits(padded, axis=1, bitorder="little")
    return by.reshape(n, nw, 4).view("<u4").reshape(n, nw).astype(np.uint32)


def unpack_bits(words: np.ndarray, length: int) -> np.ndarray:
    words = np.ascontiguousarray(np.asarray(words, dtype="<u4"))
    n, nw = words.shape
    by = words.view(np.uint8).reshape(n, nw * 4)
    return np.unpackbits(by, axis=1, bitorder="little")[:, :length]


def _f32_words(v: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(v, dtype=np.float32)).view(np.uint32)


def _words_f32(w: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(w, dtype=np.uint32)).view(np.float32).astype(np.float64)


@dataclass
class Encoded:
    records: np.ndarray        # (N, words) uint32
    idx: np.ndarray            # (N, d) int
    z: np.ndarray              # (N, d) float64: the exact z the decision is taken on
    n: np.ndarray              # (N,) float64
    flags: np.ndarray          # (N,) bool: rejected input
    gamma: np.ndarray | None = None   # (N,) float64
    proj: np.ndarray | None = None    # (N, m) float64, S rho * sqrt(d) (sign decides s)


def _rotate(qz: Quantizer, X: np.ndarray) -> np.ndarray:
    """u = H (D x) for each row (dense matrix product); Haar: u = R x."""
    if qz.rotation == ROT_HAAR:
        return X @ qz.R.T
    H = hadamard(qz.d)
    return (X * qz.D[None, :]) @ H.T


def rotate(qz: Quantizer, X) -> tuple[np.ndarray, np.ndarray]:
    """(u, n): u = H(D x) per row and n = |x| (float64)."""
    X = np.asarray(X, dtype=np.float64)
    return _rotate(qz, X), np.sqrt(np.sum(X * X, axis=1))


def encode(qz: Quantizer, X) -> Encoded:
    """Encode the rows of X (N x d, the exact input values) with quantizer qz."""
    X = np.asarray(X, dtype=np.float64)
    if X.ndim != 2 or X.shape[1] != qz.d:
        raise OracleError("DIMENSION_MISMATCH", f"expected (N, {qz.d}), got {X.shape}")
    N = X.shape[0]
    finite = np.isfinite(X).all(axis=1)
    Xs = np.where(finite[:, None], X, 0.0)
    sq = np.sum(Xs * Xs, axis=1)
    flags = ~finite | (sq > FLT_MAX)
    n = np.sqrt(sq)
    n32 = n.astype(np.float32).astype(np.float64)
    U = _rotate(qz, Xs)
    safe_n = np.where(n > 0, n, 1.0)
    z = np.where(n[:, None] > 0, U / safe_n[:, None], 0.0)
    idx = np.searchsorted(qz.t32, z.ravel(), side="left").reshape(N, qz.d)

    parts = [pack_bits((idx >> p) & 1) for p in range(qz.k)]
    gamma = proj = None
    if qz.role == ROLE_KEY:
        W = U - n32[:, None] * qz.c32[idx]          # sqrt(d) * rho
        gamma = np.sqrt(np.sum(W * W, axis=1)) / math.sqrt(qz.d)
        proj = W @ qz.S.T
        parts.append(pack_bits(proj >= 0.0))
        parts.append(_f32_words(n32)[:, None])
        parts.append(_f32_words(gamma)[:, None])
    else:
        parts.append(_f32_words(n32)[:, None])
    rec = np.concatenate(parts, axis=1).astype(np.uint32)
    assert rec.shape[1] == qz.words
    return Encoded(rec, idx, z, n, flags, gamma, proj)


@dataclass
class Fields:
    idx: np.ndarray
    signs: np.ndarray | None
    n32: np.ndarray
    gamma32: np.ndarray | None


def unpack_record(qz: Quantizer, records) -> Fields:
    rec = np.asarray(records, dtype=np.uint32).reshape(-1, qz.words)
    W = (qz.d + 31) // 32
    idx = np.zeros((rec.shape[0], qz.d), dtype=np.int64)
    for p in range(qz.k):
        idx |= unpack_bits(rec[:, p * W:(p + 1) * W], qz.d).astype(np.int64) << p
    off = qz.k * W
    if qz.role == ROLE_KEY:
        nsw = (qz.m + 31) // 32
        signs = unpack_bits(rec[:, off:off + nsw], qz.m).astype(np.float64)
        return Fields(idx, signs, _words_f32(rec[:, off + nsw]), _words_f32(rec[:, off + nsw + 1]))
    return Fields(idx, None, _words_f32(rec[:, off]), None)


def decode_values(qz: Quantizer, records) -> np.ndarray:
    """x^ = Pi^T (n32/sqrt d) c[idx] = (n32/d) D (H c[idx])  (MSE reconstruction)."""
    f = unpack_record(qz, records)
    if qz.rotation == ROT_HAAR:                       # x^ = (n32/d) R^T c[idx]
        return (f.n32[:, None] / qz.d) * (qz.c32[f.idx] @ qz.R)
    H = hadamard(qz.d)
    return (f.n32[:, None] / qz.d) * ((qz.c32[f.idx] @ H.T) * qz.D[None, :])


def dequantize_keys(qz: Quantizer, records) -> np.ndarray:
    """x~ = Pi^T y~, y~ = (n32/sqrt d) c[idx] + sqrt(pi/2)/m * gamma32 * S^T (2s - 1)."""
    f = unpack_record(qz, records)
    y = (f.n32[:, None] / math.sqrt(qz.d)) * qz.c32[f.idx]
    y = y + (QJL_CONST / qz.m) * f.gamma32[:, None] * ((2.0 * f.signs - 1.0) @ qz.S)
    if qz.rotation == ROT_HAAR:                       # Pi^T y = R^T y / sqrt(d)
        return (y @ qz.R) / math.sqrt(qz.d)
    H = hadamard(qz.d)
    return ((y @ H.T) * qz.D[None, :]) / math.sqrt(qz.d)


def scores(qzs: list[Quantizer], krec, q, scale: float | None = None) -> np.ndarray:
    """Pre-softmax scores [B][H_q][T] = scale * <q, x~_t> by dequantize-then-dot.

    krec: [B][H_kv][T][words] records; q: [B][H_q][d].  Group (b, h) uses
    quantizer (b*H_kv + h) mod len(qzs).  Query head hq reads kv head
    floor(hq * H_kv / H_q).
    """
    krec = np.asarray(krec, dtype=np.uint32)
    q = np.asarray(q, dtype=np.float64)
    B, Hkv, T, _ = krec.shape
    Hq = q.shape[1]
    d = qzs[0].d
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((B, Hq, T))
    for b in range(B):
        for h in range(Hkv):
            qz = qzs[(b * Hkv + h) % len(qzs)]
            xt = dequantize_keys(qz, krec[b, h]) if T else np.zeros((0, d))
            for hq in range(Hq):
                if (hq * Hkv) // Hq == h:
                    out[b, hq] = scale * (xt @ q[b, hq])
    return out


def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def attend(qzs_k: list[Quantizer], krec, qzs_v: list[Quantizer], vrec, q, scale=None) -> np.ndarray:
    """o[b, hq] = sum_t softmax_t(scores[b, hq]) * x^_t (decoded values of kv head of hq)."""
    s = scores(qzs_k, krec, q, scale)
    w = softmax(s, axis=-1)
    vrec = np.asarray(vrec, dtype=np.uint32)
    B, Hkv, T, _ = vrec.shape
    Hq = s.shape[1]
    d = qzs_v[0].d
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for h in range(Hkv):
            xv = decode_values(qzs_v[(b * Hkv + h) % len(qzs_v)], vrec[b, h])
            for hq in range(Hq):
                if (hq * Hkv) // Hq == h:
                    out[b, hq] = w[b, hq] @ xv
    return out


def compressed_score_terms(qz: Quantizer, records, q) -> np.ndarray:
    """The same score written the way a no-decode kernel evaluates it:
    (n32/d) sum_j qt_j c[idx_j] + sqrt(pi/2)/m gamma32 sum_i p_i (2 s_i - 1),
    with qt = H(D q) and p = S qt / sqrt(d).  Unscaled (no 1/sqrt d)."""
    f = unpack_record(qz, records)
    if qz.rotation == ROT_HAAR:
        qt = qz.R @ np.asarray(q, dtype=np.float64)
    else:
        qt = hadamard(qz.d) @ (qz.D * np.asarray(q, dtype=np.float64))
    mse = (f.n32 / qz.d) * (qz.c32[f.idx] @ qt)
    if qz.role != ROLE_KEY:
        return mse
    p = qz.S @ qt / math.sqrt(qz.d)
    return mse + (QJL_CONST / qz.m) * f.gamma32 * ((2.0 * f.signs - 1.0) @ p)


# ---------------------------------------------------------------------------
# Memory footprint ("Modules" utils; "Compression formats" table).
# ---------------------------------------------------------------------------
def bits_per_value(d: int, bits: int, m: int, role: int) -> float:
    return record_words(d, bits, m, role) * 32.0 / d


def memory_stats(d: int, k_bits: int, v_bits: int, m: int, seq_len: int, layers: int, kv_heads: int) -> dict:
    """Footprint of a K+V cache of seq_len tokens x layers x kv_heads head vectors."""
    vecs = seq_len * layers * kv_heads
    rec = 4 * (record_words(d, k_bits, m, ROLE_KEY) + record_words(d, v_bits, m, ROLE_VALUE))
    orig16 = 2 * vecs * d * 2
    orig32 = 2 * vecs * d * 4
    comp = vecs * rec
    return {"orig_fp16_bytes": float(orig16), "orig_f32_bytes": float(orig32),
            "compressed_bytes": float(comp),
            "ratio_vs_fp16": orig16 / comp if comp else 1.0}
