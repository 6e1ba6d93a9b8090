"""Gram-table scoring of block-codebook codes (FibQuant style), written out
plainly in float64.

Test infrastructure only (see ``oracle/__init__.py``).  Dense matrices: the
rotation is an explicit Sylvester-Hadamard matrix, encoding compares every
block against every codeword, and the Gram table is the product of the
codebook with its transpose.

What it follows (page: "fib-quant 0.1.0-beta.4 README"):
  * opening section: a vector is split into blocks, each block is replaced by
    the index of a codeword of a small codebook, and only the indices are
    kept;
  * "What's in the box", Codec (encode/decode), Rotation (fast Walsh-Hadamard
    rotation), Profiles (ambient dim, block dim, codebook size; k = 4, N = 32
    in the examples);
  * "New modules", Scoring: the Gram table G[i, j] = <codeword_i, codeword_j>
    (4 KB at N = 32) estimates the inner product of a query with a stored
    code without decoding it (no inverse rotation, no norm scaling).

Readings where the pages are silent:
  G1  the codebook (N codewords of dimension k) is an input.  The pages build
      it by spherical-Beta seeding and Lloyd refinement, which they leave
      underspecified; the scorer works for any codebook.
  G2  encode: n = |x| (float64, stored as float32 n32); u = H(D x) / (sqrt(d)
      n32) with the sign diagonal D given as bits (bit j set: coordinate j
      negated) and H the Sylvester-Hadamard matrix; block b = u[b k : (b+1) k]
      takes the index of the nearest codeword in Euclidean distance, the
      lowest index on ties.  A zero vector has u = 0.  The decision is the
      plain definition, the nearest codeword of the exact (float64) u, with
      float64 distances to the float32 codewords.  The pages fix no working
      precision; a kernel that rounds u may differ only for blocks whose u
      lies within that rounding of the boundary between two codewords, which
      the parity band absorbs.
  G3  record: the d/k indices of w = log2(N) bits each, LSB first, index b at
      bit offset b w of the little-endian 32-bit words (an index may straddle
      two words), ceil(d w / (k 32)) words, then float32 n32.
  G4  decode: x^ = n32 D H c / sqrt(d), c the concatenated codewords.
  G5  the query is encoded with the same quantizer (the Gram table holds
      codeword-codeword products, so both sides are codes):
        s(q, t) = scale * n_q * n_t * sum_b G[cq_b, ct_b]
      which equals scale * <q^, x^_t> for the decoded vectors (the rotation is
      orthogonal).  scale <= 0 means 1/sqrt(d), the attention-logit scale.
  G6  a vector with a non-finite element, or whose squared norm exceeds the
      binary32 range, is flagged; its record is unspecified.

Pins: tests/test_oracle_gram.py (polarization identity for the table,
score = inner product of decoded vectors, exact codeword round trip,
nearest-codeword brute force, a hand-packed record, zero vector).
"""
from __future__ import annotations

import math

import numpy as np

from .turboquant import FLT_MAX, OracleError, hadamard


def check_args(d: int, k: int, N: int) -> int:
    """Validate (head_dim, block_dim, codebook_size); return w = log2(N)."""
    if d == 0:
        raise OracleError("ZERO_DIMENSION")
    if d < 2 or d > 512 or (d & (d - 1)) != 0:
        raise OracleError("BAD_DIMENSION", f"head_dim {d} must be a power of two in [2, 512]")
    if k not in (1, 2, 4, 8) or k > d:
        raise OracleError("BAD_DIMENSION", f"block_dim {k} not in {{1, 2, 4, 8}} or above head_dim")
    if N < 2 or N > 256 or (N & (N - 1)) != 0:
        raise OracleError("INVALID_CODEBOOK", f"codebook size {N} must be a power of two in [2, 256]")
    return N.bit_length() - 1


def record_words(d: int, k: int, N: int) -> int:
    w = check_args(d, k, N)
    return ((d // k) * w + 31) // 32 + 1


def pack_record(idx: np.ndarray, n32: np.ndarray, d: int, k: int, N: int) -> np.ndarray:
    """(M, d/k) indices and (M,) float32 norms -> (M, words) uint32 (reading G3).
    Bit j of index b goes to bit (b w + j) of the record, bit i of the record
    being bit i mod 32 of word i // 32."""
    w = check_args(d, k, N)
    idx = np.asarray(idx, dtype=np.int64)
    M, nb = idx.shape
    nw = record_words(d, k, N)
    out = np.zeros((M, nw), dtype=np.uint64)
    for b in range(nb):
        for j in range(w):
            pos = b * w + j
            out[:, pos // 32] |= ((idx[:, b] >> j) & 1).astype(np.uint64) << np.uint64(pos % 32)
    out[:, nw - 1] = np.asarray(n32, dtype=np.float32).view(np.uint32)
    return out.astype(np.uint32)


def unpack_record(rec: np.ndarray, d: int, k: int, N: int) -> tuple[np.ndarray, np.ndarray]:
    """(M, words) uint32 -> ((M, d/k) indices, (M,) norms as float64)."""
    w = check_args(d, k, N)
    rec = np.asarray(rec, dtype=np.uint32)
    nb = d // k
    idx = np.zeros((rec.shape[0], nb), dtype=np.int64)
    for b in range(nb):
        for j in range(w):
            pos = b * w + j
            idx[:, b] |= ((rec[:, pos // 32].astype(np.int64) >> (pos % 32)) & 1) << j
    n = np.ascontiguousarray(rec[:, -1]).view(np.float32).astype(np.float64)
    return idx, n


def sign_vector(signs: np.ndarray, d: int) -> np.ndarray:
    """Sign-bit words -> the diagonal of D as +-1.0 (bit set: -1)."""
    signs = np.asarray(signs, dtype=np.uint32)
    bits = np.array([(int(signs[j // 32]) >> (j % 32)) & 1 for j in range(d)])
    return np.where(bits == 1, -1.0, 1.0)


def rotation_matrix(signs: np.ndarray, d: int) -> np.ndarray:
    """Pi = H D / sqrt(d) (orthogonal), so u = Pi x / n32."""
    return hadamard(d) * sign_vector(signs, d)[None, :] / math.sqrt(d)


def encode(codebook: np.ndarray, signs: np.ndarray, X, d: int, k: int):
    """Records of the rows of X (reading G2, G3), and the per-row flag of G6.
    Every block is compared with every codeword by its squared distance."""
    C = np.asarray(codebook, dtype=np.float64)
    N = C.shape[0]
    check_args(d, k, N)
    X = np.asarray(X, dtype=np.float64).reshape(-1, d)
    finite = np.all(np.isfinite(X), axis=1)
    Xs = np.where(finite[:, None], X, 0.0)
    ss = np.sum(Xs * Xs, axis=1)
    flags = ~finite | (ss > FLT_MAX)
    n32 = np.sqrt(ss).astype(np.float32)
    n = n32.astype(np.float64)
    U = Xs @ rotation_matrix(signs, d).T
    U = np.where(n[:, None] > 0, U / np.where(n > 0, n, 1.0)[:, None], 0.0)
    nb = d // k
    blocks = U.reshape(-1, nb, k)
    dist = np.sum((blocks[:, :, None, :] - C[None, None, :, :]) ** 2, axis=3)   # (M, nb, N)
    idx = np.argmin(dist, axis=2)        # first minimum: the lowest index on ties
    return pack_record(idx, n32, d, k, N), flags, dist


def decode(codebook: np.ndarray, signs: np.ndarray, rec, d: int, k: int) -> np.ndarray:
    """x^ = n32 Pi^T c (reading G4)."""
    C = np.asarray(codebook, dtype=np.float64)
    idx, n = unpack_record(rec, d, k, C.shape[0])
    c = C[idx].reshape(idx.shape[0], d)
    return n[:, None] * (c @ rotation_matrix(signs, d))


def gram_table(codebook: np.ndarray) -> np.ndarray:
    """G[i, j] = <codeword_i, codeword_j> ("New modules", Scoring)."""
    C = np.asarray(codebook, dtype=np.float64)
    return C @ C.T


def scores(codebook: np.ndarray, qrec, krec, d: int, k: int, scale: float | None = None) -> np.ndarray:
    """s[b, hq, t] = scale n_q n_t sum_b G[cq_b, ct_b] (reading G5).
    qrec (B, H_q, words), krec (B, H_kv, T, words); query head hq reads kv head
    hq * H_kv // H_q."""
    C = np.asarray(codebook, dtype=np.float64)
    N = C.shape[0]
    G = gram_table(C)
    qrec = np.asarray(qrec, dtype=np.uint32)
    krec = np.asarray(krec, dtype=np.uint32)
    B, Hq, nw = qrec.shape
    _, Hkv, T, _ = krec.shape
    sc = 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)
    out = np.zeros((B, Hq, T))
    for b in range(B):
        for hq in range(Hq):
            h = hq * Hkv // Hq
            cq, nq = unpack_record(qrec[b, hq][None, :], d, k, N)
            ct, nt = unpack_record(krec[b, h], d, k, N)
            acc = np.sum(G[cq[0][None, :], ct], axis=1)        # (T,)
            out[b, hq] = sc * nq[0] * nt * acc
    return out
