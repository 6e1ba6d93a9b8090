"""Seeded synthetic inputs shaped like the pages' KV workloads.

Holds no codec arithmetic: only random draws, per-group so any group can be
regenerated alone on the CPU.  Every stream is NumPy PCG64 keyed by
SeedSequence([seed, stream, group]).
  * kv_normal:      i.i.d. N(0,1) head vectors [G][N][d] (float32).
  * kv_outliers:    N(0,1) K and V with `n_out` fixed channels per group scaled
                    by `scale`; the channels are drawn first from the group's
                    stream and shared by K and V.
  * kv_channel_std: N(0,1) times a per-(group, channel) std drawn
                    log-uniformly in [lo, hi].
  * queries:        N(0,1) query heads [B][H_q][d].
  * block_codebook: N codewords of dimension k, i.i.d. N(0, 1/d) per
                    coordinate (the scale of a k-block of a unit vector in R^d).
  * sign_bits:      ceil(d/32) uint32 words of fair random bits.
  * block_codes:    uniform indices in [0, N) [M][nb] and norms [M] drawn as
                    |N(0, I_d)| (chi with d degrees of freedom), float32.
  * plane_words:    fair random uint32 words [G][N][n_words] (random bit
                    planes of value codes) and chi(d) norms [G][N], float32.
bf16 inputs are the float32 draws rounded to nearest-even by torch.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

STREAM_K, STREAM_V, STREAM_Q, STREAM_OUTLIER, STREAM_SIGMA = 1, 2, 3, 4, 5
STREAM_CODEBOOK, STREAM_SIGNS, STREAM_CODES = 6, 7, 8


def _rng(seed: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed & ((1 << 63) - 1), *keys])))


def _fill(G: int, fn, threads: int = 8) -> None:
    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(fn, range(G)))


def kv_normal(seed: int, G: int, N: int, d: int, stream: int = STREAM_K, groups=None) -> np.ndarray:
    gl = list(range(G)) if groups is None else list(groups)
    out = np.empty((len(gl), N, d), dtype=np.float32)

    def one(i):
        out[i] = _rng(seed, stream, gl[i]).standard_normal((N, d), dtype=np.float32)
    _fill(len(gl), one)
    return out


def kv_outliers(seed: int, G: int, N: int, d: int, n_out: int = 4, scale: float = 8.0, groups=None):
    gl = list(range(G)) if groups is None else list(groups)
    K = np.empty((len(gl), N, d), dtype=np.float32)
    V = np.empty((len(gl), N, d), dtype=np.float32)
    chans = np.empty((len(gl), n_out), dtype=np.int64)

    def one(i):
        r = _rng(seed, STREAM_OUTLIER, gl[i])
        ch = r.choice(d, n_out, replace=False)
        k = r.standard_normal((N, d), dtype=np.float32)
        v = r.standard_normal((N, d), dtype=np.float32)
        k[:, ch] *= np.float32(scale)
        v[:, ch] *= np.float32(scale)
        K[i], V[i], chans[i] = k, v, ch
    _fill(len(gl), one)
    return K, V, chans


def kv_channel_std(seed: int, G: int, N: int, d: int, lo: float = 0.5, hi: float = 8.0,
                   stream: int = STREAM_K, groups=None):
    gl = list(range(G)) if groups is None else list(groups)
    out = np.empty((len(gl), N, d), dtype=np.float32)
    sig = np.empty((len(gl), d), dtype=np.float32)

    def one(i):
        r = _rng(seed, STREAM_SIGMA, stream, gl[i])
        s = np.exp(r.uniform(math.log(lo), math.log(hi), d)).astype(np.float32)
        out[i] = r.standard_normal((N, d), dtype=np.float32) * s[None, :]
        sig[i] = s
    _fill(len(gl), one)
    return out, sig


def queries(seed: int, B: int, Hq: int, d: int) -> np.ndarray:
    return _rng(seed, STREAM_Q).standard_normal((B, Hq, d), dtype=np.float32)


def block_codebook(seed: int, N: int, k: int, d: int) -> np.ndarray:
    return (_rng(seed, STREAM_CODEBOOK).standard_normal((N, k)) / math.sqrt(d)).astype(np.float32)


def sign_bits(seed: int, d: int) -> np.ndarray:
    return _rng(seed, STREAM_SIGNS).integers(0, 1 << 32, (d + 31) // 32, dtype=np.uint64).astype(np.uint32)


def block_codes(seed: int, M: int, nb: int, N: int, d: int, stream: int = STREAM_CODES, group: int = 0):
    r = _rng(seed, stream, group)
    idx = r.integers(0, N, (M, nb), dtype=np.int64)
    norms = np.sqrt(r.chisquare(d, M)).astype(np.float32)
    return idx, norms


def plane_words(seed: int, G: int, N: int, n_words: int, d: int, stream: int = STREAM_CODES):
    r = _rng(seed, stream)
    words = r.integers(0, 1 << 32, (G, N, n_words), dtype=np.uint64).astype(np.uint32)
    norms = np.sqrt(r.chisquare(d, (G, N))).astype(np.float32)
    return words, norms


def to_torch(a: np.ndarray, dtype: str = "bf16", device=None):
    """float32 draws -> torch tensor of the given dtype (bf16/f16: round to nearest even)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    t = {"bf16": t.to(torch.bfloat16), "f16": t.to(torch.float16), "f32": t}[dtype]
    return t if device is None else t.to(device)


def exact_values(t) -> np.ndarray:
    """The exact values a tensor holds, as float64 (what the oracle consumes)."""
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()
