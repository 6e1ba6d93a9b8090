"""Seeded randomness of the codec: the sign diagonal D and the QJL matrix S.

Test infrastructure only (see ``oracle/__init__.py``).

The pages fix only that the quantizer is "fully determined" by
``(head_dim, bits, projections, seed)`` (bitpolar ``KvCacheConfig``) and that
the rotation is random (turboquant-plus-rs README, "Architecture" step 1) and
the QJL stage a random Gaussian sign projection ("Architecture" step 2,
"Modules" ``qjl``).  They do not name a generator, so this codec defines one:

* SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
  generators", OOPSLA 2014; finaliser constants as in Vigna's public
  ``splitmix64.c``).  It is counter based: output ``i`` of the stream started
  at state ``seed`` is ``mix(seed + (i + 1) * GAMMA)``, so every entry can be
  produced independently.
* Counter ranges: D uses outputs ``[0, ceil(d/64))``; S uses outputs from
  ``1 << 32``; the dense Haar rotation (mixed-precision layers) uses outputs
  from ``2 << 32``.
* D_j = -1 when bit ``j mod 64`` of output ``j // 64`` is set, else +1.
* Gaussians by Box-Muller on consecutive output pairs (x1, x2):
  ``u1 = ((x1 >> 11) + 1) * 2**-53`` in (0, 1], ``u2 = (x2 >> 11) * 2**-53``,
  ``g_even = sqrt(-2 ln u1) cos(2 pi u2)``, ``g_odd = sqrt(-2 ln u1) sin(2 pi u2)``
  in float64 with the host libm.
* S entries are those Gaussians rounded to IEEE binary16 (round to nearest,
  ties to even): the matrix is stored at 16-bit precision.  Reading: the pages
  leave the storage precision of S open; 11 significant bits keep the entries
  standard normal to within 2**-12 relative.

Pins (tests/test_oracle_prng.py): published SplitMix64 outputs for seed 0;
binary16 rounding against hand-worked ties and NumPy's converter;
Box-Muller invariant g0**2 + g1**2 = -2 ln u1; moments / KS of the Gaussians;
balance of D.
"""
from __future__ import annotations

import math

import numpy as np

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15
MIX1 = 0xBF58476D1CE4E5B9
MIX2 = 0x94D049BB133111EB

STREAM_D = 0
STREAM_S = 1 << 32
STREAM_HAAR = 2 << 32

TWO_PI = 2.0 * math.pi
TWO_M53 = 2.0 ** -53


def splitmix64(seed: int, i: int) -> int:
    """Output ``i`` (0-based) of the SplitMix64 stream whose state starts at ``seed``."""
    z = (seed + (i + 1) * GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * MIX1) & MASK64
    z = ((z ^ (z >> 27)) * MIX2) & MASK64
    return z ^ (z >> 31)


def round_to_half(x: float) -> float:
    """Nearest IEEE binary16 value to ``x`` (ties to even), returned as a float.

    Written from the binary16 format definition (IEEE 754-2008: 11 significant
    bits, exponent range [-14, 15], subnormal quantum 2**-24, max 65504).
    """
    if x != x or math.isinf(x):
        return x
    if x == 0.0:
        return x
    a = abs(x)
    _, e = math.frexp(a)          # a = f * 2**e, f in [0.5, 1)
    lead = e - 1                  # exponent of the leading bit
    quantum = 2.0 ** (max(lead, -14) - 10)
    q = round(a / quantum)        # exact division (power of two); round() ties to even
    r = q * quantum
    if r > 65504.0:
        r = math.inf
    return math.copysign(r, x)


def sign_diagonal(seed: int, d: int) -> np.ndarray:
    """D as a float64 vector of +-1 (length d)."""
    out = np.empty(d, dtype=np.float64)
    for j in range(d):
        word = splitmix64(seed, STREAM_D + j // 64)
        out[j] = -1.0 if (word >> (j % 64)) & 1 else 1.0
    return out


def gaussian_pair(seed: int, counter: int) -> tuple[float, float]:
    """Box-Muller pair from outputs ``counter`` and ``counter + 1`` (float64)."""
    x1 = splitmix64(seed, counter)
    x2 = splitmix64(seed, counter + 1)
    u1 = ((x1 >> 11) + 1) * TWO_M53
    u2 = (x2 >> 11) * TWO_M53
    r = math.sqrt(-2.0 * math.log(u1))
    ang = TWO_PI * u2
    return r * math.cos(ang), r * math.sin(ang)


def gaussians(seed: int, count: int, base: int) -> np.ndarray:
    """``count`` standard normals (float64, not rounded) from stream ``base``.

    Entry ``e`` is the even (cos) or odd (sin) member of pair ``e // 2``, whose
    outputs are ``base + 2 * (e // 2)`` and ``base + 2 * (e // 2) + 1``.
    """
    out = np.empty(count, dtype=np.float64)
    for p in range((count + 1) // 2):
        g0, g1 = gaussian_pair(seed, base + 2 * p)
        out[2 * p] = g0
        if 2 * p + 1 < count:
            out[2 * p + 1] = g1
    return out


def haar_gaussian(seed: int, d: int) -> np.ndarray:
    """d x d standard normals (float64, row-major entry e = i*d + j) from the
    Haar stream: the matrix whose orthogonal QR factor is the dense rotation."""
    return gaussians(seed, d * d, STREAM_HAAR).reshape(d, d)


def qjl_matrix(seed: int, m: int, d: int) -> np.ndarray:
    """S (m x d, row-major entry e = i*d + j) as float64 values of binary16 numbers."""
    g = gaussians(seed, m * d, STREAM_S)
    return np.array([round_to_half(v) for v in g], dtype=np.float64).reshape(m, d)


# ---------------------------------------------------------------------------
# Vectorised variant, used only where many seeds are needed (the statistical
# unbiasedness check).  It follows the same definition with NumPy ufuncs,
# whose log/cos/sin may differ from the host libm in the last bit; the tests
# check that the binary16-rounded S agrees with ``qjl_matrix``.
# ---------------------------------------------------------------------------
def _splitmix64_vec(seed: int, idx: np.ndarray) -> np.ndarray:
    z = (np.uint64(seed) + (idx.astype(np.uint64) + np.uint64(1)) * np.uint64(GAMMA))
    z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX2)
    return z ^ (z >> np.uint64(31))


def qjl_matrix_fast(seed: int, m: int, d: int) -> np.ndarray:
    count = m * d
    npairs = (count + 1) // 2
    with np.errstate(over="ignore"):
        base = np.uint64(STREAM_S) + 2 * np.arange(npairs, dtype=np.uint64)
        x1 = _splitmix64_vec(seed, base)
        x2 = _splitmix64_vec(seed, base + np.uint64(1))
    u1 = ((x1 >> np.uint64(11)) + np.uint64(1)).astype(np.float64) * TWO_M53
    u2 = (x2 >> np.uint64(11)).astype(np.float64) * TWO_M53
    r = np.sqrt(-2.0 * np.log(u1))
    ang = TWO_PI * u2
    g = np.empty(2 * npairs, dtype=np.float64)
    g[0::2] = r * np.cos(ang)
    g[1::2] = r * np.sin(ang)
    return g[:count].astype(np.float16).astype(np.float64).reshape(m, d)


def sign_diagonal_fast(seed: int, d: int) -> np.ndarray:
    nw = (d + 63) // 64
    with np.errstate(over="ignore"):
        words = _splitmix64_vec(seed, np.arange(nw, dtype=np.uint64) + np.uint64(STREAM_D))
    j = np.arange(d)
    bits = (words[j // 64] >> (j % 64).astype(np.uint64)) & np.uint64(1)
    return np.where(bits == 1, -1.0, 1.0)
