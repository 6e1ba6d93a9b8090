"""CPU oracle for the TurboQuant KV-cache codec and the Gram-table scorer of
block-codebook codes (test infrastructure only).

This package is the slow, obviously-correct reference that the HIP path is
checked against.  It is plain Python + NumPy in float64, uses dense matrices
(an explicit Sylvester-Hadamard matrix, an explicit Gaussian projection
matrix) and decode-then-dot scoring, and shares no code with the GPU path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  The product library never calls into it.

Pages cited in docstrings (the method statement and the API evidence):
  * "turboquant-plus-rs 0.1.0 README" (docs.rs), sections "Architecture",
    "Compression formats", "Modules", "Usage";
  * "bitpolar 0.3.3 src/kv_cache.rs" (docs.rs), ``KvCacheConfig``,
    ``KvCacheCompressor::{push, attention_scores, decode_values,
    compression_ratio}``, ``MultiHeadKvCache::new``;
  * "fib-quant 0.1.0-beta.4 README" (docs.rs), "What's in the box" (Codec,
    Rotation, Scoring) and "New modules", Scoring (``oracle/gram.py``).

Parity status per function is listed in the header of each module.
"""
