"""TurboQuant KV-cache compression and compressed-key attention scoring for
AMD Instinct MI355X (gfx950).

The product is the C-ABI library ``libtq.so`` (header ``include/tq.h``);
``binding`` is a thin ctypes layer with the same entry-point names that
marshals torch tensors (device memory, streams) into it.  Every step of the
hot path runs in the HIP kernels; there is no CPU fallback: the binding
raises if the library is missing.
"""
__all__ = ["binding", "inputs"]
