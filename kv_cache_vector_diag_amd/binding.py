"""ctypes binding of libtq (include/tq.h): argument marshalling only.

Torch tensors supply device memory; the current torch stream of the tensor's
device is passed as the hipStream_t.  Functions keep the C names.  Errors come
back as ``TQError`` carrying the C status code.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_double, c_float, c_int, c_int64, c_size_t, c_uint64, c_void_p

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

ROLE_KEY = 0
ROLE_VALUE = 1
ROT_HADAMARD = 0
ROT_HAAR = 1
F32, BF16, F16 = 0, 1, 2
STATUS_NON_FINITE = 1
STATUS_BAD_BLOB = 2
STATUS_BAD_CHANNEL = 4

EXPORTS = ["tq_codebook_bytes", "tq_record_bytes", "tq_make_codebook", "tq_encode_keys",
           "tq_encode_values", "tq_encode_kv", "tq_decode_values", "tq_scores", "tq_attend_workspace_bytes",
           "tq_attend", "tq_rotate", "tq_memory_stats", "tq_status_string", "tq_codebook_bytes_ex",
           "tq_record_bytes_ex", "tq_make_codebook_ex", "tq_outlier_workspace_bytes", "tq_outlier_channels",
           "tq_encode_split", "tq_scores_split", "tq_decode_values_split", "tq_encode_split_workspace_bytes",
           "tq_encode_keys_ex", "tq_encode_values_ex", "tq_decode_values_ex", "tq_scores_ex", "tq_attend_ex",
           "tq_append_workspace_bytes", "tq_append_kv", "tq_scores_paged", "tq_gram_record_bytes", "tq_gram_table",
           "tq_gram_encode", "tq_gram_scores", "tq_split_codebook_bytes", "tq_make_split_codebooks",
           "tq_attend_static_scratch_bytes", "tq_attend_static"]

_lib = None


class TQError(RuntimeError):
    def __init__(self, code: int, where: str):
        msg = load().tq_status_string(code).decode() if _lib is not None else str(code)
        super().__init__(f"{where}: {msg} (code {code})")
        self.code = code


def load() -> ctypes.CDLL:
    """Load libtq.so (built in-tree by build_lib.build()).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libtq.so not found at {LIB_PATH}; run kv_cache_vector_diag_amd.build_lib.build()")
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "tq_codebook_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
        "tq_record_bytes": (c_size_t, [c_int, c_int, c_int, c_int]),
        "tq_make_codebook": (c_int, [c_int, c_int, c_int, c_uint64, c_int, c_void_p, c_size_t]),
        "tq_encode_keys": (c_int, [c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int, c_int64, c_int64,
                                   c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
        "tq_encode_values": (c_int, [c_int, c_int, c_void_p, c_int64, c_void_p, c_int, c_int64, c_int64,
                                     c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
        "tq_encode_kv": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                 c_void_p, c_int, c_int64, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p,
                                 c_void_p]),
        "tq_decode_values": (c_int, [c_int, c_int, c_void_p, c_int64, c_void_p, c_int64, c_int64, c_void_p,
                                     c_void_p, c_void_p]),
        "tq_scores": (c_int, [c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int64, c_int64, c_int64,
                              c_void_p, c_int, c_int64, c_float, c_void_p, c_void_p, c_void_p]),
        "tq_attend_workspace_bytes": (c_size_t, [c_int, c_int64, c_int64, c_int64]),
        "tq_attend": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                              c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int, c_int64, c_float, c_void_p,
                              c_void_p, c_size_t, c_void_p, c_void_p]),
        "tq_rotate": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int, c_int64, c_int64,
                              c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
        "tq_memory_stats": (c_int, [c_int, c_int, c_int, c_int, c_int64, c_int64, c_int64,
                                    ctypes.POINTER(c_double)]),
        "tq_status_string": (ctypes.c_char_p, [c_int]),
        "tq_codebook_bytes_ex": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
        "tq_record_bytes_ex": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
        "tq_make_codebook_ex": (c_int, [c_int, c_int, c_int, c_uint64, c_int, c_int, c_void_p, c_size_t]),
        "tq_outlier_workspace_bytes": (c_size_t, [c_int, c_int64, c_int64]),
        "tq_outlier_channels": (c_int, [c_int, c_int, c_void_p, c_int, c_int64, c_int64, c_int64, c_int64,
                                        c_void_p, c_void_p, c_size_t, c_void_p]),
        "tq_encode_split": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_void_p, c_int64, c_void_p, c_int,
                                    c_int64, c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p, c_void_p,
                                    c_size_t, c_void_p, c_void_p]),
        "tq_encode_split_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int64]),
        "tq_scores_split": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                                    c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int, c_int64, c_float,
                                    c_void_p, c_void_p, c_void_p]),
        "tq_decode_values_split": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_int64, c_void_p, c_void_p,
                                           c_void_p, c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
        "tq_encode_keys_ex": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int, c_int64,
                                      c_int64, c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
        "tq_encode_values_ex": (c_int, [c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int, c_int64, c_int64,
                                        c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
        "tq_decode_values_ex": (c_int, [c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int64, c_int64,
                                        c_void_p, c_void_p, c_void_p]),
        "tq_scores_ex": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int64, c_int64,
                                 c_int64, c_void_p, c_int, c_int64, c_float, c_void_p, c_void_p, c_void_p]),
        "tq_attend_ex": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int64,
                                 c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int, c_int64, c_float,
                                 c_void_p, c_void_p, c_size_t, c_void_p, c_void_p]),
        "tq_append_workspace_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int64, c_int64]),
        "tq_scores_paged": (c_int, [c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_void_p, c_int64, c_int,
                                    c_int64, c_int64, c_int64, c_int64, c_void_p, c_int, c_int64, c_float, c_void_p,
                                    c_void_p, c_void_p]),
        "tq_append_kv": (c_int, [c_int, c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                 c_void_p, c_int, c_int64, c_int64, c_void_p, c_void_p, c_int64, c_int, c_int64,
                                 c_void_p, c_void_p, c_void_p, c_size_t, c_void_p, c_void_p]),
        "tq_gram_record_bytes": (c_size_t, [c_int, c_int, c_int]),
        "tq_split_codebook_bytes": (c_size_t, [c_int, c_int, c_int, c_int, c_int]),
        "tq_make_split_codebooks": (c_int, [c_int, c_int, c_int, c_int, c_uint64, c_void_p, c_size_t, c_void_p,
                                            c_size_t]),
        "tq_attend_static_scratch_bytes": (c_size_t, []),
        "tq_attend_static": (c_int, [c_int, c_int, c_int, c_int, c_int, c_void_p, c_int64, c_void_p, c_int64,
                                     c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p, c_int, c_int64, c_float,
                                     c_void_p, c_void_p, c_void_p]),
        "tq_gram_table": (c_int, [c_int, c_int, c_void_p, c_void_p, c_void_p]),
        "tq_gram_encode": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int, c_int64, c_int64,
                                   c_int64, c_int64, c_void_p, c_void_p, c_void_p]),
        "tq_gram_scores": (c_int, [c_int, c_int, c_int, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64,
                                   c_int64, c_float, c_void_p, c_void_p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(rc: int, where: str) -> None:
    if rc != 0:
        raise TQError(rc, where)


# ---------------------------------------------------------------------------
# host-only calls
# ---------------------------------------------------------------------------
def tq_codebook_bytes(head_dim: int, bits: int, projections: int, role: int) -> int:
    return int(load().tq_codebook_bytes(head_dim, bits, projections, role))


def tq_record_bytes(head_dim: int, bits: int, projections: int, role: int) -> int:
    return int(load().tq_record_bytes(head_dim, bits, projections, role))


def tq_make_codebook(head_dim: int, bits: int, projections: int, seed: int, role: int) -> np.ndarray:
    """One host blob (uint8 array of tq_codebook_bytes)."""
    lib = load()
    nbytes = lib.tq_codebook_bytes(head_dim, bits, projections, role)
    buf = np.zeros(max(int(nbytes), 1), dtype=np.uint8)
    _check(lib.tq_make_codebook(head_dim, bits, projections, seed & ((1 << 64) - 1), role,
                                buf.ctypes.data, buf.nbytes), "tq_make_codebook")
    return buf


def tq_codebook_bytes_ex(head_dim: int, bits: int, projections: int, role: int, rotation: int) -> int:
    return int(load().tq_codebook_bytes_ex(head_dim, bits, projections, role, rotation))


def tq_record_bytes_ex(head_dim: int, bits: int, projections: int, role: int, rotation: int) -> int:
    return int(load().tq_record_bytes_ex(head_dim, bits, projections, role, rotation))


def tq_make_codebook_ex(head_dim: int, bits: int, projections: int, seed: int, role: int,
                        rotation: int) -> np.ndarray:
    lib = load()
    nbytes = lib.tq_codebook_bytes_ex(head_dim, bits, projections, role, rotation)
    buf = np.zeros(max(int(nbytes), 1), dtype=np.uint8)
    _check(lib.tq_make_codebook_ex(head_dim, bits, projections, seed & ((1 << 64) - 1), role, rotation,
                                   buf.ctypes.data, buf.nbytes), "tq_make_codebook_ex")
    return buf


def make_codebooks(n_cb: int, head_dim: int, bits: int, projections: int, seed: int, role: int,
                   device=None, rotation: int = ROT_HADAMARD, seeds=None):
    """n_cb blobs back to back, blob i seeded with seed + i (wrapping) or seeds[i],
    as a uint8 torch tensor on `device` (host numpy array when device is None)."""
    sl = [seed + i for i in range(n_cb)] if seeds is None else list(seeds)
    blobs = np.concatenate([tq_make_codebook_ex(head_dim, bits, projections, s, role, rotation) for s in sl])
    if device is None:
        return blobs
    import torch
    return torch.from_numpy(blobs).to(device)


def tq_memory_stats(head_dim: int, k_bits: int, v_bits: int, projections: int, seq_len: int, layers: int,
                    kv_heads: int) -> dict:
    out = (c_double * 4)()
    _check(load().tq_memory_stats(head_dim, k_bits, v_bits, projections, seq_len, layers, kv_heads, out),
           "tq_memory_stats")
    return {"orig_fp16_bytes": out[0], "orig_f32_bytes": out[1], "compressed_bytes": out[2],
            "ratio_vs_fp16": out[3]}


# ---------------------------------------------------------------------------
# device calls (torch tensors)
#
# Every caller-supplied tensor is checked before anything is enqueued: device,
# dtype, contiguity, and that it holds what the call reads or writes (records
# and pools by their exact shape, codebook arrays and scratch by byte size).
# The kernels take raw pointers and sizes, so a mismatch here would otherwise
# become an out-of-bounds device access.  Checks raise ValueError; the last
# one, that the tensors live on a GPU, comes after every shape check.
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    codes = {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}
    if t.dtype not in codes:
        raise ValueError(f"unsupported dtype {t.dtype} (float32, bfloat16 or float16)")
    return codes[t.dtype]


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _tensor(t, name, dev):
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.device != dev:
        raise ValueError(f"{name} is on {t.device}, the call's tensors are on {dev}")
    return t


def _buf(t, name, dev, nbytes, dtypes=None):
    """A contiguous caller buffer on dev holding at least nbytes (of one of dtypes)."""
    _tensor(t, name, dev)
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {list(dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {nbytes}")
    return t


def _shaped(t, name, dev, shape, dtype):
    """A contiguous tensor on dev of exactly `shape` and `dtype`."""
    _tensor(t, name, dev)
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _i32():
    import torch
    return torch.int32


def _codebooks(cbs, name, dev, n_cb, blob_bytes):
    """n_cb blobs of blob_bytes each (uint8); invalid parameters are left to the library's own check."""
    import torch
    if n_cb > 0 and blob_bytes > 0:
        _buf(cbs, name, dev, n_cb * blob_bytes, (torch.uint8,))
    else:
        _tensor(cbs, name, dev)


def _status(status, dev):
    if status is not None:
        _buf(status, "status", dev, 4, (_i32(),))


def _on_gpu(dev):
    if dev.type != "cuda":
        raise ValueError(f"libtq runs on the GPU: the call's tensors are on {dev}")


def _groups(x, head_dim):
    """(G, N, sx_g, sx_n) of x viewed as [G][N][head_dim] with a contiguous last dim."""
    import torch
    if not isinstance(x, torch.Tensor):
        raise ValueError(f"x must be a torch tensor, got {type(x).__name__}")
    if x.dim() != 3 or x.shape[2] != head_dim or x.stride(2) != 1:
        raise ValueError(f"expected [G][N][{head_dim}] with contiguous last dim, got {tuple(x.shape)}")
    if x.stride(0) < 0 or x.stride(1) < 0:
        raise ValueError("negative strides are not supported")
    _dtype_code(x)
    return x.shape[0], x.shape[1], x.stride(0), x.stride(1)


def _query(q, B, head_dim, name="q"):
    import torch
    if not isinstance(q, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor, got {type(q).__name__}")
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != head_dim or not q.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B={B}][H_q][{head_dim}], got {tuple(q.shape)}")
    _dtype_code(q)
    return q.shape[1]


def _key_cache(krec, name, words):
    """(B, H_kv, T) of a contiguous int32 record tensor [B][H_kv][T][words]."""
    import torch
    if not isinstance(krec, torch.Tensor) or krec.dim() != 4:
        raise ValueError(f"{name} must be a [B][H_kv][T][words] tensor")
    B, Hkv, T = krec.shape[0], krec.shape[1], krec.shape[2]
    _shaped(krec, name, krec.device, (B, Hkv, T, words), _i32())
    return B, Hkv, T


def _words(nbytes, what):
    if nbytes <= 0:
        raise ValueError(f"invalid parameters for {what}")
    return nbytes // 4


# A `rotation` other than ROT_HADAMARD calls the rotation-named (_ex) entry point.
def tq_encode_keys(cbs, n_cb, x, head_dim, bits, projections, rec=None, status=None, rotation=ROT_HADAMARD):
    import torch
    G, N, sg, sn = _groups(x, head_dim)
    dev = x.device
    words = _words(tq_record_bytes_ex(head_dim, bits, projections, ROLE_KEY, rotation), "key records")
    _codebooks(cbs, "cbs", dev, n_cb, tq_codebook_bytes_ex(head_dim, bits, projections, ROLE_KEY, rotation))
    if rec is not None:
        _shaped(rec, "rec", dev, (G, N, words), _i32())
    _status(status, dev)
    _on_gpu(dev)
    if rec is None:
        rec = torch.empty((G, N, words), dtype=torch.int32, device=dev)
    if rotation == ROT_HADAMARD:
        rc = load().tq_encode_keys(head_dim, bits, projections, _ptr(cbs), n_cb, _ptr(x), _dtype_code(x), G, N,
                                   sg, sn, _ptr(rec), _ptr(status), _stream(x))
    else:
        rc = load().tq_encode_keys_ex(head_dim, bits, projections, rotation, _ptr(cbs), n_cb, _ptr(x),
                                      _dtype_code(x), G, N, sg, sn, _ptr(rec), _ptr(status), _stream(x))
    _check(rc, "tq_encode_keys")
    return rec


def tq_encode_kv(kcbs, n_kcb, vcbs, n_vcb, k, v, head_dim, k_bits, v_bits, projections, krec=None, vrec=None,
                 status=None):
    """Keys k and values v of the same tokens ([G][N][head_dim] each, same dtype
    and strides) -> (key records, value records), as tq_encode_keys and
    tq_encode_values give them; one launch where the library can share it."""
    import torch
    G, N, sg, sn = _groups(k, head_dim)
    dev = k.device
    _tensor(v, "v", dev)
    if tuple(v.shape) != tuple(k.shape) or v.dtype != k.dtype or v.stride() != k.stride():
        raise ValueError(f"v must match k in shape, dtype and strides (k {tuple(k.shape)} {k.dtype} {k.stride()}, "
                         f"v {tuple(v.shape)} {v.dtype} {v.stride()})")
    kw = _words(tq_record_bytes(head_dim, k_bits, projections, ROLE_KEY), "key records")
    vw = _words(tq_record_bytes(head_dim, v_bits, 0, ROLE_VALUE), "value records")
    _codebooks(kcbs, "kcbs", dev, n_kcb, tq_codebook_bytes(head_dim, k_bits, projections, ROLE_KEY))
    _codebooks(vcbs, "vcbs", dev, n_vcb, tq_codebook_bytes(head_dim, v_bits, 0, ROLE_VALUE))
    if krec is not None:
        _shaped(krec, "krec", dev, (G, N, kw), _i32())
    if vrec is not None:
        _shaped(vrec, "vrec", dev, (G, N, vw), _i32())
    _status(status, dev)
    _on_gpu(dev)
    if krec is None:
        krec = torch.empty((G, N, kw), dtype=torch.int32, device=dev)
    if vrec is None:
        vrec = torch.empty((G, N, vw), dtype=torch.int32, device=dev)
    rc = load().tq_encode_kv(head_dim, k_bits, v_bits, projections, _ptr(kcbs), n_kcb, _ptr(vcbs), n_vcb, _ptr(k),
                             _ptr(v), _dtype_code(k), G, N, sg, sn, _ptr(krec), _ptr(vrec), _ptr(status), _stream(k))
    _check(rc, "tq_encode_kv")
    return krec, vrec


def tq_encode_values(cbs, n_cb, x, head_dim, bits, rec=None, status=None, rotation=ROT_HADAMARD):
    import torch
    G, N, sg, sn = _groups(x, head_dim)
    dev = x.device
    words = _words(tq_record_bytes_ex(head_dim, bits, 0, ROLE_VALUE, rotation), "value records")
    _codebooks(cbs, "cbs", dev, n_cb, tq_codebook_bytes_ex(head_dim, bits, 0, ROLE_VALUE, rotation))
    if rec is not None:
        _shaped(rec, "rec", dev, (G, N, words), _i32())
    _status(status, dev)
    _on_gpu(dev)
    if rec is None:
        rec = torch.empty((G, N, words), dtype=torch.int32, device=dev)
    if rotation == ROT_HADAMARD:
        rc = load().tq_encode_values(head_dim, bits, _ptr(cbs), n_cb, _ptr(x), _dtype_code(x), G, N, sg, sn,
                                     _ptr(rec), _ptr(status), _stream(x))
    else:
        rc = load().tq_encode_values_ex(head_dim, bits, rotation, _ptr(cbs), n_cb, _ptr(x), _dtype_code(x), G, N,
                                        sg, sn, _ptr(rec), _ptr(status), _stream(x))
    _check(rc, "tq_encode_values")
    return rec


def tq_decode_values(cbs, n_cb, rec, head_dim, bits, out=None, status=None, rotation=ROT_HADAMARD):
    import torch
    words = _words(tq_record_bytes_ex(head_dim, bits, 0, ROLE_VALUE, rotation), "value records")
    if not isinstance(rec, torch.Tensor) or rec.dim() != 3:
        raise ValueError("rec must be a [G][N][words] tensor")
    G, N = rec.shape[0], rec.shape[1]
    dev = rec.device
    _shaped(rec, "rec", dev, (G, N, words), _i32())
    _codebooks(cbs, "cbs", dev, n_cb, tq_codebook_bytes_ex(head_dim, bits, 0, ROLE_VALUE, rotation))
    if out is not None:
        _shaped(out, "out", dev, (G, N, head_dim), torch.float32)
    _status(status, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty((G, N, head_dim), dtype=torch.float32, device=dev)
    if rotation == ROT_HADAMARD:
        rc = load().tq_decode_values(head_dim, bits, _ptr(cbs), n_cb, _ptr(rec), G, N, _ptr(out), _ptr(status),
                                     _stream(rec))
    else:
        rc = load().tq_decode_values_ex(head_dim, bits, rotation, _ptr(cbs), n_cb, _ptr(rec), G, N, _ptr(out),
                                        _ptr(status), _stream(rec))
    _check(rc, "tq_decode_values")
    return out


def tq_scores(cbs, n_cb, krec, q, head_dim, bits, projections, scale=0.0, out=None, status=None,
              rotation=ROT_HADAMARD):
    """krec [B][H_kv][T][words] (int32 view of uint32), q [B][H_q][head_dim] -> [B][H_q][T] float32."""
    import torch
    words = _words(tq_record_bytes_ex(head_dim, bits, projections, ROLE_KEY, rotation), "key records")
    B, Hkv, T = _key_cache(krec, "krec", words)
    dev = krec.device
    Hq = _query(q, B, head_dim)
    _tensor(q, "q", dev)
    _codebooks(cbs, "cbs", dev, n_cb, tq_codebook_bytes_ex(head_dim, bits, projections, ROLE_KEY, rotation))
    if out is not None:
        _shaped(out, "out", dev, (B, Hq, T), torch.float32)
    _status(status, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    if rotation == ROT_HADAMARD:
        rc = load().tq_scores(head_dim, bits, projections, _ptr(cbs), n_cb, _ptr(krec), B, Hkv, T, _ptr(q),
                              _dtype_code(q), Hq, scale, _ptr(out), _ptr(status), _stream(q))
    else:
        rc = load().tq_scores_ex(head_dim, bits, projections, rotation, _ptr(cbs), n_cb, _ptr(krec), B, Hkv, T,
                                 _ptr(q), _dtype_code(q), Hq, scale, _ptr(out), _ptr(status), _stream(q))
    _check(rc, "tq_scores")
    return out


def tq_attend_workspace_bytes(head_dim, B, Hq, T) -> int:
    return int(load().tq_attend_workspace_bytes(head_dim, B, Hq, T))


def tq_attend(kcbs, n_kcb, vcbs, n_vcb, krec, vrec, q, head_dim, k_bits, v_bits, projections, scale=0.0,
              out=None, work=None, status=None, rotation=ROT_HADAMARD):
    import torch
    kw = _words(tq_record_bytes_ex(head_dim, k_bits, projections, ROLE_KEY, rotation), "key records")
    vw = _words(tq_record_bytes_ex(head_dim, v_bits, 0, ROLE_VALUE, rotation), "value records")
    B, Hkv, T = _key_cache(krec, "krec", kw)
    dev = krec.device
    _shaped(vrec, "vrec", dev, (B, Hkv, T, vw), _i32())
    Hq = _query(q, B, head_dim)
    _tensor(q, "q", dev)
    _codebooks(kcbs, "kcbs", dev, n_kcb, tq_codebook_bytes_ex(head_dim, k_bits, projections, ROLE_KEY, rotation))
    _codebooks(vcbs, "vcbs", dev, n_vcb, tq_codebook_bytes_ex(head_dim, v_bits, 0, ROLE_VALUE, rotation))
    if out is not None:
        _shaped(out, "out", dev, (B, Hq, head_dim), torch.float32)
    need = tq_attend_workspace_bytes(head_dim, B, Hq, T)
    if work is not None:
        _buf(work, "work", dev, need)
    _status(status, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty((B, Hq, head_dim), dtype=torch.float32, device=dev)
    if work is None:
        work = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    args = (_ptr(kcbs), n_kcb, _ptr(vcbs), n_vcb, _ptr(krec), _ptr(vrec), B, Hkv, T, _ptr(q), _dtype_code(q), Hq,
            scale, _ptr(out), _ptr(work), work.numel() * work.element_size(), _ptr(status), _stream(q))
    if rotation == ROT_HADAMARD:
        rc = load().tq_attend(head_dim, k_bits, v_bits, projections, *args)
    else:
        rc = load().tq_attend_ex(head_dim, k_bits, v_bits, projections, rotation, *args)
    _check(rc, "tq_attend")
    return out


def tq_attend_static(kcbs, n_kcb, vcbs, n_vcb, krec, vrec, q, head_dim, k_bits, v_bits, projections, scale=0.0,
                     out=None, status=None, rotation=ROT_HADAMARD):
    """tq_attend without a workspace: the library's static device scratch (the
    allocation-free entry point; `out` is allocated here only when None)."""
    import torch
    kw = _words(tq_record_bytes_ex(head_dim, k_bits, projections, ROLE_KEY, rotation), "key records")
    vw = _words(tq_record_bytes_ex(head_dim, v_bits, 0, ROLE_VALUE, rotation), "value records")
    B, Hkv, T = _key_cache(krec, "krec", kw)
    dev = krec.device
    _shaped(vrec, "vrec", dev, (B, Hkv, T, vw), _i32())
    Hq = _query(q, B, head_dim)
    _tensor(q, "q", dev)
    _codebooks(kcbs, "kcbs", dev, n_kcb, tq_codebook_bytes_ex(head_dim, k_bits, projections, ROLE_KEY, rotation))
    _codebooks(vcbs, "vcbs", dev, n_vcb, tq_codebook_bytes_ex(head_dim, v_bits, 0, ROLE_VALUE, rotation))
    if out is not None:
        _shaped(out, "out", dev, (B, Hq, head_dim), torch.float32)
    _status(status, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty((B, Hq, head_dim), dtype=torch.float32, device=dev)
    _check(load().tq_attend_static(head_dim, k_bits, v_bits, projections, rotation, _ptr(kcbs), n_kcb, _ptr(vcbs),
                                   n_vcb, _ptr(krec), _ptr(vrec), B, Hkv, T, _ptr(q), _dtype_code(q), Hq, scale,
                                   _ptr(out), _ptr(status), _stream(q)), "tq_attend_static")
    return out


def tq_append_workspace_bytes(head_dim, k_bits, v_bits, projections, B, Hkv) -> int:
    return int(load().tq_append_workspace_bytes(head_dim, k_bits, v_bits, projections, B, Hkv))


def tq_append_kv(kcbs, n_kcb, vcbs, n_vcb, k_new, v_new, head_dim, k_bits, v_bits, projections, pos, page_table,
                 tokens_per_page, kpool, vpool, work=None, status=None):
    """One new token per sequence, all kv heads: k_new, v_new [B][H_kv][head_dim]; pos [B] int32;
    page_table [B][max_pages] int32; pools [num_pages][H_kv][tokens_per_page][record words] int32."""
    import torch
    if not isinstance(k_new, torch.Tensor) or k_new.dim() != 3:
        raise ValueError("k_new must be a [B][H_kv][head_dim] tensor")
    B, Hkv = k_new.shape[0], k_new.shape[1]
    dev = k_new.device
    if not (k_new.is_contiguous() and k_new.shape[2] == head_dim):
        raise ValueError("k_new, v_new must be contiguous [B][H_kv][head_dim]")
    _shaped(v_new, "v_new", dev, (B, Hkv, head_dim), k_new.dtype)
    _dtype_code(k_new)
    kw = _words(tq_record_bytes(head_dim, k_bits, projections, ROLE_KEY), "key records")
    vw = _words(tq_record_bytes(head_dim, v_bits, 0, ROLE_VALUE), "value records")
    _codebooks(kcbs, "kcbs", dev, n_kcb, tq_codebook_bytes(head_dim, k_bits, projections, ROLE_KEY))
    _codebooks(vcbs, "vcbs", dev, n_vcb, tq_codebook_bytes(head_dim, v_bits, 0, ROLE_VALUE))
    _buf(pos, "pos", dev, 4 * B, (_i32(),))
    _tensor(page_table, "page_table", dev)
    if page_table.dim() != 2 or page_table.shape[0] < B or page_table.dtype != torch.int32 \
            or not page_table.is_contiguous():
        raise ValueError(f"page_table must be contiguous int32 [B={B}][max_pages], got {tuple(page_table.shape)}")
    _tensor(kpool, "kpool", dev)
    if kpool.dim() != 4:
        raise ValueError("kpool must be [num_pages][H_kv][tokens_per_page][words]")
    num_pages = kpool.shape[0]
    _shaped(kpool, "kpool", dev, (num_pages, Hkv, tokens_per_page, kw), _i32())
    _shaped(vpool, "vpool", dev, (num_pages, Hkv, tokens_per_page, vw), _i32())
    need = tq_append_workspace_bytes(head_dim, k_bits, v_bits, projections, B, Hkv)
    if work is not None:
        _buf(work, "work", dev, need)
    _status(status, dev)
    _on_gpu(dev)
    if work is None:
        work = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    # the pool rows of the table: the first B rows are read
    _check(load().tq_append_kv(head_dim, k_bits, v_bits, projections, _ptr(kcbs), n_kcb, _ptr(vcbs), n_vcb,
                               _ptr(k_new), _ptr(v_new), _dtype_code(k_new), B, Hkv, _ptr(pos), _ptr(page_table),
                               page_table.shape[1], tokens_per_page, num_pages, _ptr(kpool), _ptr(vpool),
                               _ptr(work), work.numel() * work.element_size(), _ptr(status), _stream(k_new)),
           "tq_append_kv")


def tq_scores_paged(cbs, n_cb, kpool, page_table, tokens_per_page, T, q, head_dim, bits, projections, scale=0.0,
                    out=None, status=None):
    """kpool [num_pages][H_kv][tokens_per_page][words], page_table [B][max_pages] -> scores [B][H_q][T]."""
    import torch
    if not isinstance(q, torch.Tensor) or q.dim() != 3:
        raise ValueError("q must be a [B][H_q][head_dim] tensor")
    B = q.shape[0]
    Hq = _query(q, B, head_dim)
    dev = q.device
    kw = _words(tq_record_bytes(head_dim, bits, projections, ROLE_KEY), "key records")
    _tensor(kpool, "kpool", dev)
    if kpool.dim() != 4:
        raise ValueError("kpool must be [num_pages][H_kv][tokens_per_page][words]")
    num_pages, Hkv = kpool.shape[0], kpool.shape[1]
    _shaped(kpool, "kpool", dev, (num_pages, Hkv, tokens_per_page, kw), _i32())
    _tensor(page_table, "page_table", dev)
    if page_table.dim() != 2 or page_table.shape[0] < B or page_table.dtype != torch.int32 \
            or not page_table.is_contiguous():
        raise ValueError(f"page_table must be contiguous int32 [B={B}][max_pages], got {tuple(page_table.shape)}")
    if T < 0 or T > page_table.shape[1] * tokens_per_page:
        raise ValueError(f"T={T} exceeds the page table's {page_table.shape[1]} pages of {tokens_per_page}")
    _codebooks(cbs, "cbs", dev, n_cb, tq_codebook_bytes(head_dim, bits, projections, ROLE_KEY))
    if out is not None:
        _shaped(out, "out", dev, (B, Hq, T), torch.float32)
    _status(status, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    _check(load().tq_scores_paged(head_dim, bits, projections, _ptr(cbs), n_cb, _ptr(kpool), _ptr(page_table),
                                  page_table.shape[1], tokens_per_page, num_pages, B, Hkv, T, _ptr(q),
                                  _dtype_code(q), Hq, scale, _ptr(out), _ptr(status), _stream(q)),
           "tq_scores_paged")
    return out


def tq_split_codebook_bytes(role: int, head_dim: int, n_outlier: int, bits: int, part: int) -> int:
    return int(load().tq_split_codebook_bytes(role, head_dim, n_outlier, bits, part))


def split_codebooks(n_cb: int, head_dim: int, n_outlier: int, bits: int, seed: int, role: int, device=None):
    """(normal-part blobs, outlier-part blobs) of n_cb groups whose head seeds are
    seed + i (wrapping), each pair made by tq_make_split_codebooks (which holds
    the parts' seed rule); uint8 torch tensors on `device` (numpy when None)."""
    lib = load()
    nb = tq_split_codebook_bytes(role, head_dim, n_outlier, bits, 0)
    ob = tq_split_codebook_bytes(role, head_dim, n_outlier, bits, 1)
    if nb == 0 or ob == 0:
        raise ValueError("invalid split parameters")
    normal = np.zeros(n_cb * nb, dtype=np.uint8)
    outlier = np.zeros(n_cb * ob, dtype=np.uint8)
    for i in range(n_cb):
        _check(lib.tq_make_split_codebooks(role, head_dim, n_outlier, bits, (seed + i) & ((1 << 64) - 1),
                                           normal.ctypes.data + i * nb, nb, outlier.ctypes.data + i * ob, ob),
               "tq_make_split_codebooks")
    if device is None:
        return normal, outlier
    import torch
    return torch.from_numpy(normal).to(device), torch.from_numpy(outlier).to(device)


def split_record_words(head_dim: int, n_outlier: int, bits: int, role: int) -> tuple[int, int]:
    dn = head_dim - n_outlier
    key = role == ROLE_KEY
    return (tq_record_bytes_ex(dn, bits, dn if key else 0, role, ROT_HAAR) // 4,
            tq_record_bytes_ex(n_outlier, bits + 1, n_outlier if key else 0, role, ROT_HADAMARD) // 4)


def _split_codebook_arrays(cbs_normal, cbs_outlier, dev, n_cb, role, head_dim, n_outlier, bits):
    _codebooks(cbs_normal, "cbs_normal", dev, n_cb, tq_split_codebook_bytes(role, head_dim, n_outlier, bits, 0))
    _codebooks(cbs_outlier, "cbs_outlier", dev, n_cb, tq_split_codebook_bytes(role, head_dim, n_outlier, bits, 1))


def tq_outlier_workspace_bytes(head_dim, G, N) -> int:
    return int(load().tq_outlier_workspace_bytes(head_dim, G, N))


def tq_outlier_channels(x, head_dim, n_outlier, chan=None, work=None):
    import torch
    G, N, sg, sn = _groups(x, head_dim)
    dev = x.device
    if chan is not None:
        _shaped(chan, "chan", dev, (G, head_dim), _i32())
    need = tq_outlier_workspace_bytes(head_dim, G, N)
    if work is not None:
        _buf(work, "work", dev, need)
    _on_gpu(dev)
    if chan is None:
        chan = torch.empty((G, head_dim), dtype=torch.int32, device=dev)
    if work is None:
        work = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(load().tq_outlier_channels(head_dim, n_outlier, _ptr(x), _dtype_code(x), G, N, sg, sn, _ptr(chan),
                                      _ptr(work), work.numel() * work.element_size(), _stream(x)),
           "tq_outlier_channels")
    return chan


def tq_encode_split_workspace_bytes(role, head_dim, n_outlier, bits, G) -> int:
    return int(load().tq_encode_split_workspace_bytes(role, head_dim, n_outlier, bits, G))


def tq_encode_split(role, cbs_normal, cbs_outlier, n_cb, x, head_dim, n_outlier, bits, chan,
                    rec_normal=None, rec_outlier=None, status=None, work=None, use_workspace=True):
    """Split encode; `work` is scratch for the MFMA path (allocated here when None
    and use_workspace; use_workspace=False runs the generic kernels)."""
    import torch
    G, N, sg, sn = _groups(x, head_dim)
    dev = x.device
    wn, wo = split_record_words(head_dim, n_outlier, bits, role)
    if wn == 0 or wo == 0:
        raise ValueError("invalid split parameters")
    _split_codebook_arrays(cbs_normal, cbs_outlier, dev, n_cb, role, head_dim, n_outlier, bits)
    _shaped(chan, "chan", dev, (G, head_dim), _i32())
    if rec_normal is not None:
        _shaped(rec_normal, "rec_normal", dev, (G, N, wn), _i32())
    if rec_outlier is not None:
        _shaped(rec_outlier, "rec_outlier", dev, (G, N, wo), _i32())
    if work is not None:
        _buf(work, "work", dev, 0)
    _status(status, dev)
    _on_gpu(dev)
    if rec_normal is None:
        rec_normal = torch.empty((G, N, wn), dtype=torch.int32, device=dev)
    if rec_outlier is None:
        rec_outlier = torch.empty((G, N, wo), dtype=torch.int32, device=dev)
    if work is None and use_workspace:
        need = tq_encode_split_workspace_bytes(role, head_dim, n_outlier, bits, G)
        work = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    wbytes = 0 if work is None else work.numel() * work.element_size()
    _check(load().tq_encode_split(role, head_dim, n_outlier, bits, _ptr(cbs_normal), _ptr(cbs_outlier), n_cb,
                                  _ptr(x), _dtype_code(x), G, N, sg, sn, _ptr(chan), _ptr(rec_normal),
                                  _ptr(rec_outlier), _ptr(work), wbytes, _ptr(status), _stream(x)),
           "tq_encode_split")
    return rec_normal, rec_outlier


def tq_scores_split(cbs_normal, cbs_outlier, n_cb, chan, krec_normal, krec_outlier, q, head_dim, n_outlier, bits,
                    scale=0.0, out=None, status=None):
    import torch
    wn, wo = split_record_words(head_dim, n_outlier, bits, ROLE_KEY)
    if wn == 0 or wo == 0:
        raise ValueError("invalid split parameters")
    B, Hkv, T = _key_cache(krec_normal, "krec_normal", wn)
    dev = krec_normal.device
    _shaped(krec_outlier, "krec_outlier", dev, (B, Hkv, T, wo), _i32())
    Hq = _query(q, B, head_dim)
    _tensor(q, "q", dev)
    _split_codebook_arrays(cbs_normal, cbs_outlier, dev, n_cb, ROLE_KEY, head_dim, n_outlier, bits)
    _shaped(chan, "chan", dev, (B * Hkv, head_dim), _i32())
    if out is not None:
        _shaped(out, "out", dev, (B, Hq, T), torch.float32)
    _status(status, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    _check(load().tq_scores_split(head_dim, n_outlier, bits, _ptr(cbs_normal), _ptr(cbs_outlier), n_cb, _ptr(chan),
                                  _ptr(krec_normal), _ptr(krec_outlier), B, Hkv, T, _ptr(q), _dtype_code(q), Hq,
                                  scale, _ptr(out), _ptr(status), _stream(q)), "tq_scores_split")
    return out


def tq_decode_values_split(cbs_normal, cbs_outlier, n_cb, chan, rec_normal, rec_outlier, head_dim, n_outlier, bits,
                           out=None, status=None):
    import torch
    wn, wo = split_record_words(head_dim, n_outlier, bits, ROLE_VALUE)
    if wn == 0 or wo == 0:
        raise ValueError("invalid split parameters")
    if not isinstance(rec_normal, torch.Tensor) or rec_normal.dim() != 3:
        raise ValueError("rec_normal must be a [G][N][words] tensor")
    G, N = rec_normal.shape[0], rec_normal.shape[1]
    dev = rec_normal.device
    _shaped(rec_normal, "rec_normal", dev, (G, N, wn), _i32())
    _shaped(rec_outlier, "rec_outlier", dev, (G, N, wo), _i32())
    _split_codebook_arrays(cbs_normal, cbs_outlier, dev, n_cb, ROLE_VALUE, head_dim, n_outlier, bits)
    _shaped(chan, "chan", dev, (G, head_dim), _i32())
    if out is not None:
        _shaped(out, "out", dev, (G, N, head_dim), torch.float32)
    _status(status, dev)
    _on_gpu(dev)
    if out is None:
        out = torch.empty((G, N, head_dim), dtype=torch.float32, device=dev)
    _check(load().tq_decode_values_split(head_dim, n_outlier, bits, _ptr(cbs_normal), _ptr(cbs_outlier), n_cb,
                                         _ptr(chan), _ptr(rec_normal), _ptr(rec_outlier), G, N, _ptr(out),
                                         _ptr(status), _stream(rec_normal)), "tq_decode_values_split")
    return out


def tq_rotate(cbs, n_cb, x, head_dim, bits, projections, role):
    import torch
    G, N, sg, sn = _groups(x, head_dim)
    dev = x.device
    _codebooks(cbs, "cbs", dev, n_cb, tq_codebook_bytes(head_dim, bits, projections, role))
    _on_gpu(dev)
    u = torch.empty((G, N, head_dim), dtype=torch.float32, device=dev)
    norms = torch.empty((G, N), dtype=torch.float32, device=dev)
    _check(load().tq_rotate(head_dim, bits, projections, role, _ptr(cbs), n_cb, _ptr(x), _dtype_code(x), G, N,
                            sg, sn, _ptr(u), _ptr(norms), _stream(x)), "tq_rotate")
    return u, norms


# ---- Gram-table scoring of block-codebook codes
def tq_gram_record_bytes(head_dim: int, block_dim: int, codebook_size: int) -> int:
    return int(load().tq_gram_record_bytes(head_dim, block_dim, codebook_size))


def _gram_codebook(codebook):
    import torch
    if not isinstance(codebook, torch.Tensor) or codebook.dim() != 2:
        raise ValueError("codebook must be a [N][k] tensor")
    if codebook.dtype != torch.float32 or not codebook.is_contiguous():
        raise ValueError("codebook must be contiguous float32 [N][k]")
    return codebook.shape


def tq_gram_table(codebook, out=None):
    """codebook [N][k] float32 (device) -> G [N][N] float32."""
    import torch
    N, k = _gram_codebook(codebook)
    dev = codebook.device
    if out is not None:
        _shaped(out, "out", dev, (N, N), torch.float32)
    _on_gpu(dev)
    if out is None:
        out = torch.empty((N, N), dtype=torch.float32, device=dev)
    _check(load().tq_gram_table(k, N, _ptr(codebook), _ptr(out), _stream(codebook)), "tq_gram_table")
    return out


def tq_gram_encode(codebook, signs, x, head_dim, rec=None, status=None):
    """x [G][N][head_dim] -> records [G][N][words] (int32 view of uint32)."""
    import torch
    N_cb, k = _gram_codebook(codebook)
    G, N, sg, sn = _groups(x, head_dim)
    dev = x.device
    _tensor(codebook, "codebook", dev)
    words = _words(tq_gram_record_bytes(head_dim, k, N_cb), "Gram records")
    _buf(signs, "signs", dev, 4 * ((head_dim + 31) // 32), (_i32(),))
    if rec is not None:
        _shaped(rec, "rec", dev, (G, N, words), _i32())
    _status(status, dev)
    _on_gpu(dev)
    if rec is None:
        rec = torch.empty((G, N, words), dtype=torch.int32, device=dev)
    rc = load().tq_gram_encode(head_dim, k, N_cb, _ptr(codebook), _ptr(signs), _ptr(x), _dtype_code(x), G, N, sg,
                               sn, _ptr(rec), _ptr(status), _stream(x))
    _check(rc, "tq_gram_encode")
    return rec


def tq_gram_scores(table, qrec, krec, head_dim, block_dim, scale=0.0, out=None):
    """qrec [B][H_q][words], krec [B][H_kv][T][words] -> [B][H_q][T] float32."""
    import torch
    if not isinstance(table, torch.Tensor) or table.dim() != 2:
        raise ValueError("table must be a [N][N] tensor")
    N_cb = table.shape[0]
    words = _words(tq_gram_record_bytes(head_dim, block_dim, N_cb), "Gram records")
    B, Hkv, T = _key_cache(krec, "krec", words)
    dev = krec.device
    _shaped(table, "table", dev, (N_cb, N_cb), torch.float32)
    _tensor(qrec, "qrec", dev)
    if qrec.dim() != 3 or qrec.shape[0] != B:
        raise ValueError(f"qrec must be [B={B}][H_q][{words}], got {tuple(qrec.shape)}")
    Hq = qrec.shape[1]
    _shaped(qrec, "qrec", dev, (B, Hq, words), _i32())
    if out is not None:
        _shaped(out, "out", dev, (B, Hq, T), torch.float32)
    _on_gpu(dev)
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    rc = load().tq_gram_scores(head_dim, block_dim, N_cb, _ptr(table), _ptr(qrec), _ptr(krec), B, Hkv, T, Hq, scale,
                               _ptr(out), _stream(krec))
    _check(rc, "tq_gram_scores")
    return out
