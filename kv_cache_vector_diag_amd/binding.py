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
OUTLIER_SEED_XOR = 0x9E3779B97F4A7C15   # seed of an outlier part = head seed XOR this

EXPORTS = ["tq_codebook_bytes", "tq_record_bytes", "tq_make_codebook", "tq_encode_keys",
           "tq_encode_values", "tq_decode_values", "tq_scores", "tq_attend_workspace_bytes",
           "tq_attend", "tq_rotate", "tq_memory_stats", "tq_status_string", "tq_codebook_bytes_ex",
           "tq_record_bytes_ex", "tq_make_codebook_ex", "tq_outlier_workspace_bytes", "tq_outlier_channels",
           "tq_encode_split", "tq_scores_split", "tq_decode_values_split", "tq_encode_split_workspace_bytes",
           "tq_encode_keys_ex", "tq_encode_values_ex", "tq_decode_values_ex", "tq_scores_ex", "tq_attend_ex",
           "tq_append_workspace_bytes", "tq_append_kv", "tq_scores_paged", "tq_gram_record_bytes", "tq_gram_table",
           "tq_gram_encode", "tq_gram_scores"]

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
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch
    return {torch.float32: F32, torch.bfloat16: BF16, torch.float16: F16}[t.dtype]


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _groups(x, head_dim):
    """(G, N, sx_g, sx_n) of x viewed as [G][N][head_dim] with a contiguous last dim."""
    if x.dim() != 3 or x.shape[2] != head_dim or x.stride(2) != 1:
        raise ValueError(f"expected [G][N][{head_dim}] with contiguous last dim, got {tuple(x.shape)}")
    return x.shape[0], x.shape[1], x.stride(0), x.stride(1)


# A `rotation` other than ROT_HADAMARD calls the rotation-named (_ex) entry point.
def tq_encode_keys(cbs, n_cb, x, head_dim, bits, projections, rec=None, status=None, rotation=ROT_HADAMARD):
    import torch
    G, N, sg, sn = _groups(x, head_dim)
    words = tq_record_bytes_ex(head_dim, bits, projections, ROLE_KEY, rotation) // 4
    if rec is None:
        rec = torch.empty((G, N, words), dtype=torch.int32, device=x.device)
    if rotation == ROT_HADAMARD:
        rc = load().tq_encode_keys(head_dim, bits, projections, _ptr(cbs), n_cb, _ptr(x), _dtype_code(x), G, N,
                                   sg, sn, _ptr(rec), _ptr(status), _stream(x))
    else:
        rc = load().tq_encode_keys_ex(head_dim, bits, projections, rotation, _ptr(cbs), n_cb, _ptr(x),
                                      _dtype_code(x), G, N, sg, sn, _ptr(rec), _ptr(status), _stream(x))
    _check(rc, "tq_encode_keys")
    return rec


def tq_encode_values(cbs, n_cb, x, head_dim, bits, rec=None, status=None, rotation=ROT_HADAMARD):
    import torch
    G, N, sg, sn = _groups(x, head_dim)
    words = tq_record_bytes_ex(head_dim, bits, 0, ROLE_VALUE, rotation) // 4
    if rec is None:
        rec = torch.empty((G, N, words), dtype=torch.int32, device=x.device)
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
    G, N = rec.shape[0], rec.shape[1]
    if out is None:
        out = torch.empty((G, N, head_dim), dtype=torch.float32, device=rec.device)
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
    B, Hkv, T = krec.shape[0], krec.shape[1], krec.shape[2]
    Hq = q.shape[1]
    if not q.is_contiguous() or q.shape[0] != B or q.shape[2] != head_dim:
        raise ValueError("q must be contiguous [B][H_q][head_dim]")
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if rotation == ROT_HADAMARD:
        rc = load().tq_scores(head_dim, bits, projections, _ptr(cbs), n_cb, _ptr(krec), B, Hkv, T, _ptr(q),
                              _dtype_code(q), Hq, scale, _ptr(out), _ptr(status), _stream(q))
    else:
        rc = load().tq_scores_ex(head_dim, bits, projections, rotation, _ptr(cbs), n_cb, _ptr(krec), B, Hkv, T,
                                 _ptr(q), _dtype_code(q), Hq, scale, _ptr(out), _ptr(status), _stream(q))
    _check(rc, "tq_scores")
    return out


def tq_attend(kcbs, n_kcb, vcbs, n_vcb, krec, vrec, q, head_dim, k_bits, v_bits, projections, scale=0.0,
              out=None, work=None, status=None, rotation=ROT_HADAMARD):
    import torch
    B, Hkv, T = krec.shape[0], krec.shape[1], krec.shape[2]
    Hq = q.shape[1]
    if out is None:
        out = torch.empty((B, Hq, head_dim), dtype=torch.float32, device=q.device)
    need = int(load().tq_attend_workspace_bytes(head_dim, B, Hq, T))
    if work is None:
        work = torch.empty(need, dtype=torch.uint8, device=q.device)
    args = (_ptr(kcbs), n_kcb, _ptr(vcbs), n_vcb, _ptr(krec), _ptr(vrec), B, Hkv, T, _ptr(q), _dtype_code(q), Hq,
            scale, _ptr(out), _ptr(work), work.numel(), _ptr(status), _stream(q))
    if rotation == ROT_HADAMARD:
        rc = load().tq_attend(head_dim, k_bits, v_bits, projections, *args)
    else:
        rc = load().tq_attend_ex(head_dim, k_bits, v_bits, projections, rotation, *args)
    _check(rc, "tq_attend")
    return out


def tq_append_kv(kcbs, n_kcb, vcbs, n_vcb, k_new, v_new, head_dim, k_bits, v_bits, projections, pos, page_table,
                 tokens_per_page, kpool, vpool, work=None, status=None):
    """One new token per sequence, all kv heads: k_new, v_new [B][H_kv][head_dim]; pos [B] int32;
    page_table [B][max_pages] int32; pools [num_pages][H_kv][tokens_per_page][record words] int32."""
    import torch
    B, Hkv = k_new.shape[0], k_new.shape[1]
    if not (k_new.is_contiguous() and v_new.is_contiguous()) or k_new.shape[2] != head_dim:
        raise ValueError("k_new, v_new must be contiguous [B][H_kv][head_dim]")
    need = int(load().tq_append_workspace_bytes(head_dim, k_bits, v_bits, projections, B, Hkv))
    if work is None:
        work = torch.empty(max(need, 1), dtype=torch.uint8, device=k_new.device)
    _check(load().tq_append_kv(head_dim, k_bits, v_bits, projections, _ptr(kcbs), n_kcb, _ptr(vcbs), n_vcb,
                               _ptr(k_new), _ptr(v_new), _dtype_code(k_new), B, Hkv, _ptr(pos), _ptr(page_table),
                               page_table.shape[1], tokens_per_page, kpool.shape[0], _ptr(kpool), _ptr(vpool),
                               _ptr(work), work.numel(), _ptr(status), _stream(k_new)), "tq_append_kv")


def tq_scores_paged(cbs, n_cb, kpool, page_table, tokens_per_page, T, q, head_dim, bits, projections, scale=0.0,
                    out=None, status=None):
    """kpool [num_pages][H_kv][tokens_per_page][words], page_table [B][max_pages] -> scores [B][H_q][T]."""
    import torch
    B, Hq = q.shape[0], q.shape[1]
    Hkv = kpool.shape[1]
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check(load().tq_scores_paged(head_dim, bits, projections, _ptr(cbs), n_cb, _ptr(kpool), _ptr(page_table),
                                  page_table.shape[1], tokens_per_page, kpool.shape[0], B, Hkv, T, _ptr(q),
                                  _dtype_code(q), Hq, scale, _ptr(out), _ptr(status), _stream(q)),
           "tq_scores_paged")
    return out


def split_codebooks(n_cb: int, head_dim: int, n_outlier: int, bits: int, seed: int, role: int, device=None):
    """(normal-part blobs, outlier-part blobs) for groups seeded seed + i: Haar at
    `bits` over head_dim - n_outlier channels, Walsh-Hadamard at bits + 1 over
    n_outlier channels with seed (seed + i) XOR OUTLIER_SEED_XOR."""
    dn = head_dim - n_outlier
    key = role == ROLE_KEY
    seeds = [(seed + i) & ((1 << 64) - 1) for i in range(n_cb)]
    normal = make_codebooks(n_cb, dn, bits, dn if key else 0, seed, role, device, ROT_HAAR, seeds)
    outlier = make_codebooks(n_cb, n_outlier, bits + 1, n_outlier if key else 0, seed, role, device,
                             ROT_HADAMARD, [s ^ OUTLIER_SEED_XOR for s in seeds])
    return normal, outlier


def split_record_words(head_dim: int, n_outlier: int, bits: int, role: int) -> tuple[int, int]:
    dn = head_dim - n_outlier
    key = role == ROLE_KEY
    return (tq_record_bytes_ex(dn, bits, dn if key else 0, role, ROT_HAAR) // 4,
            tq_record_bytes_ex(n_outlier, bits + 1, n_outlier if key else 0, role, ROT_HADAMARD) // 4)


def tq_outlier_channels(x, head_dim, n_outlier, chan=None, work=None):
    import torch
    G, N, sg, sn = _groups(x, head_dim)
    if chan is None:
        chan = torch.empty((G, head_dim), dtype=torch.int32, device=x.device)
    need = int(load().tq_outlier_workspace_bytes(head_dim, G, N))
    if work is None:
        work = torch.empty(need, dtype=torch.uint8, device=x.device)
    _check(load().tq_outlier_channels(head_dim, n_outlier, _ptr(x), _dtype_code(x), G, N, sg, sn, _ptr(chan),
                                      _ptr(work), work.numel(), _stream(x)), "tq_outlier_channels")
    return chan


def tq_encode_split_workspace_bytes(role, head_dim, n_outlier, bits, G) -> int:
    return int(load().tq_encode_split_workspace_bytes(role, head_dim, n_outlier, bits, G))


def tq_encode_split(role, cbs_normal, cbs_outlier, n_cb, x, head_dim, n_outlier, bits, chan,
                    rec_normal=None, rec_outlier=None, status=None, work=None, use_workspace=True):
    """Split encode; `work` is scratch for the MFMA path (allocated here when None
    and use_workspace; use_workspace=False runs the generic kernels)."""
    import torch
    G, N, sg, sn = _groups(x, head_dim)
    wn, wo = split_record_words(head_dim, n_outlier, bits, role)
    if rec_normal is None:
        rec_normal = torch.empty((G, N, wn), dtype=torch.int32, device=x.device)
    if rec_outlier is None:
        rec_outlier = torch.empty((G, N, wo), dtype=torch.int32, device=x.device)
    if work is None and use_workspace:
        need = tq_encode_split_workspace_bytes(role, head_dim, n_outlier, bits, G)
        work = torch.empty(need, dtype=torch.uint8, device=x.device) if need else None
    wbytes = 0 if work is None else work.numel() * work.element_size()
    _check(load().tq_encode_split(role, head_dim, n_outlier, bits, _ptr(cbs_normal), _ptr(cbs_outlier), n_cb,
                                  _ptr(x), _dtype_code(x), G, N, sg, sn, _ptr(chan), _ptr(rec_normal),
                                  _ptr(rec_outlier), _ptr(work), wbytes, _ptr(status), _stream(x)),
           "tq_encode_split")
    return rec_normal, rec_outlier


def tq_scores_split(cbs_normal, cbs_outlier, n_cb, chan, krec_normal, krec_outlier, q, head_dim, n_outlier, bits,
                    scale=0.0, out=None, status=None):
    import torch
    B, Hkv, T = krec_normal.shape[0], krec_normal.shape[1], krec_normal.shape[2]
    Hq = q.shape[1]
    if not q.is_contiguous() or q.shape[0] != B or q.shape[2] != head_dim:
        raise ValueError("q must be contiguous [B][H_q][head_dim]")
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _check(load().tq_scores_split(head_dim, n_outlier, bits, _ptr(cbs_normal), _ptr(cbs_outlier), n_cb, _ptr(chan),
                                  _ptr(krec_normal), _ptr(krec_outlier), B, Hkv, T, _ptr(q), _dtype_code(q), Hq,
                                  scale, _ptr(out), _ptr(status), _stream(q)), "tq_scores_split")
    return out


def tq_decode_values_split(cbs_normal, cbs_outlier, n_cb, chan, rec_normal, rec_outlier, head_dim, n_outlier, bits,
                           out=None, status=None):
    import torch
    G, N = rec_normal.shape[0], rec_normal.shape[1]
    if out is None:
        out = torch.empty((G, N, head_dim), dtype=torch.float32, device=rec_normal.device)
    _check(load().tq_decode_values_split(head_dim, n_outlier, bits, _ptr(cbs_normal), _ptr(cbs_outlier), n_cb,
                                         _ptr(chan), _ptr(rec_normal), _ptr(rec_outlier), G, N, _ptr(out),
                                         _ptr(status), _stream(rec_normal)), "tq_decode_values_split")
    return out


def tq_rotate(cbs, n_cb, x, head_dim, bits, projections, role):
    import torch
    G, N, sg, sn = _groups(x, head_dim)
    u = torch.empty((G, N, head_dim), dtype=torch.float32, device=x.device)
    norms = torch.empty((G, N), dtype=torch.float32, device=x.device)
    _check(load().tq_rotate(head_dim, bits, projections, role, _ptr(cbs), n_cb, _ptr(x), _dtype_code(x), G, N,
                            sg, sn, _ptr(u), _ptr(norms), _stream(x)), "tq_rotate")
    return u, norms


# ---- Gram-table scoring of block-codebook codes
def tq_gram_record_bytes(head_dim: int, block_dim: int, codebook_size: int) -> int:
    return int(load().tq_gram_record_bytes(head_dim, block_dim, codebook_size))


def tq_gram_table(codebook, out=None):
    """codebook [N][k] float32 (device) -> G [N][N] float32."""
    import torch
    N, k = codebook.shape
    if codebook.dtype != torch.float32 or not codebook.is_contiguous():
        raise ValueError("codebook must be contiguous float32 [N][k]")
    if out is None:
        out = torch.empty((N, N), dtype=torch.float32, device=codebook.device)
    _check(load().tq_gram_table(k, N, _ptr(codebook), _ptr(out), _stream(codebook)), "tq_gram_table")
    return out


def tq_gram_encode(codebook, signs, x, head_dim, rec=None, status=None):
    """x [G][N][head_dim] -> records [G][N][words] (int32 view of uint32)."""
    import torch
    N_cb, k = codebook.shape
    G, N, sg, sn = _groups(x, head_dim)
    words = tq_gram_record_bytes(head_dim, k, N_cb) // 4
    if words == 0:
        raise ValueError("bad Gram codec shape")
    if rec is None:
        rec = torch.empty((G, N, words), dtype=torch.int32, device=x.device)
    rc = load().tq_gram_encode(head_dim, k, N_cb, _ptr(codebook), _ptr(signs), _ptr(x), _dtype_code(x), G, N, sg,
                               sn, _ptr(rec), _ptr(status), _stream(x))
    _check(rc, "tq_gram_encode")
    return rec


def tq_gram_scores(table, qrec, krec, head_dim, block_dim, scale=0.0, out=None):
    """qrec [B][H_q][words], krec [B][H_kv][T][words] -> [B][H_q][T] float32."""
    import torch
    N_cb = table.shape[0]
    B, Hkv, T = krec.shape[0], krec.shape[1], krec.shape[2]
    Hq = qrec.shape[1]
    words = tq_gram_record_bytes(head_dim, block_dim, N_cb) // 4
    if qrec.shape != (B, Hq, words) or krec.shape[3] != words or not (qrec.is_contiguous() and krec.is_contiguous()):
        raise ValueError("records must be contiguous [B][H_q][words] and [B][H_kv][T][words]")
    if out is None:
        out = torch.empty((B, Hq, T), dtype=torch.float32, device=krec.device)
    rc = load().tq_gram_scores(head_dim, block_dim, N_cb, _ptr(table), _ptr(qrec), _ptr(krec), B, Hkv, T, Hq, scale,
                               _ptr(out), _stream(krec))
    _check(rc, "tq_gram_scores")
    return out

