"""ctypes wrapper around the fp64 CPU oracle (zl_oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package.  The GPU library never imports it
and shares no code with it; the product path fails loudly when its HIP
library is missing instead of falling back here.

All inputs are raw 16-bit patterns (numpy uint16); every element is decoded
exactly to double inside the oracle.  Outputs are float64.
"""
import ctypes
import os
import threading

import numpy as np

from . import build as _build

F16 = 0
BF16 = 1

_lib = None
_lock = threading.Lock()

_u16p = ctypes.POINTER(ctypes.c_uint16)
_i32p = ctypes.POINTER(ctypes.c_int32)
_f64p = ctypes.POINTER(ctypes.c_double)


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = os.environ.get("ZL_ORACLE_LIBRARY")  # another build (a sanitizer build, say)
        if not path:
            path = _build.LIB
            if not os.path.exists(path):
                _build.build()
        _lib = load_library(path)
        return _lib


def load_library(path: str):
    """Load an oracle shared library from `path` and declare its signatures."""
    lib = ctypes.CDLL(path)
    lib.zo_gqa_decode.argtypes = [_u16p, _u16p, _u16p, _i32p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                  _i32p, ctypes.c_int, _f64p, _f64p, ctypes.c_int]
    lib.zo_gqa_decode.restype = ctypes.c_int
    lib.zo_mla_decode.argtypes = [_u16p, _u16p, _i32p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_int,
                                  _i32p, ctypes.c_int, _f64p, _f64p, ctypes.c_int]
    lib.zo_mla_decode.restype = ctypes.c_int
    lib.zo_decode_attn.argtypes = [_u16p, _u16p, _u16p, _i32p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_long,
                                   ctypes.c_long, ctypes.c_double, ctypes.c_int, _i32p,
                                   ctypes.c_int, _f64p, _f64p, ctypes.c_int]
    lib.zo_decode_attn.restype = ctypes.c_int
    lib.zo_varlen_attn.argtypes = [_u16p, _u16p, _u16p, _i32p, _i32p, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_long,
                                   ctypes.c_long, ctypes.c_double, ctypes.c_int, ctypes.c_int, _i32p,
                                   ctypes.c_int, _f64p, _f64p, ctypes.c_int]
    lib.zo_varlen_attn.restype = ctypes.c_int
    lib.zo_combine.argtypes = [_f64p, _f64p, ctypes.c_int, ctypes.c_long, ctypes.c_int,
                               _f64p, _f64p]
    lib.zo_combine.restype = None
    lib.zo_decode_array.argtypes = [_u16p, ctypes.c_long, ctypes.c_int, _f64p]
    lib.zo_decode_array.restype = None
    lib.zo_max_threads.argtypes = []
    lib.zo_max_threads.restype = ctypes.c_int
    return lib


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        a = a.view(np.uint16) if a.dtype.itemsize == 2 else None
        if a is None:
            raise TypeError("oracle inputs are raw 16-bit patterns")
    return a, a.ctypes.data_as(_u16p)


def _i32(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(_i32p)


def _pairs(pairs):
    if pairs is None:
        return None, None, 0
    p = np.ascontiguousarray(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
    return p, p.ctypes.data_as(_i32p), int(p.shape[0])


def max_threads() -> int:
    return int(_load().zo_max_threads())


def decode(bits, dtype: int) -> np.ndarray:
    """Exact decode of 16-bit patterns (F16 or BF16) to float64."""
    a, ap = _u16(bits)
    out = np.empty(a.shape, dtype=np.float64)
    _load().zo_decode_array(ap, a.size, dtype, out.ctypes.data_as(_f64p))
    return out


def gqa_decode(q, k, v, cu_seqlens, num_kv_heads: int, scale: float, dtype: int,
               pairs=None, threads: int = 0):
    """Decode attention, q [B, Hq, D], k/v [T, Hkv, D] (uint16 patterns).

    Returns (out [B, Hq, D] float64, lse [B, Hq] float64).  With `pairs`
    (an iterable of (b, h)), only those rows are computed; the others are
    left as NaN.
    """
    lib = _load()
    q, qp = _u16(q)
    k, kp = _u16(k)
    v, vp = _u16(v)
    cu, cup = _i32(cu_seqlens)
    B, Hq, D = q.shape
    if k.shape[1] != num_kv_heads or k.shape[2] != D or v.shape != k.shape:
        raise ValueError("k/v shape mismatch")
    if cu.shape[0] != B + 1 or cu[-1] > k.shape[0]:
        raise ValueError("cu_seqlens mismatch")
    p, pp, npairs = _pairs(pairs)
    out = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    rc = lib.zo_gqa_decode(qp, kp, vp, cup, B, Hq, num_kv_heads, D, float(scale), dtype,
                           pp, npairs, out.ctypes.data_as(_f64p), lse.ctypes.data_as(_f64p),
                           threads)
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return out, lse


def mla_decode(q, latent, cu_seqlens, scale: float, dtype: int, kv_lora_rank: int = 512,
               rope_dim: int = 64, pairs=None, threads: int = 0):
    """Absorbed MLA decode, q [B, H, rank+rope], latent [T, rank+rope].

    K is the whole latent row, V its first `kv_lora_rank` columns.
    Returns (out [B, H, rank] float64, lse [B, H] float64).
    """
    lib = _load()
    q, qp = _u16(q)
    c, cp = _u16(latent)
    cu, cup = _i32(cu_seqlens)
    B, H, Dk = q.shape
    if Dk != kv_lora_rank + rope_dim or c.shape[1] != Dk:
        raise ValueError("latent width mismatch")
    if cu.shape[0] != B + 1 or cu[-1] > c.shape[0]:
        raise ValueError("cu_seqlens mismatch")
    p, pp, npairs = _pairs(pairs)
    out = np.full((B, H, kv_lora_rank), np.nan)
    lse = np.full((B, H), np.nan)
    rc = lib.zo_mla_decode(qp, cp, cup, B, H, kv_lora_rank, rope_dim, float(scale), dtype,
                           pp, npairs, out.ctypes.data_as(_f64p), lse.ctypes.data_as(_f64p),
                           threads)
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return out, lse


def decode_attn(q, k, v, cu_seqlens, num_kv_heads: int, dk: int, dv: int, k_row_stride: int,
                v_row_stride: int, scale: float, dtype: int, pairs=None, threads: int = 0):
    """General form: K(t,g,d) = k[t*k_row_stride + g*dk + d], V likewise with dv."""
    lib = _load()
    q, qp = _u16(q)
    k, kp = _u16(k)
    v, vp = _u16(v)
    cu, cup = _i32(cu_seqlens)
    B, Hq, _ = q.shape
    p, pp, npairs = _pairs(pairs)
    out = np.full((B, Hq, dv), np.nan)
    lse = np.full((B, Hq), np.nan)
    rc = lib.zo_decode_attn(qp, kp, vp, cup, B, Hq, num_kv_heads, dk, dv, k_row_stride,
                            v_row_stride, float(scale), dtype, pp, npairs,
                            out.ctypes.data_as(_f64p), lse.ctypes.data_as(_f64p), threads)
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return out, lse


def varlen_attn(q, k, v, cu_seqlens_q, cu_seqlens_k, num_kv_heads: int, dk: int, dv: int,
                k_row_stride: int, v_row_stride: int, scale: float, dtype: int, causal: bool = True,
                rows=None, threads: int = 0):
    """Several new query tokens per sequence: q [Tq, Hq, dk] (sequence b owns
    query rows cu_q[b] .. cu_q[b+1]-1), keys/values as in decode_attn with
    cu_k.  New token i of Lq sits at cache position Lk - Lq + i and, with
    `causal`, sees cache rows 0 .. Lk - Lq + i.  Returns (out [Tq, Hq, dv],
    lse [Tq, Hq]); with `rows` (an iterable of (t, h)) only those rows are
    computed and the others are NaN."""
    lib = _load()
    q, qp = _u16(q)
    k, kp = _u16(k)
    v, vp = _u16(v)
    cq, cqp = _i32(cu_seqlens_q)
    ck, ckp = _i32(cu_seqlens_k)
    Tq, Hq, _ = q.shape
    B = cq.shape[0] - 1
    if ck.shape[0] != B + 1 or cq[-1] != Tq:
        raise ValueError("cu_seqlens mismatch")
    p, pp, n = _pairs(rows)
    out = np.full((Tq, Hq, dv), np.nan)
    lse = np.full((Tq, Hq), np.nan)
    rc = lib.zo_varlen_attn(qp, kp, vp, cqp, ckp, B, Hq, num_kv_heads, dk, dv, k_row_stride,
                            v_row_stride, float(scale), int(bool(causal)), dtype, pp, n,
                            out.ctypes.data_as(_f64p), lse.ctypes.data_as(_f64p), threads)
    if rc != 0:
        raise ValueError("oracle rejected arguments")
    return out, lse


def gqa_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, num_kv_heads: int, scale: float, dtype: int,
               causal: bool = True, rows=None, threads: int = 0):
    """varlen_attn with K/V [T, Hkv, D] (GQA/MQA/MHA)."""
    D = np.asarray(q).shape[2]
    stride = num_kv_heads * D
    return varlen_attn(q, k, v, cu_seqlens_q, cu_seqlens_k, num_kv_heads, D, D, stride, stride, scale,
                       dtype, causal, rows, threads)


def mla_varlen(q, latent, cu_seqlens_q, cu_seqlens_k, scale: float, dtype: int, causal: bool = True,
               kv_lora_rank: int = 512, rope_dim: int = 64, rows=None, threads: int = 0):
    """varlen_attn for absorbed MLA: K = the whole latent row, V its first
    kv_lora_rank columns."""
    row = kv_lora_rank + rope_dim
    return varlen_attn(q, latent, latent, cu_seqlens_q, cu_seqlens_k, 1, row, kv_lora_rank, row, row, scale,
                       dtype, causal, rows, threads)


def combine(part_out, part_lse):
    """Log-sum-exp combine: part_out [S, ..., Dv], part_lse [S, ...] -> (out, lse)."""
    po = np.ascontiguousarray(part_out, dtype=np.float64)
    pl = np.ascontiguousarray(part_lse, dtype=np.float64)
    S = po.shape[0]
    dv = po.shape[-1]
    rows = int(np.prod(pl.shape[1:])) if pl.ndim > 1 else 1
    if po.shape[:-1] != pl.shape:
        raise ValueError("partial shapes disagree")
    out = np.empty(po.shape[1:], dtype=np.float64)
    lse = np.empty(pl.shape[1:], dtype=np.float64)
    _load().zo_combine(po.ctypes.data_as(_f64p), pl.ctypes.data_as(_f64p), S, rows, dv,
                       out.ctypes.data_as(_f64p), lse.ctypes.data_as(_f64p))
    return out, lse


def gather_paged(pages, block_table, cu_seqlens, page_size: int):
    """Paged cache -> packed rows: row cu[b] + i of the result is row
    i % page_size of page block_table[b, i // page_size] (the paged layout's
    definition; pure data movement, no arithmetic).  pages [P, page_size, ...]."""
    pages = np.asarray(pages)
    table = np.asarray(block_table)
    cu = np.asarray(cu_seqlens).astype(np.int64)
    if pages.shape[1] != page_size:
        raise ValueError("pages must be [num_pages, page_size, ...]")
    T = int(cu[-1])
    out = np.empty((T,) + pages.shape[2:], dtype=pages.dtype)
    for b in range(len(cu) - 1):
        for i in range(int(cu[b + 1] - cu[b])):
            out[cu[b] + i] = pages[table[b, i // page_size], i % page_size]
    return out


def gqa_decode_paged(q, k_pages, v_pages, block_table, cu_seqlens, num_kv_heads: int, scale: float,
                     dtype: int, pairs=None, threads: int = 0):
    """Decode attention over paged caches: the plain definition applied to
    the gathered rows."""
    ps = np.asarray(k_pages).shape[1]
    k = gather_paged(k_pages, block_table, cu_seqlens, ps)
    v = gather_paged(v_pages, block_table, cu_seqlens, ps)
    return gqa_decode(q, k, v, cu_seqlens, num_kv_heads, scale, dtype, pairs=pairs, threads=threads)


def mla_decode_paged(q, kv_pages, block_table, cu_seqlens, scale: float, dtype: int, kv_lora_rank: int = 512,
                     rope_dim: int = 64, pairs=None, threads: int = 0):
    """Absorbed MLA decode over a paged latent pool (gather, then the plain form)."""
    ps = np.asarray(kv_pages).shape[1]
    c = gather_paged(kv_pages, block_table, cu_seqlens, ps)
    return mla_decode(q, c, cu_seqlens, scale, dtype, kv_lora_rank, rope_dim, pairs=pairs, threads=threads)
