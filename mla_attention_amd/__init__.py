"""Python binding of libzl_attn.so, the MI355X fused batched decode attention.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/zl_attn.h.  PyTorch supplies
device memory and streams.  There is no fallback: if the library is missing
or no GPU is present, the calls raise.

Entry points (same names as the C ABI):
  zl_decode_attn_gqa      grouped-query decode attention over a packed ragged cache
  zl_decode_attn_mla      absorbed multi-head latent attention decode
  zl_decode_attn_gqa_paged / zl_decode_attn_mla_paged
                          the same over paged caches (block table)
  zl_attn_varlen_gqa / zl_attn_varlen_mla (+ _paged)
                          several new query tokens per sequence (draft tokens, chunks)
  zl_attn_prefill_gqa / zl_attn_prefill_gqa_paged
                          long runs of new tokens (prefill, large chunks)
  zl_attn_combine         log-sum-exp combine of split partial results
  zl_decode_attn_workspace_size / zl_decode_attn_mla_workspace_size
  zl_status_string
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch  # loads the HIP runtime first; the library reuses it (same soname)

_HERE = os.path.dirname(os.path.abspath(__file__))
# ZL_ATTN_LIBRARY names another build of the same library (a host-side
# sanitizer build, for instance); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("ZL_ATTN_LIBRARY") or os.path.join(_HERE, "libzl_attn.so")
_lib = None
_lock = threading.Lock()

ZL_OK = 0
ZL_ERR_INVALID_ARGUMENT = 1
ZL_ERR_UNSUPPORTED = 2
ZL_ERR_WORKSPACE_TOO_SMALL = 3
ZL_ERR_HIP = 4

_DTYPE = {torch.float16: 0, torch.bfloat16: 1}

# Every symbol include/zl_attn.h declares, with its ctypes signature.
_c_int, _c_size, _c_float, _vp = ctypes.c_int, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p
SIGNATURES = {
    "zl_decode_attn_workspace_size": (_c_size, [_c_int] * 6),
    "zl_decode_attn_workspace_size_ex": (_c_size, [_c_int] * 7),
    "zl_decode_attn_gqa": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_float, _c_int, _vp, _vp, _vp, _c_size, _vp]),
    "zl_decode_attn_gqa_ex": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_float, _c_int, _vp, _vp, _c_int, _c_int, _vp, _c_size, _vp]),
    "zl_decode_attn_mla_workspace_size": (_c_size, [_c_int] * 6),
    "zl_decode_attn_mla_workspace_size_ex": (_c_size, [_c_int] * 7),
    "zl_decode_attn_mla": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_float,
                                    _c_int, _vp, _vp, _vp, _c_size, _vp]),
    "zl_decode_attn_mla_ex": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_float, _c_int, _vp, _vp, _c_int, _c_int, _vp, _c_size, _vp]),
    "zl_decode_attn_gqa_paged": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _vp, _c_int, _c_int,
                                          _c_int, _c_int, _c_int, _c_float, _c_int, _vp, _vp, _vp,
                                          _c_size, _vp]),
    "zl_decode_attn_gqa_paged_ex": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _vp, _c_int, _c_int,
                                             _c_int, _c_int, _c_int, _c_float, _c_int, _vp, _vp, _c_int,
                                             _c_int, _vp, _c_size, _vp]),
    "zl_decode_attn_mla_paged": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _vp, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _c_float, _c_int, _vp, _vp, _vp, _c_size, _vp]),
    "zl_decode_attn_mla_paged_ex": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _vp, _c_int, _c_int, _c_int,
                                             _c_int, _c_int, _c_float, _c_int, _vp, _vp, _c_int, _c_int,
                                             _vp, _c_size, _vp]),
    "zl_attn_varlen_gqa": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_float, _c_int, _c_int, _vp, _vp, _vp, _c_size, _vp]),
    "zl_attn_varlen_gqa_ex": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_float, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _vp, _c_size, _vp]),
    "zl_attn_varlen_mla": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                    _c_float, _c_int, _c_int, _vp, _vp, _vp, _c_size, _vp]),
    "zl_attn_varlen_mla_ex": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                       _c_float, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _vp, _c_size, _vp]),
    "zl_attn_varlen_gqa_paged": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _c_int, _c_float, _c_int, _c_int, _vp, _vp, _vp,
                                          _c_size, _vp]),
    "zl_attn_varlen_gqa_paged_ex": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int,
                                             _c_int, _c_int, _c_int, _c_int, _c_float, _c_int, _c_int, _vp, _vp,
                                             _c_int, _c_int, _vp, _c_size, _vp]),
    "zl_attn_varlen_mla_paged": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                                          _c_int, _c_int, _c_int, _c_float, _c_int, _c_int, _vp, _vp, _vp,
                                          _c_size, _vp]),
    "zl_attn_varlen_mla_paged_ex": (_c_int, [_vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                                             _c_int, _c_int, _c_int, _c_float, _c_int, _c_int, _vp, _vp, _c_int,
                                             _c_int, _vp, _c_size, _vp]),
    "zl_attn_combine": (_c_int, [_vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _vp, _vp, _vp]),
    "zl_attn_prefill_gqa": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int, _c_int,
                                     _c_float, _c_int, _c_int, _vp, _vp, _vp]),
    "zl_attn_prefill_gqa_paged": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _c_int, _c_int, _c_int,
                                           _c_int, _c_int, _c_int, _c_float, _c_int, _c_int, _vp, _vp, _vp]),
    "zl_int8_quantize": (_c_int, [_vp, _c_int, ctypes.c_longlong, _c_int, _vp, _vp, _vp]),
    "zl_int8_dequantize": (_c_int, [_vp, _vp, ctypes.c_longlong, _c_int, _c_int, _vp, _vp]),
    "zl_int8_reduce_step": (_c_int, [_vp, _vp, _vp, _c_int, ctypes.c_longlong, _c_int, _vp, _vp, _vp, _vp]),
    "zl_hbm_read_probe": (_c_int, [_vp, _c_size, _c_int, _c_int, _vp, _vp]),
    "zl_decode_attn_gqa_no_alloc": (_c_int, [_vp, _vp, _vp, _vp, _c_int, _c_int, _c_int, _c_int, _c_int,
                                             _c_float, _c_int, _vp, _vp, _vp]),
    "zl_status_string": (ctypes.c_char_p, [_c_int]),
}


class ZlError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {zl_status_string(status)}")


def library():
    """Load libzl_attn.so (built in-tree by mla_attention_amd/build.py); raise if absent."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                                  "or python mla_attention_amd/build.py")
            lib = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in SIGNATURES.items():
                fn = getattr(lib, name)
                fn.restype = res
                fn.argtypes = args
            _lib = lib
        return _lib


def zl_status_string(status: int) -> str:
    return library().zl_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != ZL_OK:
        raise ZlError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, device) -> ctypes.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def zl_decode_attn_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, max_seqlen_k,
                                  dtype: torch.dtype, num_workers: int = 0) -> int:
    return int(library().zl_decode_attn_workspace_size_ex(batch, num_q_heads, num_kv_heads, head_dim,
                                                           max_seqlen_k, _DTYPE[dtype], num_workers))


def zl_decode_attn_mla_workspace_size(batch, num_q_heads, kv_lora_rank, rope_dim, max_seqlen_k,
                                      dtype: torch.dtype, num_workers: int = 0) -> int:
    return int(library().zl_decode_attn_mla_workspace_size_ex(batch, num_q_heads, kv_lora_rank,
                                                               rope_dim, max_seqlen_k, _DTYPE[dtype],
                                                               num_workers))


def new_workspace(nbytes: int, device) -> torch.Tensor:
    """A workspace buffer (no initialisation needed)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def zl_decode_attn_gqa(q, k_cache, v_cache, cu_seqlens, max_seqlen_k: int, softmax_scale: float,
                       out=None, lse=None, workspace=None, num_workers: int = 0, stream=None,
                       return_lse: bool = False, phases: int = 3):
    """out[b,h] = softmax(scale * q[b,h] . K[seq b, h // G]) V[seq b, h // G].

    q [B, Hq, D], k_cache/v_cache [T, Hkv, D] (fp16 or bf16, packed ragged),
    cu_seqlens int32 [B+1].  Returns out (and lse [B, Hq] fp32 if return_lse
    or lse is given).  workspace: uint8 tensor of at least
    zl_decode_attn_workspace_size() bytes, allocated here when omitted.
    phases: 1 = decode kernel, 2 = merge kernel, 3 = both.
    """
    _need(q, "q", ndim=3)
    dev = q.device
    if q.dtype not in _DTYPE:
        raise ValueError("q must be float16 or bfloat16")
    _need(k_cache, "k_cache", q.dtype, 3, dev)
    _need(v_cache, "v_cache", q.dtype, 3, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[2] != D or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must be [T, Hkv, head_dim] like q")
    if cu_seqlens.numel() != B + 1:
        raise ValueError("cu_seqlens must have batch + 1 entries")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, 3, dev)
    if out.shape != q.shape:
        raise ValueError("out must be [B, Hq, head_dim]")
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    nbytes = zl_decode_attn_workspace_size(B, Hq, Hkv, D, max_seqlen_k, q.dtype, num_workers)
    if workspace is None:
        workspace = new_workspace(nbytes, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = library().zl_decode_attn_gqa_ex(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens), B, Hq, Hkv, D, int(max_seqlen_k),
        float(softmax_scale), _DTYPE[q.dtype], _ptr(out), _ptr(lse), int(num_workers), int(phases),
        _ptr(workspace), workspace.numel(), _stream(stream, dev))
    _check(st, "zl_decode_attn_gqa")
    return (out, lse) if lse is not None else out


def zl_decode_attn_gqa_no_alloc(q, k_cache, v_cache, cu_seqlens, max_seqlen_k: int, softmax_scale: float,
                                out=None, lse=None, stream=None, return_lse: bool = False):
    """zl_decode_attn_gqa with the library's fixed device workspace (no
    workspace argument, nothing allocated by the library; out / lse are
    allocated here when omitted)."""
    _need(q, "q", ndim=3)
    dev = q.device
    if q.dtype not in _DTYPE:
        raise ValueError("q must be float16 or bfloat16")
    _need(k_cache, "k_cache", q.dtype, 3, dev)
    _need(v_cache, "v_cache", q.dtype, 3, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[2] != D or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must be [T, Hkv, head_dim] like q")
    if cu_seqlens.numel() != B + 1:
        raise ValueError("cu_seqlens must have batch + 1 entries")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, 3, dev)
    if out.shape != q.shape:
        raise ValueError("out must be [B, Hq, head_dim]")
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    st = library().zl_decode_attn_gqa_no_alloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens), B, Hq, Hkv, D, int(max_seqlen_k),
        float(softmax_scale), _DTYPE[q.dtype], _ptr(out), _ptr(lse), _stream(stream, dev))
    _check(st, "zl_decode_attn_gqa_no_alloc")
    return (out, lse) if lse is not None else out


def zl_decode_attn_mla(q, kv_cache, cu_seqlens, max_seqlen_k: int, softmax_scale: float,
                       kv_lora_rank: int = 512, rope_dim: int = 64, out=None, lse=None,
                       workspace=None, num_workers: int = 0, stream=None, return_lse: bool = False,
                       phases: int = 3):
    """Absorbed MLA decode: q [B, H, rank+rope], kv_cache [T, rank+rope];
    K = whole latent row, V = its first kv_lora_rank columns.  Returns out [B, H, rank]."""
    _need(q, "q", ndim=3)
    dev = q.device
    if q.dtype not in _DTYPE:
        raise ValueError("q must be float16 or bfloat16")
    _need(kv_cache, "kv_cache", q.dtype, 2, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
    B, H, Dk = q.shape
    if Dk != kv_lora_rank + rope_dim or kv_cache.shape[1] != Dk:
        raise ValueError("q and kv_cache rows must be kv_lora_rank + rope_dim wide")
    if cu_seqlens.numel() != B + 1:
        raise ValueError("cu_seqlens must have batch + 1 entries")
    if out is None:
        out = torch.empty(B, H, kv_lora_rank, dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, 3, dev)
    if tuple(out.shape) != (B, H, kv_lora_rank):
        raise ValueError("out must be [B, H, kv_lora_rank]")
    if lse is None and return_lse:
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    nbytes = zl_decode_attn_mla_workspace_size(B, H, kv_lora_rank, rope_dim, max_seqlen_k, q.dtype,
                                               num_workers)
    if workspace is None:
        workspace = new_workspace(nbytes, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = library().zl_decode_attn_mla_ex(
        _ptr(q), _ptr(kv_cache), _ptr(cu_seqlens), B, H, kv_lora_rank, rope_dim, int(max_seqlen_k),
        float(softmax_scale), _DTYPE[q.dtype], _ptr(out), _ptr(lse), int(num_workers), int(phases),
        _ptr(workspace), workspace.numel(), _stream(stream, dev))
    _check(st, "zl_decode_attn_mla")
    return (out, lse) if lse is not None else out


def _paging_args(block_table, dev):
    _need(block_table, "block_table", torch.int32, 2, dev)
    return _ptr(block_table), int(block_table.shape[1])


def zl_decode_attn_gqa_paged(q, k_pages, v_pages, block_table, cu_seqlens, max_seqlen_k: int,
                             softmax_scale: float, out=None, lse=None, workspace=None, num_workers: int = 0,
                             stream=None, return_lse: bool = False, phases: int = 3):
    """zl_decode_attn_gqa over paged caches: k_pages/v_pages [pages, page_size, Hkv, D],
    block_table int32 [B, max_pages]; token i of sequence b is row i % page_size of page
    block_table[b, i // page_size].  cu_seqlens int32 [B+1] holds the length prefix sums."""
    _need(q, "q", ndim=3)
    dev = q.device
    if q.dtype not in _DTYPE:
        raise ValueError("q must be float16 or bfloat16")
    _need(k_pages, "k_pages", q.dtype, 4, dev)
    _need(v_pages, "v_pages", q.dtype, 4, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
    table, max_pages = _paging_args(block_table, dev)
    B, Hq, D = q.shape
    _, page_size, Hkv, Dk = k_pages.shape
    if Dk != D or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages / v_pages must be [pages, page_size, Hkv, head_dim] like q")
    if cu_seqlens.numel() != B + 1 or block_table.shape[0] != B:
        raise ValueError("cu_seqlens must have batch + 1 entries and block_table batch rows")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", q.dtype, 3, dev)
    if out.shape != q.shape:
        raise ValueError("out must be [B, Hq, head_dim]")
    if lse is None and return_lse:
        lse = torch.empty(B, Hq, dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    nbytes = zl_decode_attn_workspace_size(B, Hq, Hkv, D, max_seqlen_k, q.dtype, num_workers)
    if workspace is None:
        workspace = new_workspace(nbytes, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = library().zl_decode_attn_gqa_paged_ex(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), table, max_pages, int(page_size), _ptr(cu_seqlens), B, Hq, Hkv,
        D, int(max_seqlen_k), float(softmax_scale), _DTYPE[q.dtype], _ptr(out), _ptr(lse), int(num_workers),
        int(phases), _ptr(workspace), workspace.numel(), _stream(stream, dev))
    _check(st, "zl_decode_attn_gqa_paged")
    return (out, lse) if lse is not None else out


def zl_decode_attn_mla_paged(q, kv_pages, block_table, cu_seqlens, max_seqlen_k: int, softmax_scale: float,
                             kv_lora_rank: int = 512, rope_dim: int = 64, out=None, lse=None, workspace=None,
                             num_workers: int = 0, stream=None, return_lse: bool = False, phases: int = 3):
    """zl_decode_attn_mla over a paged latent pool kv_pages [pages, page_size, rank+rope]."""
    _need(q, "q", ndim=3)
    dev = q.device
    if q.dtype not in _DTYPE:
        raise ValueError("q must be float16 or bfloat16")
    _need(kv_pages, "kv_pages", q.dtype, 3, dev)
    _need(cu_seqlens, "cu_seqlens", torch.int32, 1, dev)
    table, max_pages = _paging_args(block_table, dev)
    B, H, Dk = q.shape
    page_size = kv_pages.shape[1]
    if Dk != kv_lora_rank + rope_dim or kv_pages.shape[2] != Dk:
        raise ValueError("q and kv_pages rows must be kv_lora_rank + rope_dim wide")
    if cu_seqlens.numel() != B + 1 or block_table.shape[0] != B:
        raise ValueError("cu_seqlens must have batch + 1 entries and block_table batch rows")
    if out is None:
        out = torch.empty(B, H, kv_lora_rank, dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, 3, dev)
    if tuple(out.shape) != (B, H, kv_lora_rank):
        raise ValueError("out must be [B, H, kv_lora_rank]")
    if lse is None and return_lse:
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    nbytes = zl_decode_attn_mla_workspace_size(B, H, kv_lora_rank, rope_dim, max_seqlen_k, q.dtype,
                                               num_workers)
    if workspace is None:
        workspace = new_workspace(nbytes, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = library().zl_decode_attn_mla_paged_ex(
        _ptr(q), _ptr(kv_pages), table, max_pages, int(page_size), _ptr(cu_seqlens), B, H, kv_lora_rank,
        rope_dim, int(max_seqlen_k), float(softmax_scale), _DTYPE[q.dtype], _ptr(out), _ptr(lse),
        int(num_workers), int(phases), _ptr(workspace), workspace.numel(), _stream(stream, dev))
    _check(st, "zl_decode_attn_mla_paged")
    return (out, lse) if lse is not None else out


def _varlen_common(q, cu_seqlens_q, cu_seqlens_k, dv, out, lse, return_lse):
    _need(q, "q", ndim=3)
    dev = q.device
    if q.dtype not in _DTYPE:
        raise ValueError("q must be float16 or bfloat16")
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1, dev)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1, dev)
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both have batch + 1 entries")
    Tq, Hq, _ = q.shape
    if out is None:
        out = torch.empty(Tq, Hq, dv, dtype=q.dtype, device=dev)
    _need(out, "out", q.dtype, 3, dev)
    if tuple(out.shape) != (Tq, Hq, dv):
        raise ValueError(f"out must be [total_q, num_q_heads, {dv}]")
    if lse is None and return_lse:
        lse = torch.empty(Tq, Hq, dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    return dev, cu_seqlens_q.numel() - 1, out, lse


def zl_attn_varlen_gqa(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, max_seqlen_k: int,
                       softmax_scale: float, causal: bool = True, out=None, lse=None, workspace=None,
                       num_workers: int = 0, stream=None, return_lse: bool = False, phases: int = 3):
    """Several new query tokens per sequence (chunked prefill, draft tokens).

    q [total_q, Hq, D]: sequence b's new tokens are rows cu_seqlens_q[b] ..
    cu_seqlens_q[b+1]-1, and their keys/values are already the last ones of
    its cache rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of k_cache/v_cache
    [T, Hkv, D].  With causal, new token i of nq sees cache rows up to
    lk - nq + i.  Returns out [total_q, Hq, D] (and lse [total_q, Hq])."""
    dev, B, out, lse = _varlen_common(q, cu_seqlens_q, cu_seqlens_k, q.shape[2], out, lse, return_lse)
    _need(k_cache, "k_cache", q.dtype, 3, dev)
    _need(v_cache, "v_cache", q.dtype, 3, dev)
    Tq, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[2] != D or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must be [T, Hkv, head_dim] like q")
    nbytes = zl_decode_attn_workspace_size(B, Hq, Hkv, D, max_seqlen_k, q.dtype, num_workers)
    if workspace is None:
        workspace = new_workspace(nbytes, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = library().zl_attn_varlen_gqa_ex(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Tq, Hq, Hkv, D,
        int(max_seqlen_k), float(softmax_scale), int(bool(causal)), _DTYPE[q.dtype], _ptr(out), _ptr(lse),
        int(num_workers), int(phases), _ptr(workspace), workspace.numel(), _stream(stream, dev))
    _check(st, "zl_attn_varlen_gqa")
    return (out, lse) if lse is not None else out


def zl_attn_prefill_gqa(q, k_cache, v_cache, cu_seqlens_q, cu_seqlens_k, max_seqlen_k: int,
                        softmax_scale: float, causal: bool = True, out=None, lse=None, stream=None,
                        return_lse: bool = False):
    """zl_attn_varlen_gqa through the prefill kernel (many new tokens per
    sequence; no workspace)."""
    dev, B, out, lse = _varlen_common(q, cu_seqlens_q, cu_seqlens_k, q.shape[2], out, lse, return_lse)
    _need(k_cache, "k_cache", q.dtype, 3, dev)
    _need(v_cache, "v_cache", q.dtype, 3, dev)
    Tq, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    if k_cache.shape[2] != D or v_cache.shape != k_cache.shape:
        raise ValueError("k_cache / v_cache must be [T, Hkv, head_dim] like q")
    st = library().zl_attn_prefill_gqa(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Tq, Hq, Hkv, D,
        int(max_seqlen_k), float(softmax_scale), int(bool(causal)), _DTYPE[q.dtype], _ptr(out), _ptr(lse),
        _stream(stream, dev))
    _check(st, "zl_attn_prefill_gqa")
    return (out, lse) if lse is not None else out


def zl_attn_prefill_gqa_paged(q, k_pages, v_pages, block_table, cu_seqlens_q, cu_seqlens_k, max_seqlen_k: int,
                              softmax_scale: float, causal: bool = True, out=None, lse=None, stream=None,
                              return_lse: bool = False):
    """zl_attn_prefill_gqa over page pools k_pages/v_pages [pages, page_size, Hkv, D]
    with block_table int32 [B, max_pages] (as zl_decode_attn_gqa_paged);
    cu_seqlens_k gives the cache lengths."""
    dev, B, out, lse = _varlen_common(q, cu_seqlens_q, cu_seqlens_k, q.shape[2], out, lse, return_lse)
    _need(k_pages, "k_pages", q.dtype, 4, dev)
    _need(v_pages, "v_pages", q.dtype, 4, dev)
    table, max_pages = _paging_args(block_table, dev)
    Tq, Hq, D = q.shape
    _, page_size, Hkv, Dk = k_pages.shape
    if Dk != D or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages / v_pages must be [pages, page_size, Hkv, head_dim] like q")
    if block_table.shape[0] != B:
        raise ValueError("block_table must have batch rows")
    st = library().zl_attn_prefill_gqa_paged(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), table, max_pages, int(page_size), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), B, Tq, Hq, Hkv, D, int(max_seqlen_k), float(softmax_scale), int(bool(causal)),
        _DTYPE[q.dtype], _ptr(out), _ptr(lse), _stream(stream, dev))
    _check(st, "zl_attn_prefill_gqa_paged")
    return (out, lse) if lse is not None else out


def zl_attn_varlen_mla(q, kv_cache, cu_seqlens_q, cu_seqlens_k, max_seqlen_k: int, softmax_scale: float,
                       causal: bool = True, kv_lora_rank: int = 512, rope_dim: int = 64, out=None, lse=None,
                       workspace=None, num_workers: int = 0, stream=None, return_lse: bool = False,
                       phases: int = 3):
    """zl_attn_varlen_gqa for absorbed MLA: q [total_q, H, rank+rope], kv_cache
    [T, rank+rope] (V = its first kv_lora_rank columns); out [total_q, H, rank]."""
    dev, B, out, lse = _varlen_common(q, cu_seqlens_q, cu_seqlens_k, kv_lora_rank, out, lse, return_lse)
    _need(kv_cache, "kv_cache", q.dtype, 2, dev)
    Tq, H, Dk = q.shape
    if Dk != kv_lora_rank + rope_dim or kv_cache.shape[1] != Dk:
        raise ValueError("q and kv_cache rows must be kv_lora_rank + rope_dim wide")
    nbytes = zl_decode_attn_mla_workspace_size(B, H, kv_lora_rank, rope_dim, max_seqlen_k, q.dtype,
                                               num_workers)
    if workspace is None:
        workspace = new_workspace(nbytes, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = library().zl_attn_varlen_mla_ex(
        _ptr(q), _ptr(kv_cache), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Tq, H, kv_lora_rank, rope_dim,
        int(max_seqlen_k), float(softmax_scale), int(bool(causal)), _DTYPE[q.dtype], _ptr(out), _ptr(lse),
        int(num_workers), int(phases), _ptr(workspace), workspace.numel(), _stream(stream, dev))
    _check(st, "zl_attn_varlen_mla")
    return (out, lse) if lse is not None else out


def zl_attn_varlen_gqa_paged(q, k_pages, v_pages, block_table, cu_seqlens_q, cu_seqlens_k, max_seqlen_k: int,
                             softmax_scale: float, causal: bool = True, out=None, lse=None, workspace=None,
                             num_workers: int = 0, stream=None, return_lse: bool = False, phases: int = 3):
    """zl_attn_varlen_gqa over paged caches k_pages/v_pages [pages, page_size, Hkv, D]
    with block_table int32 [B, max_pages] (as zl_decode_attn_gqa_paged);
    cu_seqlens_k gives the cache lengths."""
    dev, B, out, lse = _varlen_common(q, cu_seqlens_q, cu_seqlens_k, q.shape[2], out, lse, return_lse)
    _need(k_pages, "k_pages", q.dtype, 4, dev)
    _need(v_pages, "v_pages", q.dtype, 4, dev)
    table, max_pages = _paging_args(block_table, dev)
    Tq, Hq, D = q.shape
    _, page_size, Hkv, Dk = k_pages.shape
    if Dk != D or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages / v_pages must be [pages, page_size, Hkv, head_dim] like q")
    if block_table.shape[0] != B:
        raise ValueError("block_table must have batch rows")
    nbytes = zl_decode_attn_workspace_size(B, Hq, Hkv, D, max_seqlen_k, q.dtype, num_workers)
    if workspace is None:
        workspace = new_workspace(nbytes, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = library().zl_attn_varlen_gqa_paged_ex(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), table, max_pages, int(page_size), _ptr(cu_seqlens_q),
        _ptr(cu_seqlens_k), B, Tq, Hq, Hkv, D, int(max_seqlen_k), float(softmax_scale), int(bool(causal)),
        _DTYPE[q.dtype], _ptr(out), _ptr(lse), int(num_workers), int(phases), _ptr(workspace), workspace.numel(),
        _stream(stream, dev))
    _check(st, "zl_attn_varlen_gqa_paged")
    return (out, lse) if lse is not None else out


def zl_attn_varlen_mla_paged(q, kv_pages, block_table, cu_seqlens_q, cu_seqlens_k, max_seqlen_k: int,
                             softmax_scale: float, causal: bool = True, kv_lora_rank: int = 512,
                             rope_dim: int = 64, out=None, lse=None, workspace=None, num_workers: int = 0,
                             stream=None, return_lse: bool = False, phases: int = 3):
    """zl_attn_varlen_mla over a paged latent pool kv_pages [pages, page_size, rank+rope]."""
    dev, B, out, lse = _varlen_common(q, cu_seqlens_q, cu_seqlens_k, kv_lora_rank, out, lse, return_lse)
    _need(kv_pages, "kv_pages", q.dtype, 3, dev)
    table, max_pages = _paging_args(block_table, dev)
    Tq, H, Dk = q.shape
    _, page_size, Dc = kv_pages.shape
    if Dk != kv_lora_rank + rope_dim or Dc != Dk:
        raise ValueError("q and kv_pages rows must be kv_lora_rank + rope_dim wide")
    if block_table.shape[0] != B:
        raise ValueError("block_table must have batch rows")
    nbytes = zl_decode_attn_mla_workspace_size(B, H, kv_lora_rank, rope_dim, max_seqlen_k, q.dtype,
                                               num_workers)
    if workspace is None:
        workspace = new_workspace(nbytes, dev)
    _need(workspace, "workspace", torch.uint8, 1, dev)
    st = library().zl_attn_varlen_mla_paged_ex(
        _ptr(q), _ptr(kv_pages), table, max_pages, int(page_size), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Tq,
        H, kv_lora_rank, rope_dim, int(max_seqlen_k), float(softmax_scale), int(bool(causal)), _DTYPE[q.dtype],
        _ptr(out), _ptr(lse), int(num_workers), int(phases), _ptr(workspace), workspace.numel(),
        _stream(stream, dev))
    _check(st, "zl_attn_varlen_mla_paged")
    return (out, lse) if lse is not None else out


def zl_attn_combine(partial_out, partial_lse, out_dtype: torch.dtype = torch.bfloat16, out=None,
                    lse=None, stream=None, return_lse: bool = False):
    """Merge split results: partial_out [S, B, H, Dv] fp32 (normalised),
    partial_lse [S, B, H] fp32 (natural log, -inf = empty) -> out [B, H, Dv]."""
    _need(partial_out, "partial_out", torch.float32, 4)
    dev = partial_out.device
    _need(partial_lse, "partial_lse", torch.float32, 3, dev)
    S, B, H, Dv = partial_out.shape
    if tuple(partial_lse.shape) != (S, B, H):
        raise ValueError("partial_lse must be [S, B, H]")
    if out is None:
        out = torch.empty(B, H, Dv, dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, 3, dev)
    if lse is None and return_lse:
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2, dev)
    st = library().zl_attn_combine(_ptr(partial_out), _ptr(partial_lse), S, B, H, Dv,
                                   _DTYPE[out_dtype], _ptr(out), _ptr(lse), _stream(stream, dev))
    _check(st, "zl_attn_combine")
    return (out, lse) if lse is not None else out


# --------------------------------------------------------- INT8 payload codec
def _codec_nchunks(n: int, chunk: int) -> int:
    return (n + chunk - 1) // chunk


def zl_int8_quantize(x, chunk: int = 512, codes=None, scales=None, stream=None):
    """Per-chunk INT8 codes of a 16-bit payload x (any shape, contiguous):
    returns (codes int8 [x.numel()], scales fp32 [ceil(numel / chunk)])."""
    _need(x, "x")
    if x.dtype not in _DTYPE:
        raise ValueError("x must be float16 or bfloat16")
    dev, n = x.device, x.numel()
    if codes is None:
        codes = torch.empty(n, dtype=torch.int8, device=dev)
    if scales is None:
        scales = torch.empty(_codec_nchunks(n, chunk), dtype=torch.float32, device=dev)
    _need(codes, "codes", torch.int8, 1, dev)
    _need(scales, "scales", torch.float32, 1, dev)
    if codes.numel() != n or scales.numel() < _codec_nchunks(n, chunk):
        raise ValueError("codes must have x.numel() entries and scales one per chunk")
    st = library().zl_int8_quantize(_ptr(x), _DTYPE[x.dtype], n, int(chunk), _ptr(codes), _ptr(scales),
                                    _stream(stream, dev))
    _check(st, "zl_int8_quantize")
    return codes, scales


def zl_int8_dequantize(codes, scales, dtype: torch.dtype = torch.float16, chunk: int = 512, out=None, stream=None):
    """Values code * scale rounded to dtype: returns out [codes.numel()]."""
    _need(codes, "codes", torch.int8, 1)
    dev, n = codes.device, codes.numel()
    _need(scales, "scales", torch.float32, 1, dev)
    if dtype not in _DTYPE:
        raise ValueError("dtype must be float16 or bfloat16")
    if out is None:
        out = torch.empty(n, dtype=dtype, device=dev)
    _need(out, "out", dtype, 1, dev)
    if out.numel() != n or scales.numel() < _codec_nchunks(n, chunk):
        raise ValueError("out must have codes.numel() entries and scales one per chunk")
    st = library().zl_int8_dequantize(_ptr(codes), _ptr(scales), n, int(chunk), _DTYPE[dtype], _ptr(out),
                                      _stream(stream, dev))
    _check(st, "zl_int8_dequantize")
    return out


def zl_int8_reduce_step(codes_in, scales_in, local, chunk: int = 512, code_out: bool = True,
                        write_sum: bool = True, codes_out=None, scales_out=None, sum_out=None, stream=None):
    """One ring-all-reduce hop: y = code_in * scale_in + local (fp32); returns
    (codes_out, scales_out, sum_out) with the parts not asked for as None."""
    _need(local, "local")
    if local.dtype not in _DTYPE:
        raise ValueError("local must be float16 or bfloat16")
    dev, n = local.device, local.numel()
    _need(codes_in, "codes_in", torch.int8, 1, dev)
    _need(scales_in, "scales_in", torch.float32, 1, dev)
    if codes_in.numel() != n or scales_in.numel() < _codec_nchunks(n, chunk):
        raise ValueError("codes_in must have local.numel() entries and scales_in one per chunk")
    if code_out:
        codes_out = torch.empty(n, dtype=torch.int8, device=dev) if codes_out is None else codes_out
        scales_out = (torch.empty(_codec_nchunks(n, chunk), dtype=torch.float32, device=dev)
                      if scales_out is None else scales_out)
        _need(codes_out, "codes_out", torch.int8, 1, dev)
        _need(scales_out, "scales_out", torch.float32, 1, dev)
    else:
        codes_out = scales_out = None
    if write_sum:
        sum_out = torch.empty(n, dtype=local.dtype, device=dev) if sum_out is None else sum_out
        _need(sum_out, "sum_out", local.dtype, 1, dev)
    else:
        sum_out = None
    st = library().zl_int8_reduce_step(_ptr(codes_in), _ptr(scales_in), _ptr(local), _DTYPE[local.dtype], n,
                                       int(chunk), _ptr(codes_out), _ptr(scales_out), _ptr(sum_out),
                                       _stream(stream, dev))
    _check(st, "zl_int8_reduce_step")
    return codes_out, scales_out, sum_out


# ------------------------------------------------------------- measurement aid
def zl_hbm_read_probe(src: torch.Tensor, head_dim_k: int, workgroups: int = 0, sink=None, stream=None):
    """Stream src's bytes (whole 1 KB blocks) through LDS at the launch shape
    of the decode kernel for head_dim_k (64 / 128: GQA, 576: MLA), with no
    arithmetic.  sink: uint32-sized int32 tensor of one word per workgroup
    (allocated here when omitted).  Returns sink."""
    _need(src, "src")
    dev = src.device
    wg = workgroups or {64: 1536, 128: 768, 576: 256}.get(head_dim_k, 8)
    if sink is None:
        sink = torch.empty(wg, dtype=torch.int32, device=dev)
    _need(sink, "sink", torch.int32, 1, dev)
    if sink.numel() < wg:
        raise ValueError("sink needs one word per workgroup")
    st = library().zl_hbm_read_probe(_ptr(src), src.numel() * src.element_size(), int(head_dim_k), int(workgroups),
                                      _ptr(sink), _stream(stream, dev))
    _check(st, "zl_hbm_read_probe")
    return sink
