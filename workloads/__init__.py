"""Seeded synthetic decode-attention workloads.

This module only draws inputs: shapes, lengths and 16-bit Q/K/V (or latent)
values from a seeded torch CPU generator.  It holds none of the attention
arithmetic.  Both the GPU path and the fp64 oracle consume exactly the bytes
it returns.

Recipe (the pages measure only end-to-end serving on trained models, so these
stand in for the workload; no dataset or weights are involved):
  * generator: torch.Generator('cpu').manual_seed(seed); seed defaults to the
    configuration number;
  * draw order: lengths (torch.randint(lo, hi + 1), inclusive), then Q, then
    K, then V (MLA: lengths, Q, latent), each as float32 torch.randn, then
    rounded once (round-to-nearest-even) to the 16-bit dtype;
  * fixed length lists are used in their listed order;
  * layout: Q [B, Hq, Dk]; K, V [T, Hkv, D] packed in sequence order;
    latent [T, Dk]; cu_seqlens int32 [B+1] with cu[0] = 0.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional, Sequence, Tuple, Union

import numpy as np
import torch

Lens = Union[Tuple[int, ...], Tuple[str, int, int]]


@dataclasses.dataclass(frozen=True)
class Spec:
    name: str
    kind: str            # "gqa" or "mla"
    batch: int
    num_q_heads: int
    num_kv_heads: int    # 1 for MLA (one shared latent)
    head_dim_k: int
    head_dim_v: int
    lens: Lens           # explicit tuple, or ("uniform", lo, hi) inclusive
    dtype: str           # "f16" or "bf16"
    scale: float         # already rounded to float32
    seed: int

    @property
    def torch_dtype(self):
        return torch.float16 if self.dtype == "f16" else torch.bfloat16

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _f32(x: float) -> float:
    return float(np.float32(x))


WORKLOADS = {
    1: Spec("tiny-gqa-b4-h8kv2-d64", "gqa", 4, 8, 2, 64, 64, (17, 64, 100, 128), "f16",
            _f32(1.0 / math.sqrt(64)), 1),
    2: Spec("llama3-8b-decode-b32-h32kv8-d128", "gqa", 32, 32, 8, 128, 128, ("uniform", 512, 4096),
            "f16", _f32(1.0 / math.sqrt(128)), 2),
    3: Spec("70b-tp8-share-b64-h8kv1-d128", "gqa", 64, 8, 1, 128, 128, ("uniform", 1024, 8192),
            "f16", _f32(1.0 / math.sqrt(128)), 3),
    4: Spec("long-ctx-b8-h32kv8-d128-L32768", "gqa", 8, 32, 8, 128, 128, (32768,) * 8, "bf16",
            _f32(1.0 / math.sqrt(128)), 4),
    5: Spec("mla-absorbed-b32-h16-r512-rope64", "mla", 32, 16, 1, 576, 512, ("uniform", 1024, 8192),
            "bf16", _f32(1.0 / math.sqrt(192)), 5),
}


@dataclasses.dataclass
class Inputs:
    spec: Spec
    lens: np.ndarray                  # int64 [B]
    cu_seqlens: torch.Tensor          # int32 [B+1] (CPU)
    q: torch.Tensor                   # 16-bit [B, Hq, Dk] (CPU)
    k: Optional[torch.Tensor] = None  # 16-bit [T, Hkv, D]
    v: Optional[torch.Tensor] = None  # 16-bit [T, Hkv, D]
    latent: Optional[torch.Tensor] = None  # 16-bit [T, Dk] (MLA)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self) -> int:
        return int(self.lens.max()) if len(self.lens) else 0

    def kv_bytes(self) -> int:
        """Bytes of K and V (or of the latent rows) that one decode step must read once."""
        if self.latent is not None:
            return self.latent.numel() * 2
        return (self.k.numel() + self.v.numel()) * 2

    def bits(self, name: str) -> np.ndarray:
        """Raw uint16 patterns of a 16-bit tensor, as numpy (for the oracle)."""
        t = getattr(self, name)
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    def sha256(self) -> str:
        h = hashlib.sha256()
        h.update(self.cu_seqlens.numpy().tobytes())
        for name in ("q", "k", "v", "latent"):
            t = getattr(self, name)
            if t is not None:
                h.update(t.contiguous().view(torch.int16).numpy().tobytes())
        return h.hexdigest()


def draw_lens(spec: Spec, gen: torch.Generator) -> np.ndarray:
    if isinstance(spec.lens[0], str):
        _, lo, hi = spec.lens
        return torch.randint(lo, hi + 1, (spec.batch,), generator=gen).numpy().astype(np.int64)
    if len(spec.lens) != spec.batch:
        raise ValueError("explicit length list must have one entry per sequence")
    return np.asarray(spec.lens, dtype=np.int64)


def cu_from_lens(lens: Sequence[int]) -> torch.Tensor:
    cu = np.zeros(len(lens) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lens, dtype=np.int64))
    if cu[-1] > np.iinfo(np.int32).max:
        raise ValueError("total tokens exceed int32")
    return torch.from_numpy(cu.astype(np.int32))


def make_inputs(spec: Spec, seed: Optional[int] = None, lens: Optional[Sequence[int]] = None,
                q_mult: float = 1.0) -> Inputs:
    """Draw one batch for `spec`.

    seed   : overrides spec.seed.
    lens   : overrides the length draw (edge cases: zeros, ragged tails ...);
             the generator still draws nothing for lengths in that case.
    q_mult : multiplies Q before rounding ("peaked" scores for stress tests).
    """
    gen = torch.Generator("cpu")
    gen.manual_seed(spec.seed if seed is None else seed)
    if lens is None:
        lens_np = draw_lens(spec, gen)
    else:
        lens_np = np.asarray(lens, dtype=np.int64)
        if len(lens_np) != spec.batch:
            raise ValueError("lens must have batch entries")
    cu = cu_from_lens(lens_np)
    T = int(cu[-1])
    dt = spec.torch_dtype
    q = torch.randn(spec.batch, spec.num_q_heads, spec.head_dim_k, generator=gen)
    if q_mult != 1.0:
        q = q * q_mult
    q = q.to(dt)
    if spec.kind == "mla":
        latent = torch.randn(T, spec.head_dim_k, generator=gen).to(dt)
        return Inputs(spec, lens_np, cu, q, latent=latent)
    k = torch.randn(T, spec.num_kv_heads, spec.head_dim_k, generator=gen).to(dt)
    v = torch.randn(T, spec.num_kv_heads, spec.head_dim_v, generator=gen).to(dt)
    return Inputs(spec, lens_np, cu, q, k=k, v=v)


def with_shape(spec: Spec, **changes) -> Spec:
    """A copy of `spec` with some fields replaced (for edge-case tests)."""
    return dataclasses.replace(spec, **changes)


@dataclasses.dataclass
class PagedInputs:
    """The caches of an Inputs batch laid out in fixed-size pages, as a serving
    engine's page pool holds them: pages of each sequence are placed at
    seeded random pool positions (pool pages that no sequence uses stay filled
    with other random data), and block_table lists each sequence's pages in
    order.  Token i of sequence b is row i % page_size of page
    block_table[b, i // page_size]."""
    page_size: int
    block_table: torch.Tensor          # int32 [B, max_pages]
    k_pages: Optional[torch.Tensor] = None   # [pages, page_size, Hkv, D]
    v_pages: Optional[torch.Tensor] = None
    kv_pages: Optional[torch.Tensor] = None  # [pages, page_size, Dk] (MLA)

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])


def make_paged(x: Inputs, page_size: int, seed: int = 0, spare_pages: int = 3) -> PagedInputs:
    """Scatter the packed caches of `x` into a shuffled page pool (data layout
    only).  Unused table entries and spare pool pages hold values that a
    correct kernel never reads."""
    gen = torch.Generator("cpu")
    gen.manual_seed(1000 + seed)
    lens = [int(v) for v in x.lens]
    cu = x.cu_seqlens.numpy().astype(np.int64)
    npages_seq = [(L + page_size - 1) // page_size for L in lens]
    max_pages = max(1, max(npages_seq) if npages_seq else 1)
    total = sum(npages_seq) + spare_pages
    perm = torch.randperm(total, generator=gen).numpy()
    table = np.full((len(lens), max_pages), total - 1, dtype=np.int32)  # unused entries: some valid id
    nxt = 0
    for b, npg in enumerate(npages_seq):
        for i in range(npg):
            table[b, i] = perm[nxt]
            nxt += 1
    rows_of = []  # (pool page, packed token range) for the scatter
    for b, npg in enumerate(npages_seq):
        for i in range(npg):
            t0 = cu[b] + i * page_size
            t1 = min(cu[b + 1], t0 + page_size)
            rows_of.append((table[b, i], t0, t1))

    def scatter(src: torch.Tensor) -> torch.Tensor:
        pool = torch.randn((total, page_size) + tuple(src.shape[1:]), generator=gen).to(src.dtype)
        for page, t0, t1 in rows_of:
            pool[page, : t1 - t0] = src[t0:t1]
        return pool

    bt = torch.from_numpy(table)
    if x.latent is not None:
        return PagedInputs(page_size, bt, kv_pages=scatter(x.latent))
    return PagedInputs(page_size, bt, k_pages=scatter(x.k), v_pages=scatter(x.v))


@dataclasses.dataclass
class VarlenQuery:
    """Several new query tokens per sequence over the caches of an Inputs
    batch: sequence b's q_lens[b] new tokens are rows cu_q[b] .. cu_q[b+1]-1
    of q, and their keys/values are the last q_lens[b] rows of its cache."""
    q_lens: np.ndarray
    cu_q: torch.Tensor      # int32 [B + 1]
    q: torch.Tensor         # [total_q, Hq, Dk]

    @property
    def total_q(self) -> int:
        return int(self.cu_q[-1])


def make_varlen_query(x: Inputs, q_lens, seed: int = 0, q_mult: float = 1.0) -> VarlenQuery:
    """Seeded N(0,1) query rows (rounded once to the batch's dtype) for
    q_lens[b] new tokens of each sequence.  q_lens may exceed a cache length
    (the first tokens then see no key under the causal mask)."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    if len(q_lens) != x.spec.batch:
        raise ValueError("q_lens must have batch entries")
    gen = torch.Generator("cpu")
    gen.manual_seed(2000 + seed)
    cu_q = cu_from_lens(q_lens)
    q = torch.randn(int(cu_q[-1]), x.spec.num_q_heads, x.spec.head_dim_k, generator=gen)
    if q_mult != 1.0:
        q = q * q_mult
    return VarlenQuery(q_lens, cu_q, q.to(x.spec.torch_dtype))


@dataclasses.dataclass
class RawCache:
    """A cache whose cu_seqlens need not be a valid prefix sum: cu_raw may
    start above 0, decrease, or give lengths above max_seqlen.  Sequence b
    owns L_b = clamp(cu_raw[b+1] - cu_raw[b], 0, max_seqlen) rows from row
    cu_raw[b] of the buffers.  `clamped` holds the same rows gathered into a
    valid packed batch (lengths L_b, the same Q), the batch that such a call
    means."""
    cu_raw: torch.Tensor                  # int32 [B+1]
    max_seqlen: int
    k: Optional[torch.Tensor] = None      # [rows, Hkv, D]
    v: Optional[torch.Tensor] = None
    latent: Optional[torch.Tensor] = None  # [rows, Dk]
    clamped: Optional[Inputs] = None


def make_raw_cache(spec: Spec, cu_raw: Sequence[int], max_seqlen: int, seed: int) -> RawCache:
    """Seeded buffers of max(cu_raw) rows (draw order Q, then K and V, or the
    latent, as make_inputs) addressed by an unchecked cu_raw."""
    cu = np.asarray(cu_raw, dtype=np.int64)
    if len(cu) != spec.batch + 1 or cu.min() < 0 or cu.max() > np.iinfo(np.int32).max:
        raise ValueError("cu_raw must have batch + 1 non-negative int32 entries")
    lens = np.clip(np.diff(cu), 0, max_seqlen)
    rows = int(cu.max())
    gen = torch.Generator("cpu")
    gen.manual_seed(seed)
    dt = spec.torch_dtype
    q = torch.randn(spec.batch, spec.num_q_heads, spec.head_dim_k, generator=gen).to(dt)
    idx = torch.from_numpy(np.concatenate([np.arange(cu[b], cu[b] + lens[b]) for b in range(spec.batch)]
                                          + [np.zeros(0, np.int64)]))
    cspec = with_shape(spec, lens=tuple(int(v) for v in lens))
    cu_t = torch.from_numpy(cu.astype(np.int32))
    if spec.kind == "mla":
        latent = torch.randn(rows, spec.head_dim_k, generator=gen).to(dt)
        x = Inputs(cspec, lens, cu_from_lens(lens), q, latent=latent[idx])
        return RawCache(cu_t, max_seqlen, latent=latent, clamped=x)
    k = torch.randn(rows, spec.num_kv_heads, spec.head_dim_k, generator=gen).to(dt)
    v = torch.randn(rows, spec.num_kv_heads, spec.head_dim_v, generator=gen).to(dt)
    x = Inputs(cspec, lens, cu_from_lens(lens), q, k=k[idx], v=v[idx])
    return RawCache(cu_t, max_seqlen, k=k, v=v, clamped=x)
