"""Guarded device buffers for the GPU parity tests.

Every output a test hands to the library is pre-filled so that an element the
kernels fail to write cannot pass the parity gate: `out` holds NaN and `lse`
holds +inf (the gate rejects non-finite outputs and +inf log-sum-exps).  Each
buffer, the workspace included, also sits between two 4 KB canary regions
filled with the same pattern (0xA5 bytes for the workspace); after the call the
canaries must be bitwise unchanged, so a store before or past either end of
out, lse or the workspace fails the test that caused it.
"""
from __future__ import annotations

import math

import torch

GUARD_BYTES = 4096  # keeps the guarded view 256-byte aligned


class Guarded:
    """A tensor of `shape` inside a larger allocation whose head and tail are
    canaries holding `fill` (as is the tensor itself until a kernel writes it)."""

    def __init__(self, shape, dtype, device, fill):
        esize = torch.empty((), dtype=dtype).element_size()
        self.g = GUARD_BYTES // esize
        self.n = math.prod(shape)
        self.buf = torch.full((2 * self.g + self.n,), fill, dtype=dtype, device=device)
        self.head = self.buf[: self.g].clone()
        self.tail = self.buf[self.g + self.n:].clone()
        self.t = self.buf[self.g: self.g + self.n].view(tuple(shape))

    @staticmethod
    def _bits(x):
        return x.contiguous().view(torch.uint8)

    def check(self, what: str, where: str = ""):
        assert torch.equal(self._bits(self.buf[: self.g]), self._bits(self.head)), \
            f"{where}: a store landed in the canary before {what}"
        assert torch.equal(self._bits(self.buf[self.g + self.n:]), self._bits(self.tail)), \
            f"{where}: a store landed in the canary past {what}"


class CallBuffers:
    """out [rows, heads, dv], lse [rows, heads] and (optionally) a workspace of
    ws_bytes for one library call, all guarded."""

    def __init__(self, rows, heads, dv, dtype, device, ws_bytes=None):
        self.out = Guarded((rows, heads, dv), dtype, device, float("nan"))
        self.lse = Guarded((rows, heads), torch.float32, device, float("inf"))
        self.ws = Guarded((max(int(ws_bytes), 256),), torch.uint8, device, 0xA5) if ws_bytes is not None else None

    def kwargs(self):
        kw = {"out": self.out.t, "lse": self.lse.t}
        if self.ws is not None:
            kw["workspace"] = self.ws.t
        return kw

    def check(self, where: str = ""):
        self.out.check("out", where)
        self.lse.check("lse", where)
        if self.ws is not None:
            self.ws.check("the workspace", where)
