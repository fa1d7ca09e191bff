"""Guarded output buffers for the GPU parity tests.

Each output a kernel writes is carved from the middle of a larger device
allocation.  The output itself is pre-filled with a sentinel byte, and
GUARD bytes on either side hold a fixed, position-dependent pattern.  After
the call, ``check()`` verifies the pattern is untouched, so a write past
either end of the output fails the test.  Running the same call twice with
two different sentinels (``SENTINELS``) and comparing both results with the
oracle proves every byte was written: a byte the kernel skipped equals the
sentinel, which can match the expected value in at most one of the two runs.
"""

from __future__ import annotations

import math

import numpy as np
import torch

GUARD = 4096
SENTINELS = (0xFF, 0x5A)


def _pattern(nbytes: int) -> torch.Tensor:
    return ((torch.arange(nbytes, dtype=torch.int64) * 37 + 11) % 253).to(torch.uint8)


class Out:
    """One guarded output tensor ``t`` of the given shape and dtype."""

    def __init__(self, shape, dtype, sentinel: int = 0xFF, device: str = "cuda"):
        shape = tuple(int(v) for v in shape)
        item = torch.empty((), dtype=dtype).element_size()
        self.nbytes = math.prod(shape) * item
        body = -(-self.nbytes // 16) * 16
        total = GUARD + body + GUARD
        self.pattern = _pattern(total)
        self.buf = self.pattern.to(device)
        self.buf[GUARD:GUARD + self.nbytes].fill_(sentinel)
        self.t = self.buf[GUARD:GUARD + self.nbytes].view(dtype).view(shape)
        self.shape = shape

    def check(self, what: str = "output") -> None:
        """Both guard bands still hold their pattern (call after a sync)."""
        b = self.buf.cpu()
        lo = torch.equal(b[:GUARD], self.pattern[:GUARD])
        hi = torch.equal(b[GUARD + self.nbytes:], self.pattern[GUARD + self.nbytes:])
        assert lo and hi, f"{what}: write outside the output ({'before' if not lo else 'after'} it)"

    def host(self) -> np.ndarray:
        return self.t.cpu().numpy()


def outs(specs, sentinel: int):
    """Guarded outputs for a list of (shape, dtype) pairs."""
    return [Out(shape, dtype, sentinel) for shape, dtype in specs]


def check_all(objs, what: str) -> None:
    torch.cuda.synchronize()
    for i, o in enumerate(objs):
        o.check(f"{what} (output {i})")
