"""Helpers for the GPU parity tests: guarded device buffers and bit views."""
import sys

import numpy as np
import torch

CANARY16 = 0x5A5A
CANARY32 = 0x5A5A5A5A
GUARD = 64  # elements of guard band on each side (keeps 16-byte alignment)


def say(*a):
    """Name the case before a GPU step, flushed, so a crash still names it."""
    print("[gpu]", *a, file=sys.stderr, flush=True)


class Guarded:
    """A device tensor of n elements inside a canary-filled guard band.
    `shift` elements of extra offset make the payload start off its 16-byte
    boundary."""

    def __init__(self, n: int, dtype: torch.dtype, shift: int = 0, fill=None):
        self.n, self.dtype, self.shift = n, dtype, shift
        itype = torch.int16 if torch.empty(0, dtype=dtype).element_size() == 2 else torch.int32
        canary = CANARY16 if itype == torch.int16 else CANARY32
        self.raw = torch.full((n + 2 * GUARD + shift,), canary, dtype=itype, device="cuda")
        self.canary = canary
        self.lo = GUARD + shift
        self.t = self.raw[self.lo:self.lo + n].view(dtype)
        if fill is not None:
            self.t.copy_(fill)

    def check(self):
        raw = self.raw.cpu()
        assert (raw[:self.lo] == self.canary).all(), "guard band before the buffer was written"
        assert (raw[self.lo + self.n:] == self.canary).all(), "guard band after the buffer was written"


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a tensor (any device) as numpy uint16 / uint32."""
    t = t.detach().contiguous().cpu()
    if t.element_size() == 2:
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.view(torch.int32).numpy().view(np.uint32).copy()


def from_bits(a: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16).copy()).view(dtype).to(device)
    return torch.from_numpy(a.view(np.int32).copy()).view(dtype).to(device)
