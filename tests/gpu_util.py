"""Helpers for the GPU tests: device copies, guard bands, case banners."""
from __future__ import annotations

import sys

import numpy as np
import torch


def banner(*parts):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[gpu case]", *parts, file=sys.stderr, flush=True)


def np_(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


class Guarded:
    """A device tensor with canary bands before and after it, to catch
    out-of-bounds writes.  `.t` is the view passed to the kernel."""

    PAD = 4096  # elements on each side (>= one 16-lane row of any buffer)

    def __init__(self, shape, dtype, device="cuda", init=None):
        n = int(np.prod(shape))
        self.buf = torch.empty(n + 2 * self.PAD, dtype=dtype, device=device)
        bits = {torch.float32: torch.int32, torch.float16: torch.int16}[dtype]
        self.buf.view(bits).fill_(0x5A5A if dtype == torch.float16 else 0x5A5A5A5A)
        self.canary = self.buf[:self.PAD].clone()
        self.t = self.buf[self.PAD:self.PAD + n].view(shape)
        if init is not None:
            self.t.copy_(torch.as_tensor(init).reshape(shape).to(device=device, dtype=dtype))

    def intact(self) -> bool:
        lo = self.buf[:self.PAD]
        hi = self.buf[-self.PAD:]
        bits = torch.int32 if self.buf.dtype == torch.float32 else torch.int16
        c = self.canary.view(bits)
        return bool(torch.equal(lo.view(bits), c) and torch.equal(hi.view(bits), c))
