"""Device-buffer helpers for the GPU tests: bf16 uploads, guarded slab buffers, downloads."""

import numpy as np
import torch

NAN_BF16 = 0x7FC0      # sentinel prefilled into every slab element
CANARY = 0x5EED        # guard-zone pattern around each slab
GUARD = 32             # guard elements (64 bytes) before, between and after slabs


_SPLIT_WS = None


def split_ws() -> torch.Tensor:
    """One zero-filled split workspace shared by the GPU tests, large enough for every plan
    (16 KiB of counters plus 128 MiB of partials): every call leaves the counters it used at zero, so
    calls of any shape may reuse it one after another on one stream."""
    global _SPLIT_WS
    if _SPLIT_WS is None:
        _SPLIT_WS = torch.zeros((129 << 20,), dtype=torch.uint8, device="cuda")
    return _SPLIT_WS


def to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def to_host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class GuardedSlabs:
    """P slabs [B, S/P, H, D] carved from one buffer with canary guards around each."""

    def __init__(self, P, B, S_P, H, D):
        self.shape = (B, S_P, H, D)
        self.n = B * S_P * H * D
        self.P = P
        total = GUARD + P * (self.n + GUARD)
        host = np.full(total, NAN_BF16, dtype=np.uint16)
        for p in range(P + 1):
            g0 = p * (self.n + GUARD)
            host[g0:g0 + GUARD] = CANARY
        self.buf = to_dev(host)
        self.views = [self.buf[GUARD + p * (self.n + GUARD):GUARD + p * (self.n + GUARD) + self.n].view(*self.shape)
                      for p in range(P)]

    def slabs_host(self) -> np.ndarray:
        h = to_host(self.buf)
        return np.stack([h[GUARD + p * (self.n + GUARD):GUARD + p * (self.n + GUARD) + self.n].reshape(self.shape)
                         for p in range(self.P)])

    def guards_intact(self) -> bool:
        h = to_host(self.buf)
        return all(np.all(h[p * (self.n + GUARD):p * (self.n + GUARD) + GUARD] == CANARY) for p in range(self.P + 1))
