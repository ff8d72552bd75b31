"""Seeded synthetic DiT-shaped attention inputs (bf16 bit patterns, BSHD layout).

The pages describe Ulysses sequence-parallel attention inside distributed DiT inference
(X-Stage explainer, gist.science paper 2607.23264, "Contributions", FlashAttention-A2A
item) but ship no activations; these tensors stand in for one GPU's share at the shapes of
FLUX-like image DiTs and a video DiT.

Recipe (all draws from ``numpy.random.default_rng(seed)``, PCG64):

* ``q, k, v``: ``standard_normal((B, S, H, D), dtype=float32)`` drawn in that order.
* FLUX-1024 share: ``k *= 0.5`` (exact in fp32 and bf16).
* Video share: per-head rank-1 bias on K, ``k[:, :, h, :] += amp * a_h[:, None] * u_h[None, :]``
  with ``a = standard_normal((H, S))`` (per-key coefficient) and ``u = standard_normal((H, D))``
  (the shared vector), drawn after v, computed in fp32, amp = 0.3.  A bias identical for
  every key would shift each logit of a row by the same amount and leave the softmax
  unchanged; scaling the shared vector per key is what makes some rows peaked.
* Every tensor is then cast fp32 -> bf16 with round-to-nearest-even.
"""

from __future__ import annotations

import functools
import math
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One GPU's share of a Ulysses attention layer: full-S attention over H local heads."""

    name: str
    B: int
    S: int
    H: int  # local heads (H_total / P)
    D: int
    P: int  # number of destination slabs (Ulysses degree)
    seed: int
    k_scale: float = 1.0
    k_rank1_amp: float = 0.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def flops(self) -> float:
        """Algorithmic FLOP of non-causal attention: QK^T plus PV, 4*B*S^2*D*H."""
        return 4.0 * self.B * self.S * self.S * self.D * self.H

    @property
    def out_bytes(self) -> int:
        return self.B * self.S * self.H * self.D * 2

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 256, 2, 64, 2, seed=0),
    "flux1024": Workload("flux1024", 1, 4608, 3, 128, 8, seed=1, k_scale=0.5),
    "flux2048": Workload("flux2048", 1, 16896, 3, 128, 8, seed=2),
    "video": Workload("video", 1, 32760, 5, 128, 8, seed=3, k_rank1_amp=0.3),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even; NaN stays NaN."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        rounded[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return rounded


def make_inputs(w: Workload):
    """Return (q, k, v) as uint16 bf16 bit arrays of shape [B, S, H, D]."""
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.S, w.H, w.D)
    q = rng.standard_normal(shape, dtype=np.float32)
    k = rng.standard_normal(shape, dtype=np.float32)
    v = rng.standard_normal(shape, dtype=np.float32)
    if w.k_scale != 1.0:
        k *= np.float32(w.k_scale)
    if w.k_rank1_amp != 0.0:
        a = rng.standard_normal((w.H, w.S), dtype=np.float32)
        u = rng.standard_normal((w.H, w.D), dtype=np.float32)
        amp = np.float32(w.k_rank1_amp)
        for h in range(w.H):
            k[:, :, h, :] += amp * a[h][:, None] * u[h][None, :]
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def _max_offdiag_dot(codes: np.ndarray, block: int = 2048) -> float:
    """Largest c_i . c_j over i != j for +-1 code rows (exact: integer sums below 2^24)."""
    S = codes.shape[0]
    if S < 2:
        return -math.inf
    c = codes.astype(np.float32)
    best = -math.inf
    for i0 in range(0, S, block):
        g = c[i0:i0 + block] @ c.T
        idx = np.arange(g.shape[0])
        g[idx, i0 + idx] = -np.inf
        best = max(best, float(g.max()))
    return best


@functools.lru_cache(maxsize=8)
def _probe_codes(S: int, D: int, scale: float, seed: int, margin: float):
    rng = np.random.default_rng(seed)
    while True:
        codes = (rng.integers(0, 2, size=(S, D), dtype=np.int8) * 2 - 1).astype(np.int8)
        gap = scale * 64.0 * (D - _max_offdiag_dot(codes))
        if gap >= margin:
            return codes


def make_placement_probe(B: int, S: int, H: int, D: int, scale: float, seed: int = 7, margin: float = 120.0):
    """Structured inputs whose exact attention output is V itself, with V carrying tags.

    q = k = 8 * (c_s * sigma_{b,h}) with random +-1 codes c_s (redrawn until every
    off-diagonal logit sits at least ``margin`` below the diagonal one) and a per-(b, h)
    random sign vector sigma, so a query only matches its own key within its own head.
    Every logit is an exact integer times ``scale``; all off-diagonal weights fall below
    exp(-margin), which is zero in fp32, so O[b, s, h, :] = V[b, s, h, :] exactly.

    V holds exact bf16 integers: V[...,0] = s mod 256, V[...,1] = s div 256, V[...,2] = h,
    V[...,3] = b, the rest a mix of (s, d, h, b) folded into [-128, 127].
    Returns (q, k, v) uint16 bf16 bit arrays [B, S, H, D].
    """
    if D < 4:
        raise ValueError("placement probe needs D >= 4 for its tags")
    codes = _probe_codes(S, D, float(scale), seed, float(margin))
    rng = np.random.default_rng(seed + 1)
    sigma = (rng.integers(0, 2, size=(B, H, D), dtype=np.int8) * 2 - 1).astype(np.float32)
    qk = 8.0 * codes.astype(np.float32)[None, :, None, :] * sigma[:, None, :, :]  # [B,S,H,D]
    s_idx = np.arange(S)[None, :, None, None]
    h_idx = np.arange(H)[None, None, :, None]
    b_idx = np.arange(B)[:, None, None, None]
    d_idx = np.arange(D)[None, None, None, :]
    v = ((s_idx * 7 + d_idx * 13 + h_idx * 31 + b_idx * 17) % 256 - 128).astype(np.float32)
    v = np.broadcast_to(v, (B, S, H, D)).copy()
    v[..., 0] = (np.arange(S) % 256)[None, :, None]
    v[..., 1] = (np.arange(S) // 256)[None, :, None]
    v[..., 2] = np.arange(H)[None, None, :]
    v[..., 3] = np.arange(B)[:, None, None]
    qb = f32_to_bf16_bits(qk)
    return qb, qb.copy(), f32_to_bf16_bits(v)


def make_placement_probe_torch(B: int, S: int, H: int, D: int, scale: float, device, seed: int = 7,
                               margin: float = 120.0):
    """make_placement_probe's (q, k, v), bit for bit, assembled with torch on ``device`` and
    returned as bf16 tensors: the same codes and sign vectors (drawn on the host), the same
    broadcast products and tags, cast fp32 -> bf16 with round-to-nearest-even.  For tensors
    of billions of elements, whose host-side assembly would take minutes."""
    import torch

    if D < 4:
        raise ValueError("placement probe needs D >= 4 for its tags")
    codes = _probe_codes(S, D, float(scale), seed, float(margin))
    rng = np.random.default_rng(seed + 1)
    sigma = (rng.integers(0, 2, size=(B, H, D), dtype=np.int8) * 2 - 1).astype(np.float32)
    c = torch.from_numpy(codes.astype(np.float32)).to(device)
    sg = torch.from_numpy(sigma).to(device)
    q = (8.0 * c[None, :, None, :] * sg[:, None, :, :]).to(torch.bfloat16)
    i32 = dict(device=device, dtype=torch.int32)
    s_idx = torch.arange(S, **i32)[None, :, None, None]
    h_idx = torch.arange(H, **i32)[None, None, :, None]
    b_idx = torch.arange(B, **i32)[:, None, None, None]
    d_idx = torch.arange(D, **i32)[None, None, None, :]
    v = ((s_idx * 7 + d_idx * 13 + h_idx * 31 + b_idx * 17) % 256 - 128).to(torch.float32)
    v[..., 0] = (torch.arange(S, **i32) % 256).to(torch.float32)[None, :, None]
    v[..., 1] = (torch.arange(S, **i32) // 256).to(torch.float32)[None, :, None]
    v[..., 2] = torch.arange(H, **i32).to(torch.float32)[None, None, :]
    v[..., 3] = torch.arange(B, **i32).to(torch.float32)[:, None, None]
    v = v.to(torch.bfloat16)
    return q, q.clone(), v
