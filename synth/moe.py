"""Seeded synthetic inputs of the expert-wave stand-in: token counts per expert, token
destinations, bf16 activations and weights.  No GEMM, rounding-of-results or scatter
arithmetic lives here."""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .inputs import f32_to_bf16_bits


@dataclass(frozen=True)
class MoeWorkload:
    """E experts on one GPU, grouped into waves; tokens per expert drawn uniformly from
    [rows_lo, rows_hi]; each token row goes to one of P destinations."""

    name: str
    E: int
    experts_per_wave: int
    d_model: int
    d_ff: int
    rows_lo: int
    rows_hi: int
    P: int
    seed: int

    @property
    def flops_per_token(self) -> float:
        return 4.0 * self.d_model * self.d_ff  # Linear-1 and Linear-2, 2 FLOP per MAC


# A DeepSeek-V3-sized expert (7168 model features, 2048 expert features), 32 experts on one
# GPU in waves of 8, ~256 token rows per expert, 8 destinations.
MOE_WORKLOADS = {
    "moe_small": MoeWorkload("moe_small", 5, 2, 256, 128, 0, 300, 3, seed=21),
    "moe_dsv3": MoeWorkload("moe_dsv3", 32, 8, 7168, 2048, 192, 320, 8, seed=22),
}


def moe_routing(w: MoeWorkload):
    """(offsets [E+1], dst_slab [T], dst_row [T], out_rows [P]): token counts per expert,
    then for every token a uniformly drawn destination and its arrival order there."""
    rng = np.random.default_rng(w.seed)
    rows = rng.integers(w.rows_lo, w.rows_hi + 1, size=w.E)
    offsets = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    T = int(offsets[-1])
    dst_slab = rng.integers(0, w.P, size=T).astype(np.int32)
    dst_row = np.zeros(T, dtype=np.int32)
    count = np.zeros(w.P, dtype=np.int64)
    for t in range(T):
        dst_row[t] = count[dst_slab[t]]
        count[dst_slab[t]] += 1
    return offsets, dst_slab, dst_row, count.astype(np.int32)


def moe_tensors(w: MoeWorkload, T: int):
    """bf16 bits of x [T, d_model] ~ N(0, 1), w1 [E, d_ff, d_model] ~ N(0, 1/d_model),
    w2 [E, d_model, d_ff] ~ N(0, 1/d_ff) (so both products have O(1) outputs)."""
    rng = np.random.default_rng(w.seed + 1)
    x = rng.standard_normal((T, w.d_model), dtype=np.float32)
    w1 = rng.standard_normal((w.E, w.d_ff, w.d_model), dtype=np.float32) / np.float32(np.sqrt(w.d_model))
    w2 = rng.standard_normal((w.E, w.d_model, w.d_ff), dtype=np.float32) / np.float32(np.sqrt(w.d_ff))
    return f32_to_bf16_bits(x), f32_to_bf16_bits(w1), f32_to_bf16_bits(w2)
