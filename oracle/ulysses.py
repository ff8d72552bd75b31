"""The two Ulysses all-to-alls around attention on one rank, written as plain loops (test
infrastructure).

X-Stage explainer (gist.science, arXiv 2607.23264), "Contributions", FlashAttention-A2A
item: in Ulysses-style sequence parallelism each of the P ranks holds one contiguous
sequence shard of every head before attention, and after attention the output is sent back
sequence-sharded; the fused kernel issues the post-attention all-to-all from its epilogue.
The pages do not spell out the pre-attention all-to-all or the receive-buffer layout;
readings used here (listed in the design notes):

* rank r computes attention for the heads [h0, h0 + H_local) (h0 = r * H_local in a
  Ulysses group of P ranks over H = P * H_local heads);
* before attention, rank p's shard of a tensor is [B, S/P, H, D] (its S/P sequence rows,
  all H heads); the rank gathers, from every shard p, the rows of its own heads
  (sequence -> heads all-to-all);
* after attention, destination p's receive buffer is [B, S/P, H_dst, D] (its S/P rows,
  all heads); the rank writes the head columns [h0, h0 + H_local) of every destination
  (heads -> sequence all-to-all) and nothing else.
"""

from __future__ import annotations

import numpy as np

from .attention import attention_fp64


def pre_gather(shards, h0: int, H_local: int) -> np.ndarray:
    """Sequence -> heads all-to-all: x[b, p*S/P + r, h, d] = shards[p][b, r, h0 + h, d].

    ``shards``: P arrays [B, S/P, H, D].  Returns [B, S, H_local, D]; written source by
    source, row by row."""
    P = len(shards)
    B, sp, H, D = shards[0].shape
    if not 0 <= h0 <= H - H_local:
        raise ValueError("head range outside the shards")
    x = np.empty((B, P * sp, H_local, D), dtype=shards[0].dtype)
    for p in range(P):
        for b in range(B):
            for r in range(sp):
                for h in range(H_local):
                    x[b, p * sp + r, h, :] = shards[p][b, r, h0 + h, :]
    return x


def scatter_heads(o: np.ndarray, dst, h0: int) -> None:
    """Heads -> sequence all-to-all into full-head receive buffers, in place:
    dst[p][b, r, h0 + h, d] = o[b, p*S/P + r, h, d]; every other element of dst is left as is.

    ``o``: [B, S, H_local, D]; ``dst``: P arrays [B, S/P, H_dst, D]."""
    B, S, H_local, D = o.shape
    P = len(dst)
    if S % P != 0:
        raise ValueError("Ulysses shards need S divisible by P")
    sp = S // P
    if not 0 <= h0 <= dst[0].shape[2] - H_local:
        raise ValueError("head range outside the receive buffers")
    for p in range(P):
        for b in range(B):
            for r in range(sp):
                for h in range(H_local):
                    dst[p][b, r, h0 + h, :] = o[b, p * sp + r, h, :]


def ulysses_attention(q_shards, k_shards, v_shards, scale: float, h0: int, H_local: int, dst, rows=None):
    """One rank's attention layer with both all-to-alls: gather its heads from the sequence
    shards, attention in float64 (``attention_fp64``), scatter into the receive buffers.
    With ``rows`` (query rows), only those rows are computed and scattered."""
    q = pre_gather(q_shards, h0, H_local)
    k = pre_gather(k_shards, h0, H_local)
    v = pre_gather(v_shards, h0, H_local)
    o = attention_fp64(q, k, v, scale, rows=rows)
    if rows is None:
        scatter_heads(o, dst, h0)
        return
    P = len(dst)
    sp = q.shape[1] // P
    for i, s in enumerate(np.asarray(rows)):
        p, r = int(s) // sp, int(s) % sp
        dst[p][:, r, h0:h0 + H_local, :] = o[:, i]
