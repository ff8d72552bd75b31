"""Plain float64 mixture-of-experts layer with the combine all-to-all (test infrastructure).

The stand-in for the MegaMoE kernel of the X-Stage explainer (gist.science, arXiv
2607.23264), "Contributions", MegaMoE (reshaping) item: per expert, Linear-1 and then
Linear-2, whose results go to the token's destination (the combine all-to-all).  The
pages do not spell out the layer; readings used here (listed in the design notes):

* expert e owns the token rows [offsets[e], offsets[e+1]) of x;
* weights are stored as a linear layer stores them, output features by input features:
  w1[e] is [d_ff, d_model], w2[e] is [d_model, d_ff];
* Linear-1's result H is kept in bf16 (round to nearest, ties to even) between the two
  products, and no activation is applied;
* Linear-2's row of token t goes to row dst_row[t] of destination dst_slab[t]; a token
  whose destination is out of range is not stored.

The schedule (expert waves or interleaved) only orders the work: it is not part of what
is computed, so there is none here.
"""

from __future__ import annotations

import numpy as np

from .attention import bf16_bits_to_f64, round_to_bf16_bits


def moe_layer(x, w1, w2, offsets, dst_slab, dst_row, out_rows, tokens=None):
    """x [T, d_model], w1 [E, d_ff, d_model], w2 [E, d_model, d_ff] as float64 (bf16 values).

    Returns (h, outs): h [T, d_ff] float64, Linear-1 before its bf16 rounding; outs: P
    arrays [out_rows[p], d_model] float64, NaN where no token lands.  With ``tokens`` (a
    subset of token indices), only those tokens are computed; h is then NaN elsewhere."""
    T, d_model = x.shape
    E, d_ff, _ = w1.shape
    h = np.full((T, d_ff), np.nan)
    outs = [np.full((int(n), d_model), np.nan) for n in out_rows]
    want = np.ones(T, dtype=bool) if tokens is None else np.isin(np.arange(T), np.asarray(tokens))
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        sel = np.arange(lo, hi)[want[lo:hi]]
        if sel.size == 0:
            continue
        he = x[sel] @ w1[e].T                                  # Linear-1, float64
        hb = bf16_bits_to_f64(round_to_bf16_bits(he))          # kept in bf16
        ye = hb @ w2[e].T                                      # Linear-2, float64
        h[sel] = he
        for i, t in enumerate(sel):
            p, r = int(dst_slab[t]), int(dst_row[t])
            if 0 <= p < len(outs) and 0 <= r < outs[p].shape[0]:
                outs[p][r] = ye[i]
    return h, outs
