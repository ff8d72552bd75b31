"""Burst-Gap store sweep on one GPU (driver of ``xstage_burst_gap_run``).

K producer workgroups each store V/K bytes per round into their share of a destination
set, then run an FMA gap of G microseconds; the issuer-visible burst issue time is read
from device wall-clock stamps taken with no wait for store completion (X-Stage explainer,
gist.science, arXiv 2607.23264, "Methodology": Burst-Gap model; "Contributions":
parameterised microbenchmarks measure T0_iss, R and Q).

Two destination variants: "hot" (one destination set, reused every round: it stays in
the L2 / last-level cache) and "cold" (rotating sets spanning at least 512 MiB so that
no round finds its destination cached).
"""

from __future__ import annotations

import json
import math

import numpy as np

K_SET = (32, 64, 128, 256)
V_MIB = (1, 4, 16, 64)
G_US = (0, 1, 2, 5, 10, 20)
ROUNDS = 32
DISCARD = 4
COLD_SPAN = 512 << 20


def _run(torch, xs, K, V, gap_iters, rounds, dst, n_sets, nontemporal=False):
    stamps = torch.zeros(K * rounds * 3, dtype=torch.int64, device="cuda")
    xs.xstage_burst_gap_run(K, V, gap_iters, rounds, dst, stamps, n_dst_sets=n_sets, nontemporal=nontemporal)
    torch.cuda.synchronize()
    return stamps.cpu().numpy().reshape(K, rounds, 3).astype(np.int64)


def calibrate_gap(torch, xs, hz, iters=20000):
    """Seconds per iteration of the producer's dependent FMA loop (no stores running)."""
    st = _run(torch, xs, 32, 0, iters, 8, None, 1)
    per_round = (st[:, 2:7, 2] - st[:, 2:7, 1]).astype(float) / hz  # gap only, rounds 2..6
    return float(np.median(per_round)) / iters


def measure(st, hz, V):
    """Issue times of one sweep point.

    T_iss: the issuer-visible time of a burst, i.e. the time each producer takes to issue
    its V/K bytes (stores accepted, none waited on), median over producers per round and
    over the kept rounds.  The producers are not aligned across workgroups, so the span
    from the first start to the last 'all issued' stamp of a round (``span_us``) mostly
    measures inter-workgroup skew; it is reported, not fitted.
    """
    t0 = st[:, :, 0].astype(float) / hz
    t1 = st[:, :, 1].astype(float) / hz
    t2 = st[:, :, 2].astype(float) / hz
    keep = slice(DISCARD, st.shape[1])
    per_round = np.median(t1 - t0, axis=0)
    span = t1.max(axis=0) - t0.min(axis=0)
    period = np.median(np.diff(t0, axis=1)[:, DISCARD:], axis=0)
    total = t2[:, -1].max() - t0[:, 0].min()
    rounds = st.shape[1]
    return {
        "T_iss_us": float(np.median(per_round[keep]) * 1e6),
        "T_iss_p10_us": float(np.percentile(per_round[keep], 10) * 1e6),
        "T_iss_p90_us": float(np.percentile(per_round[keep], 90) * 1e6),
        "span_us": float(np.median(span[keep]) * 1e6),
        "period_us": float(np.median(period) * 1e6) if period.size else None,
        "R_direct_GBps": float(rounds * V / total / 1e9) if total > 0 else None,
    }


def run_sweep(torch, xs, out=print, variants=("hot", "cold")):
    from .bg_model import fit

    hz = xs.xstage_wallclock_hz()
    sec_per_iter = calibrate_gap(torch, xs, hz)
    out(json.dumps({"bg_calibration": {"wallclock_hz": hz, "gap_ns_per_fma_iter": sec_per_iter * 1e9}}))
    vmax = max(V_MIB) << 20
    buf = torch.empty(max(COLD_SPAN + vmax, 2 * vmax) // 4, dtype=torch.int32, device="cuda")
    summary = {}
    for variant in variants:
        pts = []
        for K in K_SET:
            for vm in V_MIB:
                V = vm << 20
                n_sets = 1 if variant == "hot" else max(2, math.ceil(COLD_SPAN / V))
                for g in G_US:
                    iters = int(round(g * 1e-6 / sec_per_iter))
                    st = _run(torch, xs, K, V, iters, ROUNDS, buf, n_sets)
                    m = measure(st, hz, V)
                    rec = {"variant": variant, "K": K, "V_MiB": vm, "G_us": g, "gap_fma_iters": iters, **m}
                    out(json.dumps({"bg": rec}))
                    pts.append((K, V, g * 1e-6, m["T_iss_us"] * 1e-6))
        f = fit(pts)
        cap = f.get("capacity_reading")
        if cap:
            # The attention epilogue's burst: one workgroup's output tile (128 rows x 128 x 2 B)
            # from one producer; with no compute after it (G = 0) the chooser gives the chunk
            # count that no following tile could lower.
            tile = 128 * 128 * 2
            c, t = xs.xstage_bg_pacing_chunks(tile, 0.0, cap["c_s"], cap["f1_Bps"], cap["R_Bps"], cap["Q_bytes"])
            f["pacing_attention_tile"] = {"tile_bytes": tile, "G_us": 0.0, "chunks": c, "T_visible_us": t * 1e6}
        summary[variant] = f
        out(json.dumps({"bg_fit": {"variant": variant, **{k: v for k, v in f.items() if k != "T0"},
                                   "T0_us": {k: v * 1e6 for k, v in f["T0"].items()}}}))
    return summary
