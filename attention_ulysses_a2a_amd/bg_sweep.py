"""Burst-Gap store sweep on one GPU (driver of ``xstage_burst_gap_run``).

K producer workgroups each store V/K bytes per round into their share of a destination
set, then run an FMA gap of G microseconds; the issuer-visible burst issue time is read
from device wall-clock stamps taken with no wait for store completion (X-Stage explainer,
gist.science, arXiv 2607.23264, "Methodology": Burst-Gap model; "Contributions":
parameterised microbenchmarks measure T0_iss, R and Q).

Two destination variants: "hot" (one destination set, reused every round: it stays in
the L2 / last-level cache) and "cold" (rotating sets spanning at least 512 MiB so that
no round finds its destination cached).  Two more series make the capacity Q observable:
"large" (cold, K = 256, bursts of 128 MiB to 1 GiB, larger than any cache, with gaps up to
160 us, so that the gap can exceed Q/R while the burst is still drain-bound) and
"isolated" (cold, K = 256, each burst issued only after the previous one has long
drained: the capacity reading gives T_iss = max(T0, (V - Q)/R), a line in V whose slope
and intercept give R and Q).  Both start every round with a barrier across the producers,
so that a round is one aggregate burst whose issue time is the span from the first start
to the last store issued.  A plain copy kernel's write rate is the cross-check of R.
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


SYNC_TIMEOUT_S = 2e-3  # bound of each round's start barrier


def _run(torch, xs, K, V, gap_iters, rounds, dst, n_sets, nontemporal=False, sync=False, hz=1e8):
    stamps = torch.zeros(K * rounds * 3, dtype=torch.int64, device="cuda")
    sy = torch.zeros(rounds, dtype=torch.int32, device="cuda") if sync else None
    xs.xstage_burst_gap_run(K, V, gap_iters, rounds, dst, stamps, n_dst_sets=n_sets, nontemporal=nontemporal,
                            sync=sy, sync_timeout_ticks=int(SYNC_TIMEOUT_S * hz) if sync else 0)
    torch.cuda.synchronize()
    return stamps.cpu().numpy().reshape(K, rounds, 3).astype(np.int64)


def calibrate_gap(torch, xs, hz, iters=20000):
    """Seconds per iteration of the producer's dependent FMA loop (no stores running)."""
    st = _run(torch, xs, 32, 0, iters, 8, None, 1)
    per_round = (st[:, 2:7, 2] - st[:, 2:7, 1]).astype(float) / hz  # gap only, rounds 2..6
    return float(np.median(per_round)) / iters


def measure(st, hz, V, discard=DISCARD):
    """Issue times of one sweep point.

    T_iss: the issuer-visible time of a burst, i.e. the time each producer takes to issue
    its V/K bytes (stores accepted, none waited on), median over producers per round and
    over the kept rounds.  The producers are not aligned across workgroups, so the span
    from the first start to the last 'all issued' stamp of a round (``span_us``) mostly
    measures inter-workgroup skew; it is reported, not fitted.  With the start barrier
    (``sync``) the producers of a round start together (``start_spread_us``: median spread
    of their start stamps) and ``span_us`` is the issue time of the aggregate burst.
    """
    t0 = st[:, :, 0].astype(float) / hz
    t1 = st[:, :, 1].astype(float) / hz
    t2 = st[:, :, 2].astype(float) / hz
    keep = slice(discard, st.shape[1])
    per_round = np.median(t1 - t0, axis=0)
    span = t1.max(axis=0) - t0.min(axis=0)
    period = np.median(np.diff(t0, axis=1)[:, discard:], axis=0)
    total = t2[:, -1].max() - t0[:, 0].min()
    rounds = st.shape[1]
    return {
        "start_spread_us": float(np.median((t0.max(axis=0) - t0.min(axis=0))[keep]) * 1e6),
        "T_iss_us": float(np.median(per_round[keep]) * 1e6),
        "T_iss_p10_us": float(np.percentile(per_round[keep], 10) * 1e6),
        "T_iss_p90_us": float(np.percentile(per_round[keep], 90) * 1e6),
        "span_us": float(np.median(span[keep]) * 1e6),
        "period_us": float(np.median(period) * 1e6) if period.size else None,
        "R_direct_GBps": float(rounds * V / total / 1e9) if total > 0 else None,
    }


LARGE_V_MIB = (128, 256, 512, 1024)
LARGE_G_US = (0, 10, 20, 40, 80, 160)
ISO_V_MIB = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024)
ISO_IDLE_US = 50.0
LARGE_SPAN = 2 << 30
LARGE_ROUNDS, LARGE_DISCARD = 10, 2


def copy_rate(torch, xs, calls=20):
    """Plain copy (the scatter kernel) of 512 MiB into 8 slabs: bytes written per second and
    bytes moved (read + written) per second, HIP events over `calls` calls."""
    B, S, H, D, P = 1, 262144, 8, 128, 8
    src = torch.ones((B, S, H, D), dtype=torch.bfloat16, device="cuda")
    dst = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        xs.xstage_a2a_scatter(src, dst)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(calls):
        xs.xstage_a2a_scatter(src, dst)
    b.record()
    torch.cuda.synchronize()
    t = a.elapsed_time(b) / calls * 1e-3
    nbytes = B * S * H * D * 2
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_written": nbytes, "s_per_call": t, "write_GBps": nbytes / t / 1e9, "read_write_GBps": 2 * nbytes / t / 1e9}


def run_capacity_series(torch, xs, hz, sec_per_iter, free_fit, R_drain, out=print):
    # R_drain (the unsynchronised cold sweep's drain rate) only sizes the isolated gaps.
    """The "large" and "isolated" series (cold destinations, K = 256) and their fits."""
    from .bg_model import fit_synchronized

    K = 256
    vmax = max(max(LARGE_V_MIB), max(ISO_V_MIB)) << 20
    buf = torch.empty((LARGE_SPAN + vmax) // 4, dtype=torch.int32, device="cuda")
    large = []
    for vm in LARGE_V_MIB:
        V = vm << 20
        n_sets = max(2, math.ceil(LARGE_SPAN / V))
        for g in LARGE_G_US:
            iters = int(round(g * 1e-6 / sec_per_iter))
            st = _run(torch, xs, K, V, iters, LARGE_ROUNDS, buf, n_sets, sync=True, hz=hz)
            m = measure(st, hz, V, discard=LARGE_DISCARD)
            m["T_iss_us"] = m["span_us"]  # aggregate burst: first start to last store issued
            out(json.dumps({"bg": {"variant": "large", "K": K, "V_MiB": vm, "G_us": g, "gap_fma_iters": iters, **m}}))
            large.append((V, g * 1e-6, m["T_iss_us"] * 1e-6))
    iso = []
    c, f1 = free_fit["c_s"], free_fit["f1_Bps"]
    for vm in ISO_V_MIB:
        V = vm << 20
        g = V / (0.5 * R_drain) * 1e6 + ISO_IDLE_US  # at least 50 us past the drain of the previous burst
        iters = int(round(g * 1e-6 / sec_per_iter))
        n_sets = max(2, math.ceil(LARGE_SPAN / V))
        st = _run(torch, xs, K, V, iters, LARGE_ROUNDS, buf, n_sets, sync=True, hz=hz)
        m = measure(st, hz, V, discard=LARGE_DISCARD)
        m["T_iss_us"] = m["span_us"]  # aggregate burst: first start to last store issued
        t0 = c + V / (K * f1)
        out(json.dumps({"bg": {"variant": "isolated", "K": K, "V_MiB": vm, "G_us": round(g, 2), "gap_fma_iters": iters,
                               "T0_free_us": t0 * 1e6, **m}}))
        iso.append((V, m["T_iss_us"] * 1e-6, m["start_spread_us"] * 1e-6))
    fs = fit_synchronized(large, iso, c, f1, K)
    out(json.dumps({"bg_sync_fit": {"K": K, "free_c_s": c, "free_f1_Bps": f1, **fs}}))
    del buf
    torch.cuda.empty_cache()
    return {"synchronized": fs}


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
    del buf
    torch.cuda.empty_cache()
    cold = summary.get("cold")
    if cold and cold.get("capacity_reading") and cold.get("R"):
        summary.update(run_capacity_series(torch, xs, hz, sec_per_iter, cold["capacity_reading"], cold["R"], out))
    cp = copy_rate(torch, xs)
    out(json.dumps({"bg_copy": cp}))
    summary["copy"] = cp
    return summary


def summarize(lines, jsonl_path="bg_sweep.jsonl"):
    """Markdown summary of a sweep's JSON lines (the output of ``bench.py --bg``, saved at
    ``jsonl_path``)."""
    recs = [json.loads(ln) for ln in lines if ln.strip().startswith("{")]
    pts = [r["bg"] for r in recs if "bg" in r]
    fits = {r["bg_fit"]["variant"]: r["bg_fit"] for r in recs if "bg_fit" in r}
    sync = next((r["bg_sync_fit"] for r in recs if "bg_sync_fit" in r), None)
    if sync:  # recompute from the recorded points with the current analysis
        from .bg_model import fit_synchronized

        lg = [(p["V_MiB"] * 2 ** 20, p["G_us"] * 1e-6, p["T_iss_us"] * 1e-6) for p in pts if p["variant"] == "large"]
        io = [(p["V_MiB"] * 2 ** 20, p["T_iss_us"] * 1e-6, p["start_spread_us"] * 1e-6)
              for p in pts if p["variant"] == "isolated"]
        if lg and io:
            sync = {**sync, **fit_synchronized(lg, io, sync["free_c_s"], sync["free_f1_Bps"], sync["K"])}
    cp = next((r["bg_copy"] for r in recs if "bg_copy" in r), None)
    cal = next((r["bg_calibration"] for r in recs if "bg_calibration" in r), {})
    md = ["# Burst-Gap store sweep on one MI355X (xstage_burst_gap_run)", "",
          f"Command (repository root): `python bench.py --bg > {jsonl_path}`, then",
          f"`python -m attention_ulysses_a2a_amd.bg_sweep {jsonl_path}` writes this summary.", ""]
    if cal:
        md.append(f"Wall clock {cal['wallclock_hz'] / 1e6:.0f} MHz; gap loop calibrated at "
                  f"{cal['gap_ns_per_fma_iter']:.2f} ns per dependent-FMA iteration.")
    md += ["K producer workgroups (256 threads) store V/K bytes per round as 16-byte stores, then run a gap of G us.",
           "T_iss = per-producer time from burst start to 'every wave has issued its last store' (no wait on",
           "completion), median over producers and kept rounds.", ""]
    for variant in ("hot", "cold", "large"):
        f = fits.get(variant)
        vp = [p for p in pts if p["variant"] == variant]
        if not vp:
            continue
        md.append(f"## {variant} destinations" if variant != "large"
                  else "## large bursts (cold destinations, K = 256, producers started together; T_iss = aggregate span)")
        md.append("")
        if variant == "large" and sync:
            md.append(f"Aggregate drain rate R_agg = {sync['R_agg_Bps'] / 1e12:.2f} TB/s (zero-gap points).  On the "
                      f"points with a gap, the printed formula max(T0, V/R_agg - G) is off by "
                      f"{100 * sync['page_formula_rel_err_median']:.0f} % (median); the capacity reading "
                      f"max(T0, V/R_agg - min(G, Q/R_agg)) with Q from the isolated bursts by "
                      f"{100 * sync.get('capacity_reading_rel_err_median', float('nan')):.1f} %.")
            md.append("")
        if f and f.get("R"):
            line = (f"Page formula fit: R = {f['R'] / 1e12:.2f} TB/s from {f['n_drain']} drain-regime points of "
                    f"{f['n_points']}")
            if "rel_err_median_predicted" in f:
                line += (f"; held-out points (G below the longest gap): median |error| "
                         f"{100 * f['rel_err_median_predicted']:.2f} %, p90 {100 * f['rel_err_p90_predicted']:.1f} %")
            md.append(line + ".")
        cr = (f or {}).get("capacity_reading")
        if cr:
            md.append(f"Capacity reading fit: R = {cr['R_Bps'] / 1e12:.2f} TB/s, Q = {cr['Q_bytes'] / 2 ** 20:.0f} MiB, "
                      f"per-producer free rate f1 = {cr['f1_Bps'] / 1e9:.0f} GB/s, fixed cost a = {cr['c_s'] * 1e9:.0f} ns, "
                      f"median |error| {100 * cr['rel_err_median']:.1f} %.")
        pa = (f or {}).get("pacing_attention_tile")
        if pa:
            md.append(f"Pacing choice for the attention epilogue's burst (one 128 x 128 bf16 tile, {pa['tile_bytes']} B, "
                      f"from one producer, G = 0; `xstage_bg_pacing_chunks`): {pa['chunks']} chunk(s), issuer-visible "
                      f"{pa['T_visible_us']:.3f} us.")
        md.append("")
        gs = sorted(set(p["G_us"] for p in vp))
        md.append("| K | V MiB | " + " | ".join(f"G={g}us" for g in gs) + " | R_direct GB/s (G=0) |")
        md.append("|---|---|" + "---|" * len(gs) + "---|")
        for K in sorted(set(p["K"] for p in vp)):
            for vm in sorted(set(p["V_MiB"] for p in vp if p["K"] == K)):
                row = {p["G_us"]: p for p in vp if p["K"] == K and p["V_MiB"] == vm}
                rd = row.get(0, {}).get("R_direct_GBps")
                cells = " | ".join(f"{row[g]['T_iss_us']:.2f}" if g in row else "" for g in gs)
                md.append(f"| {K} | {vm} | {cells} | " + (f"{rd:.0f} |" if rd else "|"))
        md.append("")
    ip = [p for p in pts if p["variant"] == "isolated"]
    if ip:
        md += ["## isolated bursts (cold destinations, K = 256, producers started together)", "",
               f"Each burst starts at least {ISO_IDLE_US:.0f} us after the previous one has drained (gap = 2 V / R + "
               f"{ISO_IDLE_US:.0f} us); T_iss is the aggregate span (first start to last store issued); T0 is the free "
               "issue time c + V/(K f1) from the cold fit.", ""]
        iso = (sync or {}).get("isolated", {})
        if "R_iso_Bps" in iso:
            md.append(f"Line through the {iso['n_used']} points above 1.5 T0: R_iso = {iso['R_iso_Bps'] / 1e12:.2f} TB/s, "
                      f"Q_iso = {iso['Q_iso_bytes'] / 2 ** 20:.1f} MiB; with the aggregate drain rate R_agg = "
                      f"{sync['R_agg_Bps'] / 1e12:.2f} TB/s of the zero-gap large bursts, Q = median(V - R_agg T) = "
                      f"{iso['Q_bytes_at_R'] / 2 ** 20:.1f} MiB.")
            md.append("")
        md.append("| V MiB | gap us | T0 (free) us | T_iss us | start spread us |")
        md.append("|---|---|---|---|---|")
        for p in sorted(ip, key=lambda p: p["V_MiB"]):
            md.append(f"| {p['V_MiB']} | {p['G_us']:.0f} | {p['T0_free_us']:.2f} | {p['T_iss_us']:.2f} | "
                      f"{p.get('start_spread_us', float('nan')):.2f} |")
        md.append("")
    if cp:
        md += ["## plain copy (cross-check of R)", "",
               f"`xstage_a2a_scatter` of a 512 MiB tensor into 8 slabs: {cp['write_GBps']:.0f} GB/s written "
               f"({cp['read_write_GBps']:.0f} GB/s read + written), {cp['s_per_call'] * 1e6:.1f} us per call.", ""]
    return "\n".join(md) + "\n"


if __name__ == "__main__":
    import sys

    with open(sys.argv[1]) as fh:
        sys.stdout.write(summarize(fh.readlines(), sys.argv[1]))
