"""Paced epilogue bursts: the Burst-Gap model's pacing choice against measurement.

X-Stage explainer (gist.science, arXiv 2607.23264), "Significance": the Burst-Gap model as a
way to shape the communication bursts and hide their issuer-side cost; "Methodology": a
burst of aggregate volume V from K producers followed by a gap G of compute, issue time
max(T0, V/R - G).  The fused kernel's epilogue is such a burst; the paced persistent call
(``xstage_attn_a2a_fwd_paced``) can issue each finished tile in c chunks over the next
tile's first key-loop iterations.

For a workload with more tiles than the paced launch has workgroups, this measures (HIP
events on the current stream, inputs resident, three interleaved rounds after a settle
phase, medians):
  * product          the product call with its split workspace (its fastest plan);
  * product_unsplit  the product call without split workspace (the same per-tile arithmetic
                     as the paced call, non-persistent, two workgroups per CU);
  * paced_c{c}       the paced call for every allowed chunk count c;
and applies ``xstage_bg_pacing_chunks`` to the launch's burst: K = the paced launch's
workgroups, each issuing one tile's rows (128 x D bf16), so V = K x tile bytes when they
issue together; G = one tile's compute time (the c = 1 paced time over the tiles per
workgroup); R, Q, f1 and a from the Burst-Gap sweep on MI355X (``bench.py --bg``: drain
rate and capacity of producers started together, per-producer free issue rate and fixed
cost), overridable.  The model's c is compared with the measured spread over c.
"""

from __future__ import annotations

import json

import numpy as np

# Burst-Gap parameters measured on MI355X (cold destinations; 256 producers started together):
R_AGG = 5.64e12        # aggregate drain rate, B/s
Q_CAP = 6.5 * 2 ** 20  # pending capacity, bytes
F1 = 131e9             # one producer's backpressure-free issue rate, B/s
A_FIXED = 86e-9        # fixed cost per burst, s

DEFAULT_WORKLOADS = ("video", "flux2048")


def chunk_counts(D: int):
    return (1, 2, 4, 8) if D == 128 else (1, 2, 4)


def model_choice(xs, n_wg: int, tile_bytes: int, G_s: float, c_max: int, R=R_AGG, Q=Q_CAP, f1=F1, a=A_FIXED):
    """Pacing chunk count the Burst-Gap model picks for the launch's burst (K = n_wg producers
    issuing one tile each, together: V = n_wg * tile_bytes at an aggregate free rate
    n_wg * f1) and the issuer-visible time it predicts."""
    V = float(n_wg) * tile_bytes
    c, t = xs.xstage_bg_pacing_chunks(V, G_s, a, n_wg * f1, R, Q, c_max)
    return {"c": int(c), "t_visible_us": t * 1e6, "V_bytes": V, "G_us": G_s * 1e6, "R_Bps": R, "Q_bytes": Q,
            "f1_Bps": f1, "a_s": a}


def _time(torch, fn, n, warm):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(n):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / n * 1e-3


def run(torch, xs, names=DEFAULT_WORKLOADS, rounds=3, target_s=0.1, settle_s=0.3, emit=print):
    from synth import make_inputs, workload

    out = []
    for name in names:
        w = workload(name)
        qb, kb, vb = make_inputs(w)
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
                   for x in (qb, kb, vb))
        slabs = torch.empty((w.P, w.B, w.S // w.P, w.H, w.D), dtype=torch.bfloat16, device="cuda")
        ws = xs.split_workspace(w.B, w.S, w.H, w.D, "cuda")
        n_wg, n_tiles = xs.xstage_attn_a2a_paced_plan(w.B, w.S, w.H, w.D)
        legs = {
            "product": xs.bind("xstage_attn_a2a_fwd", q, k, v, slabs, w.scale, split_ws=ws),
            "product_unsplit": xs.bind("xstage_attn_a2a_fwd", q, k, v, slabs, w.scale, split_ws=None),
        }
        for c in chunk_counts(w.D):
            legs[f"paced_c{c}"] = xs.bind("xstage_attn_a2a_fwd_paced", q, k, v, slabs, c, w.scale)
        # settle: the chip's clock ramps over the first launches of a process
        legs["product"]()
        torch.cuda.synchronize()
        t1 = _time(torch, legs["product"], 3, 1)
        n_settle = max(1, int(settle_s / max(t1, 1e-6)))
        _time(torch, legs["product"], n_settle, 0)
        per = {}
        for _ in range(rounds):
            for leg, fn in legs.items():
                t = _time(torch, fn, 2, 1)
                n = max(3, int(target_s / max(t, 1e-6)))
                per.setdefault(leg, []).append(_time(torch, fn, n, 2))
        ms = {leg: float(np.median(v)) * 1e3 for leg, v in per.items()}
        paced = {c: ms[f"paced_c{c}"] for c in chunk_counts(w.D)}
        tiles_per_wg = n_tiles / n_wg
        G = paced[1] * 1e-3 / tiles_per_wg
        model = model_choice(xs, n_wg, 128 * w.D * 2, G, max(chunk_counts(w.D)))
        best = min(paced, key=paced.get)
        line = {
            "paced_study": name, "B": w.B, "S": w.S, "H": w.H, "D": w.D, "P": w.P,
            "n_tiles": n_tiles, "n_workgroups": n_wg, "rounds": rounds, "settle_launches": n_settle,
            "ms": ms,
            "paced_spread_pct": (max(paced.values()) / min(paced.values()) - 1) * 100,
            "best_c_measured": best,
            "model": model,
            "model_c_vs_best_pct": (paced[model["c"]] / paced[best] - 1) * 100,
            "round_ms": {leg: [x * 1e3 for x in v] for leg, v in per.items()},
        }
        emit(json.dumps(line))
        out.append(line)
        del legs, q, k, v, slabs, ws
        torch.cuda.empty_cache()
    return out


def summarize(lines, command: str, source_hash: str) -> str:
    """Markdown summary of the study's JSON lines."""
    md = ["# Paced epilogue bursts: Burst-Gap pacing choice against measurement (one MI355X)", "",
          "Command (repository root):", "", f"    {command}", "",
          f"Kernel source hash (attn_a2a.hip + common.hpp, sha256 prefix): `{source_hash}`.", "",
          "The paced call is persistent (one workgroup per CU: its LDS holds the K/V slots and the finished tile's "
          "rows); the product calls run two workgroups per CU.  Times are medians of interleaved rounds "
          "(HIP events, back-to-back launches, inputs resident).", ""]
    for ln in lines:
        m = ln["model"]
        md += [f"## {ln['paced_study']}: B={ln['B']} S={ln['S']} H={ln['H']} D={ln['D']} P={ln['P']}", "",
               f"{ln['n_tiles']} tiles on {ln['n_workgroups']} paced workgroups "
               f"({ln['n_tiles'] / ln['n_workgroups']:.2f} tiles each).", "",
               "| call | ms per call | vs product |", "|---|---|---|"]
        base = ln["ms"]["product"]
        for leg, t in ln["ms"].items():
            md.append(f"| {leg} | {t:.4f} | {t / base:.3f} |")
        md += ["",
               f"Spread over the chunk counts: {ln['paced_spread_pct']:.2f} % (fastest measured: c = "
               f"{ln['best_c_measured']}).",
               f"Model (`xstage_bg_pacing_chunks`, V = {m['V_bytes'] / 2 ** 20:.2f} MiB from "
               f"{ln['n_workgroups']} producers, G = {m['G_us']:.1f} us, R = {m['R_Bps'] / 1e12:.2f} TB/s, "
               f"Q = {m['Q_bytes'] / 2 ** 20:.2f} MiB, f1 = {m['f1_Bps'] / 1e9:.0f} GB/s per producer, "
               f"a = {m['a_s'] * 1e9:.0f} ns): c = {m['c']}, issuer-visible {m['t_visible_us']:.3f} us per tile; "
               f"the model's c measures {ln['model_c_vs_best_pct']:+.2f} % against the fastest c.", ""]
    return "\n".join(md) + "\n"


if __name__ == "__main__":  # python -m attention_ulysses_a2a_amd.paced_study <jsonl> <source hash> [command]
    import sys

    lines = [json.loads(x) for x in open(sys.argv[1]) if x.startswith("{\"paced_study\"")]
    cmd = sys.argv[3] if len(sys.argv) > 3 else "python bench.py --paced"
    print(summarize(lines, cmd, sys.argv[2]), end="")
