"""Per-tile store spans of the fused epilogue and its overhead against sequence length.

X-Stage explainer (gist.science, arXiv 2607.23264), technical summary, "Results",
FlashAttention-A2A: as the sequence grows, the next tile's key loop covers the drain of the
previous tile's stores, the fused kernel approaches attention alone, and the overhead stays
flat, contradicting a completion-coupled counterfactual whose overhead grows linearly with
the sequence; "Contributions", X-Stage item: neither a fully blocking nor an unbounded
asynchronous model describes the issuer.

On one GPU the stores go to local HBM.  For each sequence length this measures (HIP events,
back-to-back launches, inputs resident):
  * t_attn      attention alone, contiguous output (xstage_attn_fwd);
  * t_fused     the fused kernel (xstage_attn_a2a_fwd);
  * t_nostore   the unbounded-asynchronous bound: the traced kernel issuing no output store;
  * t_coupled   the completion-coupled counterfactual: every wave waits for its stores;
the core clock of the key loops (traced mode 3) and, from the traced kernel's per-wave
stamps, the epilogue span (end of the key loop to the
last store issued; includes the merge of key splits) and, in the coupled mode, the drain
span (last store issued to stores complete).  The completion-coupled model predicts
t_fused + rounds * drain, with rounds = workgroups per co-resident slot.
"""

from __future__ import annotations

import json
import math

import numpy as np

DEFAULT_S = (1024, 2304, 4608, 9216, 16896, 32760)


def coupled_prediction(t_fused_s: float, rounds: float, drain_s: float) -> float:
    """Completion-coupled counterfactual: each of the `rounds` workgroup generations of a
    slot additionally waits for its stores to drain."""
    return t_fused_s + rounds * drain_s


def spans_from_stamps(stamps: np.ndarray, hz: float):
    """stamps: [n_workgroups, waves, 4] ticks -> (epilogue spans, drain spans) in seconds,
    over the waves that stored output."""
    st = stamps.reshape(-1, 4).astype(np.int64)
    emit = st[:, 2] > 0
    epi = (st[emit, 2] - st[emit, 1]) / hz
    done = emit & (st[:, 3] > 0)
    drain = (st[done, 3] - st[done, 2]) / hz
    return epi, drain


def loop_clock_ghz(stamps: np.ndarray, hz: float, min_wall_s: float = 2e-6):
    """Median core clock over the waves' key loops from mode-3 stamps ([1]-[0] wall-clock
    ticks, [3]-[2] shader-clock ticks), over loops of at least ``min_wall_s``."""
    st = stamps.reshape(-1, 4).astype(np.int64)
    wall = (st[:, 1] - st[:, 0]) / hz
    use = wall >= min_wall_s
    if not use.any():
        return None
    return float(np.median((st[use, 3] - st[use, 2]) / wall[use]) / 1e9)


def _time(torch, fn, n, warm):
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(n):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / n * 1e-3


def run_study(torch, xs, S_list=DEFAULT_S, H=3, D=128, P=8, seed=11, target_s=0.05, slots=None, emit=print,
              settle_s=0.3):
    from synth import Workload, make_inputs

    hz = xs.xstage_wallclock_hz()
    if slots is None:
        slots = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    rows = []
    for S in S_list:
        S = (S // P) * P
        w = Workload(f"study{S}", 1, S, H, D, P, seed=seed)
        qb, kb, vb = make_inputs(w)

        def dev(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

        q, k, v = dev(qb), dev(kb), dev(vb)
        slabs = torch.empty((P, 1, S // P, H, D), dtype=torch.bfloat16, device="cuda")
        sl = [slabs[p] for p in range(P)]
        out1 = torch.empty((1, S, H, D), dtype=torch.bfloat16, device="cuda")
        nwg, nsp = xs.xstage_attn_a2a_plan(1, S, H, D)
        wg_rows = xs.xstage_attn_a2a_wg_rows(1, S, H, D)
        stamps = [torch.zeros(nwg * (wg_rows // 32) * 4, dtype=torch.int64, device="cuda") for _ in range(4)]
        sws = xs.split_workspace(1, S, H, D)
        calls = {
            "attn": xs.bind("xstage_attn_fwd", q, k, v, out1, w.scale, split_ws=sws),
            "fused": xs.bind("xstage_attn_a2a_fwd", q, k, v, sl, w.scale, split_ws=sws),
            "traced": xs.bind("xstage_attn_a2a_fwd_traced", q, k, v, sl, 0, stamps[0], w.scale, split_ws=sws),
            "coupled": xs.bind("xstage_attn_a2a_fwd_traced", q, k, v, sl, 1, stamps[1], w.scale, split_ws=sws),
            "nostore": xs.bind("xstage_attn_a2a_fwd_traced", q, k, v, sl, 2, stamps[2], w.scale, split_ws=sws),
            "clock": xs.bind("xstage_attn_a2a_fwd_traced", q, k, v, sl, 3, stamps[3], w.scale, split_ws=sws),
        }
        if not rows:  # settle: the chip's clock dips, then recovers, over the first ~20 ms of load
            import time as _t

            t_set = _t.perf_counter()
            while _t.perf_counter() - t_set < settle_s:
                for _ in range(20):
                    calls["fused"]()
                torch.cuda.synchronize()
        t_est = _time(torch, calls["fused"], 3, 3)
        n = max(20, min(2000, int(target_s / max(t_est, 1e-6))))
        # three interleaved rounds over the call kinds, medians
        per = {name: [] for name in calls}
        for _ in range(3):
            for name, fn in calls.items():
                per[name].append(_time(torch, fn, n, max(20, n // 8)))
        t = {name: float(np.median(v)) for name, v in per.items()}
        epi, _ = spans_from_stamps(stamps[0].cpu().numpy(), hz)
        _, drain = spans_from_stamps(stamps[1].cpu().numpy(), hz)
        ghz = loop_clock_ghz(stamps[3].cpu().numpy(), hz)
        rounds = nwg * (wg_rows // 128) / slots  # slots: 128-row (4-wave) workgroups at once
        drain_med = float(np.median(drain)) if len(drain) else 0.0
        row = {
            "S": S, "H_local": H, "D": D, "P": P, "workgroups": nwg, "wg_rows": wg_rows, "key_splits": nsp, "rounds": round(rounds, 3),
            "t_attn_us": t["attn"] * 1e6, "t_fused_us": t["fused"] * 1e6, "t_traced_us": t["traced"] * 1e6,
            "t_nostore_us": t["nostore"] * 1e6, "t_coupled_us": t["coupled"] * 1e6,
            "overhead_fused_vs_attn_us": (t["fused"] - t["attn"]) * 1e6,
            "overhead_fused_vs_nostore_us": (t["fused"] - t["nostore"]) * 1e6,
            "overhead_coupled_vs_nostore_us": (t["coupled"] - t["nostore"]) * 1e6,
            "epilogue_span_us_median": float(np.median(epi)) * 1e6 if len(epi) else None,
            "epilogue_span_us_p90": float(np.percentile(epi, 90)) * 1e6 if len(epi) else None,
            "drain_span_us_median": drain_med * 1e6,
            "drain_span_us_p90": float(np.percentile(drain, 90)) * 1e6 if len(drain) else None,
            "coupled_model_us": coupled_prediction(t["fused"], math.ceil(rounds), drain_med) * 1e6,
            "loop_clock_ghz": ghz,
            "iterations": n,
        }
        rows.append(row)
        emit(json.dumps(row))
        del q, k, v, slabs, out1, stamps, calls, sws
        torch.cuda.empty_cache()
    return rows


def summarize(lines, source_hash, jsonl_path="xstage_study.jsonl"):
    """Markdown table of a study's JSON lines (the output of ``bench.py --xstage-study``,
    saved at ``jsonl_path``)."""
    rows = [json.loads(ln) for ln in lines if ln.strip().startswith("{")]
    md = ["# Fused-epilogue overhead and store spans against sequence length (one MI355X)", "",
          f"Kernel source hash (attn_a2a.hip + common.hpp, sha256 prefix): `{source_hash}`.", "",
          f"Command (repository root): `python3 bench.py --xstage-study > {jsonl_path}`, then",
          f"`python -m attention_ulysses_a2a_amd.xstage_study {jsonl_path}` writes this table",
          "(H_local=3, D=128, P=8, seeded N(0,1) inputs, inputs resident; after a 0.3 s settle phase, every",
          "call kind timed with HIP events over back-to-back launches in three interleaved rounds, medians).",
          "Times in µs per launch; loop clock in GHz.", "",
          "* attn: attention alone into a contiguous output (`xstage_attn_fwd`); fused:",
          "  `xstage_attn_a2a_fwd`; traced / coupled / no-store: `xstage_attn_a2a_fwd_traced` modes",
          "  0 / 1 / 2 (per-wave clock stamps; 1 = every wave waits for its stores to complete, the",
          "  completion-coupled counterfactual; 2 = no output store, the unbounded-asynchronous bound).",
          "* epilogue span: end of the key loop to the last output store issued (includes the",
          "  key-split merge); drain span: last store issued to stores complete (coupled mode).",
          "* model: completion-coupled prediction t_fused + ceil(rounds) x median drain span.", "",
          "| S | workgroups | key splits | rounds | attn | fused | fused − attn | traced | no-store | coupled | "
          "traced − no-store | coupled − no-store | epilogue span (median) | drain span (median / p90) | "
          "coupled model | loop clock GHz |",
          "|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        wg = f"{r['workgroups']}" + (f" × {r['wg_rows']} rows" if r.get("wg_rows", 128) != 128 else "")
        md.append(f"| {r['S']} | {wg} | {r['key_splits']} | {r['rounds']:.2f} | {r['t_attn_us']:.1f} | "
                  f"{r['t_fused_us']:.1f} | {r['overhead_fused_vs_attn_us']:+.2f} | {r['t_traced_us']:.1f} | "
                  f"{r['t_nostore_us']:.1f} | {r['t_coupled_us']:.1f} | "
                  f"{r['t_traced_us'] - r['t_nostore_us']:+.2f} | {r['overhead_coupled_vs_nostore_us']:+.2f} | "
                  f"{r['epilogue_span_us_median']:.2f} | {r['drain_span_us_median']:.2f} / "
                  f"{r['drain_span_us_p90']:.2f} | {r['coupled_model_us']:.1f} | {r['loop_clock_ghz']:.2f} |")
    return "\n".join(md) + "\n"


if __name__ == "__main__":
    import os
    import sys

    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    import bench

    with open(sys.argv[1]) as fh:
        sys.stdout.write(summarize(fh.readlines(), bench.kernel_source_hash(), sys.argv[1]))
