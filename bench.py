#!/usr/bin/env python3
"""Benchmark of the fused attention + Ulysses all-to-all hot path on one MI355X.

A step is one call of ``xstage_attn_a2a_fwd`` on the FLUX-1024 share (B=1, S=4608,
H_local=3, D=128, P=8 destination slabs of [576, 3, 128]): non-causal attention over the full
sequence with the post-attention all-to-all written from the epilogue.  Inputs are seeded
synthetic bf16 tensors resident in HBM before the timed region.  Prints one JSON line.

Every leg runs after one common settle phase (``--settle-s`` seconds of fused launches: the
first launches of a process run up to ~6 % slow while the chip ramps up).  The headline is
one block of exactly ``--steps`` fused launches (after ``--warmup`` untimed ones) between two
synchronisations, timed with HIP events on the stream the kernel runs on.  Extra legs
(reported inside the same line) run in three interleaved rounds, every leg, the fused call
included, with the same max(steps, 100) timed and max(warmup, 20) untimed launches per
round (the clock shifts for about a millisecond when the kernel mix changes, so shorter
windows measure the shift), and every ratio is taken between the legs' medians: the serial
path (attention into a contiguous buffer,
then the separate scatter kernel), attention alone (P=1), the full-head Ulysses layouts
(strided destination; the whole layer reading its inputs from P sequence shards), and the
CPU oracle timed on a bounded sample of the same workload (``cpu_baseline``).  ``--bg``
instead runs the Burst-Gap store sweep and prints one JSON line per point plus the fitted
parameters; ``--cpu-oracle-configs`` times the oracle on every configuration; ``--paced`` times
the paced persistent epilogue for every chunk count against the Burst-Gap model's choice;
``--split-study`` every key-split count against the split-count model over a grid of shapes.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused attn+A2A-scatter TFLOP/s & % bf16 MFMA peak (S=4608, 1 GPU)"
PEAK_BF16_TFLOPS = 2500.0      # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0          # MI355X published HBM3E bandwidth
PEAK_CLOCK_GHZ = 2.4           # engine clock the published peak assumes (256 CUs x 4096 FLOP/clk)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_attn_a2a_flux1024.json")
KERNEL_SOURCES = [os.path.join(ROOT, "attention_ulysses_a2a_amd", "csrc", f)
                  for f in ("attn_a2a.hip", "common.hpp")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--settle-s", type=float, default=0.3,
                    help="seconds of fused launches before any leg (chip ramp-up; see the module docstring)")
    ap.add_argument("--cpu-oracle-configs", action="store_true",
                    help="time the float64 oracle on every workload in full (plus tiny on one core)")
    ap.add_argument("--workload", default="flux1024", help="synth workload name (tiny, flux1024, flux2048, video)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--bg", action="store_true", help="run the Burst-Gap store sweep instead")
    ap.add_argument("--xstage-study", action="store_true",
                    help="fused-epilogue overhead and store spans against sequence length (one JSON line per S)")
    ap.add_argument("--profile-launches", type=int, default=0,
                    help="only issue this many fused launches of the workload (for counter collection)")
    ap.add_argument("--split-study", action="store_true",
                    help="every key-split count against the split-count model over a grid of shapes "
                         "(one JSON line per shape)")
    ap.add_argument("--split-random", nargs=2, type=int, metavar=("SEED", "N"), default=None,
                    help="with --split-study: N shapes of a seeded random draw instead of the grid")
    ap.add_argument("--paced", action="store_true",
                    help="paced persistent epilogue: every chunk count against the product call and the "
                         "Burst-Gap model's choice (one JSON line per workload)")
    ap.add_argument("--moe", action="store_true",
                    help="expert-wave grouped-GEMM stand-in: expert waves vs interleaved schedule")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only the scatter kernel on a 512 MiB input (reference for HBM byte counters)")
    return ap.parse_args()


def timed(fn, steps, warmup, torch):
    """Average ms per call over `steps` back-to-back calls on the current stream (HIP events)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        return max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        return len(os.sched_getaffinity(0))


def cpu_baseline(w, qb, kb, vb, seconds):
    """Times the oracle (as it stands) on whole query-row blocks of the workload."""
    import numpy as np

    import oracle
    threads = blas_threads()
    q, k, v = (oracle.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    rows_done = 0
    t0 = time.perf_counter()
    rng_rows = np.arange(w.S)
    block = 512
    i = 0
    while time.perf_counter() - t0 < seconds:
        sel = rng_rows[(i * block) % w.S:(i * block) % w.S + block]
        oracle.attention_fp64(q, k, v, w.scale, rows=sel)
        rows_done += len(sel)
        i += 1
    dt = time.perf_counter() - t0
    flops = 4.0 * w.B * rows_done * w.S * w.D * w.H
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{rows_done} query rows x all {w.H} heads (blocks of {block}) of the {w.name} workload over the "
                  f"full key set, float64 numpy, {dt:.1f} s",
        "seconds": dt,
        "cpu_model": cpu_model(),
    }


def cpu_oracle_configs():
    """The float64 oracle (as it stands) on every workload in full, on this host's cores, and the
    tiny workload also on one core: one JSON line per run."""
    import oracle
    from synth import make_inputs, workload

    def run(name):
        w = workload(name)
        q, k, v = (oracle.bf16_bits_to_f64(x) for x in make_inputs(w))
        if name == "tiny":  # untimed first call: BLAS thread start-up, not the oracle
            oracle.attention_fp64(q, k, v, w.scale)
        t0 = time.perf_counter()
        o = oracle.attention_fp64(q, k, v, w.scale)
        oracle.ulysses_scatter(o, w.P)
        dt = time.perf_counter() - t0
        return w, dt

    from threadpoolctl import threadpool_limits

    lines = []
    for name, one_core in (("tiny", True), ("tiny", False), ("flux1024", False), ("flux2048", False),
                           ("video", False)):
        if one_core:
            with threadpool_limits(limits=1):
                w, dt = run(name)
                threads = 1
        else:
            w, dt = run(name)
            threads = blas_threads()
        rec = {"cpu_oracle": name, "B": w.B, "S": w.S, "H_local": w.H, "D": w.D, "P": w.P,
               "seconds": round(dt, 4), "GFLOPs": round(w.flops / dt / 1e9, 2), "threads": threads,
               "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0))}
        print(json.dumps(rec), flush=True)
        lines.append(rec)
    return lines


def traffic_entry(achieved_bytes_per_launch=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it is current."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def bench_attention(args, torch, xs):
    import numpy as np

    from synth import make_inputs, workload

    w = workload(args.workload)
    qb, kb, vb = make_inputs(w)

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)

    q, k, v = dev(qb), dev(kb), dev(vb)
    slabs = torch.empty((w.P, w.B, w.S // w.P, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty((w.B, w.S, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    out1 = torch.empty((w.B, w.S, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    slab_list = [slabs[p] for p in range(w.P)]

    # The caller-owned split workspace (zero-filled once; every call leaves it reusable).
    sws = xs.split_workspace(w.B, w.S, w.H, w.D)
    # Prepared launches (arguments validated and marshalled once): the host issues each
    # step in a few microseconds, well under the kernel time, so the GPU never waits on it.
    fused = xs.bind("xstage_attn_a2a_fwd", q, k, v, slab_list, w.scale, split_ws=sws)
    unfused = xs.bind("xstage_attn_a2a_unfused", q, k, v, ws, slab_list, w.scale, split_ws=sws)
    attn_only = xs.bind("xstage_attn_fwd", q, k, v, out1, w.scale, split_ws=sws)
    scatter_only = xs.bind("xstage_a2a_scatter", ws, slab_list)

    # settle: the first launches of a process run slow while the chip ramps up
    settle_n, t_settle = 0, time.perf_counter()
    while time.perf_counter() - t_settle < args.settle_s:
        for _ in range(50):
            fused()
        settle_n += 50
        torch.cuda.synchronize()

    # the timed region: exactly `steps` fused steps bracketed by synchronizations (the events
    # exist beforehand, so that the GPU idles as briefly as possible between the synchronize
    # and the first timed launch)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        fused()
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        fused()
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = start.elapsed_time(end) / args.steps

    # comparison legs: three interleaved rounds, every leg (the fused call included) with the
    # same warm-up and step count; the ratios are taken between the medians
    import statistics

    leg_steps, leg_warmup = max(args.steps, 100), max(args.warmup, 20)
    legs = {"fused": fused, "unfused": unfused, "attn": attn_only, "scatter": scatter_only}
    per = {n: [] for n in legs}
    for _ in range(3):
        for n, fn in legs.items():
            per[n].append(timed(fn, leg_steps, leg_warmup, torch))
    med = {n: statistics.median(v) for n, v in per.items()}
    ms_unfused, ms_attn, ms_scatter = med["unfused"], med["attn"], med["scatter"]

    # Full-head Ulysses layouts, as rank 5 of a group of P ranks over H_local * P heads:
    # the strided epilogue (receive buffers [B, S/P, H, D], this rank's head columns) and the
    # whole layer with the pre-attention all-to-all read from P sequence shards of all heads
    # (seeded N(0,1) shards; separate allocations).
    H_all, h0 = w.H * w.P, min(5, w.P - 1) * w.H
    recv = [torch.empty((w.B, w.S // w.P, H_all, w.D), dtype=torch.bfloat16, device="cuda") for _ in range(w.P)]
    gen = torch.Generator(device="cuda").manual_seed(w.seed + 1000)
    shards = [[torch.randn((w.B, w.S // w.P, H_all, w.D), generator=gen, device="cuda").to(torch.bfloat16)
               for _ in range(w.P)] for _ in range(3)]
    strided = xs.bind("xstage_attn_a2a_fwd_strided", q, k, v, recv, h0, w.scale, split_ws=sws)
    layer = xs.bind("xstage_ulysses_attn_fwd", shards[0], shards[1], shards[2], recv, w.H, h0, w.scale, split_ws=sws)
    ws4 = torch.empty((4, w.B, w.S, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    layer_serial = xs.bind("xstage_ulysses_attn_unfused", shards[0], shards[1], shards[2], ws4, recv, w.H, h0,
                           w.scale, split_ws=sws)
    layer_staged = xs.bind("xstage_ulysses_attn_fwd_kv_staged", shards[0], shards[1], shards[2], ws4[:2], recv,
                           w.H, h0, w.scale, split_ws=sws)
    # the same three interleaved rounds as above: the first round also absorbs the first
    # touches of the freshly allocated shard and receive buffers
    ulegs = {"strided": strided, "layer": layer, "layer_serial": layer_serial, "layer_staged": layer_staged}
    uper = {n: [] for n in ulegs}
    for _ in range(3):
        for n, fn in ulegs.items():
            uper[n].append(timed(fn, leg_steps, leg_warmup, torch))
    umed = {n: statistics.median(v) for n, v in uper.items()}
    ms_strided, ms_layer = umed["strided"], umed["layer"]
    ms_layer_serial, ms_layer_staged = umed["layer_serial"], umed["layer_staged"]
    del shards, recv, ws4

    # Core clock during the key loop (traced call, mode 3: shader-clock ticks against
    # wall-clock ticks per wave), right after back-to-back fused launches: the published
    # peak assumes 2.4 GHz, while a chip running dense MFMA work clocks lower.
    nwg, _ = xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D)
    waves = xs.xstage_attn_a2a_wg_rows(w.B, w.S, w.H, w.D) // 32
    stamps = torch.zeros(nwg * waves * 4, dtype=torch.int64, device="cuda")
    clocked = xs.bind("xstage_attn_a2a_fwd_traced", q, k, v, slab_list, 3, stamps, w.scale, split_ws=sws)
    for _ in range(args.warmup):
        fused()
    clocked()
    torch.cuda.synchronize()
    st = stamps.cpu().numpy().reshape(nwg * waves, 4).astype(np.int64)
    wall = (st[:, 1] - st[:, 0]) / xs.xstage_wallclock_hz()
    ticks = st[:, 3] - st[:, 2]
    use = wall > 2e-6
    loop_ghz = float(np.median(ticks[use] / wall[use]) / 1e9) if use.any() else None

    # Checks of the timed path's own output, outside the timed region and without any
    # reference implementation: the fused and the serial call write the same slabs bit for
    # bit, and on the placement probe (inputs whose exact attention output is V itself) the
    # fused call puts row s of V into slab s // (S/P), row s % (S/P), every element exact.
    from synth import make_placement_probe

    fused()
    torch.cuda.synchronize()
    slabs_fused = slabs.clone()
    unfused()
    torch.cuda.synchronize()
    fused_equals_serial = bool(torch.equal(slabs_fused.view(torch.int16), slabs.view(torch.int16)))
    probe_scale = 1.0 / math.sqrt(w.D)
    pq, pk, pv = (dev(x) for x in make_placement_probe(w.B, w.S, w.H, w.D, probe_scale))
    xs.xstage_attn_a2a_fwd(pq, pk, pv, slab_list, probe_scale, split_ws=sws)
    torch.cuda.synchronize()
    expect = pv.view(w.B, w.P, w.S // w.P, w.H, w.D).transpose(0, 1).contiguous()
    placement_exact = bool(torch.equal(slabs.view(torch.int16), expect.view(torch.int16)))
    del slabs_fused, pq, pk, pv, expect
    props = torch.cuda.get_device_properties(0)

    tflops = w.flops / (ms * 1e-3) / 1e12
    res = {
        "metric": METRIC if w.S == 4608 else METRIC.replace("(S=4608,", f"(S={w.S},"),
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) bf16, K x 0.5; inputs resident in HBM)",
        "config": {
            "workload": f"{w.name} share: B={w.B} S={w.S} H_local={w.H} D={w.D} P={w.P} slabs [{w.S // w.P},{w.H},{w.D}]",
            "global_batch": w.B,
            "seq_len": w.S,
            "parallelism": f"one GPU's Ulysses share (P={w.P} destination slabs in local HBM)",
        },
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "settle_s": round(args.settle_s, 3),
        "settle_launches": settle_n,
        "leg_steps": leg_steps,
        "leg_warmup": leg_warmup,
        "split_ws_bytes": 0 if sws is None else int(sws.numel()),
        "fused_vs_unfused": round(ms_unfused / med["fused"], 4),
        "fused_vs_attention_only": round(med["fused"] / ms_attn, 4),
        "ms_fused_interleaved": med["fused"],
        "ms_unfused": ms_unfused,
        "ms_attention_only": ms_attn,
        "ms_scatter_only": ms_scatter,
        "scatter_GBps": round(2 * w.out_bytes / (ms_scatter * 1e-3) / 1e9, 1),
        "ulysses_group": f"rank {h0 // w.H} of {w.P}, {H_all} heads, heads [{h0}, {h0 + w.H})",
        "ms_strided_destination": ms_strided,
        "strided_vs_fused": round(ms_strided / med["fused"], 4),
        "ms_ulysses_layer": ms_layer,
        "ulysses_layer_vs_fused": round(ms_layer / med["fused"], 4),
        "ulysses_layer_TFLOPs": round(w.flops / (ms_layer * 1e-3) / 1e12, 3),
        "ms_ulysses_layer_serial": ms_layer_serial,
        "ulysses_fused_vs_serial": round(ms_layer_serial / ms_layer, 4),
        "ms_ulysses_layer_kv_staged": ms_layer_staged,
        "ulysses_kv_staged_vs_in_place": round(ms_layer / ms_layer_staged, 4),
        "wall_s_timed_region": t_wall,
        "gpu": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                "compute_units": props.multi_processor_count},
        "fused_equals_serial": fused_equals_serial,
        "placement_probe_exact": placement_exact,
        "loop_clock_ghz": None if loop_ghz is None else round(loop_ghz, 3),
        "pct_of_peak_at_loop_clock": None if loop_ghz is None else
        round(100.0 * tflops / (PEAK_BF16_TFLOPS * loop_ghz / PEAK_CLOCK_GHZ), 2),
    }
    hbm = traffic_entry()
    res["roofline"] = {
        "bound": "mfma",
        "achieved": round(tflops, 3),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "traffic": hbm,
    }
    return w, (qb, kb, vb), res


def bench_moe(args, torch, xs):
    """Both schedules of the expert-wave stand-in on the DeepSeek-V3-sized expert layer
    (32 experts in waves of 8, d_model 7168, d_ff 2048, ~256 token rows per expert, 8
    destinations): one step is the whole layer (all launches of the schedule).  Reports the
    time of each schedule (interleaved A/B in one process), TFLOP/s, and the Linear-2 store
    spans from the per-wave stamps (end of the k loop to the last store issued)."""
    import numpy as np

    from synth import MOE_WORKLOADS, moe_routing

    w = MOE_WORKLOADS["moe_dsv3"]
    offsets, dst_slab, dst_row, out_rows = moe_routing(w)
    T = int(offsets[-1])
    g = torch.Generator(device="cuda").manual_seed(w.seed)
    x = torch.randn((T, w.d_model), generator=g, device="cuda").to(torch.bfloat16)
    w1 = (torch.randn((w.E, w.d_ff, w.d_model), generator=g, device="cuda") / math.sqrt(w.d_model)).to(torch.bfloat16)
    w2 = (torch.randn((w.E, w.d_model, w.d_ff), generator=g, device="cuda") / math.sqrt(w.d_ff)).to(torch.bfloat16)
    h = torch.empty((T, w.d_ff), dtype=torch.bfloat16, device="cuda")
    outs = [torch.empty((int(r), w.d_model), dtype=torch.bfloat16, device="cuda") for r in out_rows]
    ds = torch.from_numpy(dst_slab).cuda()
    dr = torch.from_numpy(dst_row).cuda()
    offs = [int(o) for o in offsets]
    runs = [xs.bind("xstage_moe_waves_run", x, w1, w2, h, offs, ds, dr, outs, w.experts_per_wave, sch)
            for sch in (0, 1)]
    steps = max(5, min(args.steps, 50))
    ms = {0: [], 1: []}
    for rep in range(3):
        for sch in (0, 1):
            ms[sch].append(timed(runs[sch], steps, max(3, args.warmup // 20), torch))
    flops = w.flops_per_token * T
    res = {"workload": f"{w.name}: E={w.E} experts in waves of {w.experts_per_wave}, T={T} token rows "
                       f"({w.rows_lo}-{w.rows_hi} per expert), d_model={w.d_model}, d_ff={w.d_ff}, P={w.P}",
           "flop_per_layer": flops, "steps": steps}
    spans = {}
    for sch in (0, 1):
        _, _, nl, nt = xs.xstage_moe_waves_plan(offs, w.d_model, w.d_ff, w.experts_per_wave, sch)
        stamps = torch.zeros(nt * 16, dtype=torch.int64, device="cuda")
        xs.xstage_moe_waves_run(x, w1, w2, h, offs, ds, dr, outs, w.experts_per_wave, sch, stamps=stamps)
        torch.cuda.synchronize()
        st = stamps.cpu().numpy().reshape(nt, 4, 4)
        l2 = st[:, 0, 3] == 1
        hz = xs.xstage_wallclock_hz()
        span = (st[l2][:, :, 2] - st[l2][:, :, 1]).ravel() / hz * 1e6
        spans[sch] = {"launches": nl, "l2_store_span_us_median": round(float(np.median(span)), 3),
                      "l2_store_span_us_p90": round(float(np.percentile(span, 90)), 3)}
        m = float(np.median(ms[sch]))
        name = "expert_waves" if sch == 0 else "interleaved"
        res[name] = {"ms": m, "TFLOPs": round(flops / (m * 1e-3) / 1e12, 2), **spans[sch]}
    res["interleaved_speedup"] = round(float(np.median(ms[0])) / float(np.median(ms[1])), 4)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py measures one GPU only: the P Ulysses destinations are local "
                                   "receive buffers; no collective or multi-GPU path exists (use --gpus 1)"}))
        sys.exit(2)
    import torch

    import attention_ulysses_a2a_amd as xs

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    xs.lib()  # fail loudly if the HIP library is missing
    if args.cpu_oracle_configs:
        cpu_oracle_configs()
        return
    if args.bg:
        from attention_ulysses_a2a_amd.bg_sweep import run_sweep

        run_sweep(torch, xs)
        return
    if args.xstage_study:
        from attention_ulysses_a2a_amd.xstage_study import run_study

        run_study(torch, xs, emit=lambda line: print(line, flush=True))
        return
    if args.split_study:
        from attention_ulysses_a2a_amd.split_study import random_shapes, run as run_split

        if args.split_random:
            seed, n = args.split_random
            run_split(torch, xs, shapes=random_shapes(seed, n), label=f"random seed {seed}, {n} shapes",
                      settle_s=args.settle_s, emit=lambda line: print(line, flush=True))
        else:
            run_split(torch, xs, settle_s=args.settle_s, emit=lambda line: print(line, flush=True))
        return
    if args.paced:
        from attention_ulysses_a2a_amd.paced_study import run as run_paced

        run_paced(torch, xs, settle_s=args.settle_s, emit=lambda line: print(line, flush=True))
        return
    if args.moe:
        print(json.dumps(bench_moe(args, torch, xs)), flush=True)
        return
    if args.profile_launches > 0:
        import numpy as np

        from synth import make_inputs, workload

        w = workload(args.workload)
        q, k, v = (torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).cuda().view(torch.bfloat16)
                   for b in make_inputs(w))
        slabs = torch.empty((w.P, w.B, w.S // w.P, w.H, w.D), dtype=torch.bfloat16, device="cuda")
        sws = xs.split_workspace(w.B, w.S, w.H, w.D)
        fused = xs.bind("xstage_attn_a2a_fwd", q, k, v, [slabs[p] for p in range(w.P)], w.scale, split_ws=sws)
        for _ in range(args.profile_launches):
            fused()
        torch.cuda.synchronize()
        print(json.dumps({"profile_launches": args.profile_launches, "workload": w.name}), flush=True)
        return
    if args.copy_calibration:
        # B=1, S=262144, H=8, D=128, P=8: 512 MiB read and 512 MiB written per call; the
        # input is filled once from the host, so no call finds it in the 4 MiB L2.
        B, S, H, D, P = 1, 262144, 8, 128, 8
        src = torch.ones((B, S, H, D), dtype=torch.bfloat16, device="cuda")
        dst = torch.empty((P, B, S // P, H, D), dtype=torch.bfloat16, device="cuda")
        for _ in range(args.steps):
            xs.xstage_a2a_scatter(src, dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration": {"bytes_read_per_call": B * S * H * D * 2,
                                               "bytes_written_per_call": B * S * H * D * 2, "calls": args.steps}}))
        return
    w, inputs, res = bench_attention(args, torch, xs)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, *inputs, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
