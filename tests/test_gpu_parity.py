"""Parity of the HIP path (through the C ABI) with the CPU oracle, on MI355X.

* values: fused slabs vs the fp64 oracle, max-abs <= 1e-2 and mean-abs <= 1e-3 against the
  unrounded oracle; every query row of every workload shape (the video share is ~25 s of
  float64 oracle on the host); sampled query rows (every head and batch, every slab and
  tile boundary included) only at the extra placement-table shapes;
* placement: the structured probe whose exact output is V, bit-exact in every slab element
  at every workload shape, with NaN-prefilled slabs and canary guards;
* the serial path (attention, then the separate scatter) must equal the fused path bit for bit;
* extra shapes: B=2, slab sizes that are odd or below one 32-row wave tile, key tails of 1
  and 63, a single key, negative and zero scale.
"""

import sys

import numpy as np
import pytest
import torch

import attention_ulysses_a2a_amd as xs
import oracle
from synth import Workload, make_inputs, make_placement_probe, make_placement_probe_torch, workload
from tests.gpu_util import split_ws, NAN_BF16, GuardedSlabs, to_dev, to_host

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3
WORKLOADS = ["tiny", "flux1024", "flux2048", "video"]
FULL_ORACLE = set(WORKLOADS)  # every query row of every workload against the fp64 oracle


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def sample_rows(S, S_P, n_random=256, seed=0):
    rows = {0, S - 1}
    for p in range(S // S_P):
        for d in (-1, 0, 1, 127, 128):
            s = p * S_P + d
            if 0 <= s < S:
                rows.add(s)
    for t in range(0, S, 128):
        for d in (-1, 0, 31, 32, 63, 64):
            if 0 <= t + d < S:
                rows.add(t + d)
    rng = np.random.default_rng(seed)
    rows.update(rng.integers(0, S, size=n_random).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def run_fused(w: Workload, qb, kb, vb, scale):
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.xstage_attn_a2a_fwd(q, k, v, g.views, scale, split_ws=split_ws())
    torch.cuda.synchronize()
    return g


def run_unfused(w: Workload, qb, kb, vb, scale):
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    ws = torch.empty((w.B, w.S, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.xstage_attn_a2a_unfused(q, k, v, ws, g.views, scale, split_ws=split_ws())
    torch.cuda.synchronize()
    return g


def compare_values(name, slabs_bits, qb, kb, vb, scale, rows=None):
    q, k, v = (oracle.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    o_gpu = oracle.ulysses_gather(oracle.bf16_bits_to_f64(slabs_bits))
    ref = oracle.attention_fp64(q, k, v, scale, rows=rows)
    got = o_gpu if rows is None else o_gpu[:, rows]
    err = np.abs(got - ref)
    # bf16 spacing at the oracle value: 2^(e-8) for |ref| in [2^(e-1), 2^e)
    _, e = np.frexp(ref)
    ulp = np.ldexp(1.0, np.maximum(e - 8, -133))
    ulp_ok = np.mean(np.abs(got - oracle.bf16_bits_to_f64(oracle.round_to_bf16_bits(ref))) <= ulp)
    log(f"[{name}] rows={'all' if rows is None else len(rows)} max_abs={err.max():.3e} mean_abs={err.mean():.3e} "
        f"max|o|={np.abs(ref).max():.3f} within_1ulp={ulp_ok:.5f}")
    assert np.isfinite(got).all()
    assert err.max() <= MAX_ABS, name
    assert err.mean() <= MEAN_ABS, name


@pytest.mark.parametrize("name", WORKLOADS)
def test_fused_values_match_oracle(name):
    w = workload(name)
    log(f"fused values: {name} B={w.B} S={w.S} H={w.H} D={w.D} P={w.P}")
    qb, kb, vb = make_inputs(w)
    g = run_fused(w, qb, kb, vb, w.scale)
    assert g.guards_intact()
    slabs = g.slabs_host()
    assert not np.any(slabs == NAN_BF16)
    rows = None if name in FULL_ORACLE else sample_rows(w.S, w.S // w.P)
    compare_values(name, slabs, qb, kb, vb, w.scale, rows)


@pytest.mark.parametrize("name", WORKLOADS)
def test_unfused_equals_fused_bitwise(name):
    w = workload(name)
    log(f"unfused == fused: {name}")
    qb, kb, vb = make_inputs(w)
    a = run_fused(w, qb, kb, vb, w.scale).slabs_host()
    g = run_unfused(w, qb, kb, vb, w.scale)
    assert g.guards_intact()
    assert np.array_equal(a, g.slabs_host())


@pytest.mark.parametrize("name", WORKLOADS)
def test_placement_probe_bit_exact(name):
    w = workload(name)
    log(f"placement probe: {name}")
    qb, kb, vb = make_placement_probe(w.B, w.S, w.H, w.D, w.scale)
    g = run_fused(w, qb, kb, vb, w.scale)
    assert g.guards_intact()
    slabs = g.slabs_host()
    expect = oracle.ulysses_scatter(vb, w.P)
    bad = np.argwhere(slabs != expect)
    if bad.size:
        log(f"  first mismatches (p, b, r, h, d): {bad[:5].tolist()}")
    assert bad.size == 0


EXTRA = [
    # (B, S, H, D, P, scale)
    (2, 1000, 2, 128, 8, None),     # B=2, S/P = 125 (odd), key tail 40
    (1, 999, 3, 64, 3, None),       # S/P = 333, D = 64
    (1, 1, 1, 128, 1, None),        # single key and query
    (1, 65, 2, 64, 1, None),        # key tail of 1
    (1, 127, 1, 128, 1, None),      # key tail of 63, partial query tile
    (1, 64, 2, 128, 8, None),       # 8-row slabs: a wave tile spans 4 slabs
    (2, 130, 2, 64, 2, None),       # S/P = 65
    (1, 300, 2, 128, 4, -0.05),     # negative scale
    (1, 200, 1, 64, 2, 0.0),        # zero scale: every row is the mean of V
]


@pytest.mark.parametrize("B,S,H,D,P,scale", EXTRA)
def test_extra_shapes(B, S, H, D, P, scale):
    w = Workload("extra", B, S, H, D, P, seed=11 + S + D)
    sc = w.scale if scale is None else scale
    log(f"extra: B={B} S={S} H={H} D={D} P={P} scale={sc}")
    qb, kb, vb = make_inputs(w)
    g = run_fused(w, qb, kb, vb, sc)
    assert g.guards_intact()
    slabs = g.slabs_host()
    assert not np.any(slabs == NAN_BF16)
    compare_values(f"extra-{B}x{S}x{H}x{D}/P{P}", slabs, qb, kb, vb, sc)
    assert np.array_equal(slabs, run_unfused(w, qb, kb, vb, sc).slabs_host())
    pq, pk, pv = make_placement_probe(B, S, H, D, 1.0 / np.sqrt(D))
    gp = run_fused(w, pq, pk, pv, 1.0 / np.sqrt(D))
    assert gp.guards_intact()
    assert np.array_equal(gp.slabs_host(), oracle.ulysses_scatter(pv, P))


# Shapes whose workgroups all fit on the device at once and so take key ranges sized to
# their CU placement (unequal ranges; 4 splits at D = 64, 2 splits at B = 2 and S = 9216).
TABLE_SHAPES = [
    # (B, S, H, D, P, full oracle)
    (1, 4608, 3, 64, 8, True),
    (2, 4608, 3, 128, 8, True),
    (1, 9216, 3, 128, 8, False),
]


@pytest.mark.parametrize("B,S,H,D,P,full", TABLE_SHAPES)
def test_placement_sized_key_ranges(B, S, H, D, P, full):
    tile, split, j0, j1 = (np.array(a) for a in xs.xstage_attn_a2a_schedule(B, S, H, D))
    assert len(set((j1 - j0).tolist())) > 1  # this shape takes the placement-sized ranges
    w = Workload("table", B, S, H, D, P, seed=23 + S + D + B)
    log(f"placement-sized key ranges: B={B} S={S} H={H} D={D} P={P} workgroups={len(tile)}")
    qb, kb, vb = make_inputs(w)
    g = run_fused(w, qb, kb, vb, w.scale)
    assert g.guards_intact()
    slabs = g.slabs_host()
    assert not np.any(slabs == NAN_BF16)
    compare_values(f"table-{B}x{S}x{H}x{D}", slabs, qb, kb, vb, w.scale, None if full else sample_rows(S, S // P))
    assert np.array_equal(slabs, run_unfused(w, qb, kb, vb, w.scale).slabs_host())
    pq, pk, pv = make_placement_probe(B, S, H, D, w.scale)
    gp = run_fused(w, pq, pk, pv, w.scale)
    assert gp.guards_intact()
    assert np.array_equal(gp.slabs_host(), oracle.ulysses_scatter(pv, P))


def test_largest_supported_tensor():
    """One tensor of B*S*H*D elements just below 2^31, the largest the entry points accept
    (element offsets are 32-bit): the placement probe through the fused call, every slab
    element bit-exact (O = V exactly), guards intact.  S = 32760 gives odd 4095-row slabs
    and a key tail of 56; the probe is assembled on the device (same bytes as the host
    generator, checked on the CPU)."""
    B, S, H, D, P = 1, 32760, 512, 128, 8
    assert B * S * H * D < 2 ** 31 <= B * S * (H + 1) * D
    scale = 1.0 / np.sqrt(D)
    log(f"largest tensor: B={B} S={S} H={H} D={D} P={P} ({B * S * H * D} elements)")
    q, k, v = make_placement_probe_torch(B, S, H, D, scale, "cuda")
    g = GuardedSlabs(P, B, S // P, H, D)
    xs.xstage_attn_a2a_fwd(q, k, v, g.views, scale, split_ws=split_ws())
    torch.cuda.synchronize()
    v_host = v.view(torch.int16).cpu().numpy().view(np.uint16)
    del q, k, v
    assert g.guards_intact()
    assert np.array_equal(g.slabs_host(), oracle.ulysses_scatter(v_host, P))


def test_split_counters_reset_between_shapes():
    """Every launch leaves the key-split arrival counters at zero: launches of shapes with
    different tile and split counts, issued back to back on one stream with no
    synchronisation between them, write the same bits as each shape run alone."""
    shapes = [Workload("ctr-a", 1, 4608, 3, 128, 8, seed=31),   # one-round launch, placement table
              Workload("ctr-b", 1, 2304, 3, 128, 8, seed=32),
              Workload("ctr-c", 2, 1000, 2, 64, 8, seed=33)]
    splits = [xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D)[1] for w in shapes]
    log(f"split counters: key splits per shape {splits}")
    assert all(n > 1 for n in splits)  # every shape merges through the counters (108, 54, 32 tiles)
    ins, alone = [], []
    for w in shapes:
        qb, kb, vb = make_inputs(w)
        ins.append(tuple(to_dev(x) for x in (qb, kb, vb)))
        alone.append(run_fused(w, qb, kb, vb, w.scale).slabs_host())
    outs = []
    for rep in range(3):
        for w, (q, k, v) in zip(shapes, ins):
            g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
            xs.xstage_attn_a2a_fwd(q, k, v, g.views, w.scale, split_ws=split_ws())
            outs.append(g)
    torch.cuda.synchronize()
    for i, g in enumerate(outs):
        assert g.guards_intact()
        assert np.array_equal(g.slabs_host(), alone[i % len(shapes)]), (i, shapes[i % len(shapes)].name)


def test_split_workspace_is_caller_owned():
    """The key-split partials meet in the caller's workspace (plain torch memory): a call on a
    newly created stream with a fresh zero-filled workspace of exactly the queried size gives
    the bits of the call with the shared workspace and leaves the counters at zero and every
    byte past the plan untouched; half that workspace (fewer splits) and none (no split)
    give the oracle's values within the tolerance."""
    w = workload("flux1024")
    qb, kb, vb = make_inputs(w)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    ref = run_fused(w, qb, kb, vb, w.scale).slabs_host()
    need = xs.xstage_attn_split_ws_size(w.B, w.S, w.H, w.D)
    n_tiles = w.B * w.H * ((w.S + 127) // 128)
    log(f"split workspace: {need} bytes for {xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D)} (workgroups, splits)")
    ws = torch.zeros(need + 65536, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    with torch.cuda.stream(s):
        xs.xstage_attn_a2a_fwd(q, k, v, g.views, w.scale, split_ws=ws[:need])
    s.synchronize()
    assert g.guards_intact() and np.array_equal(g.slabs_host(), ref)
    host = ws.cpu().numpy()
    assert np.all(host[:n_tiles * 4] == 0)
    assert np.all(host[need:] == 0)
    for nbytes in (need // 2, 0):
        nwg, nsp = xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D, nbytes)
        log(f"split workspace of {nbytes} bytes: {nwg} workgroups, {nsp} splits")
        assert nsp < xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D)[1]
        g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
        xs.xstage_attn_a2a_fwd(q, k, v, g.views, w.scale, split_ws=ws[:nbytes] if nbytes else None)
        torch.cuda.synchronize()
        assert g.guards_intact()
        compare_values(f"flux1024 split_ws={nbytes}", g.slabs_host(), qb, kb, vb, w.scale)
    assert np.all(ws.cpu().numpy()[:n_tiles * 4] == 0)


def test_attn_fwd_contiguous_matches_oracle():
    w = workload("tiny")
    qb, kb, vb = make_inputs(w)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    out = torch.full((w.B, w.S, w.H, w.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    xs.xstage_attn_fwd(q, k, v, out, w.scale, split_ws=split_ws())
    torch.cuda.synchronize()
    got = oracle.bf16_bits_to_f64(to_host(out))
    ref = oracle.attention_fp64(*(oracle.bf16_bits_to_f64(x) for x in (qb, kb, vb)), w.scale)
    assert np.abs(got - ref).max() <= MAX_ABS


def test_scatter_alone_bit_exact():
    B, S, H, D, P = 2, 4608, 3, 128, 8
    bits = np.random.default_rng(5).integers(0, 0x7F00, size=(B, S, H, D)).astype(np.uint16)
    g = GuardedSlabs(P, B, S // P, H, D)
    xs.xstage_a2a_scatter(to_dev(bits), g.views)
    torch.cuda.synchronize()
    assert g.guards_intact()
    assert np.array_equal(g.slabs_host(), oracle.ulysses_scatter(bits, P))


def test_rejected_call_touches_nothing():
    w = workload("tiny")
    qb, kb, vb = make_inputs(w)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    g = GuardedSlabs(3, 1, 256 // 3, w.H, w.D)  # 256 % 3 != 0
    with pytest.raises(xs.XStageError) as e:
        xs.xstage_attn_a2a_fwd(q, k, v, g.views, w.scale, split_ws=split_ws())
    assert e.value.status == xs.XSTAGE_ERR_INVALID
    torch.cuda.synchronize()
    assert np.all(g.slabs_host() == NAN_BF16) and g.guards_intact()


def test_burst_gap_stamps_and_payload():
    K, V, rounds, sets = 32, 1 << 20, 8, 2
    dst = torch.zeros(sets * V // 4, dtype=torch.int32, device="cuda")
    stamps = torch.zeros(K * rounds * 3, dtype=torch.int64, device="cuda")
    xs.xstage_burst_gap_run(K, V, 200, rounds, dst, stamps, n_dst_sets=sets)
    torch.cuda.synchronize()
    st = stamps.cpu().numpy().reshape(K, rounds, 3).astype(np.int64)
    assert np.all(st[:, :, 0] <= st[:, :, 1]) and np.all(st[:, :, 1] <= st[:, :, 2])
    assert np.all(st[:, 1:, 0] >= st[:, :-1, 2])
    assert xs.xstage_wallclock_hz() > 1e6
    words = dst.cpu().numpy().view(np.uint32).reshape(sets, K, V // K // 16, 4)
    tid = (np.arange(V // K // 16) % 256).astype(np.uint32)
    for s in range(sets):
        assert np.all(words[s, :, :, 0] == tid[None, :])
        assert np.all(words[s, :, :, 1] == np.arange(K, dtype=np.uint32)[:, None])
        assert np.all(words[s, :, :, 2] == 0x5A5A5A5A) and np.all(words[s, :, :, 3] == 0xA5A5A5A5)


def test_bound_launches_equal_direct_calls():
    """xs.bind(...) issues the same C calls: outputs equal the direct calls bit for bit, also
    over repeated launches (split counters and workspace reused between calls)."""
    w = workload("flux1024")
    qb, kb, vb = make_inputs(w)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    ref = run_fused(w, qb, kb, vb, w.scale).slabs_host()
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    fused = xs.bind("xstage_attn_a2a_fwd", q, k, v, g.views, w.scale, split_ws=split_ws())
    for _ in range(3):
        fused()
    torch.cuda.synchronize()
    assert g.guards_intact() and np.array_equal(g.slabs_host(), ref)
    ws = torch.empty((w.B, w.S, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    g2 = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.bind("xstage_attn_a2a_unfused", q, k, v, ws, g2.views, w.scale, split_ws=split_ws())()
    torch.cuda.synchronize()
    assert g2.guards_intact() and np.array_equal(g2.slabs_host(), ref)
    out = torch.empty((w.B, w.S, w.H, w.D), dtype=torch.bfloat16, device="cuda")
    xs.bind("xstage_attn_fwd", q, k, v, out, w.scale, split_ws=split_ws())()
    g3 = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.bind("xstage_a2a_scatter", out, g3.views)()
    torch.cuda.synchronize()
    assert np.array_equal(g3.slabs_host(), ref)


@pytest.mark.parametrize("name", ["tiny", "flux1024", "flux2048"])
def test_traced_modes(name):
    """The instrumented call: modes 0, 1 and 3 write the fused result bit for bit, mode 2
    writes nothing; per-wave stamps are ordered, exactly the waves owning output rows of a
    merged (or unsplit) tile record a store, and mode 3's shader-clock ticks give a
    plausible core clock."""
    w = workload(name)
    qb, kb, vb = make_inputs(w)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    ref = run_fused(w, qb, kb, vb, w.scale).slabs_host()
    nwg, nsp = xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D)
    rows = xs.xstage_attn_a2a_wg_rows(w.B, w.S, w.H, w.D)  # 256 (8 waves) at FLUX-2048
    waves = rows // 32
    log(f"[{name}] traced: {nwg} workgroups of {rows} rows, {nsp} key splits")
    for mode in (0, 1, 2):
        g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
        stamps = torch.zeros(nwg * waves * 4, dtype=torch.int64, device="cuda")
        xs.xstage_attn_a2a_fwd_traced(q, k, v, g.views, mode, stamps, w.scale, split_ws=split_ws())
        torch.cuda.synchronize()
        assert g.guards_intact()
        if mode == 2:
            assert np.all(g.slabs_host() == NAN_BF16)
        else:
            assert np.array_equal(g.slabs_host(), ref), mode
        st = stamps.cpu().numpy().reshape(nwg, waves, 4)
        assert np.all(st[:, :, 0] > 0) and np.all(st[:, :, 1] >= st[:, :, 0])
        emit = st[:, :, 2] > 0
        assert np.all(st[emit][:, 2] >= st[emit][:, 1])
        n_tiles = nwg // nsp
        row_waves = sum(min(waves, -(-(w.S - rows * (t % (n_tiles // (w.B * w.H)))) // 32)) for t in range(n_tiles))
        assert emit.sum() == (0 if mode == 2 else row_waves), (mode, emit.sum(), row_waves)
        if mode == 1:
            assert np.all(st[emit][:, 3] >= st[emit][:, 2]) and np.all(st[emit][:, 3] > 0)
        else:
            assert np.all(st[:, :, 3] == 0)
    # mode 3: the fused result, and shader-clock ticks at start / loop end in entries 2, 3
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    stamps = torch.zeros(nwg * waves * 4, dtype=torch.int64, device="cuda")
    xs.xstage_attn_a2a_fwd_traced(q, k, v, g.views, 3, stamps, w.scale, split_ws=split_ws())
    torch.cuda.synchronize()
    assert g.guards_intact() and np.array_equal(g.slabs_host(), ref)
    st = stamps.cpu().numpy().reshape(nwg, waves, 4).astype(np.int64)
    assert np.all(st[:, :, 3] >= st[:, :, 2]) and np.all(st[:, :, 2] > 0)
    long = (st[:, :, 1] - st[:, :, 0]) > 200  # loops of >= 2 us of wall clock
    ghz = (st[:, :, 3] - st[:, :, 2])[long] / ((st[:, :, 1] - st[:, :, 0])[long] / xs.xstage_wallclock_hz()) / 1e9
    log(f"[{name}] shader clock during the key loop: median {np.median(ghz) if ghz.size else float('nan'):.3f} GHz")
    assert ghz.size == 0 or (0.3 < np.median(ghz) < 3.5)
