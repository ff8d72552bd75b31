"""Launches of 256-row workgroups (8 waves sharing each K/V block in LDS) on MI355X.

The fused call (X-Stage explainer, "Contributions", FlashAttention-A2A item: attention
followed by the post-attention all-to-all) picks 8-wave workgroups when the 4-wave launch
would keep every CU at two workgroups without placement-sized key ranges and every (b, h)
has an even number of 128-row tiles.  Each query row then sees the same key ranges in the
same merge order as with 4 waves, so the result must be the 4-wave result bit for bit: the
paced mode (always 4 waves, unsplit, documented equal to the unsplit fused call) is the
4-wave reference for unsplit launches.  Split 8-wave launches, and six seeded random 8-wave
shapes (D 64 and 128, unsplit and split, negative scales), are checked against the fp64
oracle on sampled rows, against the serial path bit for bit, and with the placement probe.
Ragged shapes put the last 256-row tile partly (or, for some waves, wholly) past S.
"""

import sys

import numpy as np
import pytest
import torch

import attention_ulysses_a2a_amd as xs
import oracle
from synth import Workload, make_inputs, make_placement_probe
from tests.gpu_util import NAN_BF16, GuardedSlabs, split_ws, to_dev
from tests.test_gpu_parity import compare_values, sample_rows

pytestmark = pytest.mark.gpu

UNSPLIT = [
    # (B, S, H, D, P): 8-wave launches without key splits
    (1, 16300, 4, 128, 4),  # last tile: 172 rows (waves 6 and 7 own none)
    (1, 16300, 4, 64, 4),
    (2, 16300, 2, 128, 2),
]
SPLIT = [
    (1, 12288, 4, 128, 8),  # 4 key splits, 768 workgroups
    (1, 12200, 4, 128, 8),  # ragged rows and keys
]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _fused(w, qb, kb, vb, ws, scale=None):
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.xstage_attn_a2a_fwd(q, k, v, g.views, w.scale if scale is None else scale, split_ws=ws)
    torch.cuda.synchronize()
    assert g.guards_intact()
    return g.slabs_host()


@pytest.mark.parametrize("B,S,H,D,P", UNSPLIT)
def test_eight_waves_equal_four_waves(B, S, H, D, P):
    assert xs.xstage_attn_a2a_wg_rows(B, S, H, D, 0) == 256
    assert xs.xstage_attn_a2a_plan(B, S, H, D, 0)[1] == 1
    w = Workload("wide", B, S, H, D, P, seed=61 + S + D)
    log(f"8 waves vs 4: B={B} S={S} H={H} D={D} P={P}")
    qb, kb, vb = make_inputs(w)
    wide = _fused(w, qb, kb, vb, None)
    assert not np.any(wide == NAN_BF16)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.xstage_attn_a2a_fwd_paced(q, k, v, g.views, 1, w.scale)  # 4 waves, unsplit
    torch.cuda.synchronize()
    assert g.guards_intact()
    log(f"  equal bit for bit: {np.array_equal(wide, g.slabs_host())}")
    assert np.array_equal(wide, g.slabs_host())


@pytest.mark.parametrize("B,S,H,D,P", SPLIT)
def test_eight_wave_splits(B, S, H, D, P):
    assert xs.xstage_attn_a2a_wg_rows(B, S, H, D) == 256
    nwg, nsp = xs.xstage_attn_a2a_plan(B, S, H, D)
    assert nsp > 1
    w = Workload("wide-split", B, S, H, D, P, seed=71 + S)
    log(f"8-wave splits: B={B} S={S} H={H} D={D} P={P}: {nwg} workgroups, {nsp} key splits")
    qb, kb, vb = make_inputs(w)
    slabs = _fused(w, qb, kb, vb, split_ws())
    assert not np.any(slabs == NAN_BF16)
    compare_values(f"wide-{B}x{S}x{H}x{D}", slabs, qb, kb, vb, w.scale, sample_rows(S, S // P, n_random=96, seed=S))
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    ws = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.xstage_attn_a2a_unfused(q, k, v, ws, g.views, w.scale, split_ws=split_ws())
    torch.cuda.synchronize()
    assert g.guards_intact() and np.array_equal(g.slabs_host(), slabs)
    pq, pk, pv = make_placement_probe(B, S, H, D, 1.0 / np.sqrt(D))
    got = _fused(w, pq, pk, pv, split_ws(), scale=1.0 / np.sqrt(D))
    log(f"  placement probe exact: {np.array_equal(got, oracle.ulysses_scatter(pv, P))}")
    assert np.array_equal(got, oracle.ulysses_scatter(pv, P))


# Seeded draw (numpy default_rng(909): B 1-2, H 1-8, D 64/128, P in {2, 3, 4, 5, 8}, S a
# multiple of P in [3000, 20000), kept when the launch runs 256-row workgroups), with scales
# set here: unsplit and split launches, last 256-row tiles of 130-248 rows.
RANDOM_WIDE = [
    (2, 7416, 8, 64, 8, None),
    (2, 11656, 4, 64, 4, -0.1154),
    (2, 16002, 8, 128, 2, None),
    (1, 11730, 3, 64, 5, 0.2386),
    (1, 19600, 8, 128, 2, None),
    (1, 7080, 5, 64, 4, -0.0641),
]


@pytest.mark.parametrize("B,S,H,D,P,scale", RANDOM_WIDE)
def test_random_eight_wave_shapes(B, S, H, D, P, scale):
    assert xs.xstage_attn_a2a_wg_rows(B, S, H, D) == 256
    nwg, nsp = xs.xstage_attn_a2a_plan(B, S, H, D)
    w = Workload("wide-random", B, S, H, D, P, seed=S + 3 * H)
    sc = w.scale if scale is None else scale
    log(f"random 8-wave shape: B={B} S={S} H={H} D={D} P={P} scale={sc:.4f}: {nwg} workgroups, {nsp} key splits")
    qb, kb, vb = make_inputs(w)
    slabs = _fused(w, qb, kb, vb, split_ws(), scale=sc)
    assert not np.any(slabs == NAN_BF16)
    compare_values(f"wide-random-{B}x{S}x{H}x{D}/P{P}", slabs, qb, kb, vb, sc, sample_rows(S, S // P, n_random=48, seed=S))
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    ws = torch.empty((B, S, H, D), dtype=torch.bfloat16, device="cuda")
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.xstage_attn_a2a_unfused(q, k, v, ws, g.views, sc, split_ws=split_ws())
    torch.cuda.synchronize()
    assert g.guards_intact() and np.array_equal(g.slabs_host(), slabs)
    pq, pk, pv = make_placement_probe(B, S, H, D, 1.0 / np.sqrt(D))
    got = _fused(w, pq, pk, pv, split_ws(), scale=1.0 / np.sqrt(D))
    assert np.array_equal(got, oracle.ulysses_scatter(pv, P))
