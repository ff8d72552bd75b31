"""The paced persistent fused call on MI355X (xstage_attn_a2a_fwd_paced).

The Burst-Gap model used to shape the epilogue burst (X-Stage explainer, "Significance";
"Methodology"): each workgroup runs several tiles in turn and issues a finished tile's rows in
c chunks over the next tile's first key-loop iterations.  Pacing moves stores in time only,
so for every chunk count the slabs must equal the unsplit product call's bit for bit (same
per-tile arithmetic), the placement probe must come out exact, and the values must match the
fp64 oracle.  Shapes have more tiles than the launch has workgroups, so that workgroups do
carry a tile's rows into the next tile's loop: a ragged sequence (the last m-tile half
full), D = 64 with four tiles per workgroup, and a short sequence whose tiles have one
key-loop iteration (chunks left over are issued after the loop) and 25-row slabs (a wave's
rows span three slabs).
"""

import sys

import numpy as np
import pytest
import torch

import attention_ulysses_a2a_amd as xs
import oracle
from synth import Workload, make_inputs, make_placement_probe
from tests.gpu_util import NAN_BF16, GuardedSlabs, to_dev
from tests.test_gpu_parity import compare_values, sample_rows

pytestmark = pytest.mark.gpu

SHAPES = [
    # (B, S, H, D, P)
    (2, 4160, 5, 128, 8),
    (1, 8192, 16, 64, 8),
    (4, 200, 40, 128, 8),
]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def chunk_counts(D):
    return (1, 2, 4, 8) if D == 128 else (1, 2, 4)


def _run(fn, w, qb, kb, vb, scale):
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    fn(q, k, v, g.views, scale)
    torch.cuda.synchronize()
    assert g.guards_intact()
    return g.slabs_host()


@pytest.mark.parametrize("B,S,H,D,P", SHAPES)
def test_paced_equals_unsplit_product(B, S, H, D, P):
    w = Workload("paced", B, S, H, D, P, seed=23 + S + H)
    n_wg, n_tiles = xs.xstage_attn_a2a_paced_plan(B, S, H, D)
    log(f"paced: B={B} S={S} H={H} D={D} P={P}: {n_tiles} tiles on {n_wg} workgroups")
    assert n_tiles == B * H * ((S + 127) // 128)
    assert 0 < n_wg < n_tiles  # workgroups run more than one tile
    qb, kb, vb = make_inputs(w)
    ref = _run(lambda q, k, v, s, sc: xs.xstage_attn_a2a_fwd(q, k, v, s, sc, split_ws=None), w, qb, kb, vb, w.scale)
    assert not np.any(ref == NAN_BF16)
    for c in chunk_counts(D):
        got = _run(lambda q, k, v, s, sc: xs.xstage_attn_a2a_fwd_paced(q, k, v, s, c, sc), w, qb, kb, vb, w.scale)
        log(f"  chunks={c}: equal to the unsplit product call: {np.array_equal(got, ref)}")
        assert np.array_equal(got, ref), c
    rows = sample_rows(S, S // P, n_random=128, seed=S)
    compare_values(f"paced-{B}x{S}x{H}x{D}/P{P}", ref, qb, kb, vb, w.scale, rows)


@pytest.mark.parametrize("B,S,H,D,P", SHAPES)
def test_paced_placement_probe_exact(B, S, H, D, P):
    w = Workload("paced-probe", B, S, H, D, P, seed=5)
    pq, pk, pv = make_placement_probe(B, S, H, D, 1.0 / np.sqrt(D))
    want = oracle.ulysses_scatter(pv, P)
    for c in (1, chunk_counts(D)[-1]):
        got = _run(lambda q, k, v, s, sc: xs.xstage_attn_a2a_fwd_paced(q, k, v, s, c, sc), w, pq, pk, pv,
                   1.0 / np.sqrt(D))
        log(f"paced probe B={B} S={S} H={H} D={D} P={P} chunks={c}: exact {np.array_equal(got, want)}")
        assert np.array_equal(got, want), c
