"""The fused calls captured into a HIP graph and replayed, on MI355X.

No entry point allocates or synchronizes, and every call leaves its split counters at zero,
so a call can be recorded once into a graph (stream capture) and replayed.  Each case
records one call (the fused call of X-Stage explainer, "Contributions", FlashAttention-A2A
item) with the caller's split workspace: a one-round launch of 4-wave workgroups with the unit
table (the FLUX-1024 share) and a multi-round launch of 8-wave workgroups (B=1, S=12288,
H_local=4: 4 splits); and the no-allocation call (its static scratch set up by an eager call
first).  Between replays the slabs are refilled with NaN by eager work on the same stream and
the device is synchronized; every replay must write the eager call's slabs bit for bit and
leave the guards intact.  The recorded calls hold only kernel nodes (no memset nodes).
"""

import sys

import numpy as np
import pytest
import torch

import attention_ulysses_a2a_amd as xs
from synth import Workload, make_inputs, workload
from tests.gpu_util import NAN_BF16, GuardedSlabs, to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _refill(g):
    for v in g.views:
        v.view(torch.int16).fill_(NAN_BF16)


def _check_replays(name, call, g, ref):
    # one eager run on a side stream before the capture, as stream capture expects
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        _refill(g)
        graph.replay()
        torch.cuda.synchronize()
        got = g.slabs_host()
        log(f"  {name} replay {rep}: equal to the eager call {np.array_equal(got, ref)}")
        assert g.guards_intact()
        assert not np.any(got == NAN_BF16)
        assert np.array_equal(got, ref), (name, rep)
    del graph


@pytest.mark.parametrize("name", ["flux1024", "wide-split"])
def test_fused_call_replays_from_a_graph(name):
    w = workload("flux1024") if name == "flux1024" else Workload("graph-wide", 1, 12288, 4, 128, 8, seed=81)
    nwg, nsp = xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D)
    rows = xs.xstage_attn_a2a_wg_rows(w.B, w.S, w.H, w.D)
    log(f"graph: {w.name} B={w.B} S={w.S} H={w.H} D={w.D}: {nwg} workgroups of {rows} rows, {nsp} key splits")
    assert nsp > 1 and rows == (128 if name == "flux1024" else 256)
    qb, kb, vb = make_inputs(w)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    ws = xs.split_workspace(w.B, w.S, w.H, w.D)
    ref_g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.xstage_attn_a2a_fwd(q, k, v, ref_g.views, w.scale, split_ws=ws)
    torch.cuda.synchronize()
    ref = ref_g.slabs_host()
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    # the stream is taken at call time: inside the capture it is the capturing stream
    _check_replays(w.name, lambda: xs.xstage_attn_a2a_fwd(q, k, v, g.views, w.scale, split_ws=ws), g, ref)
    assert int(torch.count_nonzero(ws[:16384])) == 0


def test_noalloc_call_replays_from_a_graph():
    w = workload("flux1024")
    qb, kb, vb = make_inputs(w)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    log(f"graph: no-allocation call, {w.name}")
    ref_g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.xstage_attn_a2a_fwd_noalloc(q, k, v, ref_g.views, w.scale)  # also sets up the static scratch
    torch.cuda.synchronize()
    ref = ref_g.slabs_host()
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    _check_replays("noalloc", lambda: xs.xstage_attn_a2a_fwd_noalloc(q, k, v, g.views, w.scale), g, ref)
