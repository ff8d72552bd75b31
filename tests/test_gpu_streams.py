"""Fused calls running concurrently on two streams with separate split workspaces, on MI355X.

The header allows calls on different streams to run at once when each has its own split
workspace (the arrival counters and partial records of one launch never meet the other's).
Two shapes with key splits, a one-round launch of 4-wave workgroups with placement-sized key
ranges (the FLUX-1024 share) and a multi-round launch of 8-wave workgroups (B=1, S=12288,
H_local=4, D=128: 4 splits), are issued alternately on two streams, ten calls each, so that
their workgroups share the device; each stream's slabs must equal its shape run alone, bit
for bit (the fused call of X-Stage explainer, "Contributions", FlashAttention-A2A item), and
every guard must stay intact.
"""

import sys

import numpy as np
import pytest
import torch

import attention_ulysses_a2a_amd as xs
from synth import Workload, make_inputs, workload
from tests.gpu_util import NAN_BF16, GuardedSlabs, to_dev

pytestmark = pytest.mark.gpu


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_two_streams_with_separate_workspaces():
    shapes = [workload("flux1024"), Workload("streams-wide", 1, 12288, 4, 128, 8, seed=77)]
    runs = []
    for w in shapes:
        nwg, nsp = xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D)
        rows = xs.xstage_attn_a2a_wg_rows(w.B, w.S, w.H, w.D)
        log(f"streams: {w.name} B={w.B} S={w.S} H={w.H} D={w.D}: {nwg} workgroups of {rows} rows, {nsp} key splits")
        assert nsp > 1
        qb, kb, vb = make_inputs(w)
        q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
        # alone, on the default stream, with a workspace of its own
        ref = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
        xs.xstage_attn_a2a_fwd(q, k, v, ref.views, w.scale, split_ws=xs.split_workspace(w.B, w.S, w.H, w.D))
        torch.cuda.synchronize()
        assert ref.guards_intact()
        runs.append((w, (q, k, v), ref.slabs_host()))
    assert rows == 256 and xs.xstage_attn_a2a_wg_rows(1, 4608, 3, 128) == 128
    streams = [torch.cuda.Stream() for _ in runs]
    outs = [GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D) for w, _, _ in runs]
    wss = [xs.split_workspace(w.B, w.S, w.H, w.D) for w, _, _ in runs]
    torch.cuda.synchronize()
    calls = [xs.bind("xstage_attn_a2a_fwd", q, k, v, g.views, w.scale, split_ws=ws, stream=s)
             for (w, (q, k, v), _), g, ws, s in zip(runs, outs, wss, streams)]
    for _ in range(10):
        for c in calls:
            c()
    torch.cuda.synchronize()
    for (w, _, ref), g in zip(runs, outs):
        got = g.slabs_host()
        log(f"  {w.name}: guards intact {g.guards_intact()}, equal to the lone run {np.array_equal(got, ref)}")
        assert g.guards_intact()
        assert not np.any(got == NAN_BF16)
        assert np.array_equal(got, ref), w.name
    # both workspaces are left with their counters at zero
    for ws in wss:
        assert int(torch.count_nonzero(ws[:16384])) == 0
