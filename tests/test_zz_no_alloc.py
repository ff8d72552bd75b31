"""The no-allocation fused call (xstage_attn_a2a_fwd_noalloc), through the C ABI, on MI355X.

Its split partials live in the library's static device array instead of a caller
workspace: two calls in a row (the FLUX-1024 share, then a smaller split shape) must write
the bits xstage_attn_a2a_fwd writes with a 32 MiB workspace (the same plan), match the
fp64 oracle within the tolerance, leave every guard intact, and change no device memory
allocation (free device memory is the same before and after the calls that follow the
first).
"""

import sys

import numpy as np
import pytest
import torch

import attention_ulysses_a2a_amd as xs
import oracle
from synth import Workload, make_inputs, workload
from tests.gpu_util import NAN_BF16, GuardedSlabs, to_dev

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20
MAX_ABS, MEAN_ABS = 1e-2, 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_matches_workspace_call():
    shapes = [workload("flux1024"), Workload("noalloc-small", 1, 2304, 3, 128, 8, seed=52)]
    ins = []
    for w in shapes:
        nwg, nsp = xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D, SCRATCH_BYTES)
        log(f"no-alloc: {w.name} B={w.B} S={w.S} H={w.H} D={w.D} P={w.P}: {nwg} workgroups, {nsp} key splits")
        assert nsp > 1  # both shapes merge through the scratch
        qb, kb, vb = make_inputs(w)
        ins.append((w, (qb, kb, vb), tuple(to_dev(x) for x in (qb, kb, vb))))
    # reference: the workspace entry point with a workspace of the scratch's size
    ws = torch.zeros(SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    refs = []
    for w, _, (q, k, v) in ins:
        g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
        xs.xstage_attn_a2a_fwd(q, k, v, g.views, w.scale, split_ws=ws)
        refs.append(g)
    outs = [GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D) for w, _, _ in ins]
    torch.cuda.synchronize()
    # two no-alloc calls in a row (no synchronisation between them), the second smaller
    for (w, _, (q, k, v)), g in zip(ins, outs):
        xs.xstage_attn_a2a_fwd_noalloc(q, k, v, g.views, w.scale)
    # and once more each, after the first call's set-up: no device memory changes hands
    again = [GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D) for w, _, _ in ins]
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info()[0]
    for (w, _, (q, k, v)), g in zip(ins, again):
        xs.xstage_attn_a2a_fwd_noalloc(q, k, v, g.views, w.scale)
    torch.cuda.synchronize()
    assert torch.cuda.mem_get_info()[0] == free_before
    for (w, (qb, kb, vb), _), ref, g, g2 in zip(ins, refs, outs, again):
        got = g.slabs_host()
        assert g.guards_intact() and g2.guards_intact()
        assert not np.any(got == NAN_BF16)
        assert np.array_equal(got, ref.slabs_host()), w.name
        assert np.array_equal(g2.slabs_host(), got), w.name
        q64, k64, v64 = (oracle.bf16_bits_to_f64(x) for x in (qb, kb, vb))
        o = oracle.ulysses_gather(oracle.bf16_bits_to_f64(got))
        err = np.abs(o - oracle.attention_fp64(q64, k64, v64, w.scale))
        log(f"no-alloc [{w.name}] max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, w.name


def test_noalloc_eight_wave_launch():
    """A launch of 256-row (8-wave) workgroups whose key splits merge through the static scratch
    (B=1, S=12288, H_local=3: 3 splits in a 32 MiB scratch, 432 workgroups in ~1.7 rounds):
    the bits of the workspace call with a workspace of the scratch's size, and the oracle's
    values on sampled rows."""
    w = Workload("noalloc-wide", 1, 12288, 3, 128, 8, seed=53)
    nwg, nsp = xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D, SCRATCH_BYTES)
    rows = xs.xstage_attn_a2a_wg_rows(w.B, w.S, w.H, w.D, SCRATCH_BYTES)
    log(f"no-alloc: {w.name} B={w.B} S={w.S} H={w.H} D={w.D} P={w.P}: {nwg} workgroups of {rows} rows, {nsp} key splits")
    assert rows == 256 and nsp > 1
    qb, kb, vb = make_inputs(w)
    q, k, v = (to_dev(x) for x in (qb, kb, vb))
    ws = torch.zeros(SCRATCH_BYTES, dtype=torch.uint8, device="cuda")
    ref = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.xstage_attn_a2a_fwd(q, k, v, ref.views, w.scale, split_ws=ws)
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    xs.xstage_attn_a2a_fwd_noalloc(q, k, v, g.views, w.scale)
    torch.cuda.synchronize()
    got = g.slabs_host()
    assert g.guards_intact() and ref.guards_intact()
    assert not np.any(got == NAN_BF16)
    assert np.array_equal(got, ref.slabs_host())
    rows_s = np.unique(np.concatenate([np.arange(0, w.S, 97), np.arange(w.S - 40, w.S)]))
    q64, k64, v64 = (oracle.bf16_bits_to_f64(x) for x in (qb, kb, vb))
    o = oracle.ulysses_gather(oracle.bf16_bits_to_f64(got))[:, rows_s]
    want = oracle.attention_fp64(q64, k64, v64, w.scale, rows=rows_s)
    err = np.abs(o - want)
    log(f"no-alloc [{w.name}] sampled rows {len(rows_s)}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
