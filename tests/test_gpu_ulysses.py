"""Parity of the full-head Ulysses entry points (through the C ABI) on MI355X.

* xstage_attn_a2a_fwd_strided: destination buffers hold all H_dst heads; the call's head
  columns must equal the plain fused path's slabs bit for bit, and every other element
  (NaN-prefilled) and the canary guards must be untouched;
* xstage_ulysses_attn_fwd: inputs are P sequence shards of all H heads (separate
  allocations); the output must equal gathering the rank's heads into contiguous q, k, v
  and calling the strided path, bit for bit; values against the oracle's Ulysses layer
  (oracle.ulysses_attention: explicit gather, fp64 attention, explicit scatter), every
  query row at every shape up to the FLUX-1024 and video groups; shard sizes
  that are odd or below one 64-key block make key blocks straddle shards;
* xstage_ulysses_attn_fwd_kv_staged (K and V gathered into a workspace, Q read in place)
  equals xstage_ulysses_attn_fwd bit for bit at every layer shape;
* the placement probe (exact output = V) through both all-to-alls, bit-exact.
"""

import sys

import numpy as np
import pytest
import torch

import attention_ulysses_a2a_amd as xs
import oracle
from synth import Workload, make_inputs, make_placement_probe
from tests.gpu_util import split_ws, NAN_BF16, GuardedSlabs, to_dev

pytestmark = pytest.mark.gpu

MAX_ABS, MEAN_ABS = 1e-2, 1e-3


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def shards_of(x_bits, P):
    """[B, S, H, D] -> P contiguous arrays [B, S/P, H, D] (plain slicing)."""
    sp = x_bits.shape[1] // P
    return [np.ascontiguousarray(x_bits[:, p * sp:(p + 1) * sp]) for p in range(P)]


def sample_rows(S, P, n=192, seed=0):
    sp = S // P
    rows = {0, S - 1}
    for p in range(P):
        for d in (-1, 0, 1, 63, 64):
            if 0 <= p * sp + d < S:
                rows.add(p * sp + d)
    rows.update(np.random.default_rng(seed).integers(0, S, size=n).tolist())
    return np.array(sorted(rows), dtype=np.int64)


def check_values(name, got_bits, ref):
    got = oracle.bf16_bits_to_f64(got_bits)
    err = np.abs(got - ref)
    log(f"[{name}] max_abs={err.max():.3e} mean_abs={err.mean():.3e} max|o|={np.abs(ref).max():.3f}")
    assert np.isfinite(got).all()
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, name


STRIDED = [
    # (B, S, H_local, D, P, H_dst, h_dst0)
    (1, 256, 2, 64, 2, 4, 2),
    (2, 1000, 2, 128, 8, 6, 3),      # odd slabs (125 rows)
    (1, 64, 1, 128, 8, 3, 1),        # 8-row slabs
    (1, 4608, 3, 128, 8, 24, 15),    # FLUX-1024 group, rank 5 (placement-sized key ranges)
]


@pytest.mark.parametrize("B,S,H,D,P,Hd,h0", STRIDED)
def test_strided_destination(B, S, H, D, P, Hd, h0):
    log(f"strided: B={B} S={S} H_local={H} D={D} P={P} H_dst={Hd} h0={h0}")
    w = Workload("strided", B, S, H, D, P, seed=31 + S + H)
    qb, kb, vb = make_inputs(w)
    q, k, v = to_dev(qb), to_dev(kb), to_dev(vb)
    plain = GuardedSlabs(P, B, S // P, H, D)
    xs.xstage_attn_a2a_fwd(q, k, v, plain.views, w.scale, split_ws=split_ws())
    full = GuardedSlabs(P, B, S // P, Hd, D)
    xs.xstage_attn_a2a_fwd_strided(q, k, v, full.views, h0, w.scale, split_ws=split_ws())
    torch.cuda.synchronize()
    assert full.guards_intact()
    got = full.slabs_host()
    assert np.array_equal(got[:, :, :, h0:h0 + H], plain.slabs_host())
    assert np.all(got[:, :, :, :h0] == NAN_BF16) and np.all(got[:, :, :, h0 + H:] == NAN_BF16)
    # probe: exact output V, through the strided epilogue
    pq, pk, pv = make_placement_probe(B, S, H, D, w.scale)
    probe = GuardedSlabs(P, B, S // P, Hd, D)
    xs.xstage_attn_a2a_fwd_strided(to_dev(pq), to_dev(pk), to_dev(pv), probe.views, h0, w.scale, split_ws=split_ws())
    torch.cuda.synchronize()
    assert probe.guards_intact()
    assert np.array_equal(probe.slabs_host()[:, :, :, h0:h0 + H], oracle.ulysses_scatter(pv, P))


ULYSSES = [
    # (B, S, H, H_local, h0, D, P, full oracle)
    (1, 256, 4, 2, 2, 64, 2, True),
    (2, 1000, 4, 2, 0, 128, 8, True),     # 125-row shards: key blocks straddle shards
    (1, 64, 2, 1, 1, 128, 8, True),       # 8-row shards: one key block spans all 8
    (1, 999, 3, 1, 1, 64, 3, True),       # 333-row shards, D = 64
    (1, 4608, 24, 3, 15, 128, 8, True),   # FLUX-1024 group, rank 5
    (1, 32760, 40, 5, 15, 128, 8, True),  # video group, rank 3: 4095-row shards, key tail 56
]


@pytest.mark.parametrize("B,S,H,Hl,h0,D,P,full", ULYSSES)
def test_ulysses_layer(B, S, H, Hl, h0, D, P, full):
    log(f"ulysses: B={B} S={S} H={H} H_local={Hl} h0={h0} D={D} P={P}")
    w = Workload("ulysses", B, S, H, D, P, seed=41 + S + H)
    qb, kb, vb = make_inputs(w)
    qs, ks, vs = ([to_dev(x) for x in shards_of(t, P)] for t in (qb, kb, vb))
    out = GuardedSlabs(P, B, S // P, H, D)
    xs.xstage_ulysses_attn_fwd(qs, ks, vs, out.views, Hl, h0, w.scale, split_ws=split_ws())
    # the same heads gathered into contiguous tensors, through the strided path
    ref = GuardedSlabs(P, B, S // P, H, D)
    qc, kc, vc = (to_dev(np.ascontiguousarray(t[:, :, h0:h0 + Hl])) for t in (qb, kb, vb))
    xs.xstage_attn_a2a_fwd_strided(qc, kc, vc, ref.views, h0, w.scale, split_ws=split_ws())
    # K and V staged in a workspace, Q read from the shards
    staged = GuardedSlabs(P, B, S // P, H, D)
    ws = torch.full((2, B, S, Hl, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    xs.xstage_ulysses_attn_fwd_kv_staged(qs, ks, vs, ws, staged.views, Hl, h0, w.scale, split_ws=split_ws())
    torch.cuda.synchronize()
    assert out.guards_intact() and staged.guards_intact()
    got = out.slabs_host()
    assert np.all(got[:, :, :, :h0] == NAN_BF16) and np.all(got[:, :, :, h0 + Hl:] == NAN_BF16)
    assert np.array_equal(got, ref.slabs_host())
    assert np.array_equal(staged.slabs_host(), got)
    # values against the oracle's layer (explicit gather, fp64 attention, explicit scatter)
    rows = None if full else sample_rows(S, P)
    f64 = [[oracle.bf16_bits_to_f64(x) for x in shards_of(t, P)] for t in (qb, kb, vb)]
    dst = [np.full((B, S // P, H, D), np.nan) for _ in range(P)]
    oracle.ulysses_attention(f64[0], f64[1], f64[2], w.scale, h0, Hl, dst, rows=rows)
    dst = np.stack(dst)
    sel = np.isfinite(dst)
    assert sel.any()
    check_values(f"ulysses-{B}x{S}x{H}/{Hl}@{h0}", got[sel], dst[sel])


@pytest.mark.parametrize("B,S,H,Hl,h0,D,P", [(1, 256, 4, 2, 2, 64, 2), (2, 1000, 4, 2, 2, 128, 8), (1, 64, 2, 1, 0, 128, 8)])
def test_ulysses_placement_probe(B, S, H, Hl, h0, D, P):
    scale = 1.0 / np.sqrt(D)
    pq, pk, pv = make_placement_probe(B, S, H, D, scale)
    qs, ks, vs = ([to_dev(x) for x in shards_of(t, P)] for t in (pq, pk, pv))
    out = GuardedSlabs(P, B, S // P, H, D)
    xs.xstage_ulysses_attn_fwd(qs, ks, vs, out.views, Hl, h0, scale, split_ws=split_ws())
    staged = GuardedSlabs(P, B, S // P, H, D)
    ws = torch.empty((2, B, S, Hl, D), dtype=torch.bfloat16, device="cuda")
    xs.xstage_ulysses_attn_fwd_kv_staged(qs, ks, vs, ws, staged.views, Hl, h0, scale, split_ws=split_ws())
    torch.cuda.synchronize()
    assert out.guards_intact() and staged.guards_intact()
    got = out.slabs_host()
    assert np.array_equal(got[:, :, :, h0:h0 + Hl], oracle.ulysses_scatter(pv, P)[:, :, :, h0:h0 + Hl])
    assert np.all(got[:, :, :, :h0] == NAN_BF16) and np.all(got[:, :, :, h0 + Hl:] == NAN_BF16)
    assert np.array_equal(staged.slabs_host(), got)


def test_bound_ulysses_equals_direct():
    B, S, H, Hl, h0, D, P = 1, 512, 4, 2, 2, 64, 4
    w = Workload("bind", B, S, H, D, P, seed=5)
    qb, kb, vb = make_inputs(w)
    stacked = [to_dev(np.stack(shards_of(t, P))) for t in (qb, kb, vb)]  # [P, B, S/P, H, D]
    a = GuardedSlabs(P, B, S // P, H, D)
    b = GuardedSlabs(P, B, S // P, H, D)
    xs.xstage_ulysses_attn_fwd(*stacked, a.views, Hl, h0, w.scale, split_ws=split_ws())
    f = xs.bind("xstage_ulysses_attn_fwd", *stacked, b.views, Hl, h0, w.scale, split_ws=split_ws())
    f()
    f()
    torch.cuda.synchronize()
    assert np.array_equal(a.slabs_host(), b.slabs_host())


COPY_SHAPES = [
    # (B, S, H, H_local, h0, D, P)
    (2, 1000, 4, 2, 2, 128, 8),   # 125-row shards
    (1, 64, 2, 1, 1, 64, 8),      # 8-row shards
    (1, 4608, 24, 3, 15, 128, 8), # FLUX-1024 group, rank 5
]


@pytest.mark.parametrize("B,S,H,Hl,h0,D,P", COPY_SHAPES)
def test_separate_all_to_alls_bit_exact(B, S, H, Hl, h0, D, P):
    """The serial layer's copies: the gather equals slicing the rank's heads out of the full
    tensor, the strided scatter equals the oracle's full-head scatter, bit for bit."""
    log(f"separate all-to-alls: B={B} S={S} H={H} H_local={Hl} h0={h0} D={D} P={P}")
    rng = np.random.default_rng(S + H)
    full = rng.integers(0, 0x7F00, size=(B, S, H, D), dtype=np.uint16)
    shards = [to_dev(x) for x in shards_of(full, P)]
    out = torch.full((B, S, Hl, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    xs.xstage_ulysses_gather(shards, out, Hl, h0)
    torch.cuda.synchronize()
    from tests.gpu_util import to_host
    assert np.array_equal(to_host(out), full[:, :, h0:h0 + Hl])
    local = rng.integers(0, 0x7F00, size=(B, S, Hl, D), dtype=np.uint16)
    dst = GuardedSlabs(P, B, S // P, H, D)
    xs.xstage_a2a_scatter_strided(to_dev(local), dst.views, h0)
    torch.cuda.synchronize()
    assert dst.guards_intact()
    expect = [np.full((B, S // P, H, D), NAN_BF16, dtype=np.uint16) for _ in range(P)]
    oracle.scatter_heads(local, expect, h0)
    assert np.array_equal(dst.slabs_host(), np.stack(expect))


@pytest.mark.parametrize("B,S,H,Hl,h0,D,P", COPY_SHAPES)
def test_ulysses_unfused_equals_fused(B, S, H, Hl, h0, D, P):
    log(f"ulysses unfused == fused: B={B} S={S} H={H} H_local={Hl} h0={h0} D={D} P={P}")
    w = Workload("ulysses-serial", B, S, H, D, P, seed=61 + S + H)
    qb, kb, vb = make_inputs(w)
    qs, ks, vs = ([to_dev(x) for x in shards_of(t, P)] for t in (qb, kb, vb))
    fused = GuardedSlabs(P, B, S // P, H, D)
    xs.xstage_ulysses_attn_fwd(qs, ks, vs, fused.views, Hl, h0, w.scale, split_ws=split_ws())
    serial = GuardedSlabs(P, B, S // P, H, D)
    ws = torch.empty((4, B, S, Hl, D), dtype=torch.bfloat16, device="cuda")
    xs.xstage_ulysses_attn_unfused(qs, ks, vs, ws, serial.views, Hl, h0, w.scale, split_ws=split_ws())
    torch.cuda.synchronize()
    assert serial.guards_intact()
    got = serial.slabs_host()
    assert np.array_equal(got, fused.slabs_host())
    assert np.all(got[:, :, :, :h0] == NAN_BF16) and np.all(got[:, :, :, h0 + Hl:] == NAN_BF16)
