"""The C ABI: exported symbols match include/xstage.h; every invalid argument is rejected
with its status before anything is launched; the host-side Burst-Gap helper matches the
hand-evaluated values.  Runs without a GPU (no call here reaches a kernel launch)."""

import json
import math
import os
import re

import numpy as np
import pytest

import attention_ulysses_a2a_amd as xs
from attention_ulysses_a2a_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INVALID, UNSUPPORTED = _lib.XSTAGE_ERR_INVALID, _lib.XSTAGE_ERR_UNSUPPORTED


def _gpu_visible():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


# The error-path cases below pass fake (never dereferenced) device addresses.  They are run
# only where no device is visible, so that a missing check could never reach a launch.
no_device = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer error paths run only without a visible device")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        from attention_ulysses_a2a_amd.build import build

        build()
    return _lib.lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "xstage.h")).read()
    return sorted(set(re.findall(r"^\s*(?:int|double|const char\*)\s+(xstage_\w+)\s*\(", text, re.M)))


def test_header_and_library_agree(L):
    names = header_functions()
    assert len(names) == 27
    for n in names:
        assert hasattr(L, n), n
    assert sorted(_lib.SIGNATURES) == names


def test_status_strings(L):
    assert xs.xstage_status_str(0) == "XSTAGE_OK"
    assert xs.xstage_status_str(1) == "XSTAGE_ERR_INVALID"
    assert xs.xstage_status_str(2) == "XSTAGE_ERR_UNSUPPORTED"
    assert xs.xstage_status_str(3) == "XSTAGE_ERR_HIP"
    assert xs.xstage_status_str(99) == "XSTAGE_UNKNOWN_STATUS"


def test_bg_t_iss_hand_values(L):
    with open(os.path.join(ROOT, "tests", "golden", "burst_gap_hand_values.json")) as f:
        g = json.load(f)
    for c in g["page_formula"]:
        got = xs.xstage_bg_t_iss(c["G_s"], g["T0_s"], g["V_bytes"], g["R_bytes_per_s"])
        assert abs(got - c["T_iss_s"]) <= g["tolerance_s"]
    assert xs.xstage_bg_t_iss(0, 1e-6, 1e6, 0.0) < 0
    assert xs.xstage_bg_t_iss(float("nan"), 1e-6, 1e6, 1e9) < 0


# ---- error paths with fake addresses ------------------------------------------------------
Q, K, V = 0x10_0000_0000, 0x20_0000_0000, 0x30_0000_0000
SLAB0 = 0x40_0000_0000
GAP = 0x1_0000_0000


def slabs(P, base=SLAB0, step=GAP):
    return [base + p * step for p in range(P)]


WS = 0x60_0000_0000  # a fake split workspace


def fwd(L, q=Q, k=K, v=V, sl=None, B=1, S=256, H=2, D=64, P=2, scale=0.125, ws=None, ws_bytes=0):
    sl = slabs(P) if sl is None else sl
    arr, keep = _lib.ptr_array(sl)
    return L.xstage_attn_a2a_fwd(q, k, v, arr if sl != "null" else None, B, S, H, D, P, scale, ws, ws_bytes, None)


@no_device
@pytest.mark.parametrize("kw,code", [
    (dict(q=0), INVALID), (dict(k=0), INVALID), (dict(v=0), INVALID),
    (dict(B=0), INVALID), (dict(S=-1), INVALID), (dict(H=0), INVALID), (dict(P=0), INVALID), (dict(D=0), INVALID),
    (dict(D=96), UNSUPPORTED), (dict(D=256), UNSUPPORTED),
    (dict(S=65 * 64, P=65), UNSUPPORTED),
    (dict(S=1001, P=8), INVALID),
    (dict(q=Q + 8), INVALID), (dict(v=V + 2), INVALID),
    (dict(scale=float("nan")), INVALID), (dict(scale=float("inf")), INVALID),
    (dict(S=1 << 20, H=16, D=128, P=1), UNSUPPORTED),
])
def test_fused_rejects(L, kw, code):
    assert fwd(L, **kw) == code


def paced(L, chunks, q=Q, B=1, S=256, H=2, D=128, P=2, scale=0.125):
    arr, keep = _lib.ptr_array(slabs(P))
    return L.xstage_attn_a2a_fwd_paced(q, K, V, arr, B, S, H, D, P, scale, chunks, None)


@no_device
@pytest.mark.parametrize("kw,code", [
    (dict(chunks=0), INVALID), (dict(chunks=-1), INVALID), (dict(chunks=3), INVALID),
    (dict(chunks=16), INVALID), (dict(chunks=8, D=64), INVALID), (dict(chunks=6, D=64), INVALID),
    (dict(chunks=1, q=0), INVALID), (dict(chunks=2, S=1001, P=8), INVALID),
    (dict(chunks=4, D=96), UNSUPPORTED), (dict(chunks=1, scale=float("nan")), INVALID),
])
def test_paced_rejects(L, kw, code):
    assert paced(L, **kw) == code


def test_nsplit_ws_size_values(L):
    import ctypes

    b = ctypes.c_ulonglong(7)
    # FLUX-1024 share: 108 tiles, 72 key blocks; records of 4 waves x 9 chunks x 64 lanes x 16 B
    assert L.xstage_attn_nsplit_ws_size(1, 4608, 3, 128, 1, ctypes.byref(b)) == 0 and b.value == 0
    for k in (2, 3, 4, 8, 9, 12):
        assert L.xstage_attn_nsplit_ws_size(1, 4608, 3, 128, k, ctypes.byref(b)) == 0
        assert b.value == 16384 + 108 * k * 4 * 9 * 64 * 16
    # 16 and 0 are out of range; 5 blocks (S = 300) cannot form 4 equal non-empty ranges
    # (2 blocks each gives 3 ranges), but they form 3
    assert L.xstage_attn_nsplit_ws_size(1, 4608, 3, 128, 16, ctypes.byref(b)) == INVALID
    assert L.xstage_attn_nsplit_ws_size(1, 4608, 3, 128, 0, ctypes.byref(b)) == INVALID
    assert L.xstage_attn_nsplit_ws_size(1, 300, 1, 64, 4, ctypes.byref(b)) == INVALID
    assert L.xstage_attn_nsplit_ws_size(1, 300, 1, 64, 3, ctypes.byref(b)) == 0
    assert b.value == 16384 + 3 * 3 * 4 * 5 * 64 * 16
    # more than 4096 tiles: only n_split = 1; partials above 128 MiB: refused
    assert L.xstage_attn_nsplit_ws_size(1, 128 * 4097, 1, 64, 2, ctypes.byref(b)) == INVALID
    assert L.xstage_attn_nsplit_ws_size(1, 16896, 3, 128, 15, ctypes.byref(b)) == INVALID
    assert L.xstage_attn_nsplit_ws_size(1, 4608, 3, 128, 2, None) == INVALID


@no_device
def test_nsplit_rejects(L):
    arr, keep = _lib.ptr_array(slabs(2))
    call = lambda k, ws=WS, wsb=1 << 30, q=Q: L.xstage_attn_a2a_fwd_nsplit(q, K, V, arr, 1, 4608, 3, 128, 2, 0.1,
                                                                         k, ws, wsb, None)
    assert call(0) == INVALID
    assert call(16) == INVALID
    assert call(4, ws=None) == INVALID                    # split count needs a workspace
    assert call(4, wsb=16384) == INVALID                  # too small
    assert call(4, ws=WS + 8) == INVALID                  # misaligned
    assert call(4, ws=Q) == INVALID                       # overlaps q
    assert call(4, q=0) == INVALID
    assert L.xstage_attn_a2a_fwd_nsplit(Q, K, V, arr, 1, 4608, 3, 96, 2, 0.1, 1, None, 0, None) == UNSUPPORTED


@no_device
def test_paced_plan_needs_a_device(L):
    import ctypes

    n, t = ctypes.c_int(-1), ctypes.c_int(-1)
    assert L.xstage_attn_a2a_paced_plan(1, 256, 2, 128, None, ctypes.byref(t)) == INVALID
    assert L.xstage_attn_a2a_paced_plan(0, 256, 2, 128, ctypes.byref(n), ctypes.byref(t)) == INVALID
    assert L.xstage_attn_a2a_paced_plan(1, 256, 2, 96, ctypes.byref(n), ctypes.byref(t)) == UNSUPPORTED
    # the occupancy query has no device to ask
    assert L.xstage_attn_a2a_paced_plan(1, 256, 2, 128, ctypes.byref(n), ctypes.byref(t)) == _lib.XSTAGE_ERR_HIP


@no_device
def test_fused_rejects_bad_slabs(L):
    assert L.xstage_attn_a2a_fwd(Q, K, V, None, 1, 256, 2, 64, 2, 0.125, None, 0, None) == INVALID
    assert fwd(L, sl=[SLAB0, 0]) == INVALID                       # null slab
    assert fwd(L, sl=[SLAB0, SLAB0 + 16]) == INVALID              # slabs overlap
    assert fwd(L, sl=[SLAB0, Q + 64]) == INVALID                  # slab inside q
    assert fwd(L, sl=[SLAB0, V - 16]) == INVALID                  # slab runs into v
    assert fwd(L, sl=[SLAB0, SLAB0 + GAP + 4]) == INVALID         # misaligned slab
    # adjacent but disjoint slabs are fine up to the launch: only check they pass the
    # overlap rule by making another argument invalid afterwards
    slab_bytes = 1 * 128 * 2 * 64 * 2
    assert fwd(L, sl=[SLAB0, SLAB0 + slab_bytes], scale=float("nan")) == INVALID


@no_device
def test_fused_rejects_bad_split_workspace(L):
    """The part of the split workspace a launch uses must be aligned and disjoint from every
    other buffer; an unused workspace (no split, or too small for any) is never touched."""
    B, S, H, D, P = 1, 4608, 3, 128, 8
    need = xs.xstage_attn_split_ws_size(B, S, H, D)
    assert need > 0
    big = dict(B=B, S=S, H=H, D=D, P=P, sl=slabs(P))
    assert fwd(L, ws=WS + 8, ws_bytes=need, **big) == INVALID          # misaligned
    assert fwd(L, ws=Q + 4096, ws_bytes=need, **big) == INVALID        # overlaps q
    assert fwd(L, ws=V - 256, ws_bytes=need, **big) == INVALID         # runs into v
    assert fwd(L, ws=SLAB0 + GAP - 512, ws_bytes=need, **big) == INVALID   # runs into slab 2
    # a workspace inside q that the plan does not use is never touched: the call proceeds to
    # its other checks (here: a NaN scale)
    assert fwd(L, ws=Q + 4096, ws_bytes=16, scale=float("nan"), **big) == INVALID


def test_split_ws_size_and_plan(L):
    """The workspace query reports the fastest plan's bytes (counters padded to 256, then the
    16-bit partial records of every (tile, split) unit); a smaller workspace limits the split
    count to what fits, none gives no split."""
    B, S, H, D = 1, 4608, 3, 128
    n_tiles = B * H * ((S + 127) // 128)
    nwg, nsp = xs.xstage_attn_a2a_plan(B, S, H, D)
    rec = 4 * (2 * (D // 32) + 1) * 64 * 16
    need = xs.xstage_attn_split_ws_size(B, S, H, D)
    assert need == 16384 + nwg * rec
    assert xs.xstage_attn_a2a_plan(B, S, H, D, need) == (nwg, nsp)
    assert xs.xstage_attn_a2a_plan(B, S, H, D, 0) == (n_tiles, 1)
    assert xs.xstage_attn_a2a_plan(B, S, H, D, need - 1)[1] < nsp
    for k in range(2, nsp):
        fit = 16384 + n_tiles * k * rec
        assert xs.xstage_attn_a2a_plan(B, S, H, D, fit)[1] <= k
    assert xs.xstage_attn_split_ws_size(1, 1, 1, 64) == 0
    # large shapes are split within the 128 MiB partial cap
    assert xs.xstage_attn_split_ws_size(4, 58240, 3, 64) <= (128 << 20) + 16384
    # more than 4096 tiles: never split (the counter area holds 4096)
    assert xs.xstage_attn_a2a_plan(8, 65536, 1, 64)[1] == 1
    n = _lib.ctypes.c_ulonglong(0)
    assert L.xstage_attn_split_ws_size(1, 256, 2, 80, _lib.ctypes.byref(n)) == UNSUPPORTED
    assert L.xstage_attn_split_ws_size(0, 256, 2, 64, _lib.ctypes.byref(n)) == INVALID
    assert L.xstage_attn_split_ws_size(1, 256, 2, 64, None) == INVALID


@no_device
def test_attn_fwd_rejects(L):
    def f(*a):
        return L.xstage_attn_fwd(*a[:-1], None, 0, a[-1])

    assert f(Q, K, V, 0, 1, 256, 2, 64, 0.125, None) == INVALID
    assert f(Q, K, V, K + 32, 1, 256, 2, 64, 0.125, None) == INVALID   # out overlaps k
    assert f(Q, K, V, SLAB0 + 8, 1, 256, 2, 64, 0.125, None) == INVALID
    assert f(Q, K, V, SLAB0, 1, 256, 2, 80, 0.125, None) == UNSUPPORTED
    assert f(Q, K, V, SLAB0, 1, 0, 2, 64, 0.125, None) == INVALID
    need = xs.xstage_attn_split_ws_size(1, 4608, 3, 128)
    assert L.xstage_attn_fwd(Q, K, V, SLAB0, 1, 4608, 3, 128, 0.125, SLAB0 + 64, need, None) == INVALID


@no_device
def test_scatter_rejects(L):
    arr, keep = _lib.ptr_array(slabs(2))
    f = L.xstage_a2a_scatter
    assert f(0, arr, 1, 256, 2, 64, 2, None) == INVALID
    assert f(Q + 4, arr, 1, 256, 2, 64, 2, None) == INVALID
    assert f(Q, None, 1, 256, 2, 64, 2, None) == INVALID
    assert f(Q, arr, 1, 255, 2, 64, 2, None) == INVALID
    bad, keep2 = _lib.ptr_array([SLAB0, Q + 128])
    assert f(Q, bad, 1, 256, 2, 64, 2, None) == INVALID
    assert f(Q, arr, 1, 256, 2, 48, 2, None) == UNSUPPORTED


@no_device
def test_unfused_rejects(L):
    arr, keep = _lib.ptr_array(slabs(2))
    def f(*a):
        return L.xstage_attn_a2a_unfused(*a[:-1], None, 0, a[-1])

    W = 0x50_0000_0000
    assert f(Q, K, V, 0, arr, 1, 256, 2, 64, 2, 0.125, None) == INVALID
    assert f(Q, K, V, W + 8, arr, 1, 256, 2, 64, 2, 0.125, None) == INVALID
    assert f(Q, K, V, Q + 256, arr, 1, 256, 2, 64, 2, 0.125, None) == INVALID   # workspace overlaps q
    assert f(Q, K, V, SLAB0 + GAP - 64, arr, 1, 256, 2, 64, 2, 0.125, None) == INVALID  # overlaps slab 1
    assert f(Q, K, V, W, arr, 1, 256, 2, 64, 2, float("nan"), None) == INVALID
    assert f(Q, K, V, W, arr, 1, 256, 2, 64, 3, 0.125, None) == INVALID
    arr8, keep8 = _lib.ptr_array(slabs(8))
    need = xs.xstage_attn_split_ws_size(1, 4608, 3, 128)
    assert L.xstage_attn_a2a_unfused(Q, K, V, W, arr8, 1, 4608, 3, 128, 8, 0.125, W + 4096, need, None) == INVALID


def test_plan_counts_workgroups(L):
    """Host-only: the decomposition the traced call's stamps are sized by."""
    nwg, nsp = xs.xstage_attn_a2a_plan(1, 4608, 3, 128)
    assert nwg % nsp == 0 and nwg // nsp == 3 * 36 and 1 <= nsp <= 16
    nwg, nsp = xs.xstage_attn_a2a_plan(1, 1, 1, 64)
    assert (nwg, nsp) == (1, 1)
    n = _lib.ctypes.c_int(0)
    assert L.xstage_attn_a2a_plan(1, 256, 2, 80, 0, _lib.ctypes.byref(n), None) == UNSUPPORTED
    assert L.xstage_attn_a2a_plan(0, 256, 2, 64, 0, _lib.ctypes.byref(n), None) == INVALID
    assert L.xstage_attn_a2a_plan(1, 256, 2, 64, 0, None, None) == INVALID


SCHEDULE_SHAPES = [(1, 256, 2, 64), (1, 4608, 3, 128), (1, 4608, 3, 64), (2, 4608, 3, 128), (1, 9216, 3, 128),
                   (1, 2304, 3, 128), (1, 16896, 3, 128), (1, 32760, 5, 128), (2, 1000, 2, 128), (1, 1, 1, 64)]


@pytest.mark.parametrize("B,S,H,D", SCHEDULE_SHAPES)
def test_schedule_partitions_every_tile(L, B, S, H, D):
    """Host-only: every tile's splits cover its key blocks [0, ceil(S/64)) exactly once, in
    split order, and every workgroup has its own (tile, split); tiles are of the launch's
    rows per workgroup."""
    tile, split, j0, j1 = (np.array(a) for a in xs.xstage_attn_a2a_schedule(B, S, H, D))
    nwg, nsp = xs.xstage_attn_a2a_plan(B, S, H, D)
    rows = xs.xstage_attn_a2a_wg_rows(B, S, H, D)
    n_tiles, nkv = B * H * ((S + rows - 1) // rows), (S + 63) // 64
    assert len(tile) == nwg == n_tiles * nsp
    assert len(set(zip(tile.tolist(), split.tolist()))) == nwg
    for t in range(n_tiles):
        idx = np.where(tile == t)[0]
        o = idx[np.argsort(split[idx])]
        assert split[o].tolist() == list(range(nsp))
        assert j0[o[0]] == 0 and j1[o[-1]] == nkv
        assert np.array_equal(j1[o[:-1]], j0[o[1:]])
        assert np.all(j1[o] > j0[o])


def test_schedule_mixes_placements_in_one_round(L):
    """FLUX-1024 share: 432 workgroups on 256 CUs (8 XCDs of 32) run in one round; workgroup
    i sits at slot i // 8 of XCD i % 8, slots 0..21 share a CU with slots 32..53 (the
    younger, slower partner) and 22..31 run alone.  No tile may be all younger partners, and
    a younger partner never gets more keys than an older partner or a lone workgroup of
    its tile; each tile's blocks are shared out min-max optimally."""
    tile, split, j0, j1 = (np.array(a) for a in xs.xstage_attn_a2a_schedule(1, 4608, 3, 128))
    blocks = j1 - j0
    slot = np.arange(len(tile)) // 8
    young = slot >= 32
    assert len(set(blocks.tolist())) > 1       # ranges follow the placement
    for t in range(tile.max() + 1):
        idx = np.where(tile == t)[0]
        assert not young[idx].all()
        if young[idx].any() and (~young[idx]).any():
            assert blocks[idx][young[idx]].max() <= blocks[idx][~young[idx]].min()
    # Within a tile the blocks are shared out min-max optimally for the placement rates the
    # table assumes (lone 1.0, older sharer 0.864, younger sharer 0.58): no block can move
    # off the tile's slowest split (largest blocks / rate) to another split without that
    # split becoming at least as slow.
    rate = np.where(slot < 22, 0.864, np.where(slot < 32, 1.0, 0.58))
    for t in range(tile.max() + 1):
        idx = np.where(tile == t)[0]
        tt = blocks[idx] / rate[idx]
        worst = tt.max()
        others = np.arange(len(idx)) != np.argmax(tt)
        assert np.all((blocks[idx][others] + 1) / rate[idx][others] >= worst - 1e-12), t
    # multi-round launches keep equal ranges (the last split may be shorter)
    tile, split, j0, j1 = (np.array(a) for a in xs.xstage_attn_a2a_schedule(1, 16896, 3, 128))
    assert len(set((j1 - j0)[j1 < (16896 + 63) // 64].tolist())) == 1


# (B, S, H, D, split workspace bytes or None for the full plan) -> rows per workgroup, on
# 256 CUs (the host's default without a device)
WG_ROWS_CASES = [
    ((1, 4608, 3, 128, None), 128),   # one round of 432 with placement-sized ranges
    ((1, 16896, 3, 128, None), 256),  # 1980 4-wave workgroups in ~3.9 rounds -> 990 of 8 waves
    ((1, 32760, 5, 128, None), 256),  # 2560 -> 1280
    ((1, 16384, 4, 128, None), 256),  # 512 unsplit (two per CU) -> 256
    ((1, 16384, 4, 128, 0), 256),     # the same without workspace
    ((1, 16896, 3, 128, 0), 128),     # 396 unsplit: fewer than two per CU
    ((1, 9216, 3, 128, None), 128),   # 432 with 2 splits: the one-round table
    ((1, 12160, 4, 128, None), 128),  # 95 tiles of 128 rows per head (odd)
    ((1, 16384, 4, 64, None), 256),
    ((2, 4608, 3, 128, None), 128),   # 432 with 2 splits
    ((2, 4864, 8, 128, None), 128),   # 1216 with 2 splits: at most 5 per CU (odd)
    ((1, 10496, 5, 128, None), 128),  # 1230 with 3 splits of 55 blocks: at most 5 per CU (odd)
    ((2, 5632, 2, 128, None), 128),   # 880 with 5 splits of 18 64-key blocks (short)
    ((4, 1792, 5, 128, None), 128),   # 840 with 3 splits of 10 blocks (short)
    ((4, 6400, 1, 128, None), 256),   # 1000 with 5 splits of 20 blocks: at most 4 per CU
    ((2, 8448, 2, 128, None), 256),   # 792 with 3 splits of 44 blocks
]


@pytest.mark.parametrize("shape,rows", WG_ROWS_CASES)
def test_wg_rows_rule(L, shape, rows):
    """Host-only: 256-row (8-wave) workgroups exactly where the 4-wave launch keeps every CU at
    two workgroups without the one-round table, the most 4-wave workgroups any CU runs is even,
    every key range spans at least 20 64-key blocks and every (b, h) has an even number of
    128-row tiles; the workgroup count halves, the split count and workspace bytes stay."""
    B, S, H, D, wsb = shape
    assert xs.xstage_attn_a2a_wg_rows(B, S, H, D, wsb) == rows
    nwg, nsp = xs.xstage_attn_a2a_plan(B, S, H, D, wsb)
    tiles128 = B * H * ((S + 127) // 128)
    assert nwg * rows == tiles128 * nsp * 128
    if nsp > 1:
        assert xs.xstage_attn_split_ws_size(B, S, H, D) == 16384 + tiles128 * nsp * 4 * (2 * (D // 32) + 1) * 64 * 16
    n = _lib.ctypes.c_int(0)
    assert L.xstage_attn_a2a_wg_rows(B, S, H, D, 0, None) == INVALID
    assert L.xstage_attn_a2a_wg_rows(B, S, H, 80, 0, _lib.ctypes.byref(n)) == UNSUPPORTED
    assert L.xstage_attn_a2a_wg_rows(0, S, H, D, 0, _lib.ctypes.byref(n)) == INVALID


NAMED_PLANS = {
    # workload: (workgroups, key splits, query rows per workgroup) with the full workspace
    "tiny": (4, 1, 128),
    "flux1024": (432, 4, 128),
    "flux2048": (990, 5, 256),
    "video": (1280, 2, 256),
}


@pytest.mark.parametrize("name", sorted(NAMED_PLANS))
def test_named_workload_plans(name):
    """Host-only: the plans the committed kernel traces, counter summaries and traffic figure
    were measured on.  A change of the split model or the width rule that moves one of them
    also changes what those measurements describe, so it has to be re-measured with them."""
    from synth import workload

    w = workload(name)
    nwg, nsp = xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D)
    assert (nwg, nsp, xs.xstage_attn_a2a_wg_rows(w.B, w.S, w.H, w.D)) == NAMED_PLANS[name]


def test_schedule_rejects(L):
    n = _lib.ctypes.c_int(0)
    buf = (_lib.ctypes.c_int * 4)()
    full = _lib.WS_FULL
    assert L.xstage_attn_a2a_schedule(1, 4608, 3, 128, full, 4, buf, buf, buf, buf, _lib.ctypes.byref(n)) == INVALID
    assert n.value == xs.xstage_attn_a2a_plan(1, 4608, 3, 128)[0]
    assert L.xstage_attn_a2a_schedule(1, 256, 2, 64, full, 0, None, None, None, None, None) == INVALID
    assert L.xstage_attn_a2a_schedule(1, 256, 2, 80, full, 0, None, None, None, None,
                                      _lib.ctypes.byref(n)) == UNSUPPORTED


STAMPS = 0x50_0000_0000


@no_device
def test_traced_rejects(L):
    arr, keep = _lib.ptr_array(slabs(2))
    def f(*a):
        return L.xstage_attn_a2a_fwd_traced(*a[:-1], None, 0, a[-1])

    args = (Q, K, V, arr, 1, 256, 2, 64, 2, 0.125)
    assert f(*args, 4, STAMPS, None) == INVALID                # unknown mode
    assert f(*args, -1, STAMPS, None) == INVALID
    assert f(*args, 0, 0, None) == INVALID                     # no stamps
    assert f(*args, 0, STAMPS + 4, None) == INVALID            # misaligned stamps
    assert f(*args, 0, Q + 64, None) == INVALID                # stamps inside q
    assert f(*args, 0, SLAB0 + 64, None) == INVALID            # stamps inside a slab
    assert f(Q, K, V, arr, 1, 256, 2, 64, 2, float("nan"), 0, STAMPS, None) == INVALID
    assert f(Q, K, V, arr, 1, 255, 2, 64, 2, 0.125, 0, STAMPS, None) == INVALID


@no_device
def test_strided_rejects(L):
    def f(*a):
        return L.xstage_attn_a2a_fwd_strided(*a[:-1], None, 0, a[-1])

    arr, keep = _lib.ptr_array(slabs(2))

    def call(H=2, P=2, H_dst=8, h0=4, q=Q, sl=arr, S=256, scale=0.125):
        return f(q, K, V, sl, 1, S, H, 64, P, H_dst, h0, scale, None)

    assert call(H_dst=1) == INVALID            # fewer destination heads than local heads
    assert call(h0=-1) == INVALID
    assert call(h0=7) == INVALID               # columns 7, 8 past H_dst = 8
    assert call(sl=None) == INVALID
    assert call(q=0) == INVALID
    assert call(S=255) == INVALID              # S % P
    assert call(scale=float("nan")) == INVALID
    assert call(H_dst=1 << 17, h0=0) == UNSUPPORTED  # destination offsets reach 2^31 elements
    near, keep2 = _lib.ptr_array([SLAB0, SLAB0 + 256 * 8 * 64 - 16])  # slab 0 spans 256*8*64*2/2 bytes
    assert call(sl=near) == INVALID
    inq, keep3 = _lib.ptr_array([SLAB0, Q + 64])
    assert call(sl=inq) == INVALID


@no_device
def test_ulysses_rejects(L):
    def f(*a):
        return L.xstage_ulysses_attn_fwd(*a[:-1], None, 0, a[-1])

    P = 4
    qs = [0x10_0000_0000 + p * GAP for p in range(P)]
    ks = [0x20_0000_0000 + p * GAP for p in range(P)]
    vs = [0x30_0000_0000 + p * GAP for p in range(P)]
    ds = slabs(P)

    def call(q=qs, k=ks, v=vs, d=ds, B=1, S=256, H=8, Hl=2, h0=2, D=64, P=P, scale=0.125):
        arrs = [_lib.ptr_array(x) if x is not None else (None, None) for x in (q, k, v, d)]
        return f(arrs[0][0], arrs[1][0], arrs[2][0], arrs[3][0], B, S, H, Hl, h0, D, P, scale, None)

    assert call(Hl=0) == INVALID
    assert call(Hl=9) == INVALID
    assert call(h0=7) == INVALID
    assert call(h0=-1) == INVALID
    assert call(S=258) == INVALID
    assert call(D=96) == UNSUPPORTED
    assert call(q=None) == INVALID
    assert call(d=None) == INVALID
    assert call(q=[qs[0], 0, qs[2], qs[3]]) == INVALID
    assert call(v=[vs[0], vs[1] + 8, vs[2], vs[3]]) == INVALID
    assert call(d=[ds[0], ds[1], ds[2], ks[1] + 16]) == INVALID     # output overlaps a K shard
    assert call(d=[ds[0], ds[0] + 64, ds[2], ds[3]]) == INVALID     # outputs overlap
    assert call(scale=float("inf")) == INVALID
    big = [SLAB0 + p * GAP for p in range(33)]
    assert call(q=big, k=big, v=big, d=big, S=33 * 8, P=33) == UNSUPPORTED  # more than 32 shards
    assert call(H=1 << 14, Hl=2, h0=0, S=1 << 14, D=128, P=4) == UNSUPPORTED


@no_device
def test_burst_gap_rejects(L):
    import ctypes

    def run(**kw):
        base = dict(K=64, rounds=8, n_dst_sets=1, nontemporal=0, V_bytes=1 << 20, gap_fma_iters=10,
                    dst=SLAB0, stamps=Q, sync=None, sync_timeout_ticks=0)
        base.update(kw)
        p = _lib.BGParams(**base)
        return L.xstage_burst_gap_run(ctypes.byref(p), None)

    assert L.xstage_burst_gap_run(None, None) == INVALID
    assert run(K=0) == INVALID
    assert run(K=5000) == INVALID
    assert run(rounds=0) == INVALID
    assert run(n_dst_sets=0) == INVALID
    assert run(nontemporal=2) == INVALID
    assert run(stamps=0) == INVALID
    assert run(stamps=Q + 4) == INVALID
    assert run(V_bytes=(1 << 20) + 4096) == INVALID   # not a multiple of K * 4096
    assert run(dst=0) == INVALID
    assert run(dst=SLAB0 + 8) == INVALID
    assert run(sync=0x70_0000_0002, sync_timeout_ticks=100) == INVALID       # misaligned
    assert run(sync=0x70_0000_0000, sync_timeout_ticks=0) == INVALID         # no bound on the wait
    assert run(sync=0x70_0000_0000, sync_timeout_ticks=10 ** 10) == INVALID  # bound above 10^9 ticks
    assert run(sync=Q + 8, sync_timeout_ticks=100) == INVALID                # inside the stamps
    assert run(sync=SLAB0 + 4096, sync_timeout_ticks=100) == INVALID         # inside dst


@no_device
def test_wallclock_rejects_null(L):
    assert L.xstage_wallclock_hz(None) == INVALID


def test_xcd_unit_order_is_a_bijection():
    """Host replica of the kernel's workgroup -> unit remap (XCD i % 8 gets a contiguous range)."""
    for n in list(range(1, 70)) + [108, 216, 396, 1280, 1281, 2565]:
        q8, r8 = n >> 3, n & 7
        seen = set()
        for i in range(n):
            xcd, slot = i & 7, i >> 3
            L = xcd * (q8 + 1) + slot if xcd < r8 else r8 * (q8 + 1) + (xcd - r8) * q8 + slot
            assert 0 <= L < n
            seen.add(L)
        assert len(seen) == n


# ---- expert-wave stand-in: schedule plan (host) and argument checks -----------------------
MOE_OFFS = [0, 90, 90, 300, 301, 700]  # 5 experts, one with no tokens


@pytest.mark.parametrize("epw", [1, 2, 3, 5, 8])
def test_moe_plan_covers_every_expert_in_dependency_order(L, epw):
    E = len(MOE_OFFS) - 1
    waves = [list(range(w, min(E, w + epw))) for w in range(0, E, epw)]
    l1a, l2a, na, nta = xs.xstage_moe_waves_plan(MOE_OFFS, 256, 128, epw, 0)
    l1b, l2b, nb, ntb = xs.xstage_moe_waves_plan(MOE_OFFS, 256, 128, epw, 1)
    rows = [MOE_OFFS[e + 1] - MOE_OFFS[e] for e in range(E)]
    tiles = sum(-(-r // 128) * (128 // 128 + 256 // 128) for r in rows)
    assert nta == ntb == tiles
    assert na == 2 * len(waves) and nb == len(waves) + 1
    for wi, wave in enumerate(waves):
        for e in wave:
            assert (l1a[e], l2a[e]) == (2 * wi, 2 * wi + 1)   # expert waves: L1(w), then L2(w)
            assert (l1b[e], l2b[e]) == (wi, wi + 1)           # interleaved: L2(w) with L1(w+1)
            assert l2a[e] > l1a[e] and l2b[e] > l1b[e]
    # the interleaved launches hold Linear-2 of wave w together with Linear-1 of wave w+1
    for wi in range(len(waves) - 1):
        assert {l2b[e] for e in waves[wi]} == {l1b[e] for e in waves[wi + 1]}


@no_device
def test_moe_rejects(L):
    import ctypes

    def run(**kw):
        offs = kw.pop("offs", MOE_OFFS)
        T = offs[-1]
        base = dict(E=len(offs) - 1, d_model=256, d_ff=128, experts_per_wave=2, schedule=0, x=0x10_0000_0000,
                    w1=0x20_0000_0000, w2=0x30_0000_0000, h=0x40_0000_0000, dst_slab=0x50_0000_0000,
                    dst_row=0x50_1000_0000, P=2, stamps=None)
        outs = kw.pop("outs", [0x60_0000_0000, 0x70_0000_0000])
        rows = kw.pop("rows", [T, T])
        base.update(kw)
        oarr, keep = _lib.ptr_array(outs)
        prm = _lib.MoeParams(base["E"], base["d_model"], base["d_ff"], base["experts_per_wave"], base["schedule"],
                             (ctypes.c_int * len(offs))(*offs), base["x"], base["w1"], base["w2"], base["h"],
                             base["dst_slab"], base["dst_row"], base["P"], oarr, (ctypes.c_int * max(1, len(rows)))(*rows),
                             base["stamps"])
        return L.xstage_moe_waves_run(ctypes.byref(prm), None)

    assert L.xstage_moe_waves_run(None, None) == INVALID
    assert run(E=0) == INVALID
    assert run(d_model=200) == INVALID            # not a multiple of 128
    assert run(d_ff=0) == INVALID
    assert run(experts_per_wave=0) == INVALID
    assert run(experts_per_wave=33) == UNSUPPORTED
    assert run(schedule=2) == INVALID
    assert run(offs=[1, 90, 300, 301, 700, 700]) == INVALID   # must start at 0
    assert run(offs=[0, 90, 80, 301, 700, 700]) == INVALID    # decreasing
    assert run(x=0) == INVALID
    assert run(w2=0x30_0000_0008) == INVALID     # misaligned
    assert run(dst_row=0x50_1000_0002) == INVALID
    assert run(P=0) == INVALID
    assert run(P=65) == UNSUPPORTED
    assert run(outs=[0x60_0000_0000, 0]) == INVALID
    assert run(rows=[700, -1]) == INVALID
    assert run(h=0x10_0000_0000 + 256) == INVALID                 # h overlaps x
    assert run(outs=[0x60_0000_0000, 0x60_0000_0000 + 512]) == INVALID  # outputs overlap
    assert run(outs=[0x60_0000_0000, 0x20_0000_0000]) == INVALID  # an output overlaps w1
    assert run(stamps=0x80_0000_0004) == INVALID   # misaligned stamps
    assert run(stamps=0x40_0000_0000) == INVALID   # stamps overlap h
    n = _lib.ctypes.c_int(0)
    arr = (_lib.ctypes.c_int * 8)()
    offs = (_lib.ctypes.c_int * 6)(*MOE_OFFS)
    assert L.xstage_moe_waves_plan(5, offs, 256, 128, 2, 0, None, arr, _lib.ctypes.byref(n), _lib.ctypes.byref(n)) == INVALID
    assert L.xstage_moe_waves_plan(5, offs, 256, 100, 2, 0, arr, arr, _lib.ctypes.byref(n), _lib.ctypes.byref(n)) == INVALID


@no_device
def test_serial_ulysses_rejects(L):
    P = 4
    qs = [0x10_0000_0000 + p * GAP for p in range(P)]
    ks = [0x20_0000_0000 + p * GAP for p in range(P)]
    vs = [0x30_0000_0000 + p * GAP for p in range(P)]
    ds = slabs(P)
    WS = 0x80_0000_0000
    arr = lambda x: _lib.ptr_array(x)[0]
    g = L.xstage_ulysses_gather
    assert g(arr(qs), WS, 1, 256, 8, 0, 2, 64, P, None) == INVALID          # H_local = 0
    assert g(arr(qs), WS, 1, 256, 8, 2, 7, 64, P, None) == INVALID          # heads past H
    assert g(arr(qs), 0, 1, 256, 8, 2, 2, 64, P, None) == INVALID           # no output
    assert g(arr(qs), qs[1] + 64, 1, 256, 8, 2, 2, 64, P, None) == INVALID  # output inside a shard
    assert g(arr([qs[0], 0, qs[2], qs[3]]), WS, 1, 256, 8, 2, 2, 64, P, None) == INVALID
    assert g(arr(qs), WS, 1, 258, 8, 2, 2, 64, P, None) == INVALID          # S % P
    sc = L.xstage_a2a_scatter_strided
    assert sc(WS, arr(ds), 1, 256, 2, 64, P, 1, 0, None) == INVALID         # H_dst < H_local
    assert sc(WS, arr(ds), 1, 256, 2, 64, P, 8, 7, None) == INVALID         # columns past H_dst
    assert sc(0, arr(ds), 1, 256, 2, 64, P, 8, 2, None) == INVALID
    assert sc(ds[0] + 64, arr(ds), 1, 256, 2, 64, P, 8, 2, None) == INVALID  # input inside an output
    u = L.xstage_ulysses_attn_unfused
    args = lambda **kw: dict(q=arr(qs), k=arr(ks), v=arr(vs), ws=WS, d=arr(ds), B=1, S=256, H=8, Hl=2, h0=2,
                             D=64, P=P, scale=0.125) | kw
    call = lambda a: u(a["q"], a["k"], a["v"], a["ws"], a["d"], a["B"], a["S"], a["H"], a["Hl"], a["h0"], a["D"],
                       a["P"], a["scale"], a.get("sws"), a.get("swsb", 0), None)
    assert call(args(ws=0)) == INVALID
    assert call(args(ws=ks[2] + 16)) == INVALID                  # workspace inside a shard
    assert call(args(d=arr([ds[0], ds[1], WS + 64, ds[3]]))) == INVALID  # output inside the workspace
    assert call(args(scale=float("nan"))) == INVALID
    assert call(args(h0=7)) == INVALID
    assert call(args(D=96)) == UNSUPPORTED
    # a split workspace that the (split) plan uses may not overlap the staging workspace
    need = xs.xstage_attn_split_ws_size(1, 4608, 2, 64)
    assert need > 0
    assert call(args(S=4608, sws=WS + 64, swsb=need)) == INVALID
    # K/V-staged layer: same argument list, workspace of 2 x [B, S, H_local, D]
    kv = L.xstage_ulysses_attn_fwd_kv_staged
    kcall = lambda a: kv(a["q"], a["k"], a["v"], a["ws"], a["d"], a["B"], a["S"], a["H"], a["Hl"], a["h0"], a["D"],
                         a["P"], a["scale"], a.get("sws"), a.get("swsb", 0), None)
    tl = 1 * 256 * 2 * 64 * 2
    assert kcall(args(ws=0)) == INVALID
    assert kcall(args(ws=WS + 8)) == INVALID                     # misaligned workspace
    assert kcall(args(ws=vs[3] + 16)) == INVALID                 # workspace inside a shard
    assert kcall(args(d=arr([ds[0], WS + tl + 64, ds[2], ds[3]]))) == INVALID  # output inside its second half
    assert kcall(args(q=arr([qs[0], 0, qs[2], qs[3]]))) == INVALID
    assert kcall(args(scale=float("inf"))) == INVALID
    assert kcall(args(Hl=0)) == INVALID
    assert kcall(args(D=96)) == UNSUPPORTED
    big = [SLAB0 + p * GAP for p in range(33)]
    assert kcall(args(q=arr(big), k=arr(big), v=arr(big), d=arr(big), S=33 * 8, P=33)) == UNSUPPORTED
