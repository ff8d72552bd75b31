"""Pins for the oracle's Ulysses all-to-alls around attention (``oracle/ulysses.py``).

* hand-derived positions (tests/golden/ulysses_positions.json) for both directions;
* the pre-attention gather inverts the (separately pinned) post-attention scatter on the
  rank's head columns;
* the post-attention scatter of all P ranks writes every element of the full-head receive
  buffers exactly once, and leaves the other ranks' columns alone;
* exactness of the decomposition: the P ranks' layers together equal multi-head attention
  over all heads, scattered to sequence shards, bit for bit (heads are independent);
* P = 1 with all heads reduces to plain attention.
"""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _small_shards(B, S, H, D, P, seed):
    x = np.random.default_rng(seed).standard_normal((B, S, H, D))
    return x, list(oracle.ulysses_scatter(x, P))


def test_hand_positions_both_directions():
    with open(os.path.join(GOLDEN, "ulysses_positions.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        S, H, P, Hl, rank = c["S"], c["H"], c["P"], c["H_local"], c["rank"]
        h0 = rank * Hl
        sp = S // P
        # pre-attention: tag one element of one shard and find it in the gathered tensor
        shards = [np.zeros((1, sp, H, 1)) for _ in range(P)]
        shards[c["p"]][0, c["r"], c["col"], 0] = 1.0
        x = oracle.pre_gather(shards, h0, Hl)
        assert np.argwhere(x == 1.0).tolist() == [[0, c["s"], c["h"], 0]], c
        # post-attention: tag one output element and find where it lands
        o = np.zeros((1, S, Hl, 1))
        o[0, c["s"], c["h"], 0] = 1.0
        dst = [np.zeros((1, sp, H, 1)) for _ in range(P)]
        oracle.scatter_heads(o, dst, h0)
        hits = [(p, *idx) for p in range(P) for idx in np.argwhere(dst[p] == 1.0).tolist()]
        assert hits == [(c["p"], 0, c["r"], c["col"], 0)], c


@pytest.mark.parametrize("B,S,H,Hl,D,P", [(1, 16, 4, 2, 3, 2), (2, 30, 6, 2, 2, 3), (1, 8, 3, 3, 2, 8), (1, 12, 2, 1, 4, 1)])
def test_gather_inverts_scatter_on_rank_heads(B, S, H, Hl, D, P):
    x, shards = _small_shards(B, S, H, D, P, seed=S + H)
    for h0 in range(0, H - Hl + 1):
        assert np.array_equal(oracle.pre_gather(shards, h0, Hl), x[:, :, h0:h0 + Hl, :])


@pytest.mark.parametrize("B,S,H,D,P", [(1, 16, 4, 3, 2), (2, 30, 6, 2, 3), (1, 8, 8, 1, 8)])
def test_all_ranks_write_every_element_once(B, S, H, D, P):
    Hl = H // P
    ids = np.arange(B * S * H * D, dtype=np.float64).reshape(B, S, H, D)
    dst = [np.full((B, S // P, H, D), -1.0) for _ in range(P)]
    count = [np.zeros((B, S // P, H, D), dtype=np.int64) for _ in range(P)]
    for rank in range(P):
        h0 = rank * Hl
        before = [d.copy() for d in dst]
        oracle.scatter_heads(ids[:, :, h0:h0 + Hl, :], dst, h0)
        for p in range(P):
            changed = dst[p] != before[p]
            assert not changed[:, :, :h0].any() and not changed[:, :, h0 + Hl:].any()
            count[p] += changed
    assert all((c == 1).all() for c in count)
    assert np.array_equal(np.stack(dst), oracle.ulysses_scatter(ids, P))


@pytest.mark.parametrize("B,S,H,D,P", [(1, 24, 4, 8, 2), (2, 18, 6, 4, 3)])
def test_ranks_together_equal_full_multihead_attention(B, S, H, D, P):
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    scale = 0.37
    full = oracle.attention_fp64(q, k, v, scale)
    qs, ks, vs = (list(oracle.ulysses_scatter(t, P)) for t in (q, k, v))
    Hl = H // P
    dst = [np.full((B, S // P, H, D), np.nan) for _ in range(P)]
    for rank in range(P):
        oracle.ulysses_attention(qs, ks, vs, scale, rank * Hl, Hl, dst)
    assert np.array_equal(np.stack(dst), oracle.ulysses_scatter(full, P))


def test_rows_subset_matches_full_layer():
    rng = np.random.default_rng(8)
    B, S, H, D, P, Hl, h0 = 1, 32, 4, 4, 4, 2, 2
    qs, ks, vs = (list(oracle.ulysses_scatter(rng.standard_normal((B, S, H, D)), P)) for _ in range(3))
    full = [np.full((B, S // P, H, D), np.nan) for _ in range(P)]
    oracle.ulysses_attention(qs, ks, vs, 0.5, h0, Hl, full)
    rows = np.array([0, 7, 8, 31])
    part = [np.full((B, S // P, H, D), np.nan) for _ in range(P)]
    oracle.ulysses_attention(qs, ks, vs, 0.5, h0, Hl, part, rows=rows)
    for s in rows:
        p, r = s // (S // P), s % (S // P)
        assert np.array_equal(part[p][:, r], full[p][:, r], equal_nan=True)
        assert not np.isnan(part[p][:, r, h0:h0 + Hl]).any()
    assert np.isnan(part[0][:, 1]).all()


def test_one_rank_is_plain_attention():
    rng = np.random.default_rng(9)
    q, k, v = (rng.standard_normal((1, 10, 2, 4)) for _ in range(3))
    dst = [np.zeros((1, 10, 2, 4))]
    oracle.ulysses_attention([q[0:1]], [k[0:1]], [v[0:1]], 0.25, 0, 2, dst)
    assert np.array_equal(dst[0], oracle.attention_fp64(q, k, v, 0.25)[0:1])


def test_rejects_bad_head_ranges():
    shards = [np.zeros((1, 4, 3, 2))] * 2
    with pytest.raises(ValueError):
        oracle.pre_gather(shards, 2, 2)
    with pytest.raises(ValueError):
        oracle.scatter_heads(np.zeros((1, 8, 2, 2)), [np.zeros((1, 4, 3, 2))] * 2, 2)
