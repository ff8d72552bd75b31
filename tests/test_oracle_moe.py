"""Pins for the oracle's mixture-of-experts layer (``oracle/moe.py``).

* brute force with exact summation (math.fsum) on tiny inputs, including the bf16 rounding
  of Linear-1 (the codec itself is pinned in test_oracle_slabs.py);
* identity weights reduce the layer to a row permutation of x, exactly;
* the bf16 intermediate is observable: with Linear-2 the identity, the output is Linear-1
  rounded to bf16, not Linear-1;
* power-of-two scaling of w2 scales the output exactly;
* experts are independent: permuting experts with their tokens and weights changes nothing;
* placement: every token row lands at (dst_slab, dst_row); out-of-range destinations are
  skipped; rows that receive no token stay NaN.
"""

import math

import numpy as np
import pytest

import oracle


def _bf16(x):
    return oracle.bf16_bits_to_f64(oracle.round_to_bf16_bits(np.asarray(x, dtype=np.float64)))


def _routing(T, P, seed):
    rng = np.random.default_rng(seed)
    dst_slab = rng.integers(0, P, size=T)
    dst_row = np.zeros(T, dtype=np.int64)
    cnt = np.zeros(P, dtype=np.int64)
    for t in range(T):
        dst_row[t] = cnt[dst_slab[t]]
        cnt[dst_slab[t]] += 1
    return dst_slab, dst_row, cnt


def test_brute_force_tiny():
    rng = np.random.default_rng(3)
    E, dm, df = 2, 3, 2
    offsets = [0, 2, 3]
    x = _bf16(rng.standard_normal((3, dm)))
    w1 = _bf16(rng.standard_normal((E, df, dm)))
    w2 = _bf16(rng.standard_normal((E, dm, df)))
    dst_slab, dst_row, cnt = np.array([1, 0, 1]), np.array([0, 0, 1]), [1, 2]
    h, outs = oracle.moe_layer(x, w1, w2, offsets, dst_slab, dst_row, cnt)
    for t, e in ((0, 0), (1, 0), (2, 1)):
        he = [math.fsum(x[t, k] * w1[e, f, k] for k in range(dm)) for f in range(df)]
        hb = _bf16(he)
        ye = [math.fsum(hb[f] * w2[e, o, f] for f in range(df)) for o in range(dm)]
        assert np.allclose(h[t], he, rtol=0, atol=1e-15)
        assert np.allclose(outs[dst_slab[t]][dst_row[t]], ye, rtol=0, atol=1e-15)


def test_identity_weights_permute_rows():
    rng = np.random.default_rng(4)
    E, d, T, P = 3, 8, 10, 2
    offsets = [0, 4, 4, 10]  # expert 1 has no tokens
    x = _bf16(rng.standard_normal((T, d)))
    eye = np.stack([np.eye(d)] * E)
    dst_slab, dst_row, cnt = _routing(T, P, 5)
    h, outs = oracle.moe_layer(x, eye, eye, offsets, dst_slab, dst_row, cnt)
    assert np.array_equal(h, x)
    for t in range(T):
        assert np.array_equal(outs[dst_slab[t]][dst_row[t]], x[t])


def test_intermediate_is_rounded_to_bf16():
    d = 4
    x = np.array([[1.0, 2.0 ** -9, 0.0, 0.0]])   # Linear-1 = 1 + 2^-9: not a bf16 value
    w1 = np.stack([np.eye(d) + np.eye(d, k=1)])  # h0 = x0 + x1
    w2 = np.stack([np.eye(d)])
    h, outs = oracle.moe_layer(x, w1, w2, [0, 1], [0], [0], [1])
    assert h[0, 0] == 1.0 + 2.0 ** -9
    assert outs[0][0, 0] == 1.0  # 2^-9 is under half a bf16 step at 1 (2^-8): rounds to 1


def test_power_of_two_scaling_of_w2():
    rng = np.random.default_rng(6)
    E, dm, df, T = 2, 16, 8, 9
    offsets = [0, 5, 9]
    x = _bf16(rng.standard_normal((T, dm)))
    w1 = _bf16(rng.standard_normal((E, df, dm)) / 4)
    w2 = _bf16(rng.standard_normal((E, dm, df)) / 3)
    dst_slab, dst_row, cnt = _routing(T, 3, 7)
    _, a = oracle.moe_layer(x, w1, w2, offsets, dst_slab, dst_row, cnt)
    _, b = oracle.moe_layer(x, w1, 4.0 * w2, offsets, dst_slab, dst_row, cnt)
    for p in range(3):
        assert np.array_equal(4.0 * a[p], b[p], equal_nan=True)


def test_experts_are_independent():
    rng = np.random.default_rng(8)
    E, dm, df = 3, 8, 4
    rows = [3, 1, 4]
    offsets = np.concatenate([[0], np.cumsum(rows)])
    T = int(offsets[-1])
    x = _bf16(rng.standard_normal((T, dm)))
    w1 = _bf16(rng.standard_normal((E, df, dm)))
    w2 = _bf16(rng.standard_normal((E, dm, df)))
    dst_slab, dst_row, cnt = _routing(T, 2, 9)
    _, ref = oracle.moe_layer(x, w1, w2, offsets, dst_slab, dst_row, cnt)
    perm = [2, 0, 1]
    tok = np.concatenate([np.arange(offsets[e], offsets[e + 1]) for e in perm])
    offs2 = np.concatenate([[0], np.cumsum([rows[e] for e in perm])])
    _, got = oracle.moe_layer(x[tok], w1[perm], w2[perm], offs2, dst_slab[tok], dst_row[tok], cnt)
    for p in range(2):
        assert np.array_equal(ref[p], got[p], equal_nan=True)


def test_placement_and_skipped_destinations():
    d, T = 4, 5
    x = np.arange(T * d, dtype=np.float64).reshape(T, d)
    eye = np.stack([np.eye(d)])
    dst_slab = np.array([0, 1, -1, 1, 2])   # token 2: no such destination; token 4: slab 2 of 2
    dst_row = np.array([1, 0, 0, 5, 0])     # token 3: row 5 of a 2-row slab
    outs = oracle.moe_layer(x, eye, eye, [0, T], dst_slab, dst_row, [3, 2])[1]
    assert np.array_equal(outs[0][1], x[0]) and np.array_equal(outs[1][0], x[1])
    assert np.isnan(outs[0][0]).all() and np.isnan(outs[0][2]).all() and np.isnan(outs[1][1]).all()


def test_token_subset_matches_full():
    rng = np.random.default_rng(10)
    E, dm, df = 2, 8, 4
    offsets = [0, 6, 11]
    x = _bf16(rng.standard_normal((11, dm)))
    w1 = _bf16(rng.standard_normal((E, df, dm)))
    w2 = _bf16(rng.standard_normal((E, dm, df)))
    dst_slab, dst_row, cnt = _routing(11, 2, 11)
    hf, full = oracle.moe_layer(x, w1, w2, offsets, dst_slab, dst_row, cnt)
    toks = [0, 5, 6, 10]
    hs, sub = oracle.moe_layer(x, w1, w2, offsets, dst_slab, dst_row, cnt, tokens=toks)
    for t in toks:
        assert np.array_equal(sub[dst_slab[t]][dst_row[t]], full[dst_slab[t]][dst_row[t]])
        assert np.array_equal(hs[t], hf[t])
    assert np.isnan(hs[1]).all()
