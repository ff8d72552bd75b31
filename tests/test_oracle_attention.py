"""Pins for the float64 attention oracle, independent of the oracle's own code.

* brute force: pure-Python loops with math.exp and exactly rounded sums (math.fsum) on
  tiny shapes, without the max shift the oracle uses;
* library routine: torch's float64 CPU scaled_dot_product_attention;
* closed forms and invariants of softmax attention;
* planted mistakes: mutated copies of the oracle must fail the brute-force pin.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from synth import make_inputs, workload


def brute_attention(q, k, v, scale):
    B, S, H, D = q.shape
    Dv = v.shape[3]
    out = np.zeros((B, S, H, Dv))
    for b in range(B):
        for h in range(H):
            for i in range(S):
                logits = [scale * math.fsum(q[b, i, h, d] * k[b, j, h, d] for d in range(D)) for j in range(S)]
                ex = [math.exp(x) for x in logits]
                z = math.fsum(ex)
                for d in range(Dv):
                    out[b, i, h, d] = math.fsum(ex[j] * v[b, j, h, d] for j in range(S)) / z
    return out


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("B,S,H,D", [(1, 1, 1, 1), (1, 2, 1, 2), (2, 3, 2, 4), (1, 7, 2, 4), (1, 8, 1, 2), (2, 8, 2, 1)])
def test_brute_force(B, S, H, D):
    q, k, v = rand((B, S, H, D), 1), rand((B, S, H, D), 2), rand((B, S, H, D), 3)
    scale = 0.7
    ref = brute_attention(q, k, v, scale)
    got = oracle.attention_fp64(q, k, v, scale)
    assert np.max(np.abs(got - ref)) <= 1e-12


def test_rows_subset_matches_full():
    q, k, v = rand((2, 37, 3, 8), 4), rand((2, 37, 3, 8), 5), rand((2, 37, 3, 8), 6)
    full = oracle.attention_fp64(q, k, v, 0.3, block=5)
    rows = [0, 5, 36, 17]
    part = oracle.attention_fp64(q, k, v, 0.3, rows=rows, block=3)
    assert np.max(np.abs(part - full[:, rows])) <= 1e-14


def sdpa64(q, k, v, scale):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, scale=scale)
    return o.numpy().transpose(0, 2, 1, 3)


def test_torch_sdpa_tiny_workload():
    w = workload("tiny")
    q, k, v = (oracle.bf16_bits_to_f64(x) for x in make_inputs(w))
    got = oracle.attention_fp64(q, k, v, w.scale)
    assert np.max(np.abs(got - sdpa64(q, k, v, w.scale))) <= 1e-10


@pytest.mark.parametrize("name", ["flux1024", "flux2048", "video"])
def test_torch_sdpa_query_slices(name):
    """512 query rows of each large workload against torch's fp64 SDPA over the full key set."""
    w = workload(name)
    q, k, v = (oracle.bf16_bits_to_f64(x) for x in make_inputs(w))
    rows = np.linspace(0, w.S - 1, 512).astype(np.int64)
    got = oracle.attention_fp64(q, k, v, w.scale, rows=rows)
    ref = sdpa64(np.ascontiguousarray(q[:, rows]), k, v, w.scale)
    assert np.max(np.abs(got - ref)) <= 1e-10


def test_identical_value_rows():
    q, k = rand((1, 19, 2, 5), 7), rand((1, 19, 2, 5), 8)
    row = rand((3,), 9)
    v = np.broadcast_to(row, (1, 19, 2, 3)).copy()
    got = oracle.attention_fp64(q, k, v, 1.3)
    assert np.max(np.abs(got - row)) <= 1e-12


def test_weights_sum_to_one_and_are_positive():
    q, k = rand((2, 23, 2, 6), 10) * 3, rand((2, 23, 2, 6), 11) * 3
    for b in range(2):
        for h in range(2):
            W = oracle.attention_weights_fp64(q, k, 0.9, b, h)
            assert np.all(W > 0)
            assert np.max(np.abs(W.sum(axis=1) - 1.0)) <= 1e-12


def test_weights_match_output():
    q, k, v = rand((1, 13, 2, 4), 12), rand((1, 13, 2, 4), 13), rand((1, 13, 2, 4), 14)
    o = oracle.attention_fp64(q, k, v, 0.5)
    for h in range(2):
        W = oracle.attention_weights_fp64(q, k, 0.5, 0, h)
        assert np.max(np.abs(W @ v[0, :, h, :] - o[0, :, h, :])) <= 1e-12


@pytest.mark.parametrize("zero", ["scale", "q"])
def test_uniform_weights_give_column_mean(zero):
    q, k, v = rand((2, 17, 2, 4), 15), rand((2, 17, 2, 4), 16), rand((2, 17, 2, 4), 17)
    if zero == "q":
        q = np.zeros_like(q)
        scale = 2.0
    else:
        scale = 0.0
    got = oracle.attention_fp64(q, k, v, scale)
    mean = v.mean(axis=1, keepdims=True)
    assert np.max(np.abs(got - mean)) <= 1e-12


def test_single_key():
    q, k, v = rand((2, 1, 3, 4), 18), rand((2, 1, 3, 4), 19), rand((2, 1, 3, 4), 20)
    assert np.max(np.abs(oracle.attention_fp64(q, k, v, 5.0) - v)) <= 1e-15


def test_permutation_equivariance():
    rng = np.random.default_rng(21)
    q, k, v = rand((1, 29, 2, 4), 22), rand((1, 29, 2, 4), 23), rand((1, 29, 2, 4), 24)
    o = oracle.attention_fp64(q, k, v, 0.8)
    pk = rng.permutation(29)
    assert np.max(np.abs(oracle.attention_fp64(q, k[:, pk], v[:, pk], 0.8) - o)) <= 1e-12
    pq = rng.permutation(29)
    assert np.max(np.abs(oracle.attention_fp64(q[:, pq], k, v, 0.8) - o[:, pq])) <= 1e-12


def test_convex_hull():
    q, k, v = rand((1, 31, 2, 5), 25) * 4, rand((1, 31, 2, 5), 26) * 4, rand((1, 31, 2, 5), 27)
    o = oracle.attention_fp64(q, k, v, 1.0)
    lo = v.min(axis=1, keepdims=True)
    hi = v.max(axis=1, keepdims=True)
    assert np.all(o >= lo - 1e-12) and np.all(o <= hi + 1e-12)


def test_heads_and_batches_independent():
    q, k, v = rand((2, 9, 3, 4), 28), rand((2, 9, 3, 4), 29), rand((2, 9, 3, 4), 30)
    o = oracle.attention_fp64(q, k, v, 0.6)
    for b in range(2):
        for h in range(3):
            sl = (slice(b, b + 1), slice(None), slice(h, h + 1))
            assert np.max(np.abs(oracle.attention_fp64(q[sl], k[sl], v[sl], 0.6) - o[sl])) <= 1e-15


def test_large_logits_are_stable():
    """Logits near 1e3 overflow a shift-free exp; the max shift must keep the result finite."""
    q, k, v = rand((1, 16, 1, 4), 31) * 30, rand((1, 16, 1, 4), 32) * 30, rand((1, 16, 1, 4), 33)
    o = oracle.attention_fp64(q, k, v, 1.0)
    assert np.all(np.isfinite(o))
    W = oracle.attention_weights_fp64(q, k, 1.0, 0, 0)
    assert np.max(np.abs(W @ v[0, :, 0, :] - o[0, :, 0, :])) <= 1e-12


# --- planted mistakes: each mutated oracle must be caught by the brute-force pin -------------

def _mut_no_scale(q, k, v, scale):
    return oracle.attention_fp64(q, k, v, 1.0)


def _mut_kv_head_swap(q, k, v, scale):
    return oracle.attention_fp64(q, k[:, :, ::-1], v, scale)


def _mut_softmax_over_queries(q, k, v, scale):
    out = np.empty_like(v)
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            L = scale * q[b, :, h, :] @ k[b, :, h, :].T
            W = np.exp(L - L.max(axis=0, keepdims=True))
            W /= W.sum(axis=0, keepdims=True)
            out[b, :, h, :] = W @ v[b, :, h, :]
    return out


def _mut_transposed_scores(q, k, v, scale):
    out = np.empty_like(v)
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            L = (scale * q[b, :, h, :] @ k[b, :, h, :].T).T
            W = np.exp(L - L.max(axis=1, keepdims=True))
            W /= W.sum(axis=1, keepdims=True)
            out[b, :, h, :] = W @ v[b, :, h, :]
    return out


def _mut_drop_normaliser(q, k, v, scale):
    out = np.empty_like(v)
    for b in range(q.shape[0]):
        for h in range(q.shape[2]):
            L = scale * q[b, :, h, :] @ k[b, :, h, :].T
            W = np.exp(L - L.max(axis=1, keepdims=True))
            out[b, :, h, :] = W @ v[b, :, h, :]
    return out


@pytest.mark.parametrize("mutant", [_mut_no_scale, _mut_kv_head_swap, _mut_softmax_over_queries,
                                    _mut_transposed_scores, _mut_drop_normaliser])
def test_planted_mistakes_are_caught(mutant):
    q, k, v = rand((1, 7, 2, 4), 40), rand((1, 7, 2, 4), 41), rand((1, 7, 2, 4), 42)
    ref = brute_attention(q, k, v, 0.7)
    assert np.max(np.abs(mutant(q, k, v, 0.7) - ref)) > 1e-6
