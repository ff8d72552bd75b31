"""The seeded input generator: determinism, bf16 cast, workload structure, probe guarantee."""

import numpy as np
import pytest
import torch

import oracle
from synth import WORKLOADS, f32_to_bf16_bits, make_inputs, make_placement_probe, make_placement_probe_torch, workload


def test_bf16_cast_matches_torch_rne():
    x = np.random.default_rng(0).standard_normal(200000).astype(np.float32) * np.float32(3.0)
    x[:4] = [np.float32(1.0 + 2 ** -8), np.float32(1.0 + 3 * 2 ** -8), np.float32(3.4e38), np.float32(-0.0)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(x), ref)


def test_deterministic_and_shaped():
    w = workload("tiny")
    a = make_inputs(w)
    b = make_inputs(w)
    for x, y in zip(a, b):
        assert x.dtype == np.uint16 and x.shape == (w.B, w.S, w.H, w.D)
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], a[1])


def test_workload_table():
    t, f1, f2, vd = (WORKLOADS[n] for n in ("tiny", "flux1024", "flux2048", "video"))
    assert (t.B, t.S, t.H, t.D, t.P) == (1, 256, 2, 64, 2)
    assert (f1.B, f1.S, f1.H, f1.D, f1.P) == (1, 4608, 3, 128, 8)
    assert (f2.S, f2.H, f2.P) == (16896, 3, 8)
    assert (vd.S, vd.H, vd.P) == (32760, 5, 8)
    for w in (t, f1, f2, vd):
        assert w.S % w.P == 0
    assert abs(f1.flops - 3.2615e10) / 3.2615e10 < 1e-4


def test_flux1024_keys_are_halved():
    w = workload("flux1024").with_(S=64)
    q, k, v = make_inputs(w)
    rng = np.random.default_rng(w.seed)
    shape = (w.B, w.S, w.H, w.D)
    rng.standard_normal(shape, dtype=np.float32)
    k32 = rng.standard_normal(shape, dtype=np.float32) * np.float32(0.5)
    assert np.array_equal(k, f32_to_bf16_bits(k32))


def test_video_bias_makes_rows_peaked():
    """The per-key rank-1 bias raises every head's mean peak softmax weight and lowers its entropy."""
    w = workload("video").with_(S=2048)
    qb, kb, vb = make_inputs(w)
    q, k = oracle.bf16_bits_to_f64(qb), oracle.bf16_bits_to_f64(kb)
    k0 = oracle.bf16_bits_to_f64(make_inputs(w.with_(k_rank1_amp=0.0))[1])
    for h in range(w.H):
        W = oracle.attention_weights_fp64(q, k, w.scale, 0, h)
        W0 = oracle.attention_weights_fp64(q, k0, w.scale, 0, h)
        assert W.max(axis=1).mean() > 1.05 * W0.max(axis=1).mean()
        assert -(W * np.log(W)).sum(axis=1).mean() < -(W0 * np.log(W0)).sum(axis=1).mean()


def test_placement_probe_output_is_v_exactly():
    for (B, S, H, D) in [(1, 256, 2, 64), (2, 96, 3, 128)]:
        scale = 1.0 / np.sqrt(D)
        qb, kb, vb = make_placement_probe(B, S, H, D, scale)
        q, k, v = (oracle.bf16_bits_to_f64(x) for x in (qb, kb, vb))
        o = oracle.attention_fp64(q, k, v, scale)
        # off-diagonal weights are below exp(-120): zero in fp32, about 1e-52 in fp64
        assert np.max(np.abs(o - v)) <= 1e-40
        assert np.array_equal(oracle.bf16_bits_to_f64(oracle.round_to_bf16_bits(o)), v)  # -0 == +0
        assert np.array_equal(v[0, :, 0, 0], np.arange(S) % 256)
        assert np.array_equal(v[0, :, :, 2][0], np.arange(H))


@pytest.mark.parametrize("B,S,H,D", [(1, 64, 2, 128), (2, 130, 3, 64), (1, 40, 300, 64)])
def test_torch_probe_equals_numpy_probe(B, S, H, D):
    """The torch assembly of the placement probe (used at the largest tensor size) is the
    same bytes as the numpy one; H = 300 also covers head tags that round in bf16."""
    scale = 1.0 / np.sqrt(D)
    ref = make_placement_probe(B, S, H, D, scale)
    got = make_placement_probe_torch(B, S, H, D, scale, "cpu")
    for r, g in zip(ref, got):
        assert np.array_equal(r, g.view(torch.int16).numpy().view(np.uint16))
