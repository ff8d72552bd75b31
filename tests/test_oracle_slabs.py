"""Pins for the Ulysses slab permutation and the bf16 codecs of the oracle."""

import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_hand_computed_destinations():
    with open(os.path.join(GOLDEN, "slab_destinations.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert oracle.slab_destination(c["s"], c["S"], c["P"]) == (c["p"], c["r"]), c


@pytest.mark.parametrize("B,S,H,D,P", [(1, 256, 2, 64, 2), (2, 1000, 3, 4, 8), (1, 999, 2, 3, 3), (1, 16, 1, 2, 16), (3, 40, 2, 2, 1)])
def test_scatter_gather_identity(B, S, H, D, P):
    o = np.random.default_rng(0).standard_normal((B, S, H, D))
    slabs = oracle.ulysses_scatter(o, P)
    assert slabs.shape == (P, B, S // P, H, D)
    assert np.array_equal(oracle.ulysses_gather(slabs), o)


def test_p1_is_identity():
    o = np.random.default_rng(1).standard_normal((2, 24, 3, 5))
    assert np.array_equal(oracle.ulysses_scatter(o, 1)[0], o)


def test_every_element_written_once_and_where_destination_says():
    B, S, H, D, P = 2, 60, 3, 4, 6
    ids = np.arange(B * S * H * D, dtype=np.int64).reshape(B, S, H, D)
    slabs = oracle.ulysses_scatter(ids, P)
    flat = np.sort(slabs.ravel())
    assert np.array_equal(flat, np.arange(B * S * H * D))
    for s in range(S):
        p, r = oracle.slab_destination(s, S, P)
        assert np.array_equal(slabs[p, :, r], ids[:, s])


def test_indivisible_rejected():
    with pytest.raises(ValueError):
        oracle.ulysses_scatter(np.zeros((1, 10, 1, 1)), 3)
    with pytest.raises(ValueError):
        oracle.slab_destination(0, 1001, 8)


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(2).integers(0, 65536, size=4096, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite only
    got = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(got, ref)


def test_bf16_round_hand_values():
    cases = [
        (1.0, 0x3F80),
        (1.0 + 2.0 ** -8, 0x3F80),          # tie -> even (down)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),      # tie -> even (up)
        (1.0 + 2.0 ** -8 + 2.0 ** -30, 0x3F81),  # just above the tie (fp32 would round this to the tie)
        (-2.5, 0xC020),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (2.0 ** -133, 0x0001),             # smallest bf16 subnormal
        (2.0 ** -134, 0x0000),             # tie with zero -> even (zero)
        (3.0 * 2.0 ** -134, 0x0002),       # tie -> even
        (3.4e38, 0x7F80),                  # rounds past the largest finite -> inf
        (float("inf"), 0x7F80),
        (-float("inf"), 0xFF80),
    ]
    for x, bits in cases:
        assert int(oracle.round_to_bf16_bits(np.array([x]))[0]) == bits, (x, hex(bits))
    assert (int(oracle.round_to_bf16_bits(np.array([np.nan]))[0]) & 0x7FFF) > 0x7F80


def test_bf16_round_matches_torch_on_fp32_values():
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * np.float32(7.0)
    got = oracle.round_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
