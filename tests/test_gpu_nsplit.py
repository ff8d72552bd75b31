"""The split-count override (xstage_attn_a2a_fwd_nsplit) on MI355X.

Every available key-split count must give the attention result: the merge of n_split
partial softmax states is exact up to rounding (online softmax, X-Stage explainer,
"Contributions", FlashAttention-A2A item: the fused call computes attention followed by the
all-to-all), so each count is compared with the fp64 oracle at the value bar of the product
call (max-abs 1e-2, mean-abs 1e-3, every row), the placement probe must come out exact, and
the count the library's own model picks must reproduce xstage_attn_a2a_fwd bit for bit.
One zeroed workspace serves every call in turn (each call leaves its counters at zero).
Shapes: the FLUX-1024 share (one-round launches with placement-sized ranges up to 4 splits,
then multi-round), a ragged D = 64 sequence (16 key blocks) and B = 2 with five heads.
"""

import sys

import numpy as np
import pytest
import torch

import attention_ulysses_a2a_amd as xs
import oracle
from synth import Workload, make_inputs, make_placement_probe, workload
from tests.gpu_util import NAN_BF16, GuardedSlabs, split_ws, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [
    ("flux1024", None),
    ("ragged-d64", Workload("ragged-d64", 1, 1000, 2, 64, 8, seed=41)),
    ("b2h5", Workload("b2h5", 2, 2048, 5, 128, 4, seed=42)),
]


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def available(w):
    out = []
    for k in range(1, 16):
        try:
            need = xs.xstage_attn_nsplit_ws_size(w.B, w.S, w.H, w.D, k)
        except xs.XStageError:
            continue
        if need <= split_ws().numel():
            out.append(k)
    return out


def run(w, qb, kb, vb, scale, k=None):
    q, k_, v = to_dev(qb), to_dev(kb), to_dev(vb)
    g = GuardedSlabs(w.P, w.B, w.S // w.P, w.H, w.D)
    if k is None:
        xs.xstage_attn_a2a_fwd(q, k_, v, g.views, scale, split_ws=split_ws())
    else:
        xs.xstage_attn_a2a_fwd_nsplit(q, k_, v, g.views, k, scale, split_ws=split_ws() if k > 1 else None)
    torch.cuda.synchronize()
    assert g.guards_intact()
    return g.slabs_host()


@pytest.mark.parametrize("name,w", SHAPES)
def test_every_split_count_matches_the_oracle(name, w):
    w = w or workload(name)
    ks = available(w)
    model_k = xs.xstage_attn_a2a_plan(w.B, w.S, w.H, w.D)[1]
    log(f"nsplit {name}: B={w.B} S={w.S} H={w.H} D={w.D} P={w.P}; counts {ks}; model picks {model_k}")
    assert 1 in ks and model_k in ks
    qb, kb, vb = make_inputs(w)
    ref = oracle.attention_fp64(*(oracle.bf16_bits_to_f64(x) for x in (qb, kb, vb)), w.scale)
    product = run(w, qb, kb, vb, w.scale)
    for k in ks:
        slabs = run(w, qb, kb, vb, w.scale, k)
        assert not np.any(slabs == NAN_BF16), k
        got = oracle.ulysses_gather(oracle.bf16_bits_to_f64(slabs))
        err = np.abs(got - ref)
        log(f"  n_split={k:2d}: max_abs={err.max():.3e} mean_abs={err.mean():.3e}"
            + (" (model's count: equal to the product call)" if k == model_k else ""))
        assert np.isfinite(got).all()
        assert err.max() <= 1e-2 and err.mean() <= 1e-3, k
        if k == model_k:
            assert np.array_equal(slabs, product)


@pytest.mark.parametrize("name,w", SHAPES)
def test_split_counts_place_exactly(name, w):
    w = w or workload(name)
    ks = available(w)
    pq, pk, pv = make_placement_probe(w.B, w.S, w.H, w.D, 1.0 / np.sqrt(w.D))
    want = oracle.ulysses_scatter(pv, w.P)
    for k in (ks[1] if len(ks) > 1 else ks[0], ks[-1]):
        got = run(w, pq, pk, pv, 1.0 / np.sqrt(w.D), k)
        log(f"nsplit probe {name} n_split={k}: exact {np.array_equal(got, want)}")
        assert np.array_equal(got, want), k
