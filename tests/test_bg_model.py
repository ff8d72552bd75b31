"""The product's Burst-Gap fit (used by the sweep driver) against the oracle's fit and the
hand-evaluated values; runs on the CPU (the formula is the library's host function)."""

import numpy as np
import pytest

import oracle

bg_model = pytest.importorskip("attention_ulysses_a2a_amd.bg_model")


def synthetic(seed, fluid):
    rng = np.random.default_rng(seed)
    R, Q, c, f1 = 2.0e12, 6.0 * 2 ** 20, 1.5e-6, 40e9
    pts = []
    for K in (32, 64, 128, 256):
        for V in (1, 4, 16, 64):
            Vb = V * 2 ** 20
            T0 = float(oracle.t0_linear(K, Vb, c, f1))
            for G in (0, 1e-6, 2e-6, 5e-6, 10e-6, 20e-6):
                for _ in range(2):
                    T = oracle.t_iss_fluid(G, T0, Vb, R, Q) if fluid else oracle.t_iss(G, T0, Vb, R)
                    pts.append((K, Vb, G, float(T) * (1 + 0.005 * rng.standard_normal())))
    return pts


@pytest.mark.parametrize("fluid", [False, True])
def test_product_fit_matches_oracle_fit(fluid):
    pts = synthetic(3, fluid)
    mine = bg_model.fit(pts)
    ref = oracle.fit_burst_gap(pts)
    assert abs(mine["R"] / ref["R"] - 1) < 1e-9
    for (k, v), t in ref["T0"].items():
        assert abs(mine["T0"][f"K{int(k)}_V{int(v)}"] / t - 1) < 1e-12
    assert abs(mine["rel_err_median"] - ref["rel_err_median"]) < 1e-9
    cr, fr = mine["capacity_reading"], ref["fluid"]
    assert abs(cr["R_Bps"] / fr["R"] - 1) < 0.02
    assert abs(cr["Q_bytes"] / fr["Q"] - 1) < 0.05


def test_library_formula_matches_oracle():
    G = np.linspace(0, 120e-6, 41)
    got = bg_model.t_iss(G, 10e-6, 64 * 2 ** 20, 717e9)
    assert np.allclose(got, oracle.t_iss(G, 10e-6, 64 * 2 ** 20, 717e9), rtol=0, atol=1e-15)
    got_q = bg_model.t_iss_capacity(G, 10e-6, 64 * 2 ** 20, 717e9, 8 * 2 ** 20)
    assert np.allclose(got_q, oracle.t_iss_fluid(G, 10e-6, 64 * 2 ** 20, 717e9, 8 * 2 ** 20), rtol=0, atol=1e-15)
