"""Pins for the Burst-Gap model: hand values, regimes, a brute-force queue simulation, the fit."""

import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load_hand():
    with open(os.path.join(GOLDEN, "burst_gap_hand_values.json")) as f:
        return json.load(f)


def test_hand_values_page_formula():
    g = load_hand()
    for c in g["page_formula"]:
        got = float(oracle.t_iss(c["G_s"], g["T0_s"], g["V_bytes"], g["R_bytes_per_s"]))
        assert abs(got - c["T_iss_s"]) <= g["tolerance_s"], c


def test_hand_values_fluid_reading():
    g = load_hand()
    for c in g["fluid_reading"]:
        got = float(oracle.t_iss_fluid(c["G_s"], g["T0_s"], g["V_bytes"], g["R_bytes_per_s"], g["Q_bytes"]))
        assert abs(got - c["T_iss_s"]) <= g["tolerance_s"], c


def test_regimes_slope_and_knee():
    T0, V, R = 3e-6, 8 * 2 ** 20, 1.5e12
    knee = V / R - T0
    G = np.linspace(0, 3 * knee, 301)
    T = oracle.t_iss(G, T0, V, R)
    free = G >= knee
    assert np.all(T[free] == T0)                      # backpressure-free: exactly T0
    d = G[~free]
    assert np.allclose(T[~free], V / R - d, rtol=0, atol=1e-18)  # drain-dominated
    slope = np.diff(T[~free]) / np.diff(d)
    assert np.allclose(slope, -1.0)
    assert abs(float(oracle.t_iss(knee, T0, V, R)) - T0) < 1e-18  # continuous at the knee
    reg = oracle.regime(G, T0, V, R)
    assert set(reg[free]) == {"free"} and set(reg[~free]) == {"drain"}


def test_t0_dominates_when_drain_is_fast():
    assert float(oracle.t_iss(0.0, 5e-6, 1024, 1e15)) == 5e-6


def test_fluid_reading_reduces_to_page_formula_below_q_over_r():
    T0, V, R, Q = 1e-6, 2 ** 24, 1e12, 2 ** 22
    G = np.linspace(0, Q / R, 50)
    assert np.allclose(oracle.t_iss_fluid(G, T0, V, R, Q), oracle.t_iss(G, T0, V, R), rtol=0, atol=1e-18)


def simulate_queue(V, T0, R, Q, G, periods=25, steps=4000):
    """Brute-force time-stepped fluid queue: issue at V/T0 while space remains, drain at R."""
    f = V / T0
    dt = min(T0, V / R) / steps
    backlog = 0.0
    out = []
    for _ in range(periods):
        remaining = V
        n = 0
        while remaining > 1e-12 * V:
            backlog = max(0.0, backlog - R * dt)
            iss = min(f * dt, remaining, Q - backlog)
            backlog += iss
            remaining -= iss
            n += 1
        out.append(n * dt)
        backlog = max(0.0, backlog - R * G)
    return float(np.median(out[periods // 2:])), dt


@pytest.mark.parametrize("G", [0.0, 0.1, 0.25, 0.3, 0.5, 1.0])
@pytest.mark.parametrize("Q", [0.3, 2.0])
def test_fluid_reading_matches_brute_force_queue(G, Q):
    V, T0, R = 1.0, 0.2, 1.0
    sim, dt = simulate_queue(V, T0, R, Q, G)
    model = float(oracle.t_iss_fluid(G, T0, V, R, Q))
    assert abs(sim - model) <= 5 * dt + 1e-9, (sim, model)


def test_fit_recovers_page_formula_parameters():
    """Data drawn from the printed formula with arbitrary T0(K, V): the page fit returns them."""
    rng = np.random.default_rng(0)
    R = 2.0e12
    pts, t0 = [], {}
    for K in (32, 64, 128, 256):
        for V in (1, 4, 16, 64):
            Vb = V * 2 ** 20
            t0[(K, Vb)] = float(rng.uniform(1e-6, 5e-6)) + Vb / (K * 40e9)
            for G in (0, 1e-6, 2e-6, 5e-6, 10e-6, 20e-6, 80e-6):
                for _ in range(3):
                    T = float(oracle.t_iss(G, t0[(K, Vb)], Vb, R)) * (1 + 0.01 * rng.standard_normal())
                    pts.append((K, Vb, G, T))
    fit = oracle.fit_burst_gap(pts)
    assert abs(fit["R"] / R - 1) < 0.03
    for kv, v in t0.items():
        assert abs(fit["T0"][(float(kv[0]), float(kv[1]))] / v - 1) < 0.03
    assert fit["rel_err_median"] < 0.02


def test_fit_recovers_fluid_parameters():
    """Data drawn from the capacity reading: the fluid fit returns (c, f1, R, Q)."""
    rng = np.random.default_rng(1)
    c, f1, R, Q = 1.5e-6, 40e9, 2.0e12, 6.0 * 2 ** 20
    pts = []
    for K in (32, 64, 128, 256):
        for V in (1, 4, 16, 64):
            Vb = V * 2 ** 20
            for G in (0, 1e-6, 2e-6, 5e-6, 10e-6, 20e-6):
                for _ in range(3):
                    T0 = float(oracle.t0_linear(K, Vb, c, f1))
                    T = float(oracle.t_iss_fluid(G, T0, Vb, R, Q)) * (1 + 0.005 * rng.standard_normal())
                    pts.append((K, Vb, G, T))
    fl = oracle.fit_burst_gap(pts)["fluid"]
    assert abs(fl["R"] / R - 1) < 0.03
    assert abs(fl["Q"] / Q - 1) < 0.1
    assert abs(fl["f1"] / f1 - 1) < 0.05
    assert abs(fl["c"] / c - 1) < 0.2
    assert fl["rel_err_median"] < 0.01
