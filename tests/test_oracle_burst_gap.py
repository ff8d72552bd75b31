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


def test_t0_linear_hand_values():
    """T0 read as a fixed cost c plus one producer's share V/K at its free rate f1 (hand-evaluated)."""
    # 4 producers, 8 MB: each moves 2 MB at 1 GB/s = 2 ms, plus 1 us
    assert abs(float(oracle.t0_linear(4, 8e6, 1e-6, 1e9)) - 2.001e-3) < 1e-15
    # 256 producers, 64 MiB: 262144 B each at 130 GB/s = 2.016492 us, plus 86 ns
    assert abs(float(oracle.t0_linear(256, 64 * 2 ** 20, 86e-9, 130e9)) - 2.102492308e-6) < 1e-15
    # broadcasting over (K, V)
    got = oracle.t0_linear(np.array([1, 2]), np.array([1e9, 1e9]), 0.0, 1e9)
    assert np.array_equal(got, np.array([1.0, 0.5]))


def test_t0_linear_matches_brute_force_producers():
    """K producers, each starting after c and issuing its V/K share in fixed-size pieces at f1
    (time-stepped): the last one finishes at t0_linear(K, V, c, f1)."""
    for K, V, c, f1 in ((3, 3.0e6, 2e-6, 5e8), (8, 6.4e6, 0.0, 2e9), (1, 1e6, 1e-6, 1e9)):
        dt = 1e-7
        share = V / K
        finish = []
        for _ in range(K):
            t, left = c, share
            while left > 1e-9:
                left -= min(left, f1 * dt)
                t += dt
            finish.append(t)
        assert abs(max(finish) - float(oracle.t0_linear(K, V, c, f1))) <= 2 * dt


def test_isolated_limit_of_the_fluid_reading():
    """A burst on an empty queue: the fluid reading at gaps past Q/R is max(T0, (V - Q)/R)."""
    T0, R, Q = 2e-6, 7e12, 150 * 2 ** 20
    for V in (2 ** 27, 2 ** 28, 2 ** 29, 2 ** 30):
        for G in (Q / R, 2 * Q / R, 1e-3):
            assert abs(float(oracle.t_iss_fluid(G, T0, V, R, Q)) - float(oracle.t_iss_isolated(T0, V, R, Q))) < 1e-15
    assert float(oracle.t_iss_isolated(T0, 2 ** 20, R, Q)) == T0        # absorbed entirely
    assert abs(float(oracle.t_iss_isolated(T0, 2 ** 30, R, Q)) - (2 ** 30 - Q) / R) < 1e-15


def test_simulated_isolated_bursts_agree():
    """The time-stepped queue, started empty, issues one burst in max(T0, (V - Q)/R) (fast producer)."""
    T0, R, Q = 0.01, 1.0, 0.5
    for V in (0.4, 1.0, 2.0):
        sim, dt = simulate_queue(V, T0, R, Q, G=100.0, periods=1, steps=4000)
        assert abs(sim - float(oracle.t_iss_isolated(T0, V, R, Q))) <= 5 * dt + 1e-9


def test_fit_isolated_recovers_capacity_and_rate():
    """Isolated bursts drawn from the capacity reading (with noise): the line through the
    points above T0 gives R and Q; with R given, Q is the median of V - R T."""
    rng = np.random.default_rng(3)
    R, Q, c, f1, K = 6.5e12, 160 * 2 ** 20, 1e-7, 130e9, 256
    V = np.repeat(np.array([32, 64, 128, 256, 384, 512, 768, 1024]) * 2 ** 20, 4).astype(float)
    T0 = oracle.t0_linear(K, V, c, f1)
    T = oracle.t_iss_isolated(T0, V, R, Q) * (1 + 0.01 * rng.standard_normal(V.size))
    f = oracle.fit_isolated(V, T, T0)
    assert abs(f["R_iso"] / R - 1) < 0.03 and abs(f["Q_iso"] / Q - 1) < 0.08
    g = oracle.fit_isolated(V, T, T0, R=R)
    assert abs(g["Q"] / Q - 1) < 0.08
    # bursts that all fit in the capacity identify nothing
    small = np.array([1, 2, 4, 8]) * 2 ** 20
    t0s = oracle.t0_linear(K, small, c, f1)
    assert "Q_iso" not in oracle.fit_isolated(small, oracle.t_iss_isolated(t0s, small, R, Q), t0s)
