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


def test_pacing_chunks_hand_values():
    """T(c) = max(c a + V/f1, V/R - min(G, c Q/R)), smallest c minimising it.

    Remote-like burst, with the pages' printed drain rate: V = 64 MiB, R = 717 GB/s,
    Q = 8 MiB, G = 50 us, a = 1 us, f1 = 1e12 B/s.  By hand (us): V/R = 93.5967,
    Q/R = 11.6996, V/f1 = 67.1089;  c=1: max(68.1089, 81.8971) = 81.8971;
    c=2: max(69.1089, 70.1975) = 70.1975;  c=3: max(70.1089, 58.4979) = 70.1089;
    c=4: max(71.1089, 46.7983) = 71.1089 -> c = 3, 70.1089 us."""
    import attention_ulysses_a2a_amd as xs

    c, t = xs.xstage_bg_pacing_chunks(64 * 2**20, 50e-6, 1e-6, 1e12, 717e9, 8 * 2**20, c_max=16)
    assert c == 3
    assert abs(t - 70.1089e-6) < 1e-10
    c, t = xs.xstage_bg_pacing_chunks(64 * 2**20, 50e-6, 1e-6, 1e12, 717e9, 8 * 2**20, c_max=2)
    assert c == 2 and abs(t - 70.1975e-6) < 1e-10
    c, t = xs.xstage_bg_pacing_chunks(64 * 2**20, 50e-6, 1e-6, 1e12, 717e9, 8 * 2**20, c_max=1)
    assert c == 1 and abs(t - 81.8971e-6) < 1e-10


def test_pacing_chunks_local_tile_is_unpaced():
    """A FLUX-1024 output tile (128 rows x 128 x 2 B = 32 KiB) at the local parameters fitted
    on MI355X in one sweep (R 7.55 TB/s, Q 113 MiB, f1 131 GB/s; a = 1 us assumed, G = 30 us of key loop):
    c=1 gives max(1 us + 0.250 us, 4.3 ns - 15.7 us) = 1.250 us and every extra chunk adds a,
    so the tile goes out as one burst."""
    import attention_ulysses_a2a_amd as xs

    c, t = xs.xstage_bg_pacing_chunks(32768, 30e-6, 1e-6, 131e9, 7.55e12, 113 * 2**20)
    assert c == 1 and abs(t - (1e-6 + 32768 / 131e9)) < 1e-12
    # no fixed cost and no backpressure: every c ties, the smallest wins
    assert xs.xstage_bg_pacing_chunks(32768, 30e-6, 0.0, 131e9, 7.55e12, 113 * 2**20)[0] == 1


def test_pacing_chunks_rejects():
    from attention_ulysses_a2a_amd import _lib

    L = _lib.lib()
    assert L.xstage_bg_pacing_chunks(1.0, 1.0, 1.0, 1.0, 0.0, 1.0, 4, None) == 0      # R = 0
    assert L.xstage_bg_pacing_chunks(1.0, 1.0, 1.0, 0.0, 1.0, 1.0, 4, None) == 0      # f1 = 0
    assert L.xstage_bg_pacing_chunks(1.0, -1.0, 1.0, 1.0, 1.0, 1.0, 4, None) == 0     # G < 0
    assert L.xstage_bg_pacing_chunks(float("nan"), 1.0, 1.0, 1.0, 1.0, 1.0, 4, None) == 0
    assert L.xstage_bg_pacing_chunks(1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 0, None) == 0      # c_max < 1
    assert L.xstage_bg_pacing_chunks(1.0, 1.0, 1.0, 1.0, 1.0, 1.0, 1, None) == 1


def test_product_isolated_fit_matches_oracle():
    """The sweep's isolated-burst fit and the oracle's, on bursts drawn from the capacity reading."""
    rng = np.random.default_rng(7)
    R, Q, c, f1, K = 6.8e12, 140 * 2 ** 20, 9e-8, 130e9, 256
    V = np.repeat(np.array([32, 64, 128, 256, 384, 512, 768, 1024]) * 2 ** 20, 3).astype(float)
    T0 = oracle.t0_linear(K, V, c, f1)
    T = oracle.t_iss_isolated(T0, V, R, Q) * (1 + 0.005 * rng.standard_normal(V.size))
    mine = bg_model.fit_isolated(V, T, T0, R=R)
    ref = oracle.fit_isolated(V, T, T0, R=R)
    assert abs(mine["R_iso_Bps"] / ref["R_iso"] - 1) < 1e-9
    assert abs(mine["Q_iso_bytes"] / ref["Q_iso"] - 1) < 1e-9
    assert abs(mine["Q_bytes_at_R"] / ref["Q"] - 1) < 1e-9
    assert abs(mine["Q_iso_bytes"] / Q - 1) < 0.05


def test_sweep_summary_renders_every_series():
    """The markdown summary of a sweep's JSON lines (host logic only, synthetic records)."""
    import json

    from attention_ulysses_a2a_amd import bg_sweep

    lines = [json.dumps({"bg_calibration": {"wallclock_hz": 1e8, "gap_ns_per_fma_iter": 15.0}})]
    for variant in ("hot", "cold", "large"):
        for G in (0, 1):
            lines.append(json.dumps({"bg": {"variant": variant, "K": 256, "V_MiB": 64, "G_us": G, "T_iss_us": 5.0 - G,
                                            "T_iss_p10_us": 4.0, "T_iss_p90_us": 6.0, "span_us": 5.0,
                                            "period_us": 6.0, "R_direct_GBps": 7000.0 if G == 0 else None}}))
        lines.append(json.dumps({"bg_fit": {"variant": variant, "R": 7e12, "n_drain": 2, "n_points": 2,
                                            "capacity_reading": {"R_Bps": 7.1e12, "Q_bytes": 150 * 2 ** 20,
                                                                 "f1_Bps": 1.3e11, "c_s": 8.6e-8,
                                                                 "rel_err_median": 0.03}, "T0_us": {}}}))
    # isolated bursts on T = (V - 8 MiB) / 7 TB/s, well above their free time
    for vm in (64, 256, 1024):
        t = (vm - 8) * 2 ** 20 / 7e12 * 1e6
        lines.append(json.dumps({"bg": {"variant": "isolated", "K": 256, "V_MiB": vm, "G_us": 200.0,
                                        "T0_free_us": 1.0, "T_iss_us": t, "T_iss_p10_us": t, "T_iss_p90_us": t,
                                        "start_spread_us": 0.4}}))
    lines.append(json.dumps({"bg_sync_fit": {"K": 256, "free_c_s": 8.6e-8, "free_f1_Bps": 1.3e11,
                                             "R_agg_Bps": 7e12, "page_formula_rel_err_median": 0.5,
                                             "capacity_reading_rel_err_median": 0.02,
                                             "isolated": {"n_used": 5, "R_iso_Bps": 7e12, "Q_iso_bytes": 150 * 2 ** 20,
                                                          "Q_bytes_at_R": 151 * 2 ** 20}}}))
    lines.append(json.dumps({"bg_copy": {"write_GBps": 2500.0, "read_write_GBps": 5000.0, "s_per_call": 2e-4,
                                         "bytes_written": 2 ** 29}}))
    md = bg_sweep.summarize(lines)
    for head in ("## hot destinations", "## cold destinations", "## large bursts", "## isolated bursts",
                 "## plain copy"):
        assert head in md
    assert "Q_iso = 8.0 MiB" in md and "R_iso = 7.00 TB/s" in md
    assert "| 256 | 64 | 5.00 | 4.00 | 7000 |" in md and "R_agg = 13.42 TB/s" in md


def test_synchronized_fit_prefers_the_capacity_reading():
    """Aggregate bursts drawn from the capacity reading with a small Q: the fit recovers R and Q,
    and the printed formula (which lets every gap shorten the burst) fits the gapped points worse."""
    R, Q, c, f1, K = 5.9e12, 8 * 2 ** 20, 8.6e-8, 130e9, 256
    large = []
    for vm in (128, 256, 512, 1024):
        V = vm * 2 ** 20
        for G in (0, 10e-6, 20e-6, 40e-6, 80e-6, 160e-6):
            large.append((V, G, float(oracle.t_iss_fluid(G, oracle.t0_linear(K, V, c, f1), V, R, Q))))
    iso = []
    for vm in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024):
        V = vm * 2 ** 20
        iso.append((V, float(oracle.t_iss_isolated(oracle.t0_linear(K, V, c, f1), V, R, Q))))
    f = bg_model.fit_synchronized(large, iso, c, f1, K)
    assert abs(f["R_agg_Bps"] / R - 1) < 0.01
    assert abs(f["isolated"]["Q_bytes_at_R"] / Q - 1) < 0.01
    assert f["capacity_reading_rel_err_median"] < 0.01 < f["page_formula_rel_err_median"]
