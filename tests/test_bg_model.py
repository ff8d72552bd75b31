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
