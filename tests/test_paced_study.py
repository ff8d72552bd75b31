"""Host side of the paced-epilogue study: how the launch's burst is handed to the Burst-Gap
pacing chooser (hand-evaluated values), and the summary table.  Runs without a GPU."""

import math

import pytest

import attention_ulysses_a2a_amd as xs
from attention_ulysses_a2a_amd import paced_study as ps


@pytest.fixture(scope="module", autouse=True)
def _lib():
    xs.lib()


def test_model_choice_one_tile_per_producer_is_unpaced():
    # 256 producers x one 128 x 128 bf16 tile = 8 MiB; free issue a + V / (K f1); the drain
    # term V/R - min(G, Q/R) is below it, so one chunk: t = 86 ns + 8 MiB / (256 * 131 GB/s).
    m = ps.model_choice(xs, 256, 32768, 500e-6, 8)
    V = 256 * 32768.0
    assert m["V_bytes"] == V
    assert m["c"] == 1
    assert math.isclose(m["t_visible_us"], (86e-9 + V / (256 * 131e9)) * 1e6, rel_tol=1e-12)


def test_model_choice_large_bursts_are_paced():
    # 1 MiB per producer (V = 256 MiB): T(c) = max(c a + V/(K f1), V/R - min(G, c Q/R)); with
    # G = 100 us the drain term falls by Q/R = 1.21 us per chunk and stays above the issue
    # term up to c = 8, so the chooser takes c_max.
    K, tile, G = 256, 1 << 20, 100e-6
    V = K * float(tile)
    m = ps.model_choice(xs, K, tile, G, 8)
    want = max(8 * 86e-9 + V / (K * 131e9), V / 5.64e12 - min(G, 8 * 6.5 * 2 ** 20 / 5.64e12))
    assert m["c"] == 8
    assert math.isclose(m["t_visible_us"], want * 1e6, rel_tol=1e-12)


def test_summary_table():
    line = {"paced_study": "video", "B": 1, "S": 32760, "H": 5, "D": 128, "P": 8, "n_tiles": 1280,
            "n_workgroups": 256, "ms": {"product": 2.0, "product_unsplit": 2.1, "paced_c1": 2.5, "paced_c8": 2.51},
            "paced_spread_pct": 0.4, "best_c_measured": 1, "model_c_vs_best_pct": 0.0,
            "model": ps.model_choice(xs, 256, 32768, 400e-6, 8)}
    md = ps.summarize([line], "python bench.py --paced", "abc")
    assert "| paced_c1 | 2.5000 | 1.250 |" in md
    assert "5.00 tiles each" in md
    assert "c = 1, issuer-visible 0.336 us" in md
