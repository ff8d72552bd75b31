"""Host-side pieces of the store-span study (no GPU): the completion-coupled prediction and
the span extraction and the loop clock from per-wave stamps."""

import numpy as np
import pytest

from attention_ulysses_a2a_amd import xstage_study
from attention_ulysses_a2a_amd.xstage_study import coupled_prediction, spans_from_stamps


def test_coupled_prediction_hand_values():
    # 100 us kernel, 4 generations of workgroups per slot, 2 us drain each -> 108 us
    assert abs(coupled_prediction(100e-6, 4, 2e-6) - 108e-6) < 1e-15
    assert coupled_prediction(50e-6, 0, 3e-6) == 50e-6


def test_spans_from_stamps():
    hz = 100e6  # 10 ns ticks
    st = np.zeros((2, 4, 4), dtype=np.int64)
    st[0, 0] = [100, 1100, 1300, 1500]   # stored: epilogue 200 ticks, drain 200 ticks
    st[0, 1] = [100, 1100, 1250, 0]      # stored, not waited on: epilogue only
    st[1, 2] = [100, 900, 0, 0]          # stored nothing (split that did not merge)
    epi, drain = spans_from_stamps(st, hz)
    assert np.allclose(sorted(epi), [1.5e-6, 2.0e-6])
    assert np.allclose(drain, [2.0e-6])


def test_loop_clock_from_stamps():
    hz = 100e6
    # two waves: 10 us of wall clock with 20000 and 18000 shader ticks (2.0 and 1.8 GHz); a
    # third with a 1 us loop is below the minimum span and ignored
    st = np.array([[0, 1000, 5, 20005], [10, 1010, 0, 18000], [0, 100, 0, 99999]], dtype=np.int64)
    assert xstage_study.loop_clock_ghz(st, hz) == pytest.approx(1.9)
    assert xstage_study.loop_clock_ghz(st[2:], hz) is None


def test_study_summary_table():
    """The markdown table of a study's JSON lines (host logic, a synthetic record)."""
    import json

    rec = {"S": 4608, "H_local": 3, "D": 128, "P": 8, "workgroups": 432, "key_splits": 4, "rounds": 0.84,
           "t_attn_us": 38.6, "t_fused_us": 38.5, "t_traced_us": 39.0, "t_nostore_us": 38.2, "t_coupled_us": 39.1,
           "overhead_fused_vs_attn_us": -0.1, "overhead_fused_vs_nostore_us": 0.3,
           "overhead_coupled_vs_nostore_us": 0.9, "epilogue_span_us_median": 5.3, "epilogue_span_us_p90": 6.0,
           "drain_span_us_median": 0.12, "drain_span_us_p90": 0.16, "coupled_model_us": 38.6,
           "loop_clock_ghz": 1.98, "iterations": 1300}
    md = xstage_study.summarize([json.dumps(rec)], "abc")
    assert "`abc`" in md
    assert "| 4608 | 432 | 4 | 0.84 | 38.6 | 38.5 | -0.10 | 39.0 | 38.2 | 39.1 | +0.80 | +0.90 | 5.30 | 0.12 / 0.16 | 38.6 | 1.98 |" in md
