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
