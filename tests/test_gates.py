"""Host logic of the parity gates (no GPU): the near-tie argmax rule and the
window-edge distributional gate, each shown to pass on agreeing inputs and to fail on a
planted mistake."""
import json
import os

import numpy as np
import pytest

from tests.gpu_util import F32_LOGIT_BAND, argmax_check, distributional_gate, logit_band_check, oracle_band

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_values.json")))
FLOOR = GOLD["window_edge_top1_floor"]["value"][0] / GOLD["window_edge_top1_floor"]["value"][1]
CEIL = GOLD["window_edge_logprob_ceiling"]["value"]
TOP = GOLD["window_edge_top_ids"]["value"]


def _logits(n=400, v=300, seed=0):
    return np.random.default_rng(seed).standard_normal((n, v)).astype(np.float32) * 3


def test_distributional_gate_passes_agreeing_and_small_noise():
    r = _logits()
    st = distributional_gate(r, r, TOP, FLOOR, CEIL)
    assert st["top1"] == 1.0 and st["max_gap"] == 0.0
    noisy = r + np.random.default_rng(1).standard_normal(r.shape).astype(np.float32) * 1e-3
    assert distributional_gate(noisy, r, TOP, FLOOR, CEIL)["top1"] > 0.99


def test_distributional_gate_catches_a_failed_quarter():
    r = _logits()
    g = r.copy()
    q = slice(300, 360)                                     # most of the last quarter argmaxes elsewhere
    g[q, :] = r[q, :]
    g[q, np.argmin(r[q], -1)] = r[q].max(-1) + 1.0
    agree = (np.argmax(g, -1) == np.argmax(r, -1)).mean()
    assert agree >= FLOOR                                   # the global rate alone would pass
    with pytest.raises(AssertionError):
        distributional_gate(g, r, TOP, FLOOR, 1e9)


def test_distributional_gate_catches_a_large_logprob_gap_and_nonfinite():
    r = _logits()
    g = r.copy()
    top2 = np.argsort(-r[7])[1]
    g[7, top2] -= 40.0                                      # one top-64 id pushed far down
    with pytest.raises(AssertionError):
        distributional_gate(g, r, TOP, FLOOR, CEIL)
    g = r.copy()
    g[3, 5] = np.nan
    with pytest.raises(AssertionError):
        distributional_gate(g, r, TOP, FLOOR, CEIL)


def test_argmax_check_pins_clear_winners_and_tolerates_near_ties():
    ref = np.array([[0.0, 5.0, 1.0], [2.0, 2.0 + 1e-4, 0.0]])
    pinned, near, fails = argmax_check(np.array([1, 0]), ref, 1e-3)   # row 1: a near tie, either id
    assert (pinned, near, fails) == (1, 1, [])
    pinned, near, fails = argmax_check(np.array([2, 0]), ref, 1e-3)   # row 0 pinned to 1, not 2
    assert fails and fails[0][0] == 0
    pinned, near, fails = argmax_check(np.array([1, 2]), ref, 1e-3)   # near tie, but id 2 is far below
    assert fails and fails[0][0] == 1
    # per-position allowance: a wide band turns row 0 into a near tie too
    pinned, near, fails = argmax_check(np.array([1, 0]), ref, np.array([3.0, 1e-3]))
    assert (pinned, near) == (0, 2)


def test_argmax_check_band_comes_from_the_oracle_only():
    ref = np.random.default_rng(2).standard_normal((5, 50))
    with pytest.raises(ValueError):                                    # a logits array is not a band
        argmax_check(np.argmax(ref, -1), ref, ref + 0.1)


def test_oracle_band_is_slack_times_the_bf16_rounded_deviation():
    ref = np.zeros((2, 4))
    rb = np.array([[0.0, 0.2, -0.1, 0.0], [0.05, 0.0, 0.0, -0.3]])
    np.testing.assert_allclose(oracle_band(ref, rb), [0.25, 0.375])
    np.testing.assert_allclose(oracle_band(ref, rb, slack=2.0), [0.4, 0.6])
    np.testing.assert_allclose(oracle_band(ref), [F32_LOGIT_BAND] * 2)
    d, b = logit_band_check(ref + 0.2, ref, oracle_band(ref, rb))
    assert (d, b) == (pytest.approx(0.2), pytest.approx(0.375))
