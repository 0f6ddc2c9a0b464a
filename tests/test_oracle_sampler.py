"""Pins of the oracle sampler (Step 8 of the article), CPU only."""
import numpy as np
import pytest

import oracle


def _logits(probs):
    return np.log(np.asarray(probs, dtype=np.float64)).astype(np.float32)


def test_greedy_is_argmax_with_lowest_id_on_ties():
    l = np.array([0.1, 2.0, -1.0, 2.0, 1.9], np.float32)
    assert oracle.sample(l, 0.0, 0.9, 0.5) == 1
    assert oracle.sample(np.zeros(100, np.float32), 0.0, 0.9, 0.99) == 0


def test_top_p_hand_cases():
    l = _logits([0.5, 0.3, 0.2])
    # p = 0.9: cumsum (0.5, 0.8, 1.0) -> 2 entries below 0.9 -> keep 3; plain inverse CDF
    assert oracle.sample(l, 1.0, 0.9, 0.49) == 0
    assert oracle.sample(l, 1.0, 0.9, 0.51) == 1
    assert oracle.sample(l, 1.0, 0.9, 0.81) == 2
    # p = 0.75: keep 2, renormalised to (0.625, 0.375)
    assert oracle.sample(l, 1.0, 0.75, 0.624) == 0
    assert oracle.sample(l, 1.0, 0.75, 0.626) == 1
    assert oracle.sample(l, 1.0, 0.75, 0.9999) == 1
    # order is by probability, not by id
    l2 = _logits([0.2, 0.3, 0.5])
    assert oracle.sample(l2, 1.0, 0.75, 0.1) == 2
    assert oracle.sample(l2, 1.0, 0.75, 0.7) == 1


def test_top_p_tiny_keeps_only_the_argmax():
    rng = np.random.default_rng(0)
    l = rng.standard_normal(5000).astype(np.float32)
    for u in (0.0, 0.3, 0.999999):
        assert oracle.sample(l, 0.7, 1e-9, u) == int(np.argmax(l))


def test_temperature_sharpens():
    # at T -> 0+ with top_p = 1 the draw concentrates on the argmax
    l = np.array([1.0, 1.5, 0.2], np.float32)
    assert oracle.sample(l, 1e-3, 1.0, 0.999) == 1
    # temperature divides the logits: T = 2 on l equals T = 1 on l / 2
    rng = np.random.default_rng(1)
    l = rng.standard_normal(1000).astype(np.float32)
    for u in rng.random(20):
        assert oracle.sample(l, 2.0, 0.9, u) == oracle.sample((l / 2).astype(np.float32), 1.0, 0.9, u)


def test_equal_probabilities_ordered_by_id():
    l = np.zeros(10, np.float32)
    # all equal: nucleus of p = 0.35 keeps ids 0..3 (cum 0.1..0.4); u splits them evenly
    assert oracle.sample(l, 1.0, 0.35, 0.0) == 0
    assert oracle.sample(l, 1.0, 0.35, 0.26) == 1
    assert oracle.sample(l, 1.0, 0.35, 0.99) == 3


def test_draw_frequencies_follow_the_renormalised_nucleus():
    rng = np.random.default_rng(2)
    l = (rng.standard_normal(50) * 1.5).astype(np.float32)
    T, p = 0.7, 0.9
    z = l.astype(np.float64) / T
    probs = np.exp(z - z.max())
    probs /= probs.sum()
    order = np.lexsort((np.arange(50), -l.astype(np.float64)))
    cum = np.cumsum(probs[order])
    c = int(np.sum(cum < p)) + 1
    nucleus = order[:c]
    expect = probs[nucleus] / probs[nucleus].sum()
    n = 100000
    us = rng.random(n)
    counts = np.zeros(50)
    for u in us:
        counts[oracle.sample(l, T, p, u)] += 1
    assert counts[np.setdiff1d(np.arange(50), nucleus)].sum() == 0
    obs = counts[nucleus]
    chi2 = float(np.sum((obs - n * expect) ** 2 / (n * expect)))
    # chi-square with c-1 degrees of freedom; 99.9% quantile is well below 3 * dof + 30
    assert chi2 < 3 * (c - 1) + 30, (chi2, c)


def test_margin_reports_distance_to_boundaries():
    l = _logits([0.5, 0.3, 0.2])
    assert oracle.sample_margin(l, 1.0, 0.75, 0.5) == pytest.approx(0.05, abs=1e-7)
    assert oracle.sample_margin(l, 1.0, 0.9, 0.49) == pytest.approx(0.01, abs=1e-7)
