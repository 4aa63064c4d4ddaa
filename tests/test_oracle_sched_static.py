"""Pins of the fixed-length and static-threshold verification baselines (DSpark
page, Main results: offline benchmark with fixed-length blocks; static
threshold sweep over the confidence head)."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import sched
from tests.test_oracle_verify import _enumerate, _instance, _lossless


def _survivals(rng, B, K, lo=0.05):
    return np.cumprod(rng.uniform(lo, 1.0, (B, K)), axis=1)


@pytest.mark.parametrize("gamma", [-3, 0, 1, 4, 9])
def test_fixed_length_closed_form(gamma):
    B, K = 5, 6
    res = sched.schedule_fixed(B, K, gamma)
    g = min(max(gamma, 0), K)
    assert res["n"] == [g] * B and res["N"] == B * (1 + g)


def test_threshold_counts_the_survivals_at_or_above_it():
    # rows are non-increasing, so the prefix is exactly the positions with s >= theta
    rng = np.random.default_rng(1)
    S = _survivals(rng, 40, 9)
    for theta in [0.0, 0.01, 0.1, 0.3, 0.5, 0.9, 1.0, 1.5]:
        res = sched.schedule_threshold(S, theta)
        assert res["n"] == [int((row >= theta).sum()) for row in S]
        assert res["N"] == 40 + int((S >= theta).sum())


def test_threshold_edges_and_monotonicity():
    rng = np.random.default_rng(2)
    S = _survivals(rng, 10, 7)
    assert sched.schedule_threshold(S, 0.0)["n"] == [7] * 10
    assert sched.schedule_threshold(S, 1.0 + 1e-9)["n"] == [0] * 10
    prev = None
    for theta in np.linspace(0.0, 1.0, 41):
        n = np.array(sched.schedule_threshold(S, theta)["n"])
        if prev is not None:
            assert (n <= prev).all()
        prev = n
    # equality counts as passing
    S2 = np.array([[0.5, 0.5, 0.25]])
    assert sched.schedule_threshold(S2, 0.5)["n"] == [2]


def test_threshold_is_a_prefix_even_for_a_row_that_rises():
    # the rule stops at the first position below theta
    assert sched.schedule_threshold([[0.9, 0.2, 0.8]], 0.5)["n"] == [1]


@pytest.mark.parametrize("which", ["fixed", "threshold"])
def test_baselines_are_lossless_exact(which):
    rng = np.random.default_rng(700 if which == "fixed" else 701)
    V, K = 8, 2
    inst = _instance(rng, V)
    if which == "fixed":
        for g in range(K + 1):
            per, _ = _enumerate([inst], None, lambda S, T, g=g: sched.schedule_fixed(len(S), K, g))
            assert _lossless(inst, per[0])
    else:
        for theta in [Fraction(0), Fraction(1, 4), Fraction(1, 2), Fraction(3, 4), Fraction(1)]:
            per, _ = _enumerate([inst], None, lambda S, T, th=theta: sched.schedule_threshold(S, th))
            assert _lossless(inst, per[0])
