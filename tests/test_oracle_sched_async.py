"""Pins of the oracle's asynchronous dynamic-top-k scheduler (DSpark page,
Production deployment results): the budget comes from the first-drop schedule
of survivals two steps earlier, the current candidates fill it in survival
order."""
import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import sched
from tests.test_oracle_verify import _enumerate, _instance, _lossless, _step_table


def _survivals(rng, B, K, lo=0.05):
    return np.cumprod(rng.uniform(lo, 1.0, (B, K)), axis=1)


def _tables(B, K, rng):
    n = B * (K + 1) + 1
    N = np.arange(n, dtype=np.float64)
    return [list(1.0 + 0.05 * N), list(5.0 + 0.3 * np.maximum(N - 1.5 * B, 0.0)),
            [float(x) for x in _step_table(B, K, rng)], list(np.where(N <= B + B * K // 3, 1.0, 100.0))]


@pytest.mark.parametrize("trial", range(10))
def test_same_survivals_reduce_to_the_first_drop_schedule(trial):
    # with no lag the budget is what the first-drop pass takes, and the first-drop
    # pass takes exactly the leading candidates of the same order
    rng = np.random.default_rng(300 + trial)
    B, K = int(rng.integers(1, 9)), int(rng.integers(1, 7))
    S = _survivals(rng, B, K)
    for T in _tables(B, K, rng):
        a, s = sched.schedule_async(S, S, T), sched.schedule(S, T)
        assert a["n"] == s["n"] and a["N"] == s["N"]


def test_budget_depends_on_the_lagged_survivals_only():
    rng = np.random.default_rng(7)
    B, K = 6, 5
    S_lag = _survivals(rng, B, K)
    for T in _tables(B, K, rng):
        N_ref = sched.schedule(S_lag, T)["N"]
        for _ in range(10):
            res = sched.schedule_async(S_lag, _survivals(rng, B, K), T)
            assert res["N"] == N_ref and sum(res["n"]) == N_ref - B


@pytest.mark.parametrize("trial", range(30))
def test_selection_is_the_best_prefix_closed_set_of_its_size(trial):
    # brute force: among all per-request prefixes with sum M, the chosen counts
    # maximise the expected accepted tokens sum of S over the selection
    rng = np.random.default_rng(400 + trial)
    B, K = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    S, S_lag = _survivals(rng, B, K), _survivals(rng, B, K)
    T = _tables(B, K, rng)[trial % 4]
    res = sched.schedule_async(S_lag, S, T)
    n, M = res["n"], res["M"]
    assert sum(n) == M
    best = max(sum(S[b, :c[b]].sum() for b in range(B))
               for c in itertools.product(range(K + 1), repeat=B) if sum(c) == M)
    assert sum(S[b, :n[b]].sum() for b in range(B)) == pytest.approx(best, rel=1e-12)


def test_ties_follow_the_request_then_position_order():
    S = np.array([[0.5, 0.5, 0.25], [0.5, 0.5, 0.5], [0.5, 0.25, 0.25]])
    S_lag = np.array([[0.9, 0.9, 0.9]] * 3)
    T = [1.0] * (3 * 4 + 1)                           # flat: the lagged pass takes all 9
    T = T[:3 + 4] + [100.0] * (3 * 4 + 1 - 7)         # cliff after N = 6: budget 3
    res = sched.schedule_async(S_lag, S, T)
    assert res["M"] == 3
    # candidates at 0.5 in order: (0,1) (0,2) (1,1) (1,2) (1,3) (2,1): the first three
    assert res["n"] == [2, 1, 0]


@pytest.mark.parametrize("trial", range(10))
def test_decision_does_not_look_ahead_within_a_request(trial):
    # [n_b >= j] may depend on S[b, 1..j] and on other requests, never on S[b, j+1..K]
    rng = np.random.default_rng(500 + trial)
    B, K = 5, 6
    S, S_lag = _survivals(rng, B, K), _survivals(rng, B, K)
    T = _tables(B, K, rng)[trial % 4]
    n0 = sched.schedule_async(S_lag, S, T)["n"]
    for b in range(B):
        for j in range(1, K):
            S2 = S.copy()
            S2[b, j:] *= rng.uniform(0.0, 1.0)        # later positions only, still non-increasing
            n1 = sched.schedule_async(S_lag, S2, T)["n"]
            for jj in range(1, j + 1):
                assert (n1[b] >= jj) == (n0[b] >= jj)


@pytest.mark.parametrize("trial", range(3))
def test_lossless_with_the_asynchronous_budget_exact(trial):
    # exact enumeration (fractions) of every draft and accept/reject branch, the
    # budget taken from a fixed set of lagged survivals: each emitted token given
    # the emitted prefix still follows the target
    rng = np.random.default_rng(600 + trial)
    V, K = (8, 2) if trial < 2 else (5, 2)
    B = 1 if trial < 2 else 2
    insts = [_instance(rng, V) for _ in range(B)]
    S_lag = [[Fraction(int(rng.integers(1, 20)), 20)] for _ in range(B)]
    S_lag = [[row[0], row[0] * Fraction(int(rng.integers(1, 20)), 20)] for row in S_lag]
    T = _step_table(B, K, rng)
    per, _ = _enumerate(insts, T, lambda S, T_: sched.schedule_async(S_lag, S, T_))
    for b in range(B):
        assert _lossless(insts[b], per[b])
