"""Pins of the oracle's first-drop prefix scheduler."""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import sched


def _survivals(rng, B, K, lo=0.05):
    c = rng.uniform(lo, 1.0, (B, K))
    return np.cumprod(c, axis=1)


def _objective(S, T, m):
    """f(m) = (B + sum of the m largest survivals) / T[B + m], with the method's order."""
    B = len(S)
    flat = sorted(((S[b][k], b, k) for b in range(B) for k in range(len(S[0]))),
                  key=lambda t: (-t[0], t[1], t[2]))
    return (B + sum(t[0] for t in flat[:m])) / T[B + m]


def test_flat_table_takes_everything():
    S = _survivals(np.random.default_rng(0), 7, 5)
    res = sched.schedule(S, [3.0] * (7 * 6 + 1))
    assert res["n"] == [5] * 7 and res["N"] == 42


def test_steep_table_takes_nothing():
    S = _survivals(np.random.default_rng(1), 4, 6)
    T = [1.0 + 100.0 * N for N in range(4 * 7 + 1)]
    res = sched.schedule(S, T)
    assert res["n"] == [0] * 4 and res["N"] == 4


def test_single_request_linear_table_closed_form():
    # B = 1, T(N) = a + b N:  (A + s) T(N) >= A T(N+1)  <=>  s (a + b N) >= A b.
    rng = np.random.default_rng(2)
    for trial in range(50):
        K = 8
        S = _survivals(rng, 1, K, lo=0.5)
        a, bb = rng.uniform(0.5, 2.0), rng.uniform(0.01, 0.6)
        T = [a + bb * N for N in range(K + 2)]
        A, n = 1.0, 0
        for k in range(K):
            N = 1 + n
            if S[0, k] * (a + bb * N) >= A * bb:
                A += S[0, k]
                n += 1
            else:
                break
        assert sched.schedule(S, T)["n"] == [n]


@pytest.mark.parametrize("trial", range(20))
def test_first_drop_is_the_global_optimum_for_a_unimodal_objective(trial):
    # linear or convex T with decreasing survivals make f unimodal: the early
    # stop must land on an argmax of f over all m (brute force, exact arithmetic)
    rng = np.random.default_rng(100 + trial)
    B, K = int(rng.integers(1, 5)), int(rng.integers(1, 6))
    c = [[Fraction(int(rng.integers(1, 20)), 20) for _ in range(K)] for _ in range(B)]
    S = [[Fraction(1)] * K for _ in range(B)]
    for b in range(B):
        s = Fraction(1)
        for k in range(K):
            s *= c[b][k]
            S[b][k] = s
    a, slope, curv = Fraction(int(rng.integers(1, 10))), Fraction(int(rng.integers(0, 10)), 10), \
        Fraction(int(rng.integers(0, 3)), 100)
    T = [a + slope * N + curv * N * N for N in range(B * (K + 1) + 1)]
    res = sched.schedule(S, T)
    f = [_objective(S, T, m) for m in range(B * K + 1)]
    assert f[res["taken"]] == max(f)
    assert res["N"] == B + res["taken"] == B + sum(res["n"])


def test_selection_is_a_prefix_of_every_block():
    rng = np.random.default_rng(3)
    for trial in range(30):
        B, K = 6, 7
        S = _survivals(rng, B, K)
        if trial % 3 == 0:
            S[:, 3:] = S[:, 2:3]                # exact ties along blocks (confidence 1)
        T = [1.0 + 0.05 * N + 0.002 * N * N for N in range(B * (K + 1) + 1)]
        res = sched.schedule(S, T)
        chosen = {(b, k) for (_, b, k) in res["order"][:res["taken"]]}
        for b in range(B):
            assert chosen == chosen | {(b, j) for j in range(1, res["n"][b] + 1)}
            assert all((b, j) in chosen for j in range(1, res["n"][b] + 1))
            assert all((b, j) not in chosen for j in range(res["n"][b] + 1, K + 1))


def test_decision_does_not_look_ahead():
    # whether position j of a block is taken cannot depend on the block's later survivals
    rng = np.random.default_rng(4)
    for trial in range(200):
        B, K = 3, 5
        S = _survivals(rng, B, K, lo=0.3)
        T = np.cumsum(rng.choice([0.0, 0.0, 0.3, 1.0], B * (K + 1) + 1)) + 2.0   # step-shaped
        base = sched.schedule(S, T)["n"]
        b, j = int(rng.integers(0, B)), int(rng.integers(1, K))
        S2 = S.copy()
        S2[b, j:] = S2[b, j - 1] * np.cumprod(rng.uniform(0.05, 1.0, K - j))
        new = sched.schedule(S2, T)["n"]
        assert min(base[b], j) == min(new[b], j)


@pytest.mark.parametrize("name", ["high_concurrency", "dsv4_vocab", "stress"])
def test_knee_tables_stop_exactly_at_the_knee(name):
    # flat table up to the knee, then slope/flat * A > 1 >= any survival: N = knee = 2B
    cfg = synth.get_config(name)
    T = synth.T_table(cfg)
    S = _survivals(np.random.default_rng(5), cfg.B, cfg.K, lo=0.2)
    res = sched.schedule(S, T)
    assert res["N"] == cfg.ttable[2] == 2 * cfg.B
    # the top-B survivals are the ones taken
    thr = np.sort(S.ravel())[::-1][cfg.B - 1]
    assert sum(res["n"]) == cfg.B and (S >= thr).sum() == cfg.B


def test_budget_shrinks_under_load():
    # for fixed survivals a steeper table never raises the mean verification budget
    rng = np.random.default_rng(6)
    S = _survivals(rng, 16, 8, lo=0.4)
    prev = None
    for slope in (0.0, 0.01, 0.02, 0.05, 0.1, 0.3, 1.0):
        T = [1.0 + slope * N for N in range(16 * 9 + 1)]
        tot = sum(sched.schedule(S, T)["n"])
        assert prev is None or tot <= prev
        prev = tot
