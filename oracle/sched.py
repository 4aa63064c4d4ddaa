"""Hardware-aware prefix scheduler with early stopping.

Follows the DSpark page, Method > Confidence-scheduled verification (and
Limitations):

* choosing how many draft positions to verify is posed as maximising the
  expected tokens per second of the whole system, using a step-time / SPS
  table profiled once at engine start;
* survivals are non-increasing along each block, so a greedy pass that takes
  candidates in one global order of survival respects every block's prefix;
* to keep verification lossless the decision may not look at candidates not
  yet reached, so the greedy pass stops as soon as throughput would drop;
  this is the global optimum only when the objective is unimodal.

Readings:

* objective after taking m candidates: f(m) = (B + sum_{i<=m} s_(i)) / T(B + m).
  Every request always verifies one position and emits at least one token, so
  A_0 = B expected tokens at N_0 = B verified positions; T[N] is the step time
  with N verified positions (T = 1 / SPS);
* order: survival descending, then request ascending, then position ascending
  (the position tie-break keeps each request's selection a prefix when a
  confidence rounds to exactly 1);
* the candidate (s, b, k) is taken iff f(m+1) >= f(m), evaluated without
  division as (A + s) * T[N] >= A * T[N+1]; the pass stops at the first
  candidate that fails;
* n_b = number of request b's positions taken; N = B + sum_b n_b.

The functions are written with plain Python arithmetic so that they run on
floats or on exact ``fractions.Fraction`` values alike.  schedule_async() is
the production variant (budget from lagged survivals, dynamic top-k).
"""
from __future__ import annotations

import math

import numpy as np


def _as_seq(x):
    if isinstance(x, np.ndarray):
        return x.astype(np.float64).tolist()
    return x


def schedule(S, T):
    """Greedy first-drop schedule.

    S: B x K survivals (nested sequence or array), T: sequence indexed by N of
    length >= B*(K+1)+1.  Returns dict with n (list of n_b), N, order (the
    sorted candidates as (s, b, k)), taken (number taken), margin (smallest
    relative gap |lhs - rhs| / rhs over the comparisons evaluated) and
    cut_gap (relative survival gap between the last candidate taken and the
    first refused; inf if none was refused or none taken).
    """
    S = _as_seq(S)
    T = _as_seq(T)
    B, K = len(S), len(S[0])
    cands = [(S[b][k], b, k + 1) for b in range(B) for k in range(K)]
    cands.sort(key=lambda t: (-t[0], t[1], t[2]))
    A, N = B, B
    n = [0] * B
    margin = math.inf
    taken = 0
    for s, b, k in cands:
        lhs = (A + s) * T[N]
        rhs = A * T[N + 1]
        if rhs != 0:
            margin = min(margin, float(abs(lhs - rhs) / abs(rhs)))
        if lhs >= rhs:
            A = A + s
            N += 1
            n[b] += 1
            taken += 1
        else:
            break
    cut_gap = math.inf
    if 0 < taken < len(cands):
        s_in, s_out = cands[taken - 1][0], cands[taken][0]
        if s_in != 0:
            cut_gap = float((s_in - s_out) / s_in)
    return {"n": n, "N": N, "order": cands, "taken": taken, "margin": margin, "cut_gap": cut_gap}


def schedule_async(S_lag, S, T):
    """Asynchronous dynamic-top-k schedule.

    DSpark page, Production deployment results: in production the scheduler
    runs one step behind its inputs so that it fits graph replay and the
    engine's overlapped scheduling.  It sizes the coming verification budget
    from the confidence-head outputs of two steps earlier and fills that
    budget with the current step's candidates ordered by their latest
    cumulative confidence.

    Readings: the budget is the number of candidates the first-drop schedule
    takes on the lagged survivals S_lag (same B x K shape), M = taken(S_lag);
    the current candidates are ordered as in schedule() (survival descending,
    request ascending, position ascending) and the first M are taken.  Within
    a request a later position never precedes an earlier one in that order,
    so every selection is a prefix and [n_b >= j] does not depend on the
    request's confidences after j.

    Returns dict with n, N = B + M, M, capacity_margin (the lagged schedule's
    margin) and cut_gap (relative survival gap between the M-th and the
    (M+1)-th current candidate; inf if M is 0 or every candidate is taken).
    """
    lag = schedule(S_lag, T)
    S = _as_seq(S)
    B, K = len(S), len(S[0])
    M = lag["taken"]
    cands = [(S[b][k], b, k + 1) for b in range(B) for k in range(K)]
    cands.sort(key=lambda t: (-t[0], t[1], t[2]))
    n = [0] * B
    for s, b, k in cands[:M]:
        n[b] += 1
    cut_gap = math.inf
    if 0 < M < len(cands):
        s_in, s_out = cands[M - 1][0], cands[M][0]
        if s_in != 0:
            cut_gap = float((s_in - s_out) / s_in)
    return {"n": n, "N": B + M, "M": M, "capacity_margin": lag["margin"], "cut_gap": cut_gap, "order": cands}


def schedule_fixed(B, K, gamma):
    """Fixed-length verification (DSpark page, Main results > Offline
    benchmark: the scheduler switched off, every drafter proposing a block of
    fixed length): every request verifies min(gamma, K) positions."""
    g = max(0, min(int(gamma), K))
    return {"n": [g] * B, "N": B + B * g}


def schedule_threshold(S, theta):
    """Static-threshold verification (DSpark page, Main results: the static
    threshold sweep over the confidence head).  Reading: request b verifies
    the longest prefix of positions whose survival is at least theta."""
    S = _as_seq(S)
    n = []
    for row in S:
        c = 0
        for s in row:
            if s >= theta:
                c += 1
            else:
                break
        n.append(c)
    return {"n": n, "N": len(S) + sum(n)}

