"""Pins of the oracle's decision margins.

A GPU decision (token, acceptance, scheduled length, STS pick) may differ from
the oracle's only where the oracle's margin for that decision is small, so the
margins themselves must be right: a margin stuck at zero, or taken as the
larger instead of the smaller of two gaps, would excuse real mismatches.  Each
case here is built so that its margin is known by hand:

* token (two-level sampler): chunk scores L_c + G_c and element scores
  log w_v + G_v are engineered to chosen values by subtracting the draws'
  Gumbels (the Philox stream is pinned separately by its known-answer
  vectors), so both top-two gaps are chosen numbers;
* acceptance: draft and target rows whose ratio p(x)/q(x) at the drafted token
  is a chosen number a, so the margin |u - min(1, a)| follows from the accept
  uniform u of the stream;
* scheduler: survivals and a step-time table whose comparisons
  (A + s) T[N] versus A T[N + 1] are evaluated by hand in exact fractions;
* STS: one sample and one bin, where the ECE of temperature tau is
  1 - sigmoid(z / tau) in closed form.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import philox, sampling, sched, sts, verify
from oracle.draft import draft

SEED, B_ID, K_ID = 12345, 3, 2


def _engineered_row(chunk_scores, cstar_entries, V=3 * 128, p_chunk=philox.P_DRAFT_CHUNK,
                    p_elem=philox.P_DRAFT_ELEM):
    """Log-weights whose chunk scores L_c + G_c equal chunk_scores[c] and whose
    element scores inside the winning chunk equal cstar_entries (a dict
    {offset in the chunk: element score}).  The other chunks hold one finite
    entry (offset 0) carrying their whole mass."""
    nc = V // 128
    Gc = philox.gumbels(SEED, B_ID, K_ID, p_chunk, np.arange(nc))
    L = np.asarray(chunk_scores, np.float64) - Gc
    cstar = int(np.argmax(chunk_scores))
    logw = np.full(V, -np.inf)
    for c in range(nc):
        if c != cstar:
            logw[c * 128] = L[c]
    ids = np.array([cstar * 128 + o for o in cstar_entries])
    Ge = philox.gumbels(SEED, B_ID, K_ID, p_elem, ids)
    raw = np.array([cstar_entries[o] for o in cstar_entries]) - Ge    # log w_v = score - G_v
    # shift the element weights so that the chunk's log-mass is exactly L[cstar];
    # a common shift moves every element score of the chunk by the same amount,
    # which leaves the element gap unchanged
    shift = L[cstar] - scipy.special.logsumexp(raw)
    logw[ids] = raw + shift
    return logw, cstar, ids


@pytest.mark.parametrize("chunk_gap,elem_gap", [(0.37, 0.05), (0.02, 1.5), (0.9, 0.9001)])
def test_token_margin_is_the_smaller_of_the_two_top2_gaps(chunk_gap, elem_gap):
    # chunk scores 0, chunk_gap, -1: chunk 1 wins by chunk_gap; inside it three
    # entries with element scores 4, 4 - elem_gap, 1 (the last far behind)
    logw, cstar, ids = _engineered_row([0.0, chunk_gap, -1.0], {5: 4.0, 77: 4.0 - elem_gap, 100: 1.0})
    v, margin, c = sampling.two_level_sample(logw, SEED, B_ID, K_ID, philox.P_DRAFT_CHUNK, philox.P_DRAFT_ELEM)
    assert c == cstar == 1
    assert v == ids[0]
    assert margin == pytest.approx(min(chunk_gap, elem_gap), abs=1e-9)


def test_token_margin_uses_the_winning_chunk_only():
    # a near tie between two entries of a losing chunk must not enter the margin
    logw, cstar, ids = _engineered_row([0.0, 0.5, -2.0], {3: 2.0, 4: 1.0})
    logw[2 * 128 + 1] = logw[2 * 128]           # chunk 2 now holds two equal entries
    logw[2 * 128] = np.logaddexp(logw[2 * 128], -50.0)
    _, margin, c = sampling.two_level_sample(logw, SEED, B_ID, K_ID, philox.P_DRAFT_CHUNK, philox.P_DRAFT_ELEM)
    assert c == 1
    # chunk 2's mass grew by log 2, so the chunk gap is still that of the scores given
    L2 = scipy.special.logsumexp(logw[256:384][np.isfinite(logw[256:384])])
    G = philox.gumbels(SEED, B_ID, K_ID, philox.P_DRAFT_CHUNK, np.arange(3))
    scores = np.sort(np.array([0.0, 0.5, L2 + G[2]]))
    assert margin == pytest.approx(min(scores[-1] - scores[-2], 1.0), abs=1e-9)


def test_token_margin_single_entry_in_the_winning_chunk():
    # one finite entry in c*: no element decision, the margin is the chunk gap
    logw, _, _ = _engineered_row([0.3, -0.4, 0.0], {9: 0.0})
    _, margin, c = sampling.two_level_sample(logw, SEED, B_ID, K_ID, philox.P_DRAFT_CHUNK, philox.P_DRAFT_ELEM)
    assert c == 0 and margin == pytest.approx(0.3, abs=1e-9)


def test_token_margin_of_a_draft_step_is_the_sampler_margin():
    # the draft passes the sampler's margin through: W = 0 makes ell = Z / T_s
    logw, _, _ = _engineered_row([0.0, 0.25, -1.0], {5: 4.0, 6: 3.96}, p_chunk=philox.P_DRAFT_CHUNK,
                                 p_elem=philox.P_DRAFT_ELEM)
    Z = np.full((B_ID + 1, K_ID, logw.size), -1e30, np.float64)
    Z[B_ID, K_ID - 1] = np.where(np.isfinite(logw), logw, -1e30)
    Z[:, 0] = 0.0
    E = np.zeros((logw.size, 4), np.float64)
    d = draft(Z.astype(np.float32), E.astype(np.float32), E.astype(np.float32), np.zeros(B_ID + 1, np.int64),
              1.0, SEED)
    # Z went through float32: the engineered gaps survive to ~1e-6
    assert d["margin"][B_ID, K_ID - 1] == pytest.approx(0.04, abs=2e-5)


# ---------------------------------------------------------------- acceptance margin

def _rows_with_ratio(V, x, a):
    """Target and draft log-rows (T_s = 1) with q uniform and p(x) / q(x) = a."""
    q = np.full(V, 1.0 / V)
    p = np.full(V, (1.0 - a / V) / (V - 1))
    p[x] = a / V
    return np.log(p), np.log(q)


def _verify_fixed(ratios, xs, V=8):
    """Verify one request (b = B_ID) whose positions have p/q = ratios[k] at xs[k]."""
    K = len(ratios)
    Zt = np.zeros((K + 1, V))
    Z = np.zeros((K, V))
    for k, (a, x) in enumerate(zip(ratios, xs)):
        Zt[k], Z[k] = _rows_with_ratio(V, x, a)
    E = np.zeros((V, 2))
    return verify.verify_request(B_ID, K, xs, Zt, Z, E, E, 0, 1.0, SEED)


def test_accept_margin_by_hand():
    u = [float(philox.uniforms(SEED, B_ID, k, philox.P_ACCEPT, 0)) for k in (1, 2, 3)]
    # position 1 accepted by 0.3 (or as much as fits below 1), position 2 refused
    # by 0.01, position 3 never evaluated (its margin would be 0)
    a1 = min(u[0] + 0.3, 0.999)
    a2 = u[1] - 0.01
    a3 = u[2]
    assert a2 > 0
    out = _verify_fixed([a1, a2, a3], [2, 5, 1])
    assert out["accepted"] == 1 and out["k_star"] == 2
    assert out["accept_margin"] == pytest.approx(min(a1 - u[0], 0.01), abs=1e-12)


def test_accept_margin_clips_the_ratio_at_one():
    # p/q = 1.7 accepts for sure; the margin is 1 - u, not |u - 1.7|
    u1 = float(philox.uniforms(SEED, B_ID, 1, philox.P_ACCEPT, 0))
    out = _verify_fixed([1.7], [4])
    assert out["accepted"] == 1 and out["kind"] == "bonus"
    assert out["accept_margin"] == pytest.approx(1.0 - u1, abs=1e-12)


def test_accept_margin_is_the_smallest_over_positions():
    u = [float(philox.uniforms(SEED, B_ID, k, philox.P_ACCEPT, 0)) for k in (1, 2, 3)]
    gaps = [0.2, 0.003, 0.05]
    ratios = [min(ui + g, 0.999) for ui, g in zip(u, gaps)]
    out = _verify_fixed(ratios, [0, 1, 2])
    assert out["accepted"] == 3
    assert out["accept_margin"] == pytest.approx(min(r - ui for r, ui in zip(ratios, u)), abs=1e-12)


# ---------------------------------------------------------------- scheduler margin and cut gap

S_HAND = [[Fraction(9, 10), Fraction(1, 2)], [Fraction(4, 5), Fraction(1, 10)]]


def _table(t5):
    # T[N] for N = 0..6; N starts at B = 2
    return [Fraction(1), Fraction(1), Fraction(1), Fraction(6, 5), Fraction(3, 2), t5, Fraction(3)]


def test_schedule_margin_and_cut_gap_by_hand():
    # order (0.9, b0, k1), (0.8, b1, k1), (0.5, b0, k2), (0.1, b1, k2); A = N = 2
    #   (2 + 9/10) * 1   = 29/10  vs 2 * 6/5      = 12/5   take  gap (29/10 - 12/5) / (12/5)   = 5/24
    #   (29/10 + 4/5) * 6/5 = 111/25 vs 29/10 * 3/2 = 87/20 take  gap (111/25 - 87/20) / (87/20) = 3/145
    #   (37/10 + 1/2) * 3/2 = 63/10  vs 37/10 * 2   = 37/5  refuse gap (37/5 - 63/10) / (37/5) = 11/74
    out = sched.schedule(S_HAND, _table(Fraction(2)))
    assert out["n"] == [1, 1] and out["N"] == 4 and out["taken"] == 2
    assert out["margin"] == pytest.approx(float(Fraction(3, 145)), abs=1e-15)
    assert out["cut_gap"] == pytest.approx(float((Fraction(4, 5) - Fraction(1, 2)) / Fraction(4, 5)), abs=1e-15)


def test_schedule_margin_includes_the_refused_comparison():
    # T[5] = 171/100: the refusal is the narrowest comparison
    #   (37/10 + 1/2) * 3/2 = 63/10 vs 37/10 * 171/100 = 6327/1000  gap 27/6327
    out = sched.schedule(S_HAND, _table(Fraction(171, 100)))
    assert out["n"] == [1, 1]
    assert out["margin"] == pytest.approx(27 / 6327, abs=1e-15)
    # the same margin on exact fractions
    exact = sched.schedule(S_HAND, _table(Fraction(171, 100)))
    assert exact["margin"] == pytest.approx(float(Fraction(27, 6327)), abs=1e-15)


def test_schedule_cut_gap_infinite_when_nothing_refused_or_taken():
    flat = [Fraction(1)] * 7
    out = sched.schedule(S_HAND, flat)
    assert out["taken"] == 4 and out["cut_gap"] == math.inf
    steep = [Fraction(1), Fraction(1), Fraction(1)] + [Fraction(1000)] * 4
    out = sched.schedule(S_HAND, steep)
    assert out["taken"] == 0 and out["cut_gap"] == math.inf
    # the one comparison evaluated: (2 + 9/10) * 1 vs 2 * 1000
    assert out["margin"] == pytest.approx(float((2000 - Fraction(29, 10)) / 2000), abs=1e-15)


def test_async_schedule_cut_gap_by_hand():
    # budget from the lagged survivals (same as S_HAND: 2 taken), current survivals reordered
    S_now = [[Fraction(3, 10), Fraction(1, 5)], [Fraction(7, 10), Fraction(3, 5)]]
    out = sched.schedule_async(S_HAND, S_now, _table(Fraction(2)))
    assert out["M"] == 2 and out["n"] == [0, 2]
    assert out["cut_gap"] == pytest.approx(float((Fraction(3, 5) - Fraction(3, 10)) / Fraction(3, 5)), abs=1e-15)
    assert out["capacity_margin"] == pytest.approx(3 / 145, abs=1e-15)


# ---------------------------------------------------------------- STS margin

def _one_sample_fit(c, grid):
    return sts.sts_fit(np.array([[c]], np.float32), np.array([1]), np.array([1]), np.array(grid, np.float64),
                       n_bins=1)


def test_sts_margin_closed_form():
    # one accepted sample, one bin: ECE(tau) = 1 - sigmoid(z / tau), z = logit(0.75) = ln 3;
    # the smallest tau wins (z > 0): ECE(1/2) = 1 - 9/10, runner-up ECE(1) = 1 - 3/4
    out = _one_sample_fit(0.75, [1.0, 2.0, 0.5])
    assert out["idx"][0] == 2
    assert out["margin"][0] == pytest.approx(0.9 - 0.75, abs=1e-12)
    assert out["ece_fit"][0] == pytest.approx(0.1, abs=1e-12)


def test_sts_margin_runner_up_not_last():
    # grid order must not matter: the runner-up is the second-smallest ECE
    z = math.log(3.0)
    grid = [4.0, 0.5, 2.0, 1.0]
    out = _one_sample_fit(0.75, grid)
    eces = sorted(1.0 - scipy.special.expit(z / t) for t in grid)
    assert out["margin"][0] == pytest.approx(eces[1] - eces[0], abs=1e-12)


def test_sts_margin_zero_for_duplicate_best():
    out = _one_sample_fit(0.75, [0.5, 1.0, 0.5])
    assert out["idx"][0] == 0 and out["margin"][0] == 0.0


def test_sts_margin_infinite_with_one_usable_entry():
    out = _one_sample_fit(0.75, [0.5, -1.0, float("nan")])
    assert out["idx"][0] == 0 and out["margin"][0] == math.inf
