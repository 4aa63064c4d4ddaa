"""Pins of the oracle's verification rule and of the whole cycle's losslessness.

The exact tests enumerate every draft realisation and every accept/reject
branch with exact fractions, using the oracle's own scheduler, survival,
acceptance probability and residual law; every random draw is replaced by its
branch weight.  Losslessness (DSpark page, Overview; Limitations) then says:
for each request and each emitted position j, the law of the j-th emitted
token given the tokens emitted before it (and that position j is emitted) is
the target's p_j.
"""
import itertools
import math
from collections import defaultdict
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import conf, philox, sched, verify
from oracle.draft import draft
from tests.test_oracle_sampling import _chi2_pvalue


# ---------------------------------------------------------------- exact enumeration

def _rand_dist(rng, V, zeros=0):
    w = [int(rng.integers(1, 10)) for _ in range(V)]
    for i in rng.choice(V, zeros, replace=False):
        w[i] = 0
    s = sum(w)
    return [Fraction(x, s) for x in w]


def _instance(rng, V, K=2):
    """One request: q_1 (given the anchor), q_2(. | x_1), p_1..p_3, c_1, c_2(x_1)."""
    return {
        "q": [_rand_dist(rng, V)] + [[_rand_dist(rng, V) for _ in range(V)]],
        "p": [_rand_dist(rng, V, zeros=int(rng.integers(0, 2))) for _ in range(K + 1)],
        "c1": Fraction(int(rng.integers(1, 20)), 20),
        "c2": [Fraction(int(rng.integers(1, 20)), 20) for _ in range(V)],
    }


def _emit_law(inst, xs, n_b):
    """Law of the emitted token sequence of one request given its drafts xs and budget n_b."""
    V = len(inst["p"][0])
    q_rows = [inst["q"][0], inst["q"][1][xs[0]]]
    law = defaultdict(Fraction)
    reach = Fraction(1)
    for k in range(1, n_b + 1):
        p, q, x = inst["p"][k - 1], q_rows[k - 1], xs[k - 1]
        a = verify.accept_probability(p[x], q[x])
        r = verify.residual_weights(np.array(p, dtype=object), np.array(q, dtype=object))
        mass = sum(r)
        if a != 1:
            for y in range(V):
                if r[y]:
                    law[tuple(xs[:k - 1]) + (y,)] += reach * (1 - a) * r[y] / mass
        reach *= a
    for y in range(V):
        if inst["p"][n_b][y]:
            law[tuple(xs[:n_b]) + (y,)] += reach * inst["p"][n_b][y]
    return law


def _enumerate(insts, T, scheduler):
    """Per-request law of emitted sequences, and the joint law of the first emitted tokens."""
    B, V = len(insts), len(insts[0]["p"][0])
    per = [defaultdict(Fraction) for _ in range(B)]
    first = defaultdict(Fraction)
    draft_sets = [list(itertools.product(range(V), repeat=2)) for _ in range(B)]
    for combo in itertools.product(*draft_sets):
        w = Fraction(1)
        S = []
        for inst, xs in zip(insts, combo):
            w *= inst["q"][0][xs[0]] * inst["q"][1][xs[0]][xs[1]]
            S.append(conf.survival([inst["c1"], inst["c2"][xs[0]]]))
        if w == 0:
            continue
        n = scheduler(S, T)["n"]
        laws = [_emit_law(inst, xs, n[b]) for b, (inst, xs) in enumerate(zip(insts, combo))]
        for b in range(B):
            for seq, pr in laws[b].items():
                per[b][seq] += w * pr
        if B == 2:
            f0, f1 = defaultdict(Fraction), defaultdict(Fraction)
            for seq, pr in laws[0].items():
                f0[seq[0]] += pr
            for seq, pr in laws[1].items():
                f1[seq[0]] += pr
            for u, pu in f0.items():
                for v, pv in f1.items():
                    first[(u, v)] += w * pu * pv
    return per, first


def _lossless(inst, law):
    """Check that the j-th emitted token given the emitted prefix is distributed as p_j."""
    assert sum(law.values()) == 1
    K1 = len(inst["p"])
    for j in range(1, K1 + 1):
        groups = defaultdict(lambda: defaultdict(Fraction))
        for seq, pr in law.items():
            if len(seq) >= j:
                groups[seq[:j - 1]][seq[j - 1]] += pr
        for prefix, dist in groups.items():
            tot = sum(dist.values())
            for y, pr in enumerate(inst["p"][j - 1]):
                if pr * tot != dist.get(y, 0):
                    return False
    return True


def _step_table(B, K, rng):
    T, t = [], Fraction(1)
    for N in range(B * (K + 1) + 1):
        T.append(t)
        if rng.random() < 0.5:
            t += Fraction(int(rng.integers(1, 8)), 10)
    return T


@pytest.mark.parametrize("trial", range(4))
def test_lossless_single_request_exact(trial):
    rng = np.random.default_rng(10 + trial)
    V, K = 8, 2
    inst = _instance(rng, V)
    for T in ([Fraction(1) + Fraction(N, 10) for N in range(K + 2)], _step_table(1, K, rng),
              [Fraction(1)] * (K + 2)):
        per, _ = _enumerate([inst], T, sched.schedule)
        assert _lossless(inst, per[0])


@pytest.mark.parametrize("trial", range(2))
def test_lossless_two_requests_exact(trial):
    rng = np.random.default_rng(20 + trial)
    V, K = 5, 2
    insts = [_instance(rng, V), _instance(rng, V)]
    T = _step_table(2, K, rng) if trial else [Fraction(2) + Fraction(N, 7) for N in range(2 * (K + 1) + 1)]
    per, first = _enumerate(insts, T, sched.schedule)
    for b in range(2):
        assert _lossless(insts[b], per[b])
    # the first emitted tokens of the two requests are independent draws from their p_1
    for (u, v), pr in first.items():
        assert pr == insts[0]["p"][0][u] * insts[1]["p"][0][v]


def _global_argmax_schedule(S, T):
    """A scheduler that looks ahead: it takes the best m over all m (no early stop)."""
    B, K = len(S), len(S[0])
    order = sorted(((S[b][k], b, k + 1) for b in range(B) for k in range(K)), key=lambda t: (-t[0], t[1], t[2]))
    best, best_m, A = Fraction(B) / T[B], 0, Fraction(B)
    for m, (s, b, k) in enumerate(order, start=1):
        A += s
        if A / T[B + m] > best:
            best, best_m = A / T[B + m], m
    n = [0] * B
    for s, b, k in order[:best_m]:
        n[b] += 1
    return {"n": n}


def test_negative_control_lookahead_scheduler_is_not_lossless():
    # the enumeration detects the bias of a scheduler that looks past the first
    # drop, for some step-shaped table (a random search finds one quickly)
    rng = np.random.default_rng(31)
    V, K = 6, 2
    found = False
    for trial in range(60):
        inst = _instance(rng, V)
        inst["c1"] = Fraction(7, 10)
        inst["c2"] = [Fraction(int(rng.integers(1, 20)), 20) for _ in range(V)]
        T = [Fraction(1), Fraction(1), Fraction(18, 10), Fraction(18, 10)]
        per_ok, _ = _enumerate([inst], T, sched.schedule)
        assert _lossless(inst, per_ok[0])
        per_bad, _ = _enumerate([inst], T, _global_argmax_schedule)
        if not _lossless(inst, per_bad[0]):
            found = True
            break
    assert found


def _tv(p, q):
    return sum(abs(a - b) for a, b in zip(p, q)) / 2


def test_expected_accepted_length_closed_form_exact():
    # draft rows independent of the prefix and every position verified:
    # E[accepted] = sum_k prod_{j<=k} (1 - TV(p_j, q_j))
    rng = np.random.default_rng(40)
    V, K = 7, 2
    inst = _instance(rng, V)
    q2 = _rand_dist(rng, V)
    inst["q"][1] = [q2] * V
    per, _ = _enumerate([inst], [Fraction(1)] * (K + 2), sched.schedule)
    e_acc = sum(pr * (len(seq) - 1) for seq, pr in per[0].items())
    alpha = [1 - _tv(inst["p"][k], inst["q"][0] if k == 0 else q2) for k in range(K)]
    closed = alpha[0] + alpha[0] * alpha[1]
    assert e_acc == closed


# ---------------------------------------------------------------- Monte Carlo of the full oracle

def _mc_inputs(V=64, K=4, seed=0):
    rng = np.random.default_rng(seed)
    Z = rng.normal(0, 1.5, (1, K, V)).astype(np.float32)
    Zt = np.concatenate([Z, rng.normal(0, 1.5, (1, 1, V)).astype(np.float32)], axis=1)
    Zt = (Zt + rng.normal(0, 1.0, Zt.shape)).astype(np.float32)
    return Z, Zt


def test_monte_carlo_accepted_length_and_first_token_law():
    # full oracle (Philox draws, two-level sampling, accept, residual, bonus) with a
    # fixed draft (Wt = 0) and every position verified: the mean accepted length
    # matches the closed form and the first emitted token is distributed as p_1
    V, K, T_s = 64, 4, 1.0
    Z, Zt = _mc_inputs(V, K)
    E = np.zeros((V, 4), np.float32)
    Wt = np.zeros((V, 4), np.float32)
    q = scipy.special.softmax(Z[0].astype(np.float64) / T_s, axis=1)
    p = scipy.special.softmax(Zt[0].astype(np.float64) / T_s, axis=1)
    alpha = [1 - 0.5 * np.abs(p[k] - q[k]).sum() for k in range(K)]
    closed = sum(np.prod(alpha[:k + 1]) for k in range(K))
    n_runs = 3000
    acc, first = [], []
    E64, W64 = E.astype(np.float64), Wt.astype(np.float64)
    for seed in range(n_runs):
        d = draft(Z, E, Wt, np.array([0]), T_s, seed)
        res = verify.verify_request(0, K, d["x"][0], Zt[0], Z[0], E64, W64, 0, T_s, seed)
        acc.append(res["accepted"])
        first.append(res["tokens"][0])
    acc = np.array(acc, float)
    se = acc.std(ddof=1) / math.sqrt(n_runs)
    assert abs(acc.mean() - closed) < 4 * se, (acc.mean(), closed, se)
    counts = np.bincount(first, minlength=V).astype(float)
    assert _chi2_pvalue(counts, p[0]) > 1e-3


def test_monte_carlo_every_emitted_position_follows_the_target():
    # full oracle verify with high acceptance: for every emitted position j (the
    # bonus position K+1 included) the marginal law of the j-th emitted token
    # over runs that emit it is p_j (the target rows do not depend on the prefix)
    V, K, T_s = 16, 3, 1.0
    rng = np.random.default_rng(9)
    Z = rng.normal(0, 1.0, (1, K, V)).astype(np.float32)
    extra = rng.normal(0, 1.0, (1, 1, V)).astype(np.float32)
    Zt = (np.concatenate([Z, extra], axis=1) + rng.normal(0, 0.3, (1, K + 1, V))).astype(np.float32)
    E = np.zeros((V, 2), np.float32)
    p = scipy.special.softmax(Zt[0].astype(np.float64) / T_s, axis=1)
    emitted = [[] for _ in range(K + 1)]
    for seed in range(4000):
        d = draft(Z, E, E, np.array([3]), T_s, seed)
        res = verify.verify_request(0, K, d["x"][0], Zt[0], Z[0], E.astype(float), E.astype(float), 3, T_s, seed)
        for j, y in enumerate(res["tokens"]):
            emitted[j].append(y)
    assert len(emitted[K]) > 1000
    for j in range(K + 1):
        counts = np.bincount(emitted[j], minlength=V).astype(float)
        assert _chi2_pvalue(counts, p[j]) > 1e-3, j


def test_identical_draft_and_target_always_accepts():
    # p == q: min(1, p/q) = 1 > u, so every scheduled position is kept and the
    # extra token is the bonus draw from the next target row
    V, K = 300, 3
    Z, _ = _mc_inputs(V, K, seed=2)
    Zt = np.concatenate([Z, np.random.default_rng(3).normal(0, 1, (1, 1, V)).astype(np.float32)], axis=1)
    E = np.zeros((V, 2), np.float32)
    for seed in range(20):
        d = draft(Z, E, E, np.array([5]), 1.0, seed)
        for n_b in range(K + 1):
            res = verify.verify_request(0, n_b, d["x"][0], Zt[0], Z[0], E.astype(float), E.astype(float),
                                        5, 1.0, seed)
            assert res["accepted"] == n_b and res["kind"] == "bonus"
            assert res["tokens"][:n_b] == list(d["x"][0, :n_b])


def test_disjoint_draft_and_target_resample_from_target():
    # q puts its mass on token 0, p on token 1: the draft token is rejected at
    # position 1 and the residual max(0, p - q) is essentially p
    V, K = 256, 2
    Z = np.full((1, K, V), -60.0, np.float32)
    Z[0, :, 0] = 0.0
    Zt = np.full((1, K + 1, V), -60.0, np.float32)
    Zt[0, :, 1] = 0.0
    E = np.zeros((V, 2), np.float32)
    for seed in range(10):
        d = draft(Z, E, E, np.array([0]), 1.0, seed)
        res = verify.verify_request(0, K, d["x"][0], Zt[0], Z[0], E.astype(float), E.astype(float), 0, 1.0, seed)
        assert res["accepted"] == 0 and res["kind"] == "resid" and res["tokens"] == [1]
        assert abs(res["mass"] - 1.0) < 1e-20


def test_logp_is_the_target_log_probability_of_each_verified_token():
    V, K = 500, 4
    Z, Zt = _mc_inputs(V, K, seed=4)
    E = np.zeros((V, 2), np.float32)
    d = draft(Z, E, E, np.array([1]), 0.8, 3)
    res = verify.verify_request(0, 3, d["x"][0], Zt[0], Z[0], E.astype(float), E.astype(float), 1, 0.8, 3)
    for k in range(3):
        ref = scipy.special.log_softmax(Zt[0, k].astype(np.float64) / 0.8)[d["x"][0, k]]
        assert abs(res["logp"][k] - ref) < 1e-12
    assert np.isnan(res["logp"][3])


def _markov_mc(n_runs, V=10, K=3, r=4, seed=21):
    """Draft + verify_request of the full oracle on one request whose draft rows
    depend on the prefix through a strong Markov bias (E[x_{k-1}] . Wt^T, std
    about 1.5 nats), every position verified; returns the emitted sequences,
    the outcome kinds and the target rows."""
    rng = np.random.default_rng(seed)
    Z = rng.normal(0, 1.0, (1, K, V)).astype(np.float32)
    E = rng.normal(0, 1.0, (V, r)).astype(np.float32)
    Wt = rng.normal(0, 0.75, (V, r)).astype(np.float32)
    Zt = np.concatenate([Z, rng.normal(0, 1.0, (1, 1, V)).astype(np.float32)], axis=1)
    Zt = (Zt + rng.normal(0, 0.7, Zt.shape)).astype(np.float32)
    p = scipy.special.softmax(Zt[0].astype(np.float64), axis=1)
    E64, W64 = E.astype(np.float64), Wt.astype(np.float64)
    anchor = 4
    seqs, kinds = [], []
    for s in range(n_runs):
        d = draft(Z, E, Wt, np.array([anchor]), 1.0, s)
        res = verify.verify_request(0, K, d["x"][0], Zt[0], Z[0], E64, W64, anchor, 1.0, s)
        seqs.append(res["tokens"])
        kinds.append((res["kind"], res["accepted"]))
    return seqs, kinds, p, (Z, E, Wt, anchor)


def test_monte_carlo_markov_bias_emitted_tokens_follow_the_target():
    # Prefix-dependent draft rows through the oracle's own draft and
    # verify_request (DSpark page, Overview: the output law is the target's
    # whatever the drafter).  The target rows do not depend on the prefix, so
    # the j-th emitted token, over the runs that emit it, has law p_j, and
    # given the first emitted token (the position-1 draft token accepted) the
    # second has law p_2 whatever the first was.  A verifier that used any
    # other draft row for the acceptance test or the residual (the bias of
    # another previous token, or none) would bend these laws.
    K = 3
    seqs, kinds, p, (Z, E, Wt, anchor) = _markov_mc(3000, K=K)
    V = p.shape[1]
    # the bias really moves the draft rows: the first draft row differs from softmax(Z_1) by a visible margin
    ell = Z[0, 0].astype(np.float64) + E[anchor].astype(np.float64) @ Wt.astype(np.float64).T
    q1 = scipy.special.softmax(ell)
    assert 0.5 * np.abs(q1 - scipy.special.softmax(Z[0, 0].astype(np.float64))).sum() > 0.15
    # every outcome occurs: rejections at each position (residual draws) and the bonus
    seen = set(kinds)
    for k in range(K):
        assert ("resid", k) in seen, k
    assert ("bonus", K) in seen
    for j in range(K + 1):
        ys = [s[j] for s in seqs if len(s) > j]
        assert len(ys) > 150, j
        assert _chi2_pvalue(np.bincount(ys, minlength=V).astype(float), p[j]) > 1e-3, j
    # y_2 given y_1 = a, for every a with enough runs: one chi-square over all
    # of them (the emission of y_2 selects y_1, never y_2)
    table = np.zeros((V, V))
    for s in seqs:
        if len(s) > 1:
            table[s[0], s[1]] += 1
    stat, dof, rows = 0.0, 0, 0
    for a in range(V):
        n = table[a].sum()
        if n < 60:
            continue
        rows += 1
        exp = p[1] * n
        order = np.argsort(exp)
        obs_c, exp_c, acc_o, acc_e = [], [], 0.0, 0.0
        for i in order:
            acc_o += table[a, i]
            acc_e += exp[i]
            if acc_e >= 5.0:
                obs_c.append(acc_o)
                exp_c.append(acc_e)
                acc_o = acc_e = 0.0
        if acc_e > 0:
            obs_c[-1] += acc_o
            exp_c[-1] += acc_e
        obs_c, exp_c = np.array(obs_c), np.array(exp_c)
        stat += ((obs_c - exp_c) ** 2 / exp_c).sum()
        dof += len(obs_c) - 1
    assert rows >= 3
    assert scipy.stats.chi2.sf(stat, dof) > 1e-3, (stat, dof)
