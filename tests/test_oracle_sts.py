"""Pins of the STS fitting oracle (DSpark page, Method > Confidence-scheduled
verification, the STS paragraph): ECE by hand, recovery of known temperatures
from data drawn from a temperature-scaled head, the observation rule, the
left-to-right dependence, grid handling and tie-breaks."""
from __future__ import annotations

import numpy as np
import pytest
import scipy.special

import synth
from oracle import sts


def test_logit_matches_scipy():
    c = np.array([1e-30, 1e-7, 0.1, 0.35, 0.5, 0.75, 0.999, 1 - 2.0 ** -40], dtype=np.float64)
    np.testing.assert_allclose(sts.logit(c), scipy.special.logit(c), rtol=1e-13)
    assert sts.logit(np.array([1.0]))[0] == np.inf
    assert sts.logit(np.array([0.0]))[0] == -np.inf


@pytest.mark.parametrize("pred,label,expected", [
    ([0.1, 0.1, 0.9], [0, 1, 1], (abs(0.2 - 1) + abs(0.9 - 1)) / 3),    # bins 1 and 13
    ([0.0, 1.0, 1.0, 0.5], [0, 1, 0, 1], (0 + 1 + 0.5) / 4),              # bins 0, 14 (1.0 joins the last), 7
    ([0.5, 0.5, 0.5, 0.5], [1, 0, 1, 0], 0.0),                             # calibrated
    ([0.2, 0.26], [1, 1], abs(0.46 - 2) / 2),                              # both in bin 3 ([0.2, 0.2667))
])
def test_ece_by_hand(pred, label, expected):
    assert sts.ece(pred, label, 15) == pytest.approx(expected, abs=1e-15)


def test_ece_bin_count_matters():
    # 0.2 and 0.3 share a bin with 2 bins ([0, 0.5)) and not with 10
    assert sts.ece([0.2, 0.3], [0, 1], 2) == pytest.approx(abs(0.5 - 1) / 2)
    assert sts.ece([0.2, 0.3], [0, 1], 10) == pytest.approx((0.2 + 0.7) / 2)


def _tempered_head(M, K, tau_true, seed, censor=False):
    """Data from a head whose true conditional acceptance is sigmoid(z / tau_true[k])
    while it reports c = sigmoid(z): the temperatures that calibrate it are known."""
    rng = np.random.default_rng(seed)
    z = rng.normal(1.5, 1.5, (M, K))
    c = scipy.special.expit(z).astype(np.float32)
    z32 = scipy.special.logit(c.astype(np.float64))  # the logit the fit will see
    p_true = scipy.special.expit(z32 / np.asarray(tau_true)[None, :])
    passed = rng.random((M, K)) < p_true
    chain = np.argmin(np.concatenate([passed, np.zeros((M, 1), bool)], axis=1), axis=1)
    n_ver = np.full(M, K) if not censor else np.where(rng.random(M) < 0.5, K, rng.integers(0, K + 1, M))
    return c, np.minimum(chain, n_ver).astype(np.int32), n_ver.astype(np.int32)


@pytest.mark.parametrize("censor", [False, True])
def test_recovers_known_temperatures(censor):
    tau_true = [1.6, 0.8, 1.3, 2.0]
    c, acc, nv = _tempered_head(60000, 4, tau_true, seed=3, censor=censor)
    grid = synth.sts_grid(129)
    r = sts.sts_fit(c, acc, nv, grid)
    step = np.log(grid[1] / grid[0])
    # within a few grid steps (2.2% each) of the truth at every position; the raw
    # head is visibly miscalibrated and the fit is not
    for j, t in enumerate(tau_true):
        assert abs(np.log(r["tau"][j] / t)) < 4.5 * step, (j, r["tau"][j], t)
    assert np.all(r["ece_fit"] < 0.01)
    assert r["ece_raw"][0] > 0.03


def test_raw_temperatures_of_one_recovered():
    c, acc, nv = _tempered_head(40000, 3, [1.0, 1.0, 1.0], seed=4)
    grid = synth.sts_grid(129)
    r = sts.sts_fit(c, acc, nv, grid)
    assert np.all(np.abs(np.log(r["tau"])) < 4.5 * np.log(grid[1] / grid[0]))


def test_exactly_calibrated_case_picks_one():
    # position 1: c = 0.75 four times (three accepted), c = 0.25 four times (one
    # accepted): at tau = 1 every bin is calibrated (ECE ~ 1e-16); any other grid
    # value moves both groups and costs more than 1e-3
    c = np.array([[0.75]] * 4 + [[0.25]] * 4, dtype=np.float32)
    acc = np.array([1, 1, 1, 0, 1, 0, 0, 0], dtype=np.int32)
    nv = np.ones(8, dtype=np.int32)
    grid = synth.sts_grid(65)
    r = sts.sts_fit(c, acc, nv, grid)
    assert r["idx"][0] == 32 and r["tau"][0] == 1.0
    assert r["ece_fit"][0] < 1e-15


def test_observation_rule():
    # nothing verified and nothing rejected: no sample is observed anywhere
    c = np.full((5, 3), 0.7, dtype=np.float32)
    r = sts.sts_fit(c, np.zeros(5, np.int32), np.zeros(5, np.int32), synth.sts_grid(17))
    assert np.all(r["tau"] == 1.0) and np.all(r["idx"] == -1)
    assert np.all(np.isnan(r["ece_fit"])) and np.all(np.isnan(r["ece_raw"]))
    # only verified positions enter, whatever the outcome of earlier ones
    acc, nv = np.array([0, 1]), np.array([1, 3])
    assert list(sts.observed(acc, nv, 1)) == [True, True]
    assert list(sts.observed(acc, nv, 2)) == [False, True]   # sample 0 rejected at 1, verified 1
    acc, nv = np.array([2, 1]), np.array([2, 3])
    assert list(sts.observed(acc, nv, 3)) == [False, True]


def test_selecting_on_rejections_would_bias():
    # the rule that also admits samples rejected before their verified length
    # (label 0 known) drifts from the true temperature under censoring; the
    # verified-length rule does not (the censored recovery test above)
    tau_true = [1.6, 0.8, 1.3, 2.0]
    c, acc, nv = _tempered_head(60000, 4, tau_true, seed=3, censor=True)
    grid = synth.sts_grid(129)
    orig = sts.observed
    try:
        sts.observed = lambda a, n, k: (k <= np.asarray(n)) | (np.asarray(a) < np.asarray(n))
        biased = sts.sts_fit(c, acc, nv, grid)
    finally:
        sts.observed = orig
    good = sts.sts_fit(c, acc, nv, grid)
    err = lambda r: max(abs(np.log(r["tau"][j] / t)) for j, t in enumerate(tau_true))
    assert err(biased) > 2 * err(good)


def test_unobserved_entries_do_not_matter():
    c, acc, nv = synth.make_sts_samples(3000, 6, seed=9, censor=True)
    grid = synth.sts_grid(33)
    r0 = sts.sts_fit(c, acc, nv, grid)
    c2 = c.copy()
    for j in range(6):
        hidden = ~sts.observed(acc.astype(np.int64), nv.astype(np.int64), j + 1)
        c2[hidden, j] = np.float32(0.123)
    r1 = sts.sts_fit(c2, acc, nv, grid)
    assert np.array_equal(r0["idx"], r1["idx"])
    np.testing.assert_array_equal(r0["ece_fit"], r1["ece_fit"])


def test_left_to_right():
    c, acc, nv = synth.make_sts_samples(4000, 6, seed=10)
    grid = synth.sts_grid(33)
    r0 = sts.sts_fit(c, acc, nv, grid)
    c2 = c.copy()
    c2[:, 3:] = np.float32(0.9)   # later positions changed
    r1 = sts.sts_fit(c2, acc, nv, grid)
    assert np.array_equal(r0["idx"][:3], r1["idx"][:3])
    np.testing.assert_array_equal(r0["ece_fit"][:3], r1["ece_fit"][:3])
    # an earlier temperature changes what the later positions see
    acc2 = acc.copy()
    c3 = c.copy()
    c3[:, 0] = np.float32(0.999)
    r2 = sts.sts_fit(c3, acc2, nv, grid)
    assert not np.array_equal(r0["ece_fit"][1:], r2["ece_fit"][1:])


def test_grid_handling_and_ties():
    c, acc, nv = synth.make_sts_samples(2000, 3, seed=11)
    bad = np.array([np.nan, 0.0, -1.0, np.inf])
    r = sts.sts_fit(c, acc, nv, bad)
    assert np.all(r["idx"] == -1) and np.all(r["tau"] == 1.0) and np.all(np.isnan(r["ece_fit"]))
    assert np.all(np.isfinite(r["ece_raw"]))
    g = synth.sts_grid(17)
    ref = sts.sts_fit(c, acc, nv, g)
    dup = np.concatenate([bad[:2], np.repeat(g, 2)])      # every value twice, after two invalid entries
    r = sts.sts_fit(c, acc, nv, dup)
    assert np.array_equal(r["idx"], 2 + 2 * ref["idx"])  # the first of the two equal entries
    np.testing.assert_array_equal(r["tau"], ref["tau"])


def test_fit_never_worse_than_raw_at_the_first_position():
    for seed in range(4):
        c, acc, nv = synth.make_sts_samples(2000, 4, seed=20 + seed)
        r = sts.sts_fit(c, acc, nv, synth.sts_grid(33))
        assert r["ece_fit"][0] <= r["ece_raw"][0]


def test_order_preserved():
    c, acc, nv = synth.make_sts_samples(500, 2, seed=12)
    r = sts.sts_fit(c, acc, nv, synth.sts_grid(33))
    z = sts.logit(c[:, 0])
    cal = 1.0 / (1.0 + np.exp(-z / r["tau"][0]))
    o = np.argsort(c[:, 0], kind="stable")
    assert np.all(np.diff(cal[o]) >= 0)
