"""The GPU-vs-oracle checker itself, on the CPU.

A stand-in for a GPU result is built from the oracle's own cycle (cast to the
output dtypes the library writes); differences are then planted in it.  The
checker must pass the unchanged result with every request compared, excuse a
token difference only at a low oracle margin while still comparing every other
request, and fail a high-margin difference or a residual mass off by more than
1e-5 relative.
"""
from __future__ import annotations

import copy

import numpy as np
import pytest

import synth
from oracle import cycle as ocycle
from tests import parity_util
from tests.parity_util import cycle_check


@pytest.fixture(scope="module")
def case():
    cfg = synth.get_config("tbias").replace(name="checker", B=6, K=4, V=640, r=16, d=16,
                                            ttable=("linear", 1.0, 0.001), seed=31)
    ref = ocycle.run_cycle(synth.make_inputs(cfg))
    return cfg, ref


def _as_gpu(cfg, ref):
    d = ref["draft"]
    v = ref["verify"]
    logp = np.full((cfg.B, cfg.K), np.nan, np.float32)
    for b, vr in enumerate(v):
        n = int(ref["sched"]["n"][b])
        logp[b, :n] = vr["logp"][:n]
    return {
        "tok": d["x"].astype(np.int32), "logq": d["logq"].astype(np.float32), "lse": d["lse"].astype(np.float32),
        "conf": ref["conf"].astype(np.float32), "surv": ref["surv"].astype(np.float32),
        "n_sched": np.array(ref["sched"]["n"], np.int32), "n_total": np.array([ref["sched"]["N"]], np.int32),
        "out_tok": ref["out_tok"].astype(np.int32), "n_acc": ref["n_accepted"].astype(np.int32),
        "next_anchor": ref["next_anchor"].astype(np.int32), "logp": logp,
        "resid_mass": np.array([vr["mass"] for vr in v], np.float32),
    }


def test_identical_result_compares_every_request(case):
    cfg, ref = case
    counts = cycle_check(cfg, _as_gpu(cfg, ref), ref)
    assert counts["draft"] == counts["sched"] == counts["accept"] == counts["emit"] == 0
    assert counts["draft_compared_requests"] == counts["verify_compared_requests"] == cfg.B


def test_high_margin_token_difference_fails(case):
    cfg, ref = case
    g = _as_gpu(cfg, ref)
    g["tok"][2, 1] = (g["tok"][2, 1] + 1) % cfg.V
    with pytest.raises(AssertionError, match="draft token"):
        cycle_check(cfg, g, ref)


def test_low_margin_token_difference_excludes_only_that_request(case, monkeypatch):
    cfg, ref = case
    ref2 = copy.deepcopy(ref)
    ref2["draft"]["margin"][2, 3] = 1e-6            # the oracle's decision there was a near tie
    g = _as_gpu(cfg, ref)
    g["tok"][2, 3] = (g["tok"][2, 3] + 1) % cfg.V     # last position: no later survival changes
    # 24 decisions: the 0.01% cap allows no difference at all
    with pytest.raises(AssertionError, match="low-margin differences"):
        cycle_check(cfg, g, ref2)
    monkeypatch.setattr(parity_util, "MISMATCH_RATE", 0.5)
    counts = cycle_check(cfg, g, ref2)
    assert counts["draft"] == 1
    assert counts["draft_compared_requests"] == cfg.B - 1
    assert counts["verify_compared_requests"] == cfg.B - 1


def test_residual_mass_off_by_more_than_1e5_fails(case):
    cfg, ref = case
    g = _as_gpu(cfg, ref)
    resid = [b for b, v in enumerate(ref["verify"]) if v["kind"] != "bonus"]
    assert resid, "the case needs a rejection"
    b = resid[0]
    g["resid_mass"][b] = np.float32(ref["verify"][b]["mass"] * (1 + 3e-5))
    with pytest.raises(AssertionError):
        cycle_check(cfg, g, ref)
    g["resid_mass"][b] = np.float32(ref["verify"][b]["mass"] * (1 + 5e-6))
    cycle_check(cfg, g, ref)


def test_schedule_difference_needs_an_excuse(case):
    cfg, ref = case
    g = _as_gpu(cfg, ref)
    b = int(np.argmax(g["n_sched"] < cfg.K))
    g["n_sched"][b] += 1
    ref2 = copy.deepcopy(ref)
    ref2["sched"]["margin"] = ref2["sched"]["cut_gap"] = 1.0
    with pytest.raises(AssertionError, match="schedule differs"):
        cycle_check(cfg, g, ref2)
    ref2["sched"]["cut_gap"] = 1e-6                  # survivals at the cut nearly tied: excused
    counts = cycle_check(cfg, g, ref2)
    assert counts["sched"] == 1 and counts["sched_requests_differing"] == 1
    assert counts["verify_compared_requests"] == cfg.B - 1
