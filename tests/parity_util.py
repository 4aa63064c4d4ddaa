"""Helpers of the GPU-vs-oracle parity tests.

Decision rule: a GPU decision (token, acceptance, scheduled length) may differ
from the oracle's only where the oracle's decision margin is below 1e-4, and
such mismatches must stay below 0.01% of the decisions of their kind.
Floating-point outputs: probabilities (q(x), p(x)) and the residual mass
sum_v max(0, p_v - q_v) within 1e-5 relative, confidences and survivals within
1e-6 absolute.
"""
from __future__ import annotations

import numpy as np

MARGIN = 1e-4
MISMATCH_RATE = 1e-4
PROB_RTOL = 1e-5
CONF_ATOL = 1e-6


def check_decisions(kind: str, gpu, ref, margin) -> int:
    gpu, ref, margin = (np.asarray(a).ravel() for a in (gpu, ref, margin))
    mism = gpu != ref
    high = mism & ~(margin < MARGIN)
    assert not high.any(), (f"{kind}: {int(high.sum())} mismatches with margin >= {MARGIN}: "
                            f"idx {np.flatnonzero(high)[:8]}, gpu {gpu[high][:8]}, oracle {ref[high][:8]}, "
                            f"margin {margin[high][:8]}")
    n = int(mism.sum())
    assert n <= MISMATCH_RATE * mism.size, f"{kind}: {n} low-margin mismatches of {mism.size} decisions"
    return n


def check_logprob(kind: str, gpu_log, ref_log, where=None) -> float:
    """|p_gpu / p_ref - 1| <= PROB_RTOL, with p = exp(log value)."""
    g, r = np.asarray(gpu_log, np.float64), np.asarray(ref_log, np.float64)
    if where is not None:
        g, r = g[where], r[where]
    if g.size == 0:
        return 0.0
    rel = np.abs(np.expm1(g - r))
    worst = float(rel.max())
    assert worst <= PROB_RTOL, f"{kind}: worst relative error {worst:.3e} at {np.argmax(rel)}"
    return worst


def check_abs(kind: str, gpu, ref, atol: float) -> float:
    err = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= atol, f"{kind}: worst abs error {worst:.3e} at {np.unravel_index(np.argmax(err), err.shape)}"
    return worst


def check_rel(kind: str, gpu, ref, rtol: float) -> float:
    g, r = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    rel = np.abs(g - r) / np.abs(r)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= rtol, f"{kind}: worst relative error {worst:.3e}"
    return worst


def cycle_check(cfg, g, ref, slack=None) -> dict:
    """A GPU cycle g against the oracle's own cycle ref on the same inputs.

    Nothing the GPU produced is fed to the oracle: the two cycles run
    independently and are compared stage by stage.  The first token of a request
    that differs must be a decision of oracle margin below MARGIN; that
    request's later positions, its schedule and its verification are then not
    compared (its prefixes differ), while every other request still is.  The
    whole-batch schedule must equal the oracle's unless the oracle's scheduler
    margin or survival cut gap is below MARGIN, or a draft token differed
    (then the survivals the schedule ranks differ too); where it differs, the
    requests whose scheduled lengths differ leave the verification comparison.
    ``slack`` (B x K, the RNN head's bound on logit shifts from bf16 code
    flips) widens the margins and the probability tolerances of the draft
    distribution.  Returns counts of low-margin differences per decision kind
    and of the requests each stage compared (asserted to cover every request
    that no excused difference touched)."""
    B, K = cfg.B, cfg.K
    d = ref["draft"]
    sl = np.zeros((B, K)) if slack is None else np.asarray(slack, np.float64)
    counts = {}
    same = g["tok"] == d["x"]
    prefix = np.cumprod(same, axis=1).astype(bool)                      # tokens equal through k
    prev_ok = np.concatenate([np.ones((B, 1), bool), prefix[:, :-1]], axis=1)  # equal before k
    first = prev_ok & ~same
    bad = first & ~(d["margin"] < MARGIN + 2 * sl)
    assert not bad.any(), (f"draft token: differences beyond the margin at {np.argwhere(bad)[:8].tolist()}, "
                           f"margins {d['margin'][bad][:8]}")
    counts["draft"] = int(first.sum())
    assert counts["draft"] <= MISMATCH_RATE * first.size, f"draft token: {counts['draft']} low-margin differences"
    rel = np.abs(np.expm1(g["logq"].astype(np.float64) - d["logq"]))
    assert (rel[prefix] <= PROB_RTOL + 2 * sl[prefix]).all(), f"draft q(x): worst {rel[prefix].max():.3e}"
    lse_tol = 1e-4 * max(1.0, float(np.abs(d["lse"]).max()))
    assert (np.abs(g["lse"] - d["lse"])[prefix] <= lse_tol + 2 * sl[prefix]).all(), "draft log-partition"
    for key in ("conf", "surv"):
        err = np.abs(g[key].astype(np.float64) - ref[key])[prev_ok]
        assert (err <= CONF_ATOL).all(), f"{key}: worst {err.max():.3e}"
    assert (np.diff(g["surv"], axis=1) <= 0).all(), "GPU survivals must be non-increasing"
    clean = prefix.all(axis=1)                                            # requests with every token equal
    counts["draft_compared_requests"] = int(clean.sum())
    assert counts["draft_compared_requests"] == B - int(first.any(axis=1).sum())

    sc = ref["sched"]
    n_ref = np.array(sc["n"])
    n_gpu = np.asarray(g["n_sched"])
    sched_same = n_gpu == n_ref
    if sched_same.all():
        counts["sched"] = 0
        assert int(g["n_total"][0]) == sc["N"]
    else:
        low = sc["margin"] < MARGIN or sc["cut_gap"] < MARGIN
        assert low or counts["draft"] > 0, (f"schedule differs at margin {sc['margin']:.3e}, cut gap "
                                             f"{sc['cut_gap']:.3e} with no draft token differing")
        counts["sched"] = 1
    counts["sched_requests_differing"] = int((~sched_same).sum())

    comp = clean & sched_same                                             # requests verified on equal inputs
    acc_diff = emit_diff = 0
    compared = 0
    resid_worst = 0.0
    for b in np.flatnonzero(comp):
        v = ref["verify"][b]
        nb = int(n_gpu[b])
        s_b = float(sl[b].max()) if K else 0.0
        compared += 1
        if nb:
            r = np.abs(np.expm1(g["logp"][b, :nb].astype(np.float64) - v["logp"][:nb]))
            assert (r <= PROB_RTOL).all(), f"target p(x) of request {b}: worst {r.max():.3e}"
        assert np.isnan(g["logp"][b, nb:]).all()
        if int(g["n_acc"][b]) != v["accepted"]:
            assert v["accept_margin"] < MARGIN + 2 * s_b, (b, g["n_acc"][b], v["accepted"], v["accept_margin"])
            acc_diff += 1
            continue
        if v["kind"] == "bonus":
            assert np.isnan(g["resid_mass"][b])
        else:
            tol = PROB_RTOL * abs(v["mass"]) + 2 * sl[b, v["k_star"] - 1]
            assert abs(float(g["resid_mass"][b]) - v["mass"]) <= tol, (b, g["resid_mass"][b], v["mass"])
            if v["mass"] > 0:
                resid_worst = max(resid_worst, abs(float(g["resid_mass"][b]) / v["mass"] - 1))
        if int(g["next_anchor"][b]) != v["y"]:
            assert v["token_margin"] < MARGIN + 2 * s_b, (b, g["next_anchor"][b], v["y"], v["token_margin"])
            emit_diff += 1
            continue
        row = np.full(K + 1, -1)
        row[:len(v["tokens"])] = v["tokens"]
        assert (g["out_tok"][b] == row).all(), (b, g["out_tok"][b], row)
    counts["accept"], counts["emit"] = acc_diff, emit_diff
    counts["verify_compared_requests"] = compared
    counts["resid_mass_rel_worst"] = resid_worst
    assert compared == int(comp.sum()) and compared >= 1, counts
    assert acc_diff <= MISMATCH_RATE * B and emit_diff <= MISMATCH_RATE * B, counts
    return counts
