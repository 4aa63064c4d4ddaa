"""RNN head on the GPU (dspark_draft_rnn, dspark_schedule, dspark_verify_rnn
through the C ABI) against the oracle, stage by stage.

Tolerances.  The GPU state is fp32 (gate inputs from bf16 MFMA products with
fp32 accumulation); the oracle's is fp64.  Both round the state to bf16 for the
logit projection, so where the oracle state lies within STATE_ATOL of a bf16
rounding midpoint the two codes may differ by one bf16 step; a code may differ
nowhere else.  For each (request, position) the logit shift of the entries
whose codes do differ is bounded by
  amb = sum over those entries j of 2 step_j * max_v |Wt[v, j]| / T_s
(step_j the bf16 spacing at the entry, doubled to cover a binade edge),
and every comparison downstream of the projection widens by it: a decision may
differ only where its oracle margin is below 1e-4 + 2 amb; log q within 1e-5
relative plus 2 amb; the residual mass within 1e-5 relative plus 2 amb.  Where
no code differs (amb = 0) these are the Markov head's bounds.  States are
compared to STATE_ATOL absolute (about three times the largest error seen:
3.3e-6); confidences and survivals to 1e-6."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import synth
from oracle import conf as oconf
from oracle import rnn as ornn
from oracle import sched as osched
from oracle import verify as overify
from oracle.io import f64
from parity_util import CONF_ATOL, MARGIN, check_abs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

STATE_ATOL = 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from draft_sampling_verification_markov_amd import dspark, runner
    dspark.load()
    return dspark, runner


def gpu_rnn_cycle(lib, cfg, inp, w):
    dspark, runner = lib
    P = dspark.Problem.from_config(cfg)
    x = runner.CycleInputs.upload(inp)
    o = runner.CycleOutputs(P)
    W_ih, W_hh = runner.to_device(w["W_ih"]), runner.to_device(w["W_hh"])
    b_ih, b_hh = runner.to_device(w["b_ih"]), runner.to_device(w["b_hh"])
    state = torch.full((cfg.B, cfg.K, cfg.r), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(dspark.rnn_workspace_bytes(P), dtype=torch.uint8, device="cuda")
    dspark.draft_rnn(P, x.Z, x.E, x.Wt, x.h, W_ih, b_ih, W_hh, b_hh, x.w_c, x.b_c, x.tau, x.anchor, o.tok, o.logq,
                     o.lse, o.conf, o.surv, state, ws)
    dspark.schedule(P, o.surv, x.T, o.n_sched, o.n_total, ws)
    dspark.verify_rnn(P, x.Zt, x.Z, x.E, x.Wt, x.anchor, o.tok, o.logq, o.lse, state, o.n_sched, o.out_tok, o.n_acc,
                      o.next_anchor, o.logp, o.resid_mass, ws)
    torch.cuda.synchronize()
    g = o.host()
    g["state"] = state.cpu().numpy()
    return g


def ambiguity(state, gpu_state, Wt, T_s, atol=STATE_ATOL):
    """Per (request, position): bound on the logit shift from the entries whose bf16
    codes differ between the GPU's fp32 state and the oracle's fp64 one; each such
    entry must lie within atol of a rounding midpoint."""
    code = ornn.bf16_round(state)
    _, e = np.frexp(state)
    step = np.ldexp(1.0, e - 8)                      # bf16 spacing at the value
    near = np.minimum(np.abs(state - (code + step / 2)), np.abs(state - (code - step / 2))) < atol
    flipped = ornn.bf16_round(np.asarray(gpu_state, np.float64)) != code
    assert not (flipped & ~near).any(), "a bf16 code differs away from a rounding midpoint"
    wmax = np.abs(f64(Wt)).max(axis=0)               # (r,)
    return (flipped * 2 * step * wmax).sum(axis=-1) / float(T_s)


def _decisions(kind, gpu, ref, margin, slack):
    gpu, ref, margin, slack = (np.asarray(a).ravel() for a in (gpu, ref, margin, slack))
    mism = gpu != ref
    bad = mism & ~(margin < MARGIN + 2 * slack)
    assert not bad.any(), (f"{kind}: mismatches beyond margin: idx {np.flatnonzero(bad)[:8]}, "
                           f"margin {margin[bad][:8]}, slack {slack[bad][:8]}")
    return int(mism.sum())


def staged_rnn_check(cfg, inp, w, g, requests=None):
    B, K = cfg.B, cfg.K
    reqs = np.arange(B) if requests is None else np.asarray(requests)
    counts = {}
    d = ornn.rnn_draft(inp["Z"], inp["E"], inp["Wt"], inp["h"], inp["anchor"], w["W_ih"], w["b_ih"], w["W_hh"],
                       w["b_hh"], cfg.T_s, cfg.seed, teacher_x=g["tok"], requests=reqs)
    counts["state_err"] = check_abs("state", g["state"][reqs], d["state"], STATE_ATOL)
    amb = ambiguity(d["state"], g["state"][reqs], inp["Wt"], cfg.T_s)
    counts["draft"] = _decisions("draft token", g["tok"][reqs], d["x"], d["margin"], amb)
    same = g["tok"][reqs] == d["x"]
    rel = np.abs(np.expm1(g["logq"][reqs].astype(np.float64) - d["logq"]))
    assert (rel[same] <= 1e-5 + 2 * amb[same]).all(), f"draft q(x): worst {rel[same].max():.3e}"
    counts["logq_err"] = float(rel[same].max())
    counts["codes_differ"] = int((ornn.bf16_round(g["state"][reqs].astype(np.float64)) !=
                                  ornn.bf16_round(d["state"])).sum())
    counts["logq_err_clean"] = float(rel[same & (amb == 0)].max()) if (same & (amb == 0)).any() else 0.0
    assert counts["logq_err_clean"] <= 1e-5
    c, S = oconf.confidence(inp["h"][reqs], inp["E"], inp["w_c"], inp["b_c"], inp["tau"], inp["anchor"][reqs],
                            g["tok"][reqs])
    check_abs("confidence", g["conf"][reqs], c, CONF_ATOL)
    check_abs("survival", g["surv"][reqs], S, CONF_ATOL)
    sc = osched.schedule(g["surv"].astype(np.float64), inp["T"])
    assert (g["n_sched"] == np.array(sc["n"])).all() or sc["margin"] < MARGIN
    # verification on the GPU's tokens and schedule, with the oracle's own state codes
    vec = np.zeros((B, K, cfg.r))
    vec[reqs] = ornn.bf16_round(d["state"])
    ver = overify.verify(inp["Zt"], inp["Z"], inp["E"], inp["Wt"], inp["anchor"], g["tok"], g["n_sched"], cfg.T_s,
                         cfg.seed, requests=reqs, vec=vec)
    amb_row = amb.max(axis=1)
    acc_ref = np.array([v["accepted"] for v in ver])
    counts["accept"] = _decisions("accepted length", g["n_acc"][reqs], acc_ref,
                                  np.array([v["accept_margin"] for v in ver]), amb_row)
    same_acc = g["n_acc"][reqs] == acc_ref
    y_ref = np.array([v["y"] for v in ver])
    counts["emit"] = _decisions("emitted token", g["next_anchor"][reqs][same_acc], y_ref[same_acc],
                                np.array([v["token_margin"] for v in ver])[same_acc], amb_row[same_acc])
    for i, b in enumerate(reqs):
        v = ver[i]
        if not same_acc[i]:
            continue
        if g["next_anchor"][b] == v["y"]:
            row = np.full(K + 1, -1)
            row[:len(v["tokens"])] = v["tokens"]
            assert (g["out_tok"][b] == row).all(), (b, g["out_tok"][b], row)
        if v["kind"] == "bonus":
            assert np.isnan(g["resid_mass"][b])
        else:
            ks = v["k_star"]
            tol = 1e-5 * abs(v["mass"]) + 2 * amb[i, ks - 1]
            assert abs(g["resid_mass"][b] - v["mass"]) <= tol, (b, g["resid_mass"][b], v["mass"], tol)
    counts["ambiguous_positions"] = int((amb > 0).sum())
    return counts


CASES = [
    ("tbias_bf16", None),
    ("rnn_small_r64", dict(B=33, K=3, V=1032, r=64, d=96, seed=201, ew_std=0.25, wc_std=0.2,
                           ttable=("linear", 5.0, 0.02))),
    ("rnn_k1_r32", dict(B=70, K=1, V=4104, r=32, d=64, seed=202, ew_std=0.25, wc_std=0.2,
                        ttable=("linear", 5.0, 0.02))),
    ("rnn_ragged_d", dict(B=131, K=5, V=2056, r=128, d=200, seed=203, ew_std=0.25, wc_std=0.2,
                          ttable=("linear", 5.0, 0.02))),
]


def _config(name, over):
    if over is None:
        return synth.get_config(name)
    import dataclasses
    return dataclasses.replace(synth.get_config("tbias_bf16"), name=name, **over)


@pytest.mark.parametrize("name,over", CASES, ids=[c[0] for c in CASES])
def test_rnn_staged_parity(lib, name, over):
    cfg = _config(name, over)
    _say(f"[gpu] rnn staged parity {name} B={cfg.B} K={cfg.K} V={cfg.V} r={cfg.r} d={cfg.d}")
    inp = synth.make_inputs(cfg)
    w = synth.make_rnn_weights(cfg)
    g = gpu_rnn_cycle(lib, cfg, inp, w)
    counts = staged_rnn_check(cfg, inp, w, g)
    _say(f"[gpu]   {counts}")


def test_rnn_end_to_end(lib):
    from oracle import cycle as ocycle
    cfg = synth.get_config("tbias_bf16")
    _say(f"[gpu] rnn end-to-end {cfg.name}")
    inp = synth.make_inputs(cfg)
    w = synth.make_rnn_weights(cfg)
    g = gpu_rnn_cycle(lib, cfg, inp, w)
    ref = ocycle.run_cycle_rnn(inp, w)
    d = ref["draft"]
    amb = ambiguity(d["state"], g["state"], inp["Wt"], cfg.T_s) if (g["tok"] == d["x"]).all() else \
        np.full(g["tok"].shape, np.inf)
    diff = g["tok"] != d["x"]
    assert (d["margin"][diff] < MARGIN + 2 * amb[diff]).all()
    if not diff.any():
        assert (g["n_sched"] == np.array(ref["sched"]["n"])).all()
        ok = g["n_acc"] == ref["n_accepted"]
        assert ok.mean() > 0.9
        assert (g["out_tok"][ok & (g["next_anchor"] == ref["next_anchor"])] ==
                ref["out_tok"][ok & (g["next_anchor"] == ref["next_anchor"])]).all()


def test_rnn_deterministic(lib):
    cfg = synth.get_config("tbias_bf16")
    _say("[gpu] rnn determinism")
    inp = synth.make_inputs(cfg)
    w = synth.make_rnn_weights(cfg)
    a = gpu_rnn_cycle(lib, cfg, inp, w)
    b = gpu_rnn_cycle(lib, cfg, inp, w)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_rnn_full_size_sampled(lib):
    cfg = synth.get_config("high_concurrency")
    _say(f"[gpu] rnn full-size {cfg.name} B={cfg.B} K={cfg.K} V={cfg.V} d={cfg.d}")
    inp = synth.make_inputs(cfg)
    w = synth.make_rnn_weights(cfg)
    g = gpu_rnn_cycle(lib, cfg, inp, w)
    reqs = np.random.default_rng(1).choice(cfg.B, 4, replace=False)
    counts = staged_rnn_check(cfg, inp, w, g, requests=reqs)
    _say(f"[gpu]   {counts}; N = {int(g['n_total'][0])}")
