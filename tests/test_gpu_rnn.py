"""RNN head on the GPU (dspark_draft_rnn, dspark_schedule, dspark_verify_rnn
through the C ABI) against the oracle's own RNN-head cycle on the same inputs
(nothing the GPU produced is fed to the oracle), stage by stage.

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
from oracle import cycle as ocycle
from oracle import rnn as ornn
from oracle.io import f64
from parity_util import PROB_RTOL, cycle_check

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


def ambiguity(state, gpu_state, Wt, T_s, where=None, atol=STATE_ATOL):
    """Per (request, position): bound on the logit shift from the entries whose bf16
    codes differ between the GPU's fp32 state and the oracle's fp64 one; each such
    entry must lie within atol of a rounding midpoint.  ``where`` (B x K) limits the
    check to positions whose states are comparable (zero slack elsewhere)."""
    code = ornn.bf16_round(state)
    _, e = np.frexp(state)
    step = np.ldexp(1.0, e - 8)                      # bf16 spacing at the value
    near = np.minimum(np.abs(state - (code + step / 2)), np.abs(state - (code - step / 2))) < atol
    flipped = ornn.bf16_round(np.asarray(gpu_state, np.float64)) != code
    if where is not None:
        flipped &= where[..., None]
    assert not (flipped & ~near).any(), "a bf16 code differs away from a rounding midpoint"
    wmax = np.abs(f64(Wt)).max(axis=0)               # (r,)
    return (flipped * 2 * step * wmax).sum(axis=-1) / float(T_s)


def rnn_check(cfg, inp, w, g):
    """The GPU RNN-head cycle against the oracle's own RNN-head cycle (nothing of the
    GPU's fed to the oracle), stage by stage; states where the preceding tokens agree."""
    ref = ocycle.run_cycle_rnn(inp, w)
    d = ref["draft"]
    same = g["tok"] == d["x"]
    prefix = np.cumprod(same, axis=1).astype(bool)
    prev_ok = np.concatenate([np.ones((cfg.B, 1), bool), prefix[:, :-1]], axis=1)
    err = np.abs(g["state"].astype(np.float64) - d["state"])[prev_ok]
    assert (err <= STATE_ATOL).all(), f"state: worst {err.max():.3e}"
    slack = ambiguity(d["state"], g["state"], inp["Wt"], cfg.T_s, where=prev_ok)
    counts = cycle_check(cfg, g, ref, slack)
    counts["state_err"] = float(err.max())
    counts["codes_differ"] = int((ornn.bf16_round(g["state"].astype(np.float64)) !=
                                  ornn.bf16_round(d["state"]))[prev_ok].sum())
    rel = np.abs(np.expm1(g["logq"].astype(np.float64) - d["logq"]))
    clean = prefix & (slack == 0)
    counts["logq_err_clean"] = float(rel[clean].max()) if clean.any() else 0.0
    assert counts["logq_err_clean"] <= PROB_RTOL
    counts["positions_with_flips"] = int((slack > 0).sum())
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
def test_rnn_parity(lib, name, over):
    cfg = _config(name, over)
    _say(f"[gpu] rnn parity {name} B={cfg.B} K={cfg.K} V={cfg.V} r={cfg.r} d={cfg.d}")
    inp = synth.make_inputs(cfg)
    w = synth.make_rnn_weights(cfg)
    g = gpu_rnn_cycle(lib, cfg, inp, w)
    _say(f"[gpu]   {rnn_check(cfg, inp, w, g)}")


def test_rnn_deterministic(lib):
    cfg = synth.get_config("tbias_bf16")
    _say("[gpu] rnn determinism")
    inp = synth.make_inputs(cfg)
    w = synth.make_rnn_weights(cfg)
    a = gpu_rnn_cycle(lib, cfg, inp, w)
    b = gpu_rnn_cycle(lib, cfg, inp, w)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=k)


def test_rnn_full_size(lib):
    cfg = synth.get_config("high_concurrency")
    _say(f"[gpu] rnn full-size {cfg.name} B={cfg.B} K={cfg.K} V={cfg.V} d={cfg.d}")
    inp = synth.make_inputs(cfg)
    w = synth.make_rnn_weights(cfg)
    g = gpu_rnn_cycle(lib, cfg, inp, w)
    _say("[gpu]   GPU cycle done; oracle cycle running")
    _say(f"[gpu]   {rnn_check(cfg, inp, w, g)}; N = {int(g['n_total'][0])}")
