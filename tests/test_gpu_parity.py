"""GPU (HIP, through the C ABI) vs the fp64 CPU oracle on the same seeded inputs.

Staged comparisons feed each oracle stage the GPU's own upstream results (the
draft step k gets the GPU's token x_{k-1}, the confidence head the GPU's
tokens, the scheduler the GPU's survivals, verification the GPU's tokens and
schedule), so a low-margin flip cannot cascade.  End-to-end runs compare the
whole cycle from scratch.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import synth
from oracle import conf as oconf
from oracle import cycle as ocycle
from oracle import draft as odraft
from oracle import sched as osched
from oracle import verify as overify
from tests.parity_util import CONF_ATOL, PROB_RTOL, check_abs, check_decisions, check_logprob, check_rel

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


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


def gpu_cycle(lib, cfg, inp):
    dspark, runner = lib
    P = dspark.Problem.from_config(cfg)
    x = runner.CycleInputs.upload(inp)
    o = runner.CycleOutputs(P)
    runner.run_cycle(P, x, o)
    torch.cuda.synchronize()
    return o.host()


def staged_check(cfg, inp, g, requests=None):
    """Oracle checks of every stage on the GPU's upstream results; returns mismatch counts."""
    B = cfg.B
    reqs = np.arange(B) if requests is None else np.asarray(requests)
    counts = {}
    # draft, teacher-forced on the GPU's previous tokens
    d = odraft.draft(inp["Z"], inp["E"], inp["Wt"], inp["anchor"], cfg.T_s, cfg.seed,
                     teacher_x=g["tok"], requests=reqs)
    counts["draft"] = check_decisions("draft token", g["tok"][reqs], d["x"], d["margin"])
    same = g["tok"][reqs] == d["x"]
    check_logprob("draft q(x)", g["logq"][reqs], d["logq"], where=same)
    check_abs("draft log-partition", g["lse"][reqs], d["lse"], 1e-4 * max(1.0, float(np.abs(d["lse"]).max())))
    # confidence and survival on the GPU's tokens
    c, S = oconf.confidence(inp["h"][reqs], inp["E"], inp["w_c"], inp["b_c"], inp["tau"], inp["anchor"][reqs],
                            g["tok"][reqs])
    check_abs("confidence", g["conf"][reqs], c, CONF_ATOL)
    check_abs("survival", g["surv"][reqs], S, CONF_ATOL)
    assert (np.diff(g["surv"], axis=1) <= 0).all(), "GPU survivals must be non-increasing"
    # schedule on the GPU's survivals (whole batch)
    sc = osched.schedule(g["surv"].astype(np.float64), inp["T"])
    m = np.full(B, sc["margin"])
    counts["sched"] = check_decisions("scheduled length", g["n_sched"], np.array(sc["n"]), m)
    if counts["sched"] == 0:
        assert int(g["n_total"][0]) == sc["N"]
    # verify on the GPU's tokens and schedule
    ver = overify.verify(inp["Zt"], inp["Z"], inp["E"], inp["Wt"], inp["anchor"], g["tok"], g["n_sched"],
                         cfg.T_s, cfg.seed, requests=reqs)
    acc_ref = np.array([v["accepted"] for v in ver])
    acc_m = np.array([v["accept_margin"] for v in ver])
    counts["accept"] = check_decisions("accepted length", g["n_acc"][reqs], acc_ref, acc_m)
    same = g["n_acc"][reqs] == acc_ref
    y_ref = np.array([v["y"] for v in ver])
    y_m = np.array([v["token_margin"] for v in ver])
    counts["emit"] = check_decisions("emitted token", g["next_anchor"][reqs][same], y_ref[same], y_m[same])
    K = cfg.K
    for i, b in enumerate(reqs):
        v = ver[i]
        nb = int(g["n_sched"][b])
        ok = same[i] and g["next_anchor"][b] == v["y"]
        if ok:
            row = np.full(K + 1, -1)
            row[:len(v["tokens"])] = v["tokens"]
            assert (g["out_tok"][b] == row).all(), (b, g["out_tok"][b], row)
        # log p_k(x_k) of every verified position
        if nb:
            check_logprob("target p(x)", g["logp"][b, :nb], v["logp"][:nb])
        assert np.isnan(g["logp"][b, nb:]).all()
        if same[i]:
            if v["kind"] == "bonus":
                assert np.isnan(g["resid_mass"][b])
            else:
                check_rel("residual mass", [g["resid_mass"][b]], [v["mass"]], PROB_RTOL)
    return counts


def end_to_end_check(cfg, inp, g):
    ref = ocycle.run_cycle(inp)
    d = ref["draft"]
    assert (g["tok"] == d["x"]).all() or (d["margin"][g["tok"] != d["x"]] < 1e-4).all()
    if (g["tok"] == d["x"]).all():
        assert (g["n_sched"] == np.array(ref["sched"]["n"])).all()
        assert (g["out_tok"] == ref["out_tok"]).all()
        assert (g["next_anchor"] == ref["next_anchor"]).all()


SMALL = ["tiny", "tbias", "tbias_bf16"]


@pytest.mark.parametrize("name", SMALL)
def test_staged_parity_small(lib, name):
    cfg = synth.get_config(name)
    _say(f"[gpu] staged parity {name} B={cfg.B} K={cfg.K} V={cfg.V} r={cfg.r}")
    inp = synth.make_inputs(cfg)
    g = gpu_cycle(lib, cfg, inp)
    counts = staged_check(cfg, inp, g)
    _say(f"[gpu]   mismatches {counts}")


@pytest.mark.parametrize("name", SMALL)
def test_end_to_end_small(lib, name):
    cfg = synth.get_config(name)
    _say(f"[gpu] end-to-end {name}")
    inp = synth.make_inputs(cfg)
    g = gpu_cycle(lib, cfg, inp)
    end_to_end_check(cfg, inp, g)


EDGE = [
    # one request, one position, a vocabulary smaller than one chunk
    synth.get_config("tbias").replace(name="edge_v8", B=1, K=1, V=8, r=16, d=8),
    # ragged batch (33 rows), one chunk plus a ragged tail, bf16 everything
    synth.get_config("tbias_bf16").replace(name="edge_ragged", B=33, K=3, V=136, r=32, d=64, seed=7),
    # every position scheduled (flat table), 64 positions
    synth.get_config("tbias").replace(name="edge_flat_k64", B=2, K=64, V=512, r=16, d=16,
                                      ttable=("linear", 1.0, 0.0), seed=8),
    # nothing scheduled (steep table): every request takes the bonus path
    synth.get_config("tbias").replace(name="edge_steep", B=5, K=3, V=1000, r=64, d=32,
                                      ttable=("linear", 1.0, 100.0), seed=9),
    # fp32 logits with bf16 factors, T_s != 1, 300 requests (two row passes)
    synth.get_config("tbias_bf16").replace(name="edge_two_pass", B=300, K=2, V=2048, r=128, d=32,
                                           logits_dtype="f32", T_s=0.7, seed=10),
    # bf16 everything with 300 requests: two row passes of the draft and resample kernels, ragged last wave
    synth.get_config("tbias_bf16").replace(name="edge_two_pass_bf16", B=300, K=3, V=2056, r=128, d=32, seed=12),
    # K = 32: the resample pass exceeds the buffer-offset range of its DMA kernel at the full vocabulary,
    # here a small vocabulary keeps it on that kernel while the draft spans 32 positions
    synth.get_config("tbias_bf16").replace(name="edge_k32", B=20, K=32, V=1032, r=64, d=32, seed=13),
    # identical draft and target: every scheduled position is accepted
    synth.get_config("tbias").replace(name="edge_p_eq_q", B=3, K=4, V=640, r=16, d=16, target_noise=0.0,
                                      ew_std=0.0, ttable=("linear", 1.0, 0.0), seed=11),
]


@pytest.mark.parametrize("cfg", EDGE, ids=[c.name for c in EDGE])
def test_edge_cases(lib, cfg):
    _say(f"[gpu] edge case {cfg.name} B={cfg.B} K={cfg.K} V={cfg.V} r={cfg.r}")
    inp = synth.make_inputs(cfg)
    g = gpu_cycle(lib, cfg, inp)
    staged_check(cfg, inp, g)
    end_to_end_check(cfg, inp, g)
    if cfg.name == "edge_steep":
        assert (g["n_sched"] == 0).all() and (g["n_acc"] == 0).all()
    if cfg.name == "edge_flat_k64":
        assert (g["n_sched"] == cfg.K).all()
    if cfg.name == "edge_p_eq_q":
        assert (g["n_acc"] == g["n_sched"]).all() and np.isnan(g["resid_mass"]).all()


def test_deterministic(lib):
    cfg = synth.get_config("tbias_bf16")
    _say("[gpu] determinism tbias_bf16 x3")
    inp = synth.make_inputs(cfg)
    runs = [gpu_cycle(lib, cfg, inp) for _ in range(3)]
    for r in runs[1:]:
        for k in runs[0]:
            np.testing.assert_array_equal(runs[0][k], r[k], err_msg=k)


@pytest.mark.parametrize("name,n_req", [("qwen3_4b", 6), ("high_concurrency", 6), ("dsv4_vocab", 5), ("stress", 4)])
def test_full_size_sampled(lib, name, n_req):
    # every workload at full size (the bench's, and the larger-batch ones: two
    # and four 256-row passes, 32,768 candidates in the scheduler, and a resample
    # pass past the 32-bit buffer range); the oracle checks a sample of requests,
    # and the scheduler over the whole batch
    cfg = synth.get_config(name)
    _say(f"[gpu] full-size {name} B={cfg.B} K={cfg.K} V={cfg.V}")
    inp = synth.make_inputs(cfg)
    g = gpu_cycle(lib, cfg, inp)
    reqs = np.random.default_rng(0).choice(cfg.B, n_req, replace=False)
    counts = staged_check(cfg, inp, g, requests=reqs)
    _say(f"[gpu]   mismatches {counts}; N = {int(g['n_total'][0])}")
