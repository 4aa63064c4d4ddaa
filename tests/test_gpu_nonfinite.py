"""Whole cycles on logits that break the contract (NaN, +-inf), on the GPU.

The contract asks for finite logits (the debug build flags any other); what a
cycle returns for a request whose logits are not finite is unspecified.  What is
specified is that every kernel stays inside its arrays and every id it returns
is a valid one, whatever the values: a row whose chunk scores are all NaN keeps
the best-chunk sentinel, and every selection compares it with the chunk count
and falls back to chunk 0.  These cycles plant such rows and check that

* every returned id is inside the vocabulary and every length inside its range;
* the other requests' draft outputs (tokens, log q, log-partitions, confidences,
  survivals) are bit-identical to a cycle on the clean inputs (each request's
  draft is computed on its own rows only);
* each other request whose scheduled length came out as in the clean cycle (the
  schedule ranks every request's survivals together) has the clean cycle's
  verification outputs.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

BF16_NAN, BF16_NEG_INF, BF16_POS_INF = 0x7FC0, 0xFF80, 0x7F80


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


def _cycle(lib, cfg, inp, path):
    dspark, runner = lib
    P = dspark.Problem.from_config(cfg)
    x = runner.CycleInputs.upload(inp)
    o = runner.CycleOutputs(P)
    runner.run_cycle(P, x, o, path=path)
    torch.cuda.synchronize()
    return o.host()


def _poison(cfg, inp):
    """Copies of the inputs with non-finite rows; returns (inputs, poisoned request ids)."""
    Z, Zt = inp["Z"].copy(), inp["Zt"].copy()
    bf = cfg.logits_dtype == "bf16"
    nan = np.uint16(BF16_NAN) if bf else np.float32(np.nan)
    ninf = np.uint16(BF16_NEG_INF) if bf else np.float32(-np.inf)
    pinf = np.uint16(BF16_POS_INF) if bf else np.float32(np.inf)
    B, K, V = cfg.B, cfg.K, cfg.V
    rows = {}
    rows["draft NaN"] = 1 % B
    Z[rows["draft NaN"]] = nan
    if B > 2:
        rows["draft -inf"] = 2
        Z[2] = ninf
    if B > 3:
        rows["target NaN"] = 3
        Zt[3] = nan
    if B > 5:
        rows["some +inf"] = 5
        Z[5, min(1, K - 1), V // 4: V // 4 + 300] = pinf
        Zt[5, 0, V // 2: V // 2 + 300] = pinf
    out = dict(inp)
    out["Z"], out["Zt"] = Z, Zt
    return out, sorted(set(rows.values()))


CASES = [("tbias_bf16", 0), ("tbias_bf16", 1), ("tbias_bf16_f32logits", 0), ("tbias", 0), ("tiny", 0)]


def _config(name):
    if name == "tbias_bf16_f32logits":  # the persistent draft's fp32 path and the small-batch resample pass
        return synth.get_config("tbias_bf16").replace(name=name, logits_dtype="f32")
    return synth.get_config(name)


@pytest.mark.parametrize("name,path", CASES, ids=[f"{n}-{'auto' if p == 0 else 'per_position'}" for n, p in CASES])
def test_nonfinite_logits_stay_in_range(lib, name, path):
    dspark, _ = lib
    cfg = _config(name)
    B, K, V = cfg.B, cfg.K, cfg.V
    inp = synth.make_inputs(cfg)
    bad_inp, bad = _poison(cfg, inp)
    P = dspark.Problem.from_config(cfg)
    _say(f"[gpu] non-finite logits on {name} B={B} K={K} V={V} path={path} "
         f"(dspark_draft takes {dspark.draft_path(P)}), poisoned requests {bad}")
    ref = _cycle(lib, cfg, inp, path)
    g = _cycle(lib, cfg, bad_inp, path)

    # every id valid, every length in range
    assert ((g["tok"] >= 0) & (g["tok"] < V)).all()
    assert ((g["next_anchor"] >= 0) & (g["next_anchor"] < V)).all()
    assert ((g["n_sched"] >= 0) & (g["n_sched"] <= K)).all()
    assert ((g["n_acc"] >= 0) & (g["n_acc"] <= g["n_sched"])).all()
    for b in range(B):
        emitted = g["out_tok"][b, : g["n_acc"][b] + 1]
        assert ((emitted >= 0) & (emitted < V)).all(), (b, emitted)

    # the clean requests' draft outputs do not see the poisoned rows
    clean = np.setdiff1d(np.arange(B), bad)
    for key in ("tok", "logq", "lse", "conf", "surv"):
        np.testing.assert_array_equal(g[key][clean], ref[key][clean], err_msg=key)
    # and their verification, where the whole-batch schedule gave them the same length
    same = clean[g["n_sched"][clean] == ref["n_sched"][clean]]
    _say(f"[gpu]   {len(same)} of {len(clean)} clean requests kept their scheduled length")
    for key in ("n_acc", "next_anchor", "resid_mass"):
        np.testing.assert_array_equal(g[key][same], ref[key][same], err_msg=key)
    for b in same:
        n = ref["n_acc"][b] + 1
        np.testing.assert_array_equal(g["out_tok"][b, :n], ref["out_tok"][b, :n], err_msg=f"out_tok {b}")
