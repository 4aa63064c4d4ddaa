"""The debug build (libdspark_debug.so, DSPARK_DEBUG_CHECKS) on the GPU.

A whole cycle through it gives bit-identical results to the ordinary library and
raises no flag; its input scans, run alone (no other kernel sees the planted
values), raise exactly the flag of each planted contract violation: a NaN or an
infinity among bf16 and fp32 logits, an anchor outside [0, V), a step-time
entry that is zero or NaN.  The persistent draft's bounded barrier waits, made
unreachable from the host, give up, raise their flag and let every workgroup
run to the end; normal waits afterwards give the ordinary library's tokens.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import synth

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
    dspark.load(False)
    dspark.load(True)
    yield dspark, runner
    dspark.use_debug_library(False)


def _cycle(dspark, runner, cfg, inp, debug):
    dspark.use_debug_library(debug)
    try:
        P = dspark.Problem.from_config(cfg)
        x = runner.CycleInputs.upload(inp)
        o = runner.CycleOutputs(P)
        runner.run_cycle(P, x, o)
        torch.cuda.synchronize()
        return o.host()
    finally:
        dspark.use_debug_library(False)


@pytest.mark.parametrize("name", ["tbias_bf16", "tbias"])
def test_debug_cycle_matches_and_flags_nothing(lib, name):
    dspark, runner = lib
    cfg = synth.get_config(name)
    _say(f"[gpu] debug library cycle {name} B={cfg.B} K={cfg.K} V={cfg.V}")
    inp = synth.make_inputs(cfg)
    dspark.debug_flags(clear=True)
    plain = _cycle(dspark, runner, cfg, inp, False)
    dbg = _cycle(dspark, runner, cfg, inp, True)
    assert dspark.debug_flags(clear=True) == 0
    for k in plain:
        np.testing.assert_array_equal(plain[k], dbg[k], err_msg=k)


@pytest.mark.parametrize("logits", ["bf16", "f32"])
def test_debug_input_scans_flag_planted_violations(lib, logits):
    dspark, _ = lib
    B, K, V = 5, 3, 1000
    P = dspark.Problem.make(B, K, V, 32, 64, logits, "bf16", "bf16")
    dt = torch.bfloat16 if logits == "bf16" else torch.float32
    g = torch.Generator(device="cuda").manual_seed(3)
    Z = torch.randn(B, K, V, device="cuda", generator=g).to(dt)
    Zt = torch.randn(B, K + 1, V, device="cuda", generator=g).to(dt)
    anchor = torch.randint(0, V, (B,), device="cuda", dtype=torch.int32, generator=g)
    T = torch.linspace(1.0, 2.0, B * (K + 1) + 1, device="cuda")
    dspark.debug_flags(clear=True)
    _say(f"[gpu] debug scans, {logits} logits: clean inputs")
    dspark.debug_check_inputs(P, Z, Zt, anchor, T)
    assert dspark.debug_flags(clear=True) == 0

    def flags_of(**kw):
        args = dict(Z=Z, target=Zt, anchor=anchor, T_table=T)
        args.update(kw)
        dspark.debug_check_inputs(P, **args)
        return dspark.debug_flags(clear=True)

    Zn = Z.clone()
    Zn[2, 1, 777] = float("nan")
    assert flags_of(Z=Zn) == dspark.DEBUG_LOGITS
    Zi = Z.clone()
    Zi[4, 2, V - 1] = float("inf")   # the last element of the array
    assert flags_of(Z=Zi) == dspark.DEBUG_LOGITS
    Tn = Zt.clone()
    Tn[0, K, 0] = float("-inf")
    assert flags_of(target=Tn) == dspark.DEBUG_LOGITS
    for bad in (-1, V):
        a = anchor.clone()
        a[3] = bad
        assert flags_of(anchor=a) == dspark.DEBUG_IDS, bad
    for bad in (0.0, float("nan"), -1.0):
        t = T.clone()
        t[B * (K + 1)] = bad
        assert flags_of(T_table=t) == dspark.DEBUG_SCHEDULE_INPUT, bad
    # several at once: their bits together
    assert flags_of(Z=Zn, anchor=torch.full_like(anchor, V)) == dspark.DEBUG_LOGITS | dspark.DEBUG_IDS


def test_persistent_barrier_timeout_ends_and_is_flagged(lib):
    dspark, runner = lib
    cfg = synth.get_config("tbias_bf16")
    P = dspark.Problem.from_config(cfg)
    assert dspark.draft_path(P) == dspark.DRAFT_PERSISTENT
    _say(f"[gpu] persistent draft with unreachable barriers, B={cfg.B} K={cfg.K} V={cfg.V}")
    inp = synth.make_inputs(cfg)
    x = runner.CycleInputs.upload(inp)
    o = runner.CycleOutputs(P)
    runner.draft(P, x, o)
    torch.cuda.synchronize()
    ref = o.tok.cpu().numpy().copy()
    dspark.use_debug_library(True)
    try:
        dspark.debug_flags(clear=True)
        dspark.debug_force_barrier_timeout(True)
        try:
            runner.draft(P, x, o)
            torch.cuda.synchronize()
        finally:
            dspark.debug_force_barrier_timeout(False)
        flags = dspark.debug_flags(clear=True)
        assert flags & dspark.DEBUG_BARRIER_TIMEOUT, flags
        tok = o.tok.cpu().numpy()
        assert ((tok >= 0) & (tok < cfg.V)).all()   # every workgroup ran to its end
        runner.draft(P, x, o)
        torch.cuda.synchronize()
        assert dspark.debug_flags(clear=True) == 0
        np.testing.assert_array_equal(o.tok.cpu().numpy(), ref)
    finally:
        dspark.use_debug_library(False)
