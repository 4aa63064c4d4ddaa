"""The library inside a captured HIP graph: a whole cycle (draft, schedule,
verify; Markov head and RNN head) captured once on stable buffers, replayed
several times with eager work and synchronisation between the replays, new
inputs copied into the captured input buffers between replays; every replay
must reproduce the eager cycle on the same inputs bit for bit.  The library
records no memset and no host synchronisation, so nothing in the graph
depends on host state.  Under capture the draft runs its per-position
schedule (a cooperative launch is not captured), so the eager references take
that schedule explicitly; outside capture small batches take the persistent
one, equal up to fp32 summation order."""
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
    dspark.load()
    return dspark, runner


def _copy_inputs(dst, src):
    for f in ("Z", "Zt", "E", "Wt", "h", "w_c", "tau", "anchor", "T"):
        getattr(dst, f).copy_(getattr(src, f))


def _host(o):
    return {k: np.array(v, copy=True) for k, v in o.host().items()}


def _same(a, b, what):
    for k in a:
        np.testing.assert_array_equal(a[k], b[k], err_msg=f"{what}: {k}")


@pytest.mark.parametrize("name", ["tiny", "tbias_bf16"])
def test_cycle_graph_replays(lib, name):
    dspark, runner = lib
    cfg = synth.get_config(name)
    _say(f"[gpu] graph replay {name}")
    P = dspark.Problem.from_config(cfg)
    sets = []
    for seed_shift in (0, 7):
        import dataclasses
        c = dataclasses.replace(cfg, seed=cfg.seed + seed_shift)
        sets.append(runner.CycleInputs.upload(synth.make_inputs(c)))
    # eager references, on the schedule capture records
    per_position = dspark.DRAFT_PER_POSITION
    refs = []
    for x in sets:
        o = runner.CycleOutputs(P)
        runner.run_cycle(P, x, o, path=per_position)
        torch.cuda.synchronize()
        refs.append(_host(o))
    assert not all(np.array_equal(refs[0][k], refs[1][k]) for k in refs[0])
    # stable buffers, warm-up on a side stream, capture
    xs = runner.CycleInputs.upload(synth.make_inputs(cfg))
    og = runner.CycleOutputs(P)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        runner.run_cycle(P, xs, og)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        runner.run_cycle(P, xs, og)
    torch.cuda.synchronize()
    other = runner.CycleOutputs(P)
    for rep in range(4):
        i = rep % 2
        _copy_inputs(xs, sets[i])
        og.tok.fill_(-3)
        og.n_acc.fill_(-3)
        g.replay()
        runner.run_cycle(P, sets[1 - i], other, path=per_position)   # eager work between replays
        torch.cuda.synchronize()
        _same(_host(og), refs[i], f"replay {rep}")
        _same(_host(other), refs[1 - i], f"eager after replay {rep}")


def test_rnn_cycle_graph_replays(lib):
    dspark, runner = lib
    cfg = synth.get_config("tbias_bf16")
    _say("[gpu] graph replay RNN head")
    P = dspark.Problem.from_config(cfg)
    inp = synth.make_inputs(cfg)
    w = synth.make_rnn_weights(cfg)
    x = runner.CycleInputs.upload(inp)
    W_ih, W_hh = runner.to_device(w["W_ih"]), runner.to_device(w["W_hh"])
    b_ih, b_hh = runner.to_device(w["b_ih"]), runner.to_device(w["b_hh"])

    def make_state():
        return (torch.zeros((cfg.B, cfg.K, cfg.r), dtype=torch.float32, device="cuda"),
                torch.empty(dspark.rnn_workspace_bytes(P), dtype=torch.uint8, device="cuda"))

    def cycle(o, state, ws):
        dspark.draft_rnn(P, x.Z, x.E, x.Wt, x.h, W_ih, b_ih, W_hh, b_hh, x.w_c, x.b_c, x.tau, x.anchor, o.tok, o.logq,
                         o.lse, o.conf, o.surv, state, ws)
        dspark.schedule(P, o.surv, x.T, o.n_sched, o.n_total, ws)
        dspark.verify_rnn(P, x.Zt, x.Z, x.E, x.Wt, x.anchor, o.tok, o.logq, o.lse, state, o.n_sched, o.out_tok,
                          o.n_acc, o.next_anchor, o.logp, o.resid_mass, ws)

    o_ref = runner.CycleOutputs(P)
    st_ref, ws_ref = make_state()
    cycle(o_ref, st_ref, ws_ref)
    torch.cuda.synchronize()
    ref = _host(o_ref)
    ref["state"] = st_ref.cpu().numpy()
    og = runner.CycleOutputs(P)
    st_g, ws_g = make_state()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        cycle(og, st_g, ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cycle(og, st_g, ws_g)
    for rep in range(3):
        st_g.fill_(float("nan"))
        og.tok.fill_(-3)
        g.replay()
        cycle(o_ref, st_ref, ws_ref)                # eager work between replays
        torch.cuda.synchronize()
        got = _host(og)
        got["state"] = st_g.cpu().numpy()
        _same(got, ref, f"RNN replay {rep}")
