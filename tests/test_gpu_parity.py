"""GPU (HIP, through the C ABI) vs the fp64 CPU oracle on the same seeded inputs.

The oracle runs the whole cycle on its own (nothing the GPU produced is fed to
it) and the two cycles are compared stage by stage: tokens, draft
probabilities and log-partitions, confidences and survivals, the whole-batch
schedule, accepted lengths, emitted tokens, target probabilities and residual
masses.  A low-margin difference ends the comparison of what depends on it.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import synth
from oracle import cycle as ocycle
from tests.parity_util import cycle_check

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


def gpu_cycle(lib, cfg, inp, path=0):
    dspark, runner = lib
    P = dspark.Problem.from_config(cfg)
    x = runner.CycleInputs.upload(inp)
    o = runner.CycleOutputs(P)
    runner.run_cycle(P, x, o, path=path)
    torch.cuda.synchronize()
    return o.host()


def check(cfg, inp, g):
    """The GPU cycle against the oracle's own cycle on the same inputs."""
    return cycle_check(cfg, g, ocycle.run_cycle(inp))


SMALL = ["tiny", "tbias", "tbias_bf16"]


@pytest.mark.parametrize("name", SMALL)
def test_parity_small(lib, name):
    cfg = synth.get_config(name)
    _say(f"[gpu] parity {name} B={cfg.B} K={cfg.K} V={cfg.V} r={cfg.r}")
    inp = synth.make_inputs(cfg)
    g = gpu_cycle(lib, cfg, inp)
    counts = check(cfg, inp, g)
    _say(f"[gpu]   low-margin differences {counts}")


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
    # bf16 everything at rank 16 (two 16-byte pieces per factor row): the selection and finishing kernels'
    # smallest piece layout, ragged batch and last chunk
    synth.get_config("tbias_bf16").replace(name="edge_r16_bf16", B=9, K=3, V=1000, r=16, d=32, seed=14),
    # identical draft and target: every scheduled position is accepted
    synth.get_config("tbias").replace(name="edge_p_eq_q", B=3, K=4, V=640, r=16, d=16, target_noise=0.0,
                                      ew_std=0.0, ttable=("linear", 1.0, 0.0), seed=11),
]


@pytest.mark.parametrize("cfg", EDGE, ids=[c.name for c in EDGE])
def test_edge_cases(lib, cfg):
    _say(f"[gpu] edge case {cfg.name} B={cfg.B} K={cfg.K} V={cfg.V} r={cfg.r}")
    inp = synth.make_inputs(cfg)
    g = gpu_cycle(lib, cfg, inp)
    check(cfg, inp, g)
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


@pytest.mark.parametrize("name", ["qwen3_4b", "high_concurrency", "dsv4_vocab", "stress"])
def test_full_size(lib, name):
    # every workload at full size (the bench's, and the larger-batch ones: two
    # and four 256-row passes, 32,768 candidates in the scheduler, and a resample
    # pass past the 32-bit buffer range), every request against the oracle's own cycle
    cfg = synth.get_config(name)
    _say(f"[gpu] full-size {name} B={cfg.B} K={cfg.K} V={cfg.V}")
    inp = synth.make_inputs(cfg)
    g = gpu_cycle(lib, cfg, inp)
    _say("[gpu]   GPU cycle done; oracle cycle running")
    counts = check(cfg, inp, g)
    _say(f"[gpu]   low-margin differences {counts}; N = {int(g['n_total'][0])}")


# Both schedules of the draft phase (dspark_instr.h): each where dspark_draft
# would take the other one (the persistent kernel at the full batch, the
# per-position kernels at small bf16 and fp32-logit batches), and the persistent
# kernel at its edges (fp32 logits with a ragged batch and vocabulary too): one request, one position, a vocabulary of one chunk (one workgroup
# selecting every row) and of one chunk plus a ragged 8 entries, a ragged batch
# with more rows than workgroups, and the largest batch it takes by default.
SCHEDULES = [
    ("high_concurrency", 2),
    ("tbias_bf16", 1),
    ("persist_ragged", 2),
    ("persist_b1", 2),
    ("persist_k1", 2),
    ("persist_v128", 2),
    ("persist_v136", 2),
    ("persist_b48", 2),
    ("qwen3_4b", 1),
    ("persist_f32_ragged", 2),
    ("persist_b150", 2),
    ("persist_f32_b256", 2),
]


def _schedule_cfg(name):
    base = synth.get_config("tbias_bf16")
    if name == "persist_ragged":
        # 33 rows (a ragged N-tile), V = 1000 (a ragged last chunk and M-tile), 8 chunks: 8 workgroups
        # selecting 4-5 rows each
        return base.replace(name=name, B=33, K=3, V=1000, r=256, d=64, seed=15)
    if name == "persist_b1":
        return base.replace(name=name, B=1, K=5, seed=16)
    if name == "persist_k1":
        return base.replace(name=name, K=1, seed=17)
    if name == "persist_v128":
        return base.replace(name=name, B=20, K=3, V=128, d=64, seed=18)
    if name == "persist_v136":
        return base.replace(name=name, B=20, K=3, V=136, d=64, seed=19)
    if name == "persist_f32_ragged":
        # fp32 base logits (the in-place refill of the base-logit registers), ragged batch and vocabulary
        return base.replace(name=name, B=33, K=3, V=1000, r=256, d=64, logits_dtype="f32", seed=21)
    if name == "persist_b48":
        return synth.get_config("high_concurrency").replace(name=name, B=48, K=4, seed=20)
    if name == "persist_b150":
        # five N-tiles, the last ragged (22 rows), and the second half-batch merge on a partial half
        return synth.get_config("high_concurrency").replace(name=name, B=150, K=3, seed=22)
    if name == "persist_f32_b256":
        # fp32 base logits at the full batch (dspark_draft takes the persistent schedule there)
        return synth.get_config("high_concurrency").replace(name=name, K=2, logits_dtype="f32", seed=23)
    return synth.get_config(name)


@pytest.mark.parametrize("name,path", SCHEDULES, ids=[f"{n}-{'persistent' if p == 2 else 'per_position'}"
                                                      for n, p in SCHEDULES])
def test_draft_schedules(lib, name, path):
    dspark, _ = lib
    cfg = _schedule_cfg(name)
    P = dspark.Problem.from_config(cfg)
    auto = dspark.draft_path(P)
    _say(f"[gpu] schedule {path} on {name} B={cfg.B} K={cfg.K} V={cfg.V} (dspark_draft takes {auto})")
    if name in ("high_concurrency", "tbias_bf16", "qwen3_4b"):
        assert auto != path   # the schedule dspark_draft does not take there
    inp = synth.make_inputs(cfg)
    g = gpu_cycle(lib, cfg, inp, path=path)
    counts = check(cfg, inp, g)
    _say(f"[gpu]   low-margin differences {counts}")
