"""Scheduler alone (HIP, through the C ABI) vs the oracle scheduler, at
candidate counts on both sides of the single-workgroup limit (16384) and with
exact ties between survivals, so that the (survival desc, request asc,
position asc) order is decided by the tie-break."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import synth
from oracle import sched as osched

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from draft_sampling_verification_markov_amd import dspark
    dspark.load()
    return dspark


CASES = [
    (256, 16, False),   # 4096 candidates, the batch of the throughput workload
    (512, 32, False),   # exactly 16384: the largest set ordered in LDS
    (1024, 32, False),  # 32768: ordered through global memory
    (700, 9, True),     # ties everywhere
    (3000, 7, True),    # ties, global path
]


@pytest.mark.parametrize("B,K,ties", CASES, ids=[f"B{b}_K{k}{'_ties' if t else ''}" for b, k, t in CASES])
def test_schedule_sizes(lib, B, K, ties):
    dspark = lib
    n = B * K
    print(f"[gpu] schedule B={B} K={K} n={n} ties={ties}", flush=True)
    sys.stdout.flush()
    S = synth.make_survivals(B, K, seed=5, ties=ties)
    # cliff table: flat up to N0, then 100x.  Every candidate before the cliff
    # passes exactly (s > 0) and the one at the cliff fails by a wide margin,
    # so which n/3 candidates are taken, and hence every per-request count,
    # is decided by the order alone; the comparison is exact.
    N0 = B + n // 3
    T = np.where(np.arange(B * (K + 1) + 1) <= N0, 1.0, 100.0).astype(np.float32)
    ref = osched.schedule(S.astype(np.float64), T)
    assert ref["N"] == N0
    P = dspark.Problem.make(B, K, 1024, 16, 8)
    ws = torch.empty(dspark.workspace_bytes(P), dtype=torch.uint8, device="cuda")
    surv = torch.from_numpy(S).cuda()
    T_d = torch.from_numpy(T).cuda()
    n_sched = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    n_total = torch.zeros(1, dtype=torch.int32, device="cuda")
    dspark.schedule(P, surv, T_d, n_sched, n_total, ws)
    torch.cuda.synchronize()
    g = n_sched.cpu().numpy()
    print(f"[gpu]   N = {int(n_total.item())} (oracle {ref['N']}); requests differing: "
          f"{int((g != np.array(ref['n'])).sum())}", flush=True)
    np.testing.assert_array_equal(g, np.array(ref["n"]))
    assert int(n_total.item()) == ref["N"]


ASYNC_CASES = [(256, 16, False), (700, 9, True), (1024, 32, False), (3000, 7, True)]


@pytest.mark.parametrize("B,K,ties", ASYNC_CASES, ids=[f"B{b}_K{k}{'_ties' if t else ''}" for b, k, t in ASYNC_CASES])
def test_schedule_async_sizes(lib, B, K, ties):
    # budget from survivals two steps earlier (cliff table: decided exactly), the
    # current candidates in schedule order; the comparison is exact
    dspark = lib
    n = B * K
    print(f"[gpu] schedule_async B={B} K={K} n={n} ties={ties}", flush=True)
    S_lag = synth.make_survivals(B, K, seed=6, ties=False)
    S = synth.make_survivals(B, K, seed=5, ties=ties)
    N0 = B + n // 5
    T = np.where(np.arange(B * (K + 1) + 1) <= N0, 1.0, 100.0).astype(np.float32)
    ref = osched.schedule_async(S_lag.astype(np.float64), S.astype(np.float64), T)
    assert ref["N"] == N0
    P = dspark.Problem.make(B, K, 1024, 16, 8)
    ws = torch.empty(dspark.workspace_bytes(P), dtype=torch.uint8, device="cuda")
    n_sched = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    n_total = torch.zeros(1, dtype=torch.int32, device="cuda")
    dspark.schedule_async(P, torch.from_numpy(S_lag).cuda(), torch.from_numpy(S).cuda(), torch.from_numpy(T).cuda(),
                          n_sched, n_total, ws)
    torch.cuda.synchronize()
    g = n_sched.cpu().numpy()
    print(f"[gpu]   N = {int(n_total.item())} (oracle {ref['N']}); requests differing: "
          f"{int((g != np.array(ref['n'])).sum())}", flush=True)
    np.testing.assert_array_equal(g, np.array(ref["n"]))
    assert int(n_total.item()) == ref["N"]
    # the synchronous schedule of the current survivals differs (a different budget): the lag matters
    assert ref["N"] != osched.schedule(S.astype(np.float64),
                                       np.where(np.arange(B * (K + 1) + 1) <= B + n // 3, 1.0, 100.0))["N"]


STATIC_CASES = [(256, 16, False), (1500, 7, True), (1, 1, False), (2049, 32, True)]


@pytest.mark.parametrize("B,K,ties", STATIC_CASES, ids=[f"B{b}_K{k}{'_ties' if t else ''}" for b, k, t in STATIC_CASES])
def test_schedule_baselines(lib, B, K, ties):
    """Fixed-length and static-threshold baselines, bit-exact against the oracle.
    Thresholds include values equal to a survival (the comparison is >=, and
    both sides compare the same fp32 numbers), 0, 1 and beyond."""
    dspark = lib
    print(f"[gpu] baselines B={B} K={K} ties={ties}", flush=True)
    S = synth.make_survivals(B, K, seed=11, ties=ties)
    P = dspark.Problem.make(B, K, 1024, 16, 8)
    surv = torch.from_numpy(S).cuda()
    n_sched = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    n_total = torch.zeros(1, dtype=torch.int32, device="cuda")
    for gamma in sorted({0, 1, K // 2, K}):
        dspark.schedule_fixed(P, gamma, n_sched, n_total)
        torch.cuda.synchronize()
        ref = osched.schedule_fixed(B, K, gamma)
        assert n_sched.cpu().tolist() == ref["n"] and int(n_total.item()) == ref["N"]
    thetas = [0.0, 0.5, 1.0, 1.5, -1.0, float(S[0, min(1, K - 1)]), float(S[B // 2, 0])]
    for theta in thetas:
        dspark.schedule_threshold(P, surv, theta, n_sched, n_total)
        torch.cuda.synchronize()
        ref = osched.schedule_threshold(S, np.float32(theta))
        assert n_sched.cpu().tolist() == list(ref["n"]), theta
        assert int(n_total.item()) == ref["N"], theta
    with pytest.raises(RuntimeError):
        dspark.schedule_fixed(P, K + 1, n_sched, n_total)


def _linear_table(B, K, slope):
    return (5.0 + slope * np.arange(B * (K + 1) + 1)).astype(np.float32)


def _stair_table(B, K, delta, width=64):
    N = np.arange(B * (K + 1) + 1)
    return (1.0 + delta * np.maximum(N - B, 0) // width).astype(np.float32)


def _mid_order_table(B, K, S, kind):
    """A table whose first drop lands near the middle of the candidate order, away
    from a tie: the parameter (slope, or step height) is the geometric middle of
    the interval over which the oracle takes the same number of candidates as at
    the parameter that splits the order in half (bisection on the oracle, log scale)."""
    make = _linear_table if kind == "linear" else _stair_table
    n = B * K
    S64 = S.astype(np.float64)

    def taken(x):
        return osched.schedule(S64, make(B, K, x).astype(np.float64))["taken"]

    def edge(lo, hi, keep_lo):
        # bisect [lo, hi] for the point where keep_lo(taken) stops holding
        for _ in range(50):
            mid = (lo * hi) ** 0.5
            lo, hi = (mid, hi) if keep_lo(taken(mid)) else (lo, mid)
        return lo, hi

    _, x0 = edge(1e-9, 10.0, lambda t: t > n // 2)
    t0 = taken(x0)
    a, _ = edge(1e-9, x0, lambda t: t > t0)           # below a more are taken
    _, b = edge(x0, 10.0, lambda t: t >= t0)          # above b fewer are taken
    return make(B, K, (a * b) ** 0.5)


GREEDY_CASES = [(256, 16, "linear"), (256, 16, "stair"), (512, 32, "linear"), (512, 32, "stair"),
                (1024, 32, "linear"), (1024, 32, "stair")]


@pytest.mark.parametrize("B,K,kind", GREEDY_CASES, ids=[f"B{b}_K{k}_{t}" for b, k, t in GREEDY_CASES])
def test_schedule_greedy_mid_order(lib, B, K, kind):
    """Linear and staircase step-time tables whose first drop lands mid-order: the
    greedy comparison (A + s) T[N] >= A T[N + 1] decides every candidate up to the
    stop (the GPU sums A in float64 in a parallel prefix, the oracle in order), so
    the whole schedule is compared exactly (margins and cut gap reported)."""
    dspark = lib
    n = B * K
    S = synth.make_survivals(B, K, seed=21, ties=False)
    T = _mid_order_table(B, K, S, kind)
    ref = osched.schedule(S.astype(np.float64), T.astype(np.float64))
    print(f"[gpu] schedule greedy B={B} K={K} {kind}: oracle takes {ref['taken']} of {n}, margin "
          f"{ref['margin']:.3e}, cut gap {ref['cut_gap']:.3e}", flush=True)
    assert n // 4 < ref["taken"] < 3 * n // 4
    P = dspark.Problem.make(B, K, 1024, 16, 8)
    ws = torch.empty(dspark.workspace_bytes(P), dtype=torch.uint8, device="cuda")
    n_sched = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    n_total = torch.zeros(1, dtype=torch.int32, device="cuda")
    dspark.schedule(P, torch.from_numpy(S).cuda(), torch.from_numpy(T).cuda(), n_sched, n_total, ws)
    torch.cuda.synchronize()
    g = n_sched.cpu().numpy()
    differ = int((g != np.array(ref["n"])).sum())
    print(f"[gpu]   N = {int(n_total.item())} (oracle {ref['N']}); requests differing: {differ}", flush=True)
    # Both sides evaluate every comparison in float64 on the same float32 survivals and
    # table entries; they differ only in the order of the additions that form A (a
    # relative difference of order n * 1e-16).  The comparisons' relative margins here
    # are about (survival spacing) / A, 1e-9 to 1e-8, far above that: the schedule must
    # be identical unless the oracle's margin is below 1e-12.
    if differ or int(n_total.item()) != ref["N"]:
        assert ref["margin"] < 1e-12, "schedule differs at a comparison margin above 1e-12"
    else:
        assert int(n_total.item()) == ref["N"]
