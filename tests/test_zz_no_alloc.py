"""dspark_schedule_noalloc (the scheduler with the library's static scratch, for
callers that cannot allocate) against dspark_schedule with a caller workspace,
through the C ABI: two calls in a row, the second on a smaller problem (the
scratch keeps the first call's contents), at candidate counts on both sides of
the LDS-ordered path, with exact ties; and the size limit."""
from __future__ import annotations

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from draft_sampling_verification_markov_amd import dspark
    dspark.load()
    return dspark


def _tables(B, K, S, seed):
    # a cliff at a third of the candidates, and a linear table (the greedy test decides)
    n = B * K
    cliff = np.where(np.arange(B * (K + 1) + 1) <= B + n // 3, 1.0, 100.0).astype(np.float32)
    linear = (5.0 + 0.002 * np.arange(B * (K + 1) + 1)).astype(np.float32)
    return [cliff, linear]


def _run(dspark, B, K, S, T, noalloc):
    P = dspark.Problem.make(B, K, 1024, 16, 8)
    n_sched = torch.full((B,), -7, dtype=torch.int32, device="cuda")
    n_total = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    surv, T_d = torch.from_numpy(S).cuda(), torch.from_numpy(T).cuda()
    if noalloc:
        dspark.schedule_noalloc(P, surv, T_d, n_sched, n_total)
    else:
        ws = torch.empty(dspark.workspace_bytes(P), dtype=torch.uint8, device="cuda")
        dspark.schedule(P, surv, T_d, n_sched, n_total, ws)
    torch.cuda.synchronize()
    return n_sched.cpu().numpy(), int(n_total.item())


# (first call, second call with fewer candidates)
PAIRS = [((1024, 32, False), (256, 16, True)),     # 32768 (global ordering) then 4096 (LDS ordering)
         ((512, 16, True), (300, 7, False)),       # 8192 then 2100, ties in the first
         ((2048, 16, False), (1000, 9, True))]     # 32768 then 9000 (both global)


@pytest.mark.parametrize("first,second", PAIRS, ids=[f"{a[0]}x{a[1]}_then_{b[0]}x{b[1]}" for a, b in PAIRS])
def test_noalloc_matches_workspace_schedule(lib, first, second):
    dspark = lib
    for j, (B, K, ties) in enumerate((first, second)):
        S = synth.make_survivals(B, K, seed=40 + j, ties=ties)
        for T in _tables(B, K, S, seed=j):
            print(f"[gpu] schedule_noalloc B={B} K={K} ties={ties} call {j + 1}", flush=True)
            got = _run(dspark, B, K, S, T, noalloc=True)
            ref = _run(dspark, B, K, S, T, noalloc=False)
            np.testing.assert_array_equal(got[0], ref[0])
            assert got[1] == ref[1]


def test_noalloc_rejects_more_than_32768_candidates(lib):
    dspark = lib
    B, K = 1025, 32
    P = dspark.Problem.make(B, K, 1024, 16, 8)
    S = torch.ones((B, K), dtype=torch.float32, device="cuda")
    T = torch.ones(B * (K + 1) + 1, dtype=torch.float32, device="cuda")
    n_sched = torch.zeros(B, dtype=torch.int32, device="cuda")
    n_total = torch.zeros(1, dtype=torch.int32, device="cuda")
    with pytest.raises(dspark.DsparkError) as e:
        dspark.schedule_noalloc(P, S, T, n_sched, n_total)
    assert e.value.status == dspark.E_WORKSPACE
