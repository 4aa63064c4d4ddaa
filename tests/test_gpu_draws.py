"""The device's random draws against the oracle's (both written from the
published definition of Philox4x32-10 and the cycle's uniform and Gumbel
transforms), through dspark_probe_draws: the published known-answer vectors,
10^6 random counters word for word, and every one of the 2^24 uniform values
(all values of w >> 8) with its Gumbel within 2e-6 of the float64 one."""
from __future__ import annotations

import numpy as np
import pytest

from oracle import philox
from tests.test_oracle_philox import _kat_rows

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ds():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    from draft_sampling_verification_markov_amd import dspark
    dspark.load()
    return dspark


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint32).view(np.int32)).cuda()


def test_known_answer_vectors(ds):
    for ctr, key, expected in _kat_rows():
        seed = key[0] | (key[1] << 32)
        out = torch.empty((1, 4), dtype=torch.int32, device="cuda")
        ds.probe_draws(seed, ctr=_i32(np.array([ctr])), out_words=out)
        torch.cuda.synchronize()
        assert out.cpu().numpy().view(np.uint32)[0].tolist() == expected


def test_random_counters_word_for_word(ds):
    n = 1_000_000
    rng = np.random.default_rng(2026)
    ctr = rng.integers(0, 2**32, (n, 4), dtype=np.uint64).astype(np.uint32)
    seed = 0x0123456789ABCDEF
    out = torch.empty((n, 4), dtype=torch.int32, device="cuda")
    print(f"[gpu] philox on {n} counters", flush=True)
    ds.probe_draws(seed, ctr=_i32(ctr), out_words=out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    ref = philox.philox4x32_10(ctr, np.array([seed & 0xFFFFFFFF, seed >> 32], np.uint32))
    assert (got == ref).all(), int((got != ref).any(axis=1).sum())


def test_whole_uniform_grid_and_gumbels(ds):
    m = 1 << 24
    w = (np.arange(m, dtype=np.uint64) << np.uint64(8)).astype(np.uint32)
    w[1::2] |= np.uint32(0x5A)                       # the low 8 bits are ignored by both
    u = torch.empty(m, dtype=torch.float32, device="cuda")
    g = torch.empty(m, dtype=torch.float32, device="cuda")
    print(f"[gpu] uniform and Gumbel on all {m} values of w >> 8", flush=True)
    ds.probe_draws(0, w=_i32(w), uniform=u, gumbel=g)
    torch.cuda.synchronize()
    u_ref = philox.uniform(w)
    g_ref = philox.gumbel(u_ref)
    u_got = u.cpu().numpy().astype(np.float64)
    g_got = g.cpu().numpy().astype(np.float64)
    assert (u_got == u_ref).all()
    err = np.abs(g_got - g_ref)
    worst = float(err.max())
    print(f"[gpu]   Gumbel: worst |dG| {worst:.3e} at u = {u_ref[np.argmax(err)]:.9f}, "
          f"G range [{g_ref.min():.3f}, {g_ref.max():.3f}]", flush=True)
    assert worst <= 2e-6
