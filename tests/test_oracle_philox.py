"""Pins of the oracle's Philox4x32-10, uniform and Gumbel transforms."""
import math
import os

import mpmath
import numpy as np
import pytest

from oracle import philox

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "philox_kat.txt")


def _kat_rows():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            vals = [int(t, 16) for t in line.split()]
            rows.append((vals[0:4], vals[4:6], vals[6:10]))
    return rows


@pytest.mark.parametrize("ctr,key,expected", _kat_rows())
def test_philox_known_answers(ctr, key, expected):
    out = philox.philox4x32_10(np.array(ctr, np.uint32), np.array(key, np.uint32))
    assert [int(w) for w in out] == expected


def test_philox_vectorised_matches_scalar_calls():
    rng = np.random.default_rng(7)
    ctr = rng.integers(0, 2**32, (64, 4), dtype=np.uint64).astype(np.uint32)
    key = np.array([0x12345678, 0x9ABCDEF0], np.uint32)
    batch = philox.philox4x32_10(ctr, key)
    for i in range(64):
        assert (philox.philox4x32_10(ctr[i], key) == batch[i]).all()


def test_uniform_grid_is_exact_odd_multiples():
    # every possible 24-bit value of (w >> 8): the map is exact, odd, inside (0, 1)
    w = (np.arange(2**24, dtype=np.uint64) << np.uint64(8)).astype(np.uint32)
    u = philox.uniform(w)
    assert u.min() == 2.0**-24 and u.max() == 1.0 - 2.0**-24
    assert (u.astype(np.float32).astype(np.float64) == u).all()
    m = u * 2.0**24
    assert (m == np.round(m)).all() and (np.round(m).astype(np.int64) % 2 == 1).all()
    # the low 8 bits of the word are ignored
    assert philox.uniform(np.uint32(0xFFFFFF00)) == philox.uniform(np.uint32(0xFFFFFFFF))


def test_gumbel_against_high_precision():
    us = [2.0**-24, 3 * 2.0**-24, 0.25, 0.5 - 2.0**-24, 0.5, 0.5 + 2.0**-24, 0.9, 0.999,
          1 - 2.0**-20, 1 - 3 * 2.0**-24, 1 - 2.0**-24]
    mpmath.mp.dps = 50
    for u in us:
        ref = -mpmath.log(-mpmath.log(mpmath.mpf(u)))
        got = float(philox.gumbel(u))
        assert abs(got - float(ref)) <= 4e-16 * max(1.0, abs(float(ref))), (u, got, ref)


def test_gumbel_moments_closed_form():
    # standard Gumbel: mean = Euler-Mascheroni constant, variance = pi^2 / 6
    g = philox.gumbels(2024, np.arange(1000)[:, None], 3, philox.P_DRAFT_CHUNK, np.arange(1000)[None, :]).ravel()
    n = g.size
    assert abs(g.mean() - 0.5772156649015329) < 5 * math.sqrt(math.pi**2 / 6 / n)
    assert abs(g.var() - math.pi**2 / 6) < 0.02


def test_uniform_draws_are_uniform_and_keyed():
    u = philox.uniforms(5, np.arange(512)[:, None], 1, philox.P_ACCEPT, np.arange(512)[None, :]).ravel()
    hist, _ = np.histogram(u, bins=16, range=(0, 1))
    expected = u.size / 16
    chi2 = ((hist - expected) ** 2 / expected).sum()
    assert chi2 < 45  # 15 dof, p ~ 1e-4
    # different purposes, positions, requests and seeds give different streams
    base = philox.words(1, 3, 2, philox.P_DRAFT_ELEM, np.arange(64))
    for other in (philox.words(1, 3, 2, philox.P_RESID_ELEM, np.arange(64)),
                  philox.words(1, 4, 2, philox.P_DRAFT_ELEM, np.arange(64)),
                  philox.words(1, 3, 3, philox.P_DRAFT_ELEM, np.arange(64)),
                  philox.words(2, 3, 2, philox.P_DRAFT_ELEM, np.arange(64)),
                  philox.words(1 + (1 << 32), 3, 2, philox.P_DRAFT_ELEM, np.arange(64))):
        assert (base != other).mean() > 0.9
