"""Pins of the oracle's two-level Gumbel-max sampler."""
import numpy as np
import pytest
import scipy.special
import scipy.stats

from oracle import philox, sampling


def _chi2_pvalue(counts, probs, min_expected=5.0):
    """Chi-square goodness of fit, pooling cells with a small expectation."""
    n = counts.sum()
    exp = probs * n
    order = np.argsort(exp)
    obs_c, exp_c, acc_o, acc_e = [], [], 0.0, 0.0
    for i in order:
        acc_o += counts[i]
        acc_e += exp[i]
        if acc_e >= min_expected:
            obs_c.append(acc_o)
            exp_c.append(acc_e)
            acc_o = acc_e = 0.0
    if acc_e > 0:
        obs_c[-1] += acc_o
        exp_c[-1] += acc_e
    obs_c, exp_c = np.array(obs_c), np.array(exp_c)
    stat = ((obs_c - exp_c) ** 2 / exp_c).sum()
    return scipy.stats.chi2.sf(stat, len(obs_c) - 1)


@pytest.mark.parametrize("V", [100, 128, 300, 1000])
def test_chunk_logsumexp_matches_library(V):
    x = np.random.default_rng(V).normal(0, 3, (3, V))
    x[1, 5] = -np.inf
    got = sampling.chunk_logsumexp(x)
    for c in range(sampling.n_chunks(V)):
        lo, hi = c * 128, min((c + 1) * 128, V)
        np.testing.assert_allclose(got[:, c], scipy.special.logsumexp(x[:, lo:hi], axis=1), rtol=1e-13)


def test_chunk_logsumexp_empty_chunk_is_minus_inf():
    x = np.zeros(300)
    x[128:256] = -np.inf
    got = sampling.chunk_logsumexp(x)
    assert got[1] == -np.inf and np.isfinite(got[0]) and np.isfinite(got[2])


@pytest.mark.parametrize("V,T", [(8, 1.0), (300, 1.0), (1000, 0.5)])
def test_two_level_sampler_matches_softmax(V, T):
    # chi-square of 20000 draws against softmax: an exact sampler passes
    rng = np.random.default_rng(V)
    logits = rng.normal(0, 2, V) / T
    probs = scipy.special.softmax(logits)
    n, blk = 20000, 5000
    # independent draws: one row per request index b (each b keys its own stream)
    draws = np.concatenate([sampling.two_level_sample(np.tile(logits, (blk, 1)), 77, np.arange(i, i + blk), 1,
                                                      philox.P_DRAFT_CHUNK, philox.P_DRAFT_ELEM)[0]
                            for i in range(0, n, blk)])
    counts = np.bincount(draws, minlength=V).astype(float)
    assert _chi2_pvalue(counts, probs) > 1e-3


def test_two_level_sampler_batched_rows_match_single_rows():
    rng = np.random.default_rng(1)
    logits = rng.normal(0, 3, (5, 700))
    b = np.array([0, 3, 3, 9, 1])
    k = np.array([1, 1, 2, 4, 7])
    v, m, c = sampling.two_level_sample(logits, 11, b, k, 1, 2)
    for i in range(5):
        vi, mi, ci = sampling.two_level_sample(logits[i], 11, int(b[i]), int(k[i]), 1, 2)
        assert (vi, ci) == (v[i], c[i]) and mi == m[i]


def test_single_chunk_reduces_to_flat_gumbel_max():
    # V <= C: the chunk level is trivial and the draw is plain Gumbel-max
    logits = np.random.default_rng(3).normal(0, 1, 100)
    for seed in range(200):
        a = sampling.two_level_sample(logits, seed, 2, 5, philox.P_BONUS_CHUNK, philox.P_BONUS_ELEM)[0]
        assert a == sampling.flat_sample(logits, seed, 2, 5, philox.P_BONUS_ELEM)


def test_zero_temperature_limit_is_argmax():
    logits = np.random.default_rng(4).normal(0, 1, 1000)
    for seed in range(20):
        v = sampling.two_level_sample(logits * 1e6, seed, 0, 1, 1, 2)[0]
        assert v == int(np.argmax(logits))


def test_zero_weights_never_drawn():
    logw = np.full(600, -np.inf)
    support = [3, 130, 131, 599]
    logw[support] = [0.0, 1.0, -1.0, 0.5]
    seen = {sampling.two_level_sample(logw, s, 0, 1, 4, 5)[0] for s in range(400)}
    assert seen == set(support)
