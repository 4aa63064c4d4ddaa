"""Pins of the oracle's Markov-head draft step."""
import numpy as np
import scipy.special

from oracle import draft as odraft
from oracle import philox, sampling
from tests.test_oracle_sampling import _chi2_pvalue


def test_zero_projection_gives_plain_softmax():
    # Wt = 0: no transition bias, q_k = softmax(Z_k / T_s)
    rng = np.random.default_rng(0)
    B, K, V, r = 3, 4, 1000, 16
    Z = rng.normal(0, 3, (B, K, V)).astype(np.float32)
    E = rng.normal(0, 1, (V, r)).astype(np.float32)
    Wt = np.zeros((V, r), np.float32)
    T_s = 0.7
    out = odraft.draft(Z, E, Wt, np.array([1, 2, 3]), T_s, seed=9)
    for b in range(B):
        for k in range(K):
            ls = scipy.special.log_softmax(Z[b, k].astype(np.float64) / T_s)
            assert abs(out["logq"][b, k] - ls[out["x"][b, k]]) < 1e-12
            assert abs(out["lse"][b, k] - scipy.special.logsumexp(Z[b, k].astype(np.float64) / T_s)) < 1e-12


def _permutation_chain(V=64, strength=60.0):
    """E = identity, Wt[v, j] = strength iff v == f(j): the bias row of prev is strength at f(prev)."""
    rng = np.random.default_rng(5)
    f = rng.permutation(V)
    while (f[f] == np.arange(V)).any():       # f differs from its inverse everywhere
        f = rng.permutation(V)
    E = np.eye(V, dtype=np.float32)
    Wt = np.zeros((V, V), np.float32)
    Wt[f, np.arange(V)] = strength
    return f, E, Wt


def test_markov_bias_follows_the_previous_token():
    # the transition bias dominates, so each token is f(previous token) and x_0 is the anchor
    V, K = 64, 6
    f, E, Wt = _permutation_chain(V)
    Z = np.random.default_rng(1).normal(0, 1, (2, K, V)).astype(np.float32)
    anchor = np.array([7, 40])
    out = odraft.draft(Z, E, Wt, anchor, 2.0, seed=3)
    for b in range(2):
        prev = anchor[b]
        for k in range(K):
            assert out["x"][b, k] == f[prev]
            prev = f[prev]


def test_low_rank_bias_shifts_the_draw_law():
    # with a bias of O(1) nats the law of x_1 is softmax((Z + bias) / T_s); the
    # bias row is E[anchor] . Wt^T, written here via one-hot rows of E
    rng = np.random.default_rng(2)
    V, r, T_s = 300, 3, 1.3
    E = np.zeros((V, r), np.float32)
    E[11] = [1.0, 0.0, 0.0]
    Wt = rng.normal(0, 2, (V, r)).astype(np.float32)
    z = rng.normal(0, 1, V).astype(np.float32)
    probs = scipy.special.softmax((z.astype(np.float64) + Wt[:, 0].astype(np.float64)) / T_s)
    n = 20000
    Zrows = np.tile(z, (n, 1))
    st = odraft.draft_step(Zrows, E, Wt, np.full(n, 11), T_s, 44, np.arange(n), 1)
    counts = np.bincount(st["x"], minlength=V).astype(float)
    assert _chi2_pvalue(counts, probs) > 1e-3
    # and it is not the unbiased law
    assert _chi2_pvalue(counts, scipy.special.softmax(z.astype(np.float64) / T_s)) < 1e-6


def test_teacher_forcing_with_own_tokens_reproduces_the_run():
    rng = np.random.default_rng(3)
    B, K, V, r = 2, 5, 500, 8
    Z = rng.normal(0, 3, (B, K, V)).astype(np.float32)
    E = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    Wt = rng.normal(0, 0.5, (V, r)).astype(np.float32)
    anchor = np.array([0, 499])
    a = odraft.draft(Z, E, Wt, anchor, 1.0, 8)
    b = odraft.draft(Z, E, Wt, anchor, 1.0, 8, teacher_x=a["x"])
    for key in ("x", "logq", "lse"):
        np.testing.assert_array_equal(a[key], b[key])
    # a request's steps use only its own draws: running a subset gives the same rows
    c = odraft.draft(Z, E, Wt, anchor, 1.0, 8, requests=[1])
    np.testing.assert_array_equal(c["x"][0], a["x"][1])


def test_draft_uses_position_keyed_draws():
    # position k's draw uses (b, k) streams: with a flat row the token equals the
    # argmax of the two-level scores computed from those streams alone
    V = 256
    Z = np.zeros((1, 2, V), np.float32)
    E = np.zeros((V, 4), np.float32)
    Wt = np.zeros((V, 4), np.float32)
    out = odraft.draft(Z, E, Wt, np.array([0]), 1.0, seed=12)
    for k in (1, 2):
        gc = philox.gumbels(12, 0, k, philox.P_DRAFT_CHUNK, np.arange(2))
        c = int(np.argmax(gc + np.log(128.0)))
        ge = philox.gumbels(12, 0, k, philox.P_DRAFT_ELEM, np.arange(c * 128, c * 128 + 128))
        assert out["x"][0, k - 1] == c * 128 + int(np.argmax(ge))
    assert sampling.n_chunks(V) == 2
