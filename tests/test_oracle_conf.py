"""Pins of the oracle's confidence head, STS and survival."""
import math

import numpy as np
import scipy.special

from oracle import conf


def test_sigmoid_matches_library_without_overflow():
    t = np.concatenate([np.linspace(-50, 50, 1001), [-800.0, -745.0, 745.0, 800.0]])
    np.testing.assert_allclose(conf.sigmoid(t), scipy.special.expit(t), rtol=1e-15, atol=1e-300)


def test_confidence_reads_the_previous_token_embedding():
    # h = 0, w_h arbitrary: z_k = w_e . E[x_{k-1}] + b_c; with E[v, 0] = v / 64 and
    # w_e = e_0, c_k = sigmoid((x_{k-1} / 64 + b_c) / tau_k) in closed form
    B, K, d, r, V = 2, 4, 8, 4, 256
    h = np.zeros((B, K, d), np.float32)
    E = np.zeros((V, r), np.float32)
    E[:, 0] = np.arange(V) / 64.0
    w_c = np.concatenate([np.random.default_rng(0).normal(0, 1, d), [1.0, 0, 0, 0]]).astype(np.float32)
    b_c = 0.25
    tau = np.array([0.5, 1.0, 2.0, 4.0], np.float32)
    anchor = np.array([3, 200])
    x = np.array([[10, 20, 30, 40], [100, 0, 255, 1]])
    c, S = conf.confidence(h, E, w_c, b_c, tau, anchor, x)
    for b in range(B):
        prevs = [anchor[b]] + list(x[b, :K - 1])
        for k in range(K):
            zz = (prevs[k] / 64.0 + b_c) / float(tau[k])
            assert abs(c[b, k] - 1.0 / (1.0 + math.exp(-zz))) < 1e-15


def test_confidence_hidden_part():
    # w_e = 0: z_k = w_h . h_k + b_c
    B, K, d, r, V = 1, 2, 16, 4, 8
    h = np.zeros((B, K, d), np.float32)
    h[0, 0, 3] = 2.0
    h[0, 1, 15] = -1.5
    w_c = np.zeros(d + r, np.float32)
    w_c[3] = 0.75
    w_c[15] = 2.0
    c, S = conf.confidence(h, np.ones((V, r), np.float32), w_c, -0.5, np.array([1.0, 1.0], np.float32),
                           np.array([0]), np.array([[1, 2]]))
    assert abs(c[0, 0] - scipy.special.expit(2.0 * 0.75 - 0.5)) < 1e-15
    assert abs(c[0, 1] - scipy.special.expit(-1.5 * 2.0 - 0.5)) < 1e-15


def test_survival_is_a_nonincreasing_running_product():
    rng = np.random.default_rng(1)
    B, K, d, r, V = 5, 16, 32, 8, 100
    h = rng.normal(0, 1, (B, K, d)).astype(np.float32)
    E = rng.normal(0, 1, (V, r)).astype(np.float32)
    w_c = rng.normal(0, 0.5, d + r).astype(np.float32)
    tau = rng.uniform(0.8, 2.0, K).astype(np.float32)
    x = rng.integers(0, V, (B, K))
    c, S = conf.confidence(h, E, w_c, 0.1, tau, rng.integers(0, V, B), x)
    assert ((c > 0) & (c < 1)).all()
    assert (S[:, 0] == c[:, 0]).all()
    assert (np.diff(S, axis=1) <= 0).all()
    np.testing.assert_allclose(S[:, 1:] / S[:, :-1], c[:, 1:], rtol=1e-14)


def test_temperature_scaling_preserves_order():
    z = np.sort(np.random.default_rng(2).normal(0, 3, 200))
    for tau in (0.3, 0.8, 1.0, 2.0, 7.5):
        assert (np.diff(conf.sigmoid(z / tau)) >= 0).all()
    # and tau = 1 is the plain sigmoid
    np.testing.assert_allclose(conf.sigmoid(z / 1.0), scipy.special.expit(z), rtol=1e-15)
