"""Lossless rejection-sampling verification of the scheduled draft prefix.

Follows the DSpark page, Overview and Background: the target checks the draft
tokens left to right in one pass, keeps the longest prefix consistent with its
own distribution, discards everything after the first rejection, and the
rejection-sampling rule keeps the output distributed exactly as the target.

The rule written out is the published speculative-sampling one (Leviathan,
Kalman, Matias 2023; Chen et al. 2023):

* position k (1 <= k <= n_b) with draft token x_k is accepted with probability
  min(1, p_k(x_k) / q_k(x_k)): accept iff u_k <= that value, u_k the accept
  draw (purpose 3) at (b, k);
* at the first rejection k*, the emitted token is drawn from the normalised
  residual max(0, p_k* - q_k*) (two-level Gumbel-max over log of the residual,
  purposes 4/5 at position k*), and a_b = k* - 1 draft tokens are kept;
* if all n_b positions are accepted, a bonus token is drawn from p at
  position n_b + 1 (purposes 6/7), and a_b = n_b;
* emitted: x_1 .. x_{a_b}, then the drawn token, which is the next anchor.

Readings: p_k = softmax(Zt[b, k] / T_s) (the sampling temperature applies to
the target too); q_k is the draft distribution recomputed from the prefix:
the Markov head's (``draft``) or, when the projection operands ``vec`` of the
positions are given, the one those operands define (the RNN head, ``rnn``); if the residual mass is exactly zero (possible
only through rounding) the token is drawn from p_k* with purposes 4/5.
``accept_probability`` and ``residual_weights`` use plain arithmetic so the
enumeration tests can run them on exact fractions.
"""
from __future__ import annotations

import math

import numpy as np

from . import philox
from .draft import markov_logits
from .io import f64
from .sampling import logsumexp, two_level_sample


def accept_probability(p_x, q_x):
    """min(1, p(x) / q(x))."""
    ratio = p_x / q_x
    return 1 if ratio >= 1 else ratio


def residual_weights(p, q):
    """Unnormalised residual max(0, p - q), elementwise (arrays of floats or of Fractions)."""
    d = np.asarray(p) - np.asarray(q)
    return np.where(d > 0, d, 0 * d)


def verify_request(b: int, n_b: int, x_row, Zt_b, Z_b, E64, W64, anchor_b: int, T_s: float, seed: int,
                   vec_b=None):
    """Verify request b's first n_b draft tokens.  Zt_b: (K+1, V) target rows; Z_b: (K, V) base rows;
    vec_b: (K, r) projection operands of the positions (None: E of the previous token)."""
    K = len(x_row)
    x_row = [int(t) for t in x_row]
    logp = np.full(K, np.nan)
    lp_rows = {}
    for k in range(1, n_b + 1):
        lp = f64(Zt_b[k - 1]) / float(T_s)
        lp_rows[k] = lp
        logp[k - 1] = lp[x_row[k - 1]] - logsumexp(lp)
    accept_margin = math.inf
    for k in range(1, n_b + 1):
        if vec_b is None:
            prev = int(anchor_b) if k == 1 else x_row[k - 2]
            ell = markov_logits(Z_b[k - 1][None, :], E64, W64, prev, T_s)[0]
        else:
            ell = (f64(Z_b[k - 1]) + np.asarray(vec_b[k - 1], np.float64) @ W64.T) / float(T_s)
        lse_q = logsumexp(ell)
        logq_k = ell[x_row[k - 1]] - lse_q
        a = accept_probability(math.exp(logp[k - 1]), math.exp(logq_k))
        u = float(philox.uniforms(seed, b, k, philox.P_ACCEPT, 0))
        accept_margin = min(accept_margin, abs(u - a))
        if u <= a:
            continue
        lp = lp_rows[k]
        p = np.exp(lp - logsumexp(lp))
        q = np.exp(ell - lse_q)
        r = residual_weights(p, q)
        mass = float(r.sum())
        if mass > 0:
            with np.errstate(divide="ignore"):
                logw = np.log(r)
            kind = "resid"
        else:
            logw = lp
            kind = "resid_p"
        y, tmargin, _ = two_level_sample(logw, seed, b, k, philox.P_RESID_CHUNK, philox.P_RESID_ELEM)
        return {"tokens": x_row[:k - 1] + [y], "accepted": k - 1, "y": y, "logp": logp, "mass": mass,
                "kind": kind, "k_star": k, "accept_margin": accept_margin, "token_margin": tmargin}
    lp = f64(Zt_b[n_b]) / float(T_s)
    y, tmargin, _ = two_level_sample(lp, seed, b, n_b + 1, philox.P_BONUS_CHUNK, philox.P_BONUS_ELEM)
    return {"tokens": x_row[:n_b] + [y], "accepted": n_b, "y": y, "logp": logp, "mass": float("nan"),
            "kind": "bonus", "k_star": 0, "accept_margin": accept_margin, "token_margin": tmargin}


def verify(Zt, Z, E, Wt, anchor, x, n, T_s: float, seed: int, requests=None, vec=None):
    """Verify every listed request (default: all).  Returns a list of per-request dicts.
    vec: (B, K, r) projection operands (RNN head), indexed by request like Z."""
    B = Z.shape[0]
    reqs = range(B) if requests is None else [int(b) for b in requests]
    E64, W64 = f64(E), f64(Wt)
    return [verify_request(b, int(n[b]), x[b], Zt[b], Z[b], E64, W64, int(anchor[b]), T_s, seed,
                           None if vec is None else vec[b]) for b in reqs]
