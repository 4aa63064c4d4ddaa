"""Markov-head draft sampling (the sequential stage of semi-autoregressive drafting).

Follows the DSpark page, Method > Semi-autoregressive generation:

* the parallel backbone yields one base-logit row per draft position, and the
  anchor token is itself the first prediction position, so position k = 1 is
  conditioned on the anchor (x_0 = anchor) and row k of Z predicts x_k;
* the sequential stage adds a prefix-dependent transition bias to the base
  logits; the Markov head makes it depend on the immediately preceding token
  only, through a rank-r factorisation of the V x V transition matrix into an
  embedding lookup E[prev] (V x r table) and a logit projection (stored
  vocabulary-major as Wt, V x r):  bias[v] = sum_j E[prev, j] * Wt[v, j];
* tokens are sampled one position after another, each conditioned on the one
  just sampled.

Readings: the bias is added to the raw base logits before the sampling
temperature T_s, with no extra scale, and q = softmax((Z + bias) / T_s).
Draws: two-level Gumbel-max (see ``sampling``) with chunk purpose 1 and element
purpose 2 at (request b, position k).
"""
from __future__ import annotations

import numpy as np

from . import philox
from .io import f64
from .sampling import logsumexp, two_level_sample


def markov_logits(Z_rows: np.ndarray, E: np.ndarray, Wt: np.ndarray, prev, T_s: float) -> np.ndarray:
    """ell[i, v] = (Z_rows[i, v] + E[prev_i] . Wt[v]) / T_s in float64.  Z_rows: (n, V)."""
    Z64 = f64(Z_rows)
    E64 = E if E.dtype == np.float64 else f64(E)
    W64 = Wt if Wt.dtype == np.float64 else f64(Wt)
    prev = np.atleast_1d(np.asarray(prev, np.int64))
    bias = E64[prev] @ W64.T
    return (np.atleast_2d(Z64) + bias) / float(T_s)


def draft_step(Z_rows, E, Wt, prev, T_s: float, seed: int, b, k):
    """One sequential step for the rows Z_rows (n, V) of requests b at position k.

    Returns dict with x (sampled token), logq (log q_k(x)), lse (log-partition of
    q_k in the units of ell) and margin (decision margin in nats).
    """
    ell = markov_logits(Z_rows, E, Wt, prev, T_s)
    lse = logsumexp(ell, axis=-1)
    x, margin, _ = two_level_sample(ell, seed, b, k, philox.P_DRAFT_CHUNK, philox.P_DRAFT_ELEM)
    x = np.atleast_1d(x)
    logq = ell[np.arange(ell.shape[0]), x] - lse
    return {"x": x, "logq": logq, "lse": lse, "margin": np.atleast_1d(margin)}


def draft(Z: np.ndarray, E: np.ndarray, Wt: np.ndarray, anchor: np.ndarray, T_s: float, seed: int,
          teacher_x: np.ndarray | None = None, requests=None):
    """All K sequential steps for the requests listed (default: all).

    With ``teacher_x`` (B x K tokens) the previous token of step k is
    teacher_x[b, k-2] instead of the token the oracle sampled itself, so a
    step can be checked on its own given another implementation's prefix.
    Returns x, logq, lse, margin as (n_requests, K) arrays.
    """
    B, K, V = Z.shape
    reqs = np.arange(B) if requests is None else np.asarray(requests, np.int64)
    E64, W64 = f64(E), f64(Wt)
    n = reqs.size
    out = {key: np.empty((n, K), dt) for key, dt in
           (("x", np.int64), ("logq", np.float64), ("lse", np.float64), ("margin", np.float64))}
    prev = np.asarray(anchor, np.int64)[reqs]
    for k in range(1, K + 1):
        if teacher_x is not None and k > 1:
            prev = np.asarray(teacher_x, np.int64)[reqs, k - 2]
        st = draft_step(Z[reqs, k - 1], E64, W64, prev, T_s, seed, reqs, k)
        for key in out:
            out[key][:, k - 1] = st[key]
        prev = st["x"]
    return out
