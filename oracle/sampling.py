"""Two-level Gumbel-max sampling over a vocabulary split into chunks of C = 128.

The method samples every token from a full-vocabulary softmax (DSpark page,
Method > Semi-autoregressive generation: the sequential stage samples each
draft position from base logits plus a transition bias; Overview/Background:
verification resamples from the target).  The pages do not fix the sampler.
The reading taken here is Gumbel-max (argmax of log-weight plus an independent
standard Gumbel is an exact draw from the normalised weights), applied in two
levels so that only one chunk needs per-element noise:

1. chunk log-mass  L_c = log sum_{v in c} w_v  over  c = [cC, min((c+1)C, V));
2. c* = argmax_c (L_c + G(chunk purpose, c));
3. v* = argmax_{v in c*} (log w_v + G(element purpose, v)).

P(c* = c) is proportional to e^{L_c} and P(v* = v | c*) to w_v / e^{L_c}, so v*
is an exact draw from w / sum(w).  For V <= C there is one chunk and the
scheme is plain Gumbel-max.  Ties go to the smallest chunk id, then the
smallest vocabulary id.  Entries with zero weight (log-weight -inf) never win.
"""
from __future__ import annotations

import numpy as np

from . import philox

C = 128


def n_chunks(V: int) -> int:
    return (V + C - 1) // C


def chunk_logsumexp(logw: np.ndarray) -> np.ndarray:
    """Per-chunk log-sum-exp along the last axis (ragged last chunk allowed); -inf for empty mass."""
    logw = np.asarray(logw, dtype=np.float64)
    V = logw.shape[-1]
    nc = n_chunks(V)
    pad = nc * C - V
    if pad:
        logw = np.concatenate([logw, np.full(logw.shape[:-1] + (pad,), -np.inf)], axis=-1)
    blocks = logw.reshape(logw.shape[:-1] + (nc, C))
    m = blocks.max(axis=-1)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        s = np.log(np.exp(blocks - safe_m[..., None]).sum(axis=-1))
    return np.where(np.isfinite(m), safe_m + s, -np.inf)


def logsumexp(x: np.ndarray, axis: int = -1) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    m = x.max(axis=axis, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    with np.errstate(divide="ignore"):
        return (m + np.log(np.exp(x - m).sum(axis=axis, keepdims=True))).squeeze(axis)


def _top2_gap(scores: np.ndarray) -> float:
    """Gap between the two largest finite scores (inf if fewer than two)."""
    finite = scores[np.isfinite(scores)]
    if finite.size < 2:
        return float("inf")
    top = np.partition(finite, finite.size - 2)[-2:]
    return float(top[1] - top[0])


def two_level_sample(logw: np.ndarray, seed: int, b, k, p_chunk: int, p_elem: int):
    """Draw v* from softmax(logw) row by row with the two-level scheme.

    logw is (V,) or (n, V); b and k are scalars or length-n arrays naming each
    row's draws.  Returns (v*, margin, c*) with the leading shape of logw.
    margin is the smaller of the top-two gaps of the chunk scores and of the
    element scores inside c* (in nats): a decision taken at lower precision
    can differ only where it is small.
    """
    logw = np.asarray(logw, dtype=np.float64)
    single = logw.ndim == 1
    logw = np.atleast_2d(logw)
    n, V = logw.shape
    nc = n_chunks(V)
    b = np.broadcast_to(np.asarray(b, np.int64), (n,))
    k = np.broadcast_to(np.asarray(k, np.int64), (n,))
    L = chunk_logsumexp(logw)                                         # (n, nc)
    G = philox.gumbels(seed, b[:, None], k[:, None], p_chunk, np.arange(nc)[None, :])
    sc = np.where(np.isfinite(L), L + G, -np.inf)
    cstar = np.argmax(sc, axis=1)
    # the C vocabulary ids of each row's winning chunk (ids past V in a ragged chunk are masked)
    ids = cstar[:, None] * C + np.arange(C)[None, :]
    inside = ids < V
    ids_c = np.minimum(ids, V - 1)
    lw = np.where(inside, np.take_along_axis(logw, ids_c, axis=1), -np.inf)
    ge = philox.gumbels(seed, b[:, None], k[:, None], p_elem, ids_c)
    se = np.where(np.isfinite(lw), lw + ge, -np.inf)
    v = ids[np.arange(n), np.argmax(se, axis=1)]
    margin = np.array([min(_top2_gap(sc[i]), _top2_gap(se[i])) for i in range(n)])
    if single:
        return int(v[0]), float(margin[0]), int(cstar[0])
    return v, margin, cstar


def flat_sample(logw: np.ndarray, seed: int, b: int, k: int, p_elem: int) -> int:
    """One-level Gumbel-max over the whole vocabulary (reference for tests)."""
    logw = np.asarray(logw, dtype=np.float64)
    s = logw + philox.gumbels(seed, b, k, p_elem, np.arange(logw.shape[-1]))
    return int(np.argmax(np.where(np.isfinite(logw), s, -np.inf)))
