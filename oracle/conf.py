"""Confidence head, Sequential Temperature Scaling and prefix survival.

Follows the DSpark page, Method > Confidence-scheduled verification:

* the confidence head outputs, per draft position, a value in (0, 1): the
  probability that the position passes verification given that every earlier
  position did; its inputs are the backbone hidden state of the position and
  the Markov embedding (the row of E) of the immediately preceding draft
  token; it is a light linear projection followed by a sigmoid;
* STS calibrates it with one temperature per position; temperature scaling
  keeps the order of the confidences;
* the survival of a position is the cumulative product of the per-position
  confidences up to it, and is therefore non-increasing along the block.

Readings: z = w_h . h_k + w_e . E[x_{k-1}] + b_c with w_c = [w_h (d); w_e (r)],
c_k = sigmoid(z / tau_k) (the temperature divides the logit), S_k = S_{k-1} c_k
with S_0 = 1, and x_0 = the anchor.
"""
from __future__ import annotations

import numpy as np

from .io import f64


def sigmoid(t: np.ndarray) -> np.ndarray:
    """1 / (1 + e^-t), evaluated without overflow for either sign of t."""
    t = np.asarray(t, dtype=np.float64)
    e = np.exp(-np.abs(t))
    return np.where(t >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def survival(c_row):
    """Prefix survival: running product of the confidences along a block (any number type)."""
    out, s = [], 1
    for c in c_row:
        s = s * c
        out.append(s)
    return out


def confidence(h: np.ndarray, E: np.ndarray, w_c: np.ndarray, b_c: float, tau: np.ndarray,
               anchor: np.ndarray, x: np.ndarray):
    """c[b, k] and S[b, k] for the draft tokens x (B x K); h is (B, K, d)."""
    h64 = f64(h)
    B, K, d = h64.shape
    E64 = f64(E)
    w = np.asarray(w_c, np.float64)
    w_h, w_e = w[:d], w[d:]
    prev = np.concatenate([np.asarray(anchor, np.int64)[:, None], np.asarray(x, np.int64)[:, :K - 1]], axis=1)
    z = h64 @ w_h + E64[prev] @ w_e + float(b_c)
    c = sigmoid(z / np.asarray(tau, np.float64)[None, :])
    S = np.array([survival(row) for row in c], dtype=np.float64).reshape(B, K)
    return c, S
