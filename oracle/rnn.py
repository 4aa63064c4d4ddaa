"""RNN head: the gated recurrent alternative to the Markov head.

Follows the DSpark page, Method > Semi-autoregressive generation (the second
sequential block): the RNN head keeps a recurrent state that accumulates the
whole prefix drafted so far in the block, and at every step applies a gated
update that combines the current state, the embedding of the previous token
and the backbone hidden state of the position.  Main results: it adds a small
gain over the Markov head at long draft lengths.

Readings (the pages give no gate equations):

* the gated update is a GRU cell in the form common libraries implement
  (torch.nn.GRUCell): with input u_k = [h_k; E[x_{k-1}]] (d + r) and state
  s_{k-1} (r),
      a = W_ih u_k + b_ih,  c = W_hh s_{k-1} + b_hh    (3r each, gate order reset, update, new)
      rho = sigmoid(a_r + c_r),  z = sigmoid(a_z + c_z),  n = tanh(a_n + rho * c_n)
      s_k = (1 - z) * n + z * s_{k-1},   s_0 = 0;
* the state has the Markov rank r and takes the place of E[x_{k-1}] in the
  logit projection: ell_k = (Z_k + code(s_k) . Wt^T) / T_s, where code() rounds
  to bfloat16 (nearest, ties to even), the precision of the projection's
  operands; the confidence head keeps its inputs [h_k; E[x_{k-1}]];
* sampling, verification and randomness are those of the Markov head, with
  the projection operand of position k being code(s_k) instead of E[x_{k-1}].

Arithmetic is float64 (the rounding to bfloat16 is the only narrowing).
"""
from __future__ import annotations

import numpy as np

from . import philox
from .conf import sigmoid
from .io import f64
from .sampling import logsumexp, two_level_sample


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (8 significant bits, ties to even) of float64 x, as float64.
    Normal range only (the states are in (-1, 1) and far from the subnormals)."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                    # x = m * 2^e, 0.5 <= |m| < 1
    return np.ldexp(np.rint(m * 256.0), e - 8)


def gru_cell(s: np.ndarray, u: np.ndarray, W_ih, b_ih, W_hh, b_hh) -> np.ndarray:
    """One gated update; s (n, r), u (n, d + r); weights (3r, d + r), (3r,), (3r, r), (3r,)."""
    r = s.shape[-1]
    a = u @ W_ih.T + b_ih
    c = s @ W_hh.T + b_hh
    rho = sigmoid(a[:, :r] + c[:, :r])
    z = sigmoid(a[:, r:2 * r] + c[:, r:2 * r])
    n = np.tanh(a[:, 2 * r:] + rho * c[:, 2 * r:])
    return (1.0 - z) * n + z * s


def rnn_draft(Z, E, Wt, h, anchor, W_ih, b_ih, W_hh, b_hh, T_s: float, seed: int,
              teacher_x=None, requests=None) -> dict:
    """All K steps of the RNN head for the listed requests (default: all).

    With ``teacher_x`` the previous token of step k > 1 is teacher_x[b, k-2].
    Returns x, logq, lse, margin (n, K) and state (n, K, r): s_k in float64.
    """
    B, K, V = Z.shape
    reqs = np.arange(B) if requests is None else np.asarray(requests, np.int64)
    E64, W64 = f64(E), f64(Wt)
    Wih, Whh = f64(W_ih), f64(W_hh)
    bih, bhh = np.asarray(b_ih, np.float64), np.asarray(b_hh, np.float64)
    r = E64.shape[1]
    n = reqs.size
    out = {key: np.empty((n, K), dt) for key, dt in
           (("x", np.int64), ("logq", np.float64), ("lse", np.float64), ("margin", np.float64))}
    out["state"] = np.empty((n, K, r))
    s = np.zeros((n, r))
    prev = np.asarray(anchor, np.int64)[reqs]
    for k in range(1, K + 1):
        if teacher_x is not None and k > 1:
            prev = np.asarray(teacher_x, np.int64)[reqs, k - 2]
        u = np.concatenate([f64(h[reqs, k - 1]), E64[prev]], axis=1)
        s = gru_cell(s, u, Wih, bih, Whh, bhh)
        out["state"][:, k - 1] = s
        ell = (f64(Z[reqs, k - 1]) + bf16_round(s) @ W64.T) / float(T_s)
        lse = logsumexp(ell, axis=-1)
        x, margin, _ = two_level_sample(ell, seed, reqs, k, philox.P_DRAFT_CHUNK, philox.P_DRAFT_ELEM)
        x = np.atleast_1d(x)
        out["x"][:, k - 1] = x
        out["logq"][:, k - 1] = ell[np.arange(n), x] - lse
        out["lse"][:, k - 1] = lse
        out["margin"][:, k - 1] = margin
        prev = x
    return out
