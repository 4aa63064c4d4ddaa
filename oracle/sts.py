"""Fitting the Sequential Temperature Scaling temperatures.

Follows the DSpark page, Method > Confidence-scheduled verification (the STS
paragraph), with the calibration figures of Main results:

* each confidence models a conditional acceptance probability, so by the chain
  rule the probability that a whole prefix is accepted is the running product
  of the confidences (the survival);
* STS calibrates that joint prefix probability from left to right: at each
  position the temperatures of the earlier positions stay fixed and a
  one-dimensional grid search picks the temperature that minimises the
  Expected Calibration Error (ECE);
* temperature scaling keeps the order of the confidences.

Readings (the pages fix none of these):

* the raw confidence c of a position is the head's output at temperature 1;
  a temperature tau acts on its logit: sigmoid(logit(c) / tau), with
  logit(c) = ln c - ln(1 - c);
* the quantity calibrated at position k is the survival
  S_k = S_{k-1} * sigmoid(logit(c_k) / tau_k), with the fitted temperatures
  of positions < k in S_{k-1}; its label is "the first k drafted positions
  were all accepted", i.e. accepted length >= k;
* a sample enters position k only when position k was verified
  (k <= verified length).  A rejection inside a shorter verified prefix also
  fixes the label of position k (to 0), but keeping those samples while the
  accepted ones of the same verified length stay unknown would select on the
  outcome and bias every later position towards 0; the verified length is
  chosen before verification, so selecting on it keeps the labels unbiased;
* ECE uses equal-width bins on [0, 1] (15 by default), bin = min(floor(p * n_bins), n_bins - 1),
  ECE = sum over bins of |sum of predictions - number of accepted| / (number of observed samples);
* the grid is supplied by the caller; entries that are not finite and positive
  are never chosen; ties go to the smallest grid index;
* with no observed sample at a position, or no usable grid entry, the
  position keeps tau = 1 (index -1) and its fitted ECE is NaN (the raw one
  too when nothing is observed).

Arithmetic is float64.
"""
from __future__ import annotations

import numpy as np

from .conf import sigmoid


def logit(c: np.ndarray) -> np.ndarray:
    """ln c - ln(1 - c) in float64 (c = 1 gives +inf, c = 0 gives -inf)."""
    c = np.asarray(c, dtype=np.float64)
    with np.errstate(divide="ignore"):
        return np.log(c) - np.log1p(-c)


def ece(pred: np.ndarray, label: np.ndarray, n_bins: int = 15) -> float:
    """Expected Calibration Error with equal-width bins (definition written out)."""
    pred = np.asarray(pred, dtype=np.float64)
    label = np.asarray(label, dtype=np.float64)
    n = pred.size
    if n == 0:
        return float("nan")
    b = np.minimum(np.floor(pred * n_bins), n_bins - 1).astype(np.int64)
    total = 0.0
    for i in range(n_bins):
        sel = b == i
        total += abs(float(pred[sel].sum()) - float(label[sel].sum()))
    return total / n


def observed(acc_len: np.ndarray, n_verified: np.ndarray, k: int) -> np.ndarray:
    """Samples that enter position k (1-based): those that verified it."""
    return k <= np.asarray(n_verified)


def sts_fit(c: np.ndarray, acc_len: np.ndarray, n_verified: np.ndarray, grid: np.ndarray,
            n_bins: int = 15) -> dict:
    """Sequential left-to-right grid search of one temperature per position.

    c [M][K] raw confidences (float32 values), acc_len [M] accepted drafts,
    n_verified [M] verified drafts, grid [G] candidate temperatures.
    Returns tau [K], idx [K], ece_fit [K], ece_raw [K] and the decision margin
    of each position (the runner-up ECE minus the best, over distinct grid
    indices; 0 for equal grid values).
    """
    c = np.asarray(c)
    M, K = c.shape
    acc_len = np.asarray(acc_len, dtype=np.int64)
    n_verified = np.asarray(n_verified, dtype=np.int64)
    grid = np.asarray(grid, dtype=np.float64)
    z = logit(c)
    s_fit = np.ones(M)
    s_raw = np.ones(M)
    tau = np.ones(K)
    idx = np.full(K, -1, dtype=np.int64)
    ece_fit = np.full(K, np.nan)
    ece_raw = np.full(K, np.nan)
    margin = np.full(K, np.inf)
    for j in range(K):
        k = j + 1
        obs = observed(acc_len, n_verified, k)
        y = (acc_len >= k).astype(np.float64)[obs]
        if obs.any():
            ece_raw[j] = ece(s_raw[obs] * sigmoid(z[obs, j]), y, n_bins)
            scores = []
            for g, t in enumerate(grid):
                if np.isfinite(t) and t > 0:
                    scores.append((ece(s_fit[obs] * sigmoid(z[obs, j] / t), y, n_bins), g))
            if scores:
                best_e, best_g = scores[0]
                for e, g in scores[1:]:
                    if e < best_e:
                        best_e, best_g = e, g
                tau[j], idx[j], ece_fit[j] = grid[best_g], best_g, best_e
                rest = [e for e, g in scores if g != best_g]
                if rest:
                    margin[j] = min(rest) - best_e
        s_fit = s_fit * sigmoid(z[:, j] / tau[j])
        s_raw = s_raw * sigmoid(z[:, j])
    return {"tau": tau, "idx": idx, "ece_fit": ece_fit, "ece_raw": ece_raw, "margin": margin}
