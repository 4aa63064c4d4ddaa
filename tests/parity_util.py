"""Helpers of the GPU-vs-oracle parity tests.

Decision rule: a GPU decision (token, acceptance, scheduled length) may differ
from the oracle's only where the oracle's decision margin is below 1e-4, and
such mismatches must stay below 0.01% of the decisions of their kind.
Floating-point outputs: probabilities (q(x), p(x), residual mass) within 1e-5
relative, confidences and survivals within 1e-6 absolute.
"""
from __future__ import annotations

import numpy as np

MARGIN = 1e-4
MISMATCH_RATE = 1e-4
PROB_RTOL = 1e-5
CONF_ATOL = 1e-6


def check_decisions(kind: str, gpu, ref, margin) -> int:
    gpu, ref, margin = (np.asarray(a).ravel() for a in (gpu, ref, margin))
    mism = gpu != ref
    high = mism & ~(margin < MARGIN)
    assert not high.any(), (f"{kind}: {int(high.sum())} mismatches with margin >= {MARGIN}: "
                            f"idx {np.flatnonzero(high)[:8]}, gpu {gpu[high][:8]}, oracle {ref[high][:8]}, "
                            f"margin {margin[high][:8]}")
    n = int(mism.sum())
    assert n <= MISMATCH_RATE * mism.size, f"{kind}: {n} low-margin mismatches of {mism.size} decisions"
    return n


def check_logprob(kind: str, gpu_log, ref_log, where=None) -> float:
    """|p_gpu / p_ref - 1| <= PROB_RTOL, with p = exp(log value)."""
    g, r = np.asarray(gpu_log, np.float64), np.asarray(ref_log, np.float64)
    if where is not None:
        g, r = g[where], r[where]
    if g.size == 0:
        return 0.0
    rel = np.abs(np.expm1(g - r))
    worst = float(rel.max())
    assert worst <= PROB_RTOL, f"{kind}: worst relative error {worst:.3e} at {np.argmax(rel)}"
    return worst


def check_abs(kind: str, gpu, ref, atol: float) -> float:
    err = np.abs(np.asarray(gpu, np.float64) - np.asarray(ref, np.float64))
    worst = float(err.max()) if err.size else 0.0
    assert worst <= atol, f"{kind}: worst abs error {worst:.3e} at {np.unravel_index(np.argmax(err), err.shape)}"
    return worst


def check_rel(kind: str, gpu, ref, rtol: float) -> float:
    g, r = np.asarray(gpu, np.float64), np.asarray(ref, np.float64)
    rel = np.abs(g - r) / np.abs(r)
    worst = float(rel.max()) if rel.size else 0.0
    assert worst <= rtol, f"{kind}: worst relative error {worst:.3e}"
    return worst
