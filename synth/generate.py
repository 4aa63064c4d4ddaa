"""Draw the seeded arrays of one cycle.

Every tensor is drawn from its own numpy ``default_rng([seed, tensor_id, slab])``
stream, where ``slab`` is the request index for per-request tensors and 0 for
shared ones, so that any request's rows can be regenerated on their own.

Tensor ids: 1 Z, 2 target noise, 3 E, 4 Wt, 5 h, 6 w_c, 7 tau, 8 anchor,
10 the extra base-logit row behind the bonus position (row K+1 of the target).

bf16 arrays are returned as their raw 16-bit patterns (``np.uint16``), rounded
from float32 with round-to-nearest-even; float32 arrays as ``np.float32``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import Config

TID_Z, TID_NOISE, TID_E, TID_WT, TID_H, TID_WC, TID_TAU, TID_ANCHOR, TID_ZBONUS = 1, 2, 3, 4, 5, 6, 7, 8, 10


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def _bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(cfg: Config, tid: int, slab: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, tid, slab])


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    return bf16_bits_from_f32(x32) if dtype == "bf16" else np.ascontiguousarray(x32, np.float32)


def _as_f32(stored: np.ndarray, dtype: str) -> np.ndarray:
    return _bf16_bits_to_f32(stored) if dtype == "bf16" else stored


def _base_rows(cfg: Config, rng: np.random.Generator, n: int, positions) -> np.ndarray:
    """n base-logit rows (float32) for the given 1-based positions."""
    V = cfg.V
    out = np.empty((n, V), np.float32)
    if cfg.z_kind == "zipf":
        ranked = (cfg.zipf_top - cfg.zipf_slope * np.log1p(np.arange(V, dtype=np.float64))).astype(np.float32)
        for i in range(n):
            perm = rng.permutation(V)
            out[i, perm] = ranked
            out[i] += rng.standard_normal(V, dtype=np.float32) * np.float32(cfg.zipf_noise)
    elif cfg.z_kind == "normal":
        rng.standard_normal(out=out, dtype=np.float32)
        out *= np.float32(cfg.z_std)
    else:
        raise ValueError(cfg.z_kind)
    if cfg.flatten_after is not None:
        for i, pos in enumerate(positions):
            if pos > cfg.flatten_after:
                out[i] *= np.float32(cfg.flatten_scale)
    return out


def T_table(cfg: Config) -> np.ndarray:
    """Step time T[N] for N = 0 .. B*(K+1) verified positions (float32)."""
    N = np.arange(cfg.n_max + 1, dtype=np.float64)
    kind = cfg.ttable[0]
    if kind == "linear":
        _, a, b = cfg.ttable
        t = a + b * N
    elif kind == "knee":
        _, flat, knee, slope = cfg.ttable
        t = flat + slope * np.maximum(N - knee, 0.0)
    elif kind == "table":
        t = np.asarray(cfg.ttable[1], np.float64)
        assert t.shape == N.shape
    else:
        raise ValueError(kind)
    return t.astype(np.float32)


def make_inputs(cfg: Config, threads: int | None = None) -> dict:
    """All arrays of one cycle for ``cfg`` (see the module docstring for the layout)."""
    B, K, V, r, d = cfg.B, cfg.K, cfg.V, cfg.r, cfg.d
    ldt = cfg.logits_dtype
    zdtype = np.uint16 if ldt == "bf16" else np.float32
    Z = np.empty((B, K, V), zdtype)
    Zt = np.empty((B, K + 1, V), zdtype)

    def slab(b: int) -> None:
        z32 = _base_rows(cfg, _rng(cfg, TID_Z, b), K, range(1, K + 1))
        zs = _store(z32, ldt)
        Z[b] = zs
        zb32 = _base_rows(cfg, _rng(cfg, TID_ZBONUS, b), 1, [K + 1])
        zbs = _store(zb32, ldt)
        base = np.concatenate([_as_f32(zs, ldt), _as_f32(zbs, ldt)], axis=0)
        noise = _rng(cfg, TID_NOISE, b).standard_normal((K + 1, V), dtype=np.float32)
        Zt[b] = _store(base + noise * np.float32(cfg.target_noise), ldt)

    nthreads = threads or min(16, os.cpu_count() or 1)
    if B == 1 or nthreads == 1:
        for b in range(B):
            slab(b)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(slab, range(B)))

    E32 = _rng(cfg, TID_E).standard_normal((V, r), dtype=np.float32) * np.float32(cfg.ew_std)
    W32 = _rng(cfg, TID_WT).standard_normal((V, r), dtype=np.float32) * np.float32(cfg.ew_std)
    hdt = cfg.hidden_dtype
    h = np.empty((B, K, d), np.uint16 if hdt == "bf16" else np.float32)
    for b in range(B):
        h[b] = _store(_rng(cfg, TID_H, b).standard_normal((K, d), dtype=np.float32) * np.float32(cfg.h_std), hdt)
    w_c = (_rng(cfg, TID_WC).standard_normal(d + r, dtype=np.float32) * np.float32(cfg.wc_std)).astype(np.float32)
    lo, hi = cfg.tau_range
    tau = _rng(cfg, TID_TAU).uniform(lo, hi, K).astype(np.float32)
    anchor = _rng(cfg, TID_ANCHOR).integers(0, V, B).astype(np.int32)
    return {
        "cfg": cfg,
        "Z": Z, "Zt": Zt,
        "E": _store(E32, cfg.weight_dtype), "Wt": _store(W32, cfg.weight_dtype),
        "h": h, "w_c": w_c, "b_c": float(cfg.b_c), "tau": tau,
        "anchor": anchor, "T": T_table(cfg),
    }


def make_survivals(B: int, K: int, seed: int, ties: bool = False) -> np.ndarray:
    """Scheduler-only input: float32 [B, K] rows in (0, 1], non-increasing along
    each row (sorted uniform draws).  With ``ties`` the values are rounded to
    multiples of 1/16, so that many candidates of different requests, and of the
    same request, share one survival and the tie-break decides their order."""
    rng = np.random.default_rng([seed, 90, B, K])
    u = rng.uniform(0.0, 1.0, (B, K))
    if ties:
        u = np.ceil(u * 16.0) / 16.0
    u = np.maximum(u, 2.0 ** -20)
    return -np.sort(-u, axis=1).astype(np.float32)



def make_sts_samples(M: int, K: int, seed: int, censor: bool = True) -> tuple:
    """Calibration samples for fitting per-position temperatures: raw confidences
    c float32 [M, K] in (0, 1] (1% exactly 1), accepted lengths int32 [M] and
    verified lengths int32 [M].  The acceptance chain is drawn from a head that is
    overconfident: position k passes with probability 0.5 + 0.7 (c_k - 0.5) given
    that every earlier position passed.  With ``censor`` half of the samples verify a random
    length in [0, K] (so later positions are unobserved unless a rejection came
    first); the others verify all K."""
    rng = np.random.default_rng([seed, 91, M, K])
    c = rng.uniform(0.35, 1.0, (M, K)).astype(np.float32)
    c[rng.random((M, K)) < 0.01] = 1.0
    passed = rng.random((M, K)) < 0.5 + 0.7 * (c.astype(np.float64) - 0.5)
    chain = np.argmin(np.concatenate([passed, np.zeros((M, 1), bool)], axis=1), axis=1)
    if censor:
        n_ver = np.where(rng.random(M) < 0.5, K, rng.integers(0, K + 1, M))
    else:
        n_ver = np.full(M, K)
    acc = np.minimum(chain, n_ver)
    return c, acc.astype(np.int32), n_ver.astype(np.int32)


def sts_grid(G: int = 129, lo: float = 0.25, hi: float = 4.0) -> np.ndarray:
    """Candidate temperatures: G values spaced evenly in log between lo and hi
    (float64), with the middle entry exactly 1 when G is odd and lo * hi = 1."""
    g = np.exp(np.linspace(np.log(lo), np.log(hi), G))
    if G % 2 == 1 and lo * hi == 1.0:
        g[G // 2] = 1.0
    return g


def make_rnn_weights(cfg: Config) -> dict:
    """Weights of the gated recurrent head for a workload: W_ih (3r, d + r) over the
    input [h_k; E[x_{k-1}]], W_hh (3r, r), biases b_ih, b_hh (3r,) float32.  The
    matrices are stored in the workload's factor dtype.  Scales put every
    pre-activation near unit variance: h columns 1 / (h_std sqrt(d)), E columns
    1 / (ew_std sqrt(r)), W_hh 1 / sqrt(r); biases N(0, 0.1^2)."""
    d, r = cfg.d, cfg.r
    g = _rng(cfg, 20)
    Wh = g.standard_normal((3 * r, d), dtype=np.float32) * np.float32(1.0 / (cfg.h_std * np.sqrt(d)))
    We = _rng(cfg, 21).standard_normal((3 * r, r), dtype=np.float32) * np.float32(1.0 / (cfg.ew_std * np.sqrt(r)))
    W_hh = _rng(cfg, 22).standard_normal((3 * r, r), dtype=np.float32) * np.float32(1.0 / np.sqrt(r))
    bb = _rng(cfg, 23).standard_normal((2, 3 * r), dtype=np.float32) * np.float32(0.1)
    return {"W_ih": _store(np.concatenate([Wh, We], axis=1), cfg.weight_dtype),
            "W_hh": _store(W_hh, cfg.weight_dtype),
            "b_ih": bb[0].astype(np.float32), "b_hh": bb[1].astype(np.float32)}
