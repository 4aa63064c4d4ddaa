"""Philox4x32-10 counter-based generator and the draws the cycle takes from it.

Philox4x32-10 follows its published definition (Salmon, Moraes, Dror, Shaw,
"Parallel random numbers: as easy as 1, 2, 3", SC'11): a 4x32-bit counter, a
2x32-bit key, ten rounds; each round multiplies counter words 0 and 2 by the
two round constants into 64-bit products and mixes the high halves with the
other words and the key; the key is bumped by the two Weyl constants between
rounds.

Draw layout (a reading of the method's "keyed by request, position and
purpose" randomness; the pages print none of it):

* key     = (seed & 0xffffffff, seed >> 32)
* counter = (idx >> 2, b, k, purpose); the draw is output word ``idx & 3``
* b is the 0-based request, k the 1-based draft position (K+1 for a bonus
  draw after K accepted positions), idx the chunk id, the vocabulary id, or 0.

Uniform: u = (((w >> 8) | 1)) * 2^-24, an odd multiple of 2^-24 in (0, 1),
exactly representable in float32.

Gumbel: G = -ln(E) with E = -ln(u); for u >= 1/2, E is evaluated as
-log1p(-(1 - u)) (1 - u is exact) so that the largest Gumbels, which decide
argmaxes, keep full relative accuracy as u -> 1.
"""
from __future__ import annotations

import numpy as np

M0 = 0xD2511F53
M1 = 0xCD9E8D57
W0 = 0x9E3779B9
W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)

# purposes of the draws taken in one cycle
P_DRAFT_CHUNK = 1
P_DRAFT_ELEM = 2
P_ACCEPT = 3
P_RESID_CHUNK = 4
P_RESID_ELEM = 5
P_BONUS_CHUNK = 6
P_BONUS_ELEM = 7


def philox4x32_10(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """Philox4x32 with 10 rounds.  ctr: (..., 4) uint32; key: (..., 2) uint32 (broadcast)."""
    ctr = np.asarray(ctr, dtype=np.uint32)
    key = np.asarray(key, dtype=np.uint32)
    c0 = ctr[..., 0].astype(np.uint64)
    c1 = ctr[..., 1].astype(np.uint64)
    c2 = ctr[..., 2].astype(np.uint64)
    c3 = ctr[..., 3].astype(np.uint64)
    k0 = np.broadcast_to(key[..., 0].astype(np.uint64), c0.shape)
    k1 = np.broadcast_to(key[..., 1].astype(np.uint64), c0.shape)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(W0)) & _MASK
            k1 = (k1 + np.uint64(W1)) & _MASK
        p0 = np.uint64(M0) * c0
        p1 = np.uint64(M1) * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def words(seed: int, b, k, purpose: int, idx) -> np.ndarray:
    """The 32-bit draw for (seed, request b, position k, purpose, index idx); broadcasts b, k, idx."""
    idx = np.asarray(idx, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    k = np.asarray(k, dtype=np.int64)
    shape = np.broadcast_shapes(idx.shape, b.shape, k.shape)
    idx, b, k = (np.broadcast_to(a, shape) for a in (idx, b, k))
    ctr = np.stack([(idx >> 2).astype(np.uint32), b.astype(np.uint32), k.astype(np.uint32),
                    np.full(shape, purpose, np.uint32)], axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], np.uint32)
    out = philox4x32_10(ctr, key)
    return np.take_along_axis(out, (idx & 3)[..., None], axis=-1)[..., 0]


def uniform(w) -> np.ndarray:
    """Odd multiple of 2^-24 in (0, 1) from a 32-bit word (float64, exact)."""
    w = np.asarray(w, dtype=np.uint32)
    return ((w >> np.uint32(8)) | np.uint32(1)).astype(np.float64) * 2.0 ** -24


def gumbel(u) -> np.ndarray:
    """Standard Gumbel variate -ln(-ln(u)), accurate as u -> 1."""
    u = np.asarray(u, dtype=np.float64)
    e = np.where(u >= 0.5, -np.log1p(-(1.0 - u)), -np.log(u))
    return -np.log(e)


def gumbels(seed: int, b, k, purpose: int, idx) -> np.ndarray:
    return gumbel(uniform(words(seed, b, k, purpose, idx)))


def uniforms(seed: int, b, k, purpose: int, idx) -> np.ndarray:
    return uniform(words(seed, b, k, purpose, idx))
