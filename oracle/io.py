"""Exact widening of stored inputs to float64.

bf16 arrays arrive as their raw 16-bit patterns (numpy uint16); a bf16 value is
the float32 whose upper half is those bits, so the widening is exact.
"""
from __future__ import annotations

import numpy as np


def f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if a.dtype in (np.float32, np.float64):
        return a.astype(np.float64)
    raise TypeError(f"unsupported stored dtype {a.dtype}")
