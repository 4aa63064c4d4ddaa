"""Workload definitions for the synthetic cycle inputs.

Each configuration fixes the problem shape (B requests, K draft positions,
vocabulary V, Markov rank r, hidden size d), the storage types, the value
distributions and the seed.  The five named workloads are the shapes the
method is exercised on; ``tbias*`` are test-only variants whose Markov factors
are large enough that the transition bias moves the sampled tokens (with
N(0, 0.02^2) factors the bias has a standard deviation of only
sqrt(r) * 0.02^2, far below one nat).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    K: int
    V: int
    r: int
    d: int
    logits_dtype: str = "bf16"      # "f32" | "bf16" (Z and the target logits)
    weight_dtype: str = "bf16"      # "f32" | "bf16" (E and Wt)
    hidden_dtype: str = "bf16"      # "f32" | "bf16" (h)
    T_s: float = 1.0                # sampling temperature, applied to q and p
    seed: int = 0
    z_kind: str = "normal"          # "normal" | "zipf"
    z_std: float = 3.0
    zipf_top: float = 8.0           # logit of rank i = top - slope * ln(i + 1)
    zipf_slope: float = 1.1
    zipf_noise: float = 0.5
    target_noise: float = 1.0       # target = Z + N(0, target_noise^2)
    flatten_after: Optional[int] = None   # positions k > this are scaled
    flatten_scale: float = 1.0
    ew_std: float = 0.02            # std of E and Wt entries
    wc_std: float = 0.02            # std of the confidence weights
    b_c: float = 0.0
    h_std: float = 1.0
    tau_range: Tuple[float, float] = (0.8, 2.0)
    # step-time table: ("linear", a, b) -> a + b*N ;
    #                  ("knee", flat, knee, slope) -> flat, plus slope*(N-knee) above the knee
    ttable: Tuple = ("linear", 1.0, 0.01)

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def n_max(self) -> int:
        """Largest number of verified positions: B * (K + 1)."""
        return self.B * (self.K + 1)


CONFIGS = {
    # fp32 everywhere, one request
    "tiny": Config(name="tiny", B=1, K=4, V=4096, r=32, d=128,
                   logits_dtype="f32", weight_dtype="f32", hidden_dtype="f32",
                   seed=0, z_kind="normal", z_std=3.0, target_noise=1.0,
                   ttable=("linear", 1.0, 0.01)),
    # vocabulary and hidden size of a 4B-class model; fp32 logits
    "qwen3_4b": Config(name="qwen3_4b", B=32, K=16, V=151936, r=256, d=2560,
                       logits_dtype="f32", weight_dtype="bf16", hidden_dtype="bf16",
                       seed=1, z_kind="normal", z_std=3.0, target_noise=1.0,
                       ttable=("linear", 5.0, 0.02)),
    # the headline workload: 256 concurrent requests, Zipf-shaped logits
    "high_concurrency": Config(name="high_concurrency", B=256, K=16, V=151936, r=256, d=4096,
                               seed=2, z_kind="zipf", target_noise=1.5,
                               ttable=("knee", 5.0, 512, 0.03)),
    # 129,280-entry vocabulary, low acceptance (target noise std 2)
    "dsv4_vocab": Config(name="dsv4_vocab", B=512, K=8, V=129280, r=256, d=7168,
                         seed=3, z_kind="normal", z_std=3.0, target_noise=2.0,
                         ttable=("knee", 5.0, 1024, 0.02)),
    # 1024 requests x 32 positions, late positions flattened, T_s = 0.7
    "stress": Config(name="stress", B=1024, K=32, V=151936, r=256, d=4096,
                     seed=4, z_kind="normal", z_std=3.0, target_noise=1.0,
                     flatten_after=8, flatten_scale=0.3, T_s=0.7,
                     ttable=("knee", 5.0, 2048, 0.04)),
    # test-only: tiny shape with a visible Markov bias (std ~1.4 nats at r = 32)
    "tbias": Config(name="tbias", B=4, K=4, V=4096, r=32, d=128,
                    logits_dtype="f32", weight_dtype="f32", hidden_dtype="f32",
                    seed=100, ew_std=0.5, wc_std=0.2, ttable=("linear", 1.0, 0.01)),
    # test-only: bf16 path with a visible bias at r = 256 (std ~1 nat),
    # ragged batch (not a multiple of 32) and a ragged last vocabulary chunk
    "tbias_bf16": Config(name="tbias_bf16", B=40, K=6, V=20000, r=256, d=512,
                         seed=101, ew_std=0.25, wc_std=0.2,
                         ttable=("linear", 5.0, 0.02)),
}


def get_config(name: str) -> Config:
    return CONFIGS[name]
