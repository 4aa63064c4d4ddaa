"""Seeded synthetic inputs for the draft/schedule/verify cycle.

This package holds no arithmetic of the method itself: it only draws the
arrays a cycle consumes (base draft logits, target logits, low-rank Markov
factors, hidden states, confidence weights, per-position temperatures,
anchors and the step-time table).  Both the CPU oracle (``oracle/``) and the
GPU path consume exactly the bytes produced here.
"""
from .configs import CONFIGS, Config, get_config
from .generate import (make_inputs, make_survivals, make_sts_samples, sts_grid, make_rnn_weights,
                       bf16_bits_from_f32, T_table)

__all__ = ["CONFIGS", "Config", "get_config", "make_inputs", "make_survivals", "make_sts_samples", "sts_grid", "make_rnn_weights",
           "bf16_bits_from_f32", "T_table"]
