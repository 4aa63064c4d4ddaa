"""One full cycle: draft -> confidence/survival -> schedule -> verify.

The order is the per-cycle order of the DSpark page (Method): the sequential
Markov stage samples the block, the confidence head scores it, the scheduler
picks how much of each block to verify, and verification accepts a prefix and
emits one more token per request.
"""
from __future__ import annotations

import numpy as np

from .conf import confidence
from .draft import draft
from .rnn import bf16_round, rnn_draft
from .sched import schedule
from .verify import verify


def run_cycle(inp: dict) -> dict:
    """Run the oracle on a dict of inputs as produced by ``synth.make_inputs``."""
    cfg = inp["cfg"]
    d = draft(inp["Z"], inp["E"], inp["Wt"], inp["anchor"], cfg.T_s, cfg.seed)
    c, S = confidence(inp["h"], inp["E"], inp["w_c"], inp["b_c"], inp["tau"], inp["anchor"], d["x"])
    sc = schedule(S, inp["T"])
    ver = verify(inp["Zt"], inp["Z"], inp["E"], inp["Wt"], inp["anchor"], d["x"], sc["n"], cfg.T_s, cfg.seed)
    K = cfg.K
    out_tok = np.full((cfg.B, K + 1), -1, np.int64)
    for b, vr in enumerate(ver):
        out_tok[b, :len(vr["tokens"])] = vr["tokens"]
    return {
        "draft": d, "conf": c, "surv": S, "sched": sc, "verify": ver,
        "out_tok": out_tok,
        "n_accepted": np.array([vr["accepted"] for vr in ver]),
        "next_anchor": np.array([vr["y"] for vr in ver]),
    }


def run_cycle_rnn(inp: dict, rnn: dict) -> dict:
    """The same cycle with the RNN head as the sequential block (``rnn`` holds
    W_ih, b_ih, W_hh, b_hh as produced by ``synth.make_rnn_weights``)."""
    cfg = inp["cfg"]
    d = rnn_draft(inp["Z"], inp["E"], inp["Wt"], inp["h"], inp["anchor"], rnn["W_ih"], rnn["b_ih"], rnn["W_hh"],
                  rnn["b_hh"], cfg.T_s, cfg.seed)
    c, S = confidence(inp["h"], inp["E"], inp["w_c"], inp["b_c"], inp["tau"], inp["anchor"], d["x"])
    sc = schedule(S, inp["T"])
    ver = verify(inp["Zt"], inp["Z"], inp["E"], inp["Wt"], inp["anchor"], d["x"], sc["n"], cfg.T_s, cfg.seed,
                 vec=bf16_round(d["state"]))
    K = cfg.K
    out_tok = np.full((cfg.B, K + 1), -1, np.int64)
    for b, vr in enumerate(ver):
        out_tok[b, :len(vr["tokens"])] = vr["tokens"]
    return {
        "draft": d, "conf": c, "surv": S, "sched": sc, "verify": ver,
        "out_tok": out_tok,
        "n_accepted": np.array([vr["accepted"] for vr in ver]),
        "next_anchor": np.array([vr["y"] for vr in ver]),
    }
