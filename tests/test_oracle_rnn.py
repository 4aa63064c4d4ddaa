"""Pins of the RNN-head oracle (DSpark page, Method > Semi-autoregressive
generation, the RNN head): the gated update against torch.nn.GRUCell, the
bfloat16 rounding against torch's, closed forms at saturated gates, a forced
token through the state projection, dependence on the whole prefix, and the
verification's use of the per-position projection operands."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import synth
from oracle import draft as odraft
from oracle import rnn as ornn
from oracle import verify as overify
from oracle.io import f64


def _weights(r, d, seed, scale=0.3):
    g = np.random.default_rng(seed)
    return (g.normal(0, scale, (3 * r, d + r)), g.normal(0, 0.1, 3 * r),
            g.normal(0, scale, (3 * r, r)), g.normal(0, 0.1, 3 * r))


def test_gru_cell_matches_torch():
    r, d, n = 6, 5, 7
    W_ih, b_ih, W_hh, b_hh = _weights(r, d, 1)
    g = np.random.default_rng(2)
    s, u = g.normal(0, 0.7, (n, r)), g.normal(0, 1, (n, d + r))
    cell = torch.nn.GRUCell(d + r, r).double()
    with torch.no_grad():
        cell.weight_ih.copy_(torch.from_numpy(W_ih)); cell.bias_ih.copy_(torch.from_numpy(b_ih))
        cell.weight_hh.copy_(torch.from_numpy(W_hh)); cell.bias_hh.copy_(torch.from_numpy(b_hh))
        ref = cell(torch.from_numpy(u), torch.from_numpy(s)).numpy()
    np.testing.assert_allclose(ornn.gru_cell(s, u, W_ih, b_ih, W_hh, b_hh), ref, rtol=1e-13, atol=1e-14)


def test_bf16_round_matches_torch_and_ties():
    g = np.random.default_rng(3)
    x32 = np.concatenate([g.normal(0, 1, 20000), g.normal(0, 1e-3, 2000), [0.0, -0.0, 1.0, -0.75]]).astype(np.float32)
    ref = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ornn.bf16_round(x32.astype(np.float64)), ref)
    # ties to even: 1 + 2^-8 sits halfway between 1 and 1 + 2^-7 (odd last bit) -> 1;
    # 1 + 3 * 2^-8 sits between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> 1 + 2^-6
    assert ornn.bf16_round(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert ornn.bf16_round(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6
    assert ornn.bf16_round(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == -(1 + 2.0 ** -6)
    # just above the midpoint rounds up, and 255.5 * 2^-8 units rounds into the next binade
    assert ornn.bf16_round(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7
    assert ornn.bf16_round(np.array([2.0 - 2.0 ** -9]))[0] == 2.0


def _cfg_inputs():
    cfg = synth.get_config("tbias")
    return cfg, synth.make_inputs(cfg)


def test_zero_weights_reduce_to_base_logits():
    cfg, inp = _cfg_inputs()
    r, d = cfg.r, cfg.d
    z = (np.zeros((3 * r, d + r)), np.zeros(3 * r), np.zeros((3 * r, r)), np.zeros(3 * r))
    out = ornn.rnn_draft(inp["Z"], inp["E"], inp["Wt"], inp["h"], inp["anchor"], *z, cfg.T_s, cfg.seed)
    assert np.all(out["state"] == 0)
    ref = odraft.draft(inp["Z"], inp["E"], np.zeros_like(f64(inp["Wt"])), inp["anchor"], cfg.T_s, cfg.seed)
    assert np.array_equal(out["x"], ref["x"])
    np.testing.assert_allclose(out["logq"], ref["logq"], rtol=0, atol=1e-12)


def test_saturated_gates_closed_forms():
    cfg, inp = _cfg_inputs()
    r, d = cfg.r, cfg.d
    W_ih, b_ih, W_hh, b_hh = _weights(r, d, 4, scale=0.05)
    # update gate shut (z = 1): the state never leaves 0
    b = b_ih.copy(); b[r:2 * r] = 60.0
    out = ornn.rnn_draft(inp["Z"], inp["E"], inp["Wt"], inp["h"], inp["anchor"], W_ih, b, W_hh, b_hh, cfg.T_s, cfg.seed)
    assert np.abs(out["state"]).max() < 1e-20
    # update gate open (z = 0) and no recurrent weights: s_k = tanh(W_n [h_k; E[x_{k-1}]] + b_n + rho * b_hh_n)
    b = b_ih.copy(); b[r:2 * r] = -60.0
    Whh0, bhh0 = np.zeros_like(W_hh), np.zeros_like(b_hh)
    out = ornn.rnn_draft(inp["Z"], inp["E"], inp["Wt"], inp["h"], inp["anchor"], W_ih, b, Whh0, bhh0, cfg.T_s, cfg.seed)
    E64 = f64(inp["E"])
    for k in range(1, cfg.K + 1):
        prev = inp["anchor"] if k == 1 else out["x"][:, k - 2]
        u = np.concatenate([f64(inp["h"][:, k - 1]), E64[prev]], axis=1)
        np.testing.assert_allclose(out["state"][:, k - 1], np.tanh(u @ W_ih[2 * r:].T + b[2 * r:]), rtol=1e-12,
                                   atol=1e-14)


def test_state_projection_forces_token():
    # z = 0, nothing but the new-gate bias: s_1 = tanh(b_n) = 0.5 e_0 (exact in bfloat16);
    # Wt[v, 0] = 60 only for the target token: the bias is +30 nats there
    cfg, inp = _cfg_inputs()
    r, d, V = cfg.r, cfg.d, cfg.V
    W_ih, W_hh = np.zeros((3 * r, d + r)), np.zeros((3 * r, r))
    b_ih, b_hh = np.zeros(3 * r), np.zeros(3 * r)
    b_ih[r:2 * r] = -60.0
    b_ih[2 * r] = np.arctanh(0.5)
    Wt = np.zeros((V, r))
    target = 1234
    Wt[target, 0] = 60.0
    out = ornn.rnn_draft(inp["Z"], inp["E"], Wt, inp["h"], inp["anchor"], W_ih, b_ih, W_hh, b_hh, cfg.T_s, cfg.seed)
    assert np.all(out["x"] == target)
    np.testing.assert_allclose(ornn.bf16_round(out["state"][:, :, 0]), 0.5)
    # the transposed reading (state against the vocabulary axis) would not force it
    assert np.all(out["logq"] > -1e-6)


def test_state_carries_the_whole_prefix():
    cfg, inp = _cfg_inputs()
    w = synth.make_rnn_weights(cfg)
    args = (inp["Z"], inp["E"], inp["Wt"], inp["h"], inp["anchor"], w["W_ih"], w["b_ih"], w["W_hh"], w["b_hh"],
            cfg.T_s, cfg.seed)
    base = ornn.rnn_draft(*args)
    tx = base["x"].copy()
    tx[:, 0] = (tx[:, 0] + 1) % cfg.V          # change only x_1
    alt = ornn.rnn_draft(*args, teacher_x=tx)
    # position 3's state depends on x_1 (two tokens back): the Markov operand E[x_2] would not
    assert np.all(np.abs(alt["state"][:, 2] - base["state"][:, 2]).max(axis=1) > 1e-6)
    assert np.array_equal(alt["state"][:, 0], base["state"][:, 0])


def test_verify_operands_index_positions():
    # passing the Markov operands E[x_{k-1}] as the per-position operands reproduces the Markov verification
    cfg, inp = _cfg_inputs()
    d = odraft.draft(inp["Z"], inp["E"], inp["Wt"], inp["anchor"], cfg.T_s, cfg.seed)
    n = np.full(cfg.B, cfg.K)
    prev = np.concatenate([inp["anchor"][:, None], d["x"][:, :-1]], axis=1)
    vec = f64(inp["E"])[prev]
    a = overify.verify(inp["Zt"], inp["Z"], inp["E"], inp["Wt"], inp["anchor"], d["x"], n, cfg.T_s, cfg.seed)
    b = overify.verify(inp["Zt"], inp["Z"], inp["E"], inp["Wt"], inp["anchor"], d["x"], n, cfg.T_s, cfg.seed, vec=vec)
    for ra, rb in zip(a, b):
        assert ra["tokens"] == rb["tokens"] and ra["accepted"] == rb["accepted"]
        np.testing.assert_allclose(rb["mass"], ra["mass"], rtol=1e-12, equal_nan=True)
