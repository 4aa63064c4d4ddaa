"""ctypes binding of libdspark.so: same entry points as include/dspark.h.

This module only marshals arguments: torch tensors supply device pointers and
torch supplies the current HIP stream.  Every step of the cycle runs in the
library's HIP kernels; there is no other implementation behind these calls, and
a missing library raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdspark.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libdspark_debug.so")  # built with DSPARK_DEBUG_CHECKS

OK, E_INVALID, E_DTYPE, E_UNSUPPORTED, E_WORKSPACE, E_LAUNCH, E_POINTER = 0, -1, -2, -3, -4, -5, -6
DRAFT_AUTO, DRAFT_PER_POSITION, DRAFT_PERSISTENT = 0, 1, 2  # schedules of the draft phase (dspark_instr.h)
# flag bits of the debug build's checks (dspark_instr.h)
DEBUG_LOGITS, DEBUG_FACTORS, DEBUG_IDS, DEBUG_SCHEDULE_INPUT, DEBUG_OUTPUT = 1, 2, 4, 8, 16
DEBUG_BARRIER_TIMEOUT = 32
F32, BF16 = 0, 1
_DT = {"f32": F32, "bf16": BF16}
_TORCH_DT = {F32: torch.float32, BF16: torch.bfloat16}

SYMBOLS = ("dspark_workspace_bytes", "dspark_status_string", "dspark_draft", "dspark_draft_timed", "dspark_draft_path",
           "dspark_debug_flags", "dspark_debug_check_inputs", "dspark_debug_force_barrier_timeout",
           "dspark_schedule", "dspark_schedule_async", "dspark_schedule_fixed", "dspark_schedule_threshold",
           "dspark_sts_workspace_bytes", "dspark_sts_fit", "dspark_verify", "dspark_rnn_workspace_bytes",
           "dspark_draft_rnn", "dspark_verify_rnn", "dspark_schedule_noalloc",
           "dspark_probe_draws")


class Problem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("K", ctypes.c_int32), ("V", ctypes.c_int32),
        ("r", ctypes.c_int32), ("d", ctypes.c_int32),
        ("logits_dtype", ctypes.c_int32), ("weight_dtype", ctypes.c_int32), ("hidden_dtype", ctypes.c_int32),
        ("sampling_temp", ctypes.c_float), ("seed", ctypes.c_uint64),
    ]

    @classmethod
    def make(cls, B, K, V, r, d, logits="bf16", weights="bf16", hidden="bf16", T_s=1.0, seed=0) -> "Problem":
        return cls(B, K, V, r, d, _DT[logits], _DT[weights], _DT[hidden], float(T_s), int(seed))

    @classmethod
    def from_config(cls, cfg) -> "Problem":
        return cls.make(cfg.B, cfg.K, cfg.V, cfg.r, cfg.d, cfg.logits_dtype, cfg.weight_dtype,
                        cfg.hidden_dtype, cfg.T_s, cfg.seed)


class DsparkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")
        self.status = status


_libs = {}
_use_debug = False


def use_debug_library(on: bool) -> None:
    """Route every binding of this module through libdspark_debug.so (the same
    kernels with input and output scans around each call) or back to libdspark.so."""
    global _use_debug
    _use_debug = bool(on)


def load(debug: bool | None = None) -> ctypes.CDLL:
    """Load libdspark.so, or libdspark_debug.so (both built by
    draft_sampling_verification_markov_amd.build); raises if absent."""
    debug = _use_debug if debug is None else debug
    if debug in _libs:
        return _libs[debug]
    path = DEBUG_LIB_PATH if debug else LIB_PATH
    if not os.path.exists(path):
        raise FileNotFoundError(f"{path} is missing: build it with __graft_entry__.build() "
                                "or python -m draft_sampling_verification_markov_amd.build")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(Problem)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.dspark_workspace_bytes.argtypes = [P]
    lib.dspark_workspace_bytes.restype = sz
    lib.dspark_status_string.argtypes = [i32]
    lib.dspark_status_string.restype = ctypes.c_char_p
    lib.dspark_draft.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dspark_draft.restype = i32
    lib.dspark_draft_timed.argtypes = lib.dspark_draft.argtypes + [vp, i32, i32]
    lib.dspark_draft_timed.restype = i32
    lib.dspark_draft_path.argtypes = [ctypes.POINTER(Problem)]
    lib.dspark_draft_path.restype = i32
    lib.dspark_schedule.argtypes = [P, vp, vp, vp, vp, vp, sz, vp]
    lib.dspark_schedule.restype = i32
    lib.dspark_probe_draws.argtypes = [ctypes.c_uint64, vp, i32, vp, vp, i32, vp, vp, vp]
    lib.dspark_probe_draws.restype = i32
    lib.dspark_schedule_noalloc.argtypes = [P, vp, vp, vp, vp, vp]
    lib.dspark_schedule_noalloc.restype = i32
    lib.dspark_schedule_async.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.dspark_schedule_async.restype = i32
    lib.dspark_sts_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.dspark_sts_workspace_bytes.restype = sz
    lib.dspark_sts_fit.argtypes = [i32, i32, vp, vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.dspark_sts_fit.restype = i32
    lib.dspark_schedule_fixed.argtypes = [P, i32, vp, vp, vp]
    lib.dspark_schedule_fixed.restype = i32
    lib.dspark_schedule_threshold.argtypes = [P, vp, ctypes.c_float, vp, vp, vp]
    lib.dspark_schedule_threshold.restype = i32
    lib.dspark_verify.argtypes = [P] + [vp] * 14 + [vp, sz, vp]
    lib.dspark_verify.restype = i32
    lib.dspark_rnn_workspace_bytes.argtypes = [P]
    lib.dspark_rnn_workspace_bytes.restype = sz
    lib.dspark_draft_rnn.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_float] + [vp] * 8 + [vp, sz, vp]
    lib.dspark_draft_rnn.restype = i32
    lib.dspark_verify_rnn.argtypes = [P] + [vp] * 15 + [vp, sz, vp]
    lib.dspark_verify_rnn.restype = i32
    lib.dspark_debug_flags.argtypes = [vp, i32]
    lib.dspark_debug_flags.restype = i32
    lib.dspark_debug_check_inputs.argtypes = [P, vp, vp, vp, vp, vp]
    lib.dspark_debug_check_inputs.restype = i32
    lib.dspark_debug_force_barrier_timeout.argtypes = [i32]
    lib.dspark_debug_force_barrier_timeout.restype = i32
    _libs[debug] = lib
    return lib


def workspace_bytes(P: Problem) -> int:
    return int(load().dspark_workspace_bytes(ctypes.byref(P)))


def status_string(status: int) -> str:
    return load().dspark_status_string(int(status)).decode()


def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous CUDA (HIP) tensor, checking its dtype; None passes NULL."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise DsparkError(fn, status)


def draft(P: Problem, Z, E, Wt, h, w_conf, b_conf: float, tau, anchor,
          draft_tok, draft_logq, draft_lse, conf, surv, workspace, stream=None) -> None:
    lt, wt, ht = _TORCH_DT[P.logits_dtype], _TORCH_DT[P.weight_dtype], _TORCH_DT[P.hidden_dtype]
    st = load().dspark_draft(
        ctypes.byref(P), _ptr(Z, lt, "Z"), _ptr(E, wt, "E"), _ptr(Wt, wt, "Wt"), _ptr(h, ht, "h"),
        _ptr(w_conf, torch.float32, "w_conf"), ctypes.c_float(b_conf), _ptr(tau, torch.float32, "tau"),
        _ptr(anchor, torch.int32, "anchor"), _ptr(draft_tok, torch.int32, "draft_tok"),
        _ptr(draft_logq, torch.float32, "draft_logq"), _ptr(draft_lse, torch.float32, "draft_lse"),
        _ptr(conf, torch.float32, "conf"), _ptr(surv, torch.float32, "surv"),
        _ptr(workspace, None, "workspace"), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        _stream(stream))
    _check("dspark_draft", st)


def draft_timed(P: Problem, Z, E, Wt, h, w_conf, b_conf: float, tau, anchor,
                draft_tok, draft_logq, draft_lse, conf, surv, workspace, events=None, stream=None,
                path: int = DRAFT_AUTO) -> None:
    """dspark_draft_timed: dspark_draft with schedule `path` (DRAFT_*), recording `events` (raw
    hipEvent_t handles, a ctypes array of 2 or 2 + 2K c_void_p, or None) around the draft phase and,
    with 2 + 2K, around each launch of its stream kernel."""
    lt, wt, ht = _TORCH_DT[P.logits_dtype], _TORCH_DT[P.weight_dtype], _TORCH_DT[P.hidden_dtype]
    st = load().dspark_draft_timed(
        ctypes.byref(P), _ptr(Z, lt, "Z"), _ptr(E, wt, "E"), _ptr(Wt, wt, "Wt"), _ptr(h, ht, "h"),
        _ptr(w_conf, torch.float32, "w_conf"), ctypes.c_float(b_conf), _ptr(tau, torch.float32, "tau"),
        _ptr(anchor, torch.int32, "anchor"), _ptr(draft_tok, torch.int32, "draft_tok"),
        _ptr(draft_logq, torch.float32, "draft_logq"), _ptr(draft_lse, torch.float32, "draft_lse"),
        _ptr(conf, torch.float32, "conf"), _ptr(surv, torch.float32, "surv"),
        _ptr(workspace, None, "workspace"), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        _stream(stream), None if events is None else ctypes.cast(events, ctypes.c_void_p),
        ctypes.c_int32(0 if events is None else len(events)), ctypes.c_int32(path))
    _check("dspark_draft_timed", st)


def draft_path(P: Problem) -> int:
    """dspark_draft_path: the schedule dspark_draft takes for P (DRAFT_PERSISTENT or DRAFT_PER_POSITION)."""
    r = load().dspark_draft_path(ctypes.byref(P))
    if r < 0:
        raise DsparkError("dspark_draft_path", r)
    return r


def schedule(P: Problem, surv, T_table, n_sched, n_total, workspace, stream=None) -> None:
    st = load().dspark_schedule(
        ctypes.byref(P), _ptr(surv, torch.float32, "surv"), _ptr(T_table, torch.float32, "T_table"),
        _ptr(n_sched, torch.int32, "n_sched"), _ptr(n_total, torch.int32, "n_total"),
        _ptr(workspace, None, "workspace"), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        _stream(stream))
    _check("dspark_schedule", st)


def probe_draws(seed: int, ctr=None, out_words=None, w=None, uniform=None, gumbel=None, stream=None) -> None:
    """The device's Philox words of counters ctr [n][4] (uint32 as int32 tensors) and the uniform
    and Gumbel transforms of words w [m] (instrumentation)."""
    n = 0 if ctr is None else int(ctr.shape[0])
    m = 0 if w is None else int(w.numel())
    st = load().dspark_probe_draws(ctypes.c_uint64(seed), _ptr(ctr, torch.int32, "ctr"), n,
                                   _ptr(out_words, torch.int32, "out_words"), _ptr(w, torch.int32, "w"), m,
                                   _ptr(uniform, torch.float32, "uniform"), _ptr(gumbel, torch.float32, "gumbel"),
                                   _stream(stream))
    _check("dspark_probe_draws", st)


def schedule_noalloc(P: Problem, surv, T_table, n_sched, n_total, stream=None) -> None:
    """dspark_schedule with the library's static scratch instead of a workspace (B * K <= 32768)."""
    st = load().dspark_schedule_noalloc(
        ctypes.byref(P), _ptr(surv, torch.float32, "surv"), _ptr(T_table, torch.float32, "T_table"),
        _ptr(n_sched, torch.int32, "n_sched"), _ptr(n_total, torch.int32, "n_total"), _stream(stream))
    _check("dspark_schedule_noalloc", st)


def schedule_async(P: Problem, surv_lag, surv, T_table, n_sched, n_total, workspace, stream=None) -> None:
    st = load().dspark_schedule_async(
        ctypes.byref(P), _ptr(surv_lag, torch.float32, "surv_lag"), _ptr(surv, torch.float32, "surv"),
        _ptr(T_table, torch.float32, "T_table"), _ptr(n_sched, torch.int32, "n_sched"),
        _ptr(n_total, torch.int32, "n_total"), _ptr(workspace, None, "workspace"),
        ctypes.c_size_t(workspace.numel() * workspace.element_size()), _stream(stream))
    _check("dspark_schedule_async", st)


def schedule_fixed(P: Problem, gamma: int, n_sched, n_total, stream=None) -> None:
    st = load().dspark_schedule_fixed(ctypes.byref(P), int(gamma), _ptr(n_sched, torch.int32, "n_sched"),
                                      _ptr(n_total, torch.int32, "n_total"), _stream(stream))
    _check("dspark_schedule_fixed", st)


def schedule_threshold(P: Problem, surv, theta: float, n_sched, n_total, stream=None) -> None:
    st = load().dspark_schedule_threshold(ctypes.byref(P), _ptr(surv, torch.float32, "surv"), ctypes.c_float(theta),
                                          _ptr(n_sched, torch.int32, "n_sched"),
                                          _ptr(n_total, torch.int32, "n_total"), _stream(stream))
    _check("dspark_schedule_threshold", st)


def sts_workspace_bytes(M: int, K: int, G: int, n_bins: int = 15) -> int:
    return int(load().dspark_sts_workspace_bytes(int(M), int(K), int(G), int(n_bins)))


def sts_fit(conf_raw, acc_len, n_verified, tau_grid, tau, tau_idx, ece_fit, ece_raw, workspace,
            n_bins: int = 15, stream=None) -> None:
    """Per-position STS temperatures by grid search on ECE (conf_raw [M][K] float32)."""
    M, K = (int(x) for x in conf_raw.shape)
    G = int(tau_grid.numel())
    st = load().dspark_sts_fit(M, K, _ptr(conf_raw, torch.float32, "conf_raw"),
                               _ptr(acc_len, torch.int32, "acc_len"), _ptr(n_verified, torch.int32, "n_verified"),
                               _ptr(tau_grid, torch.float64, "tau_grid"), G, int(n_bins),
                               _ptr(tau, torch.float64, "tau"), _ptr(tau_idx, torch.int32, "tau_idx"),
                               _ptr(ece_fit, torch.float64, "ece_fit"), _ptr(ece_raw, torch.float64, "ece_raw"),
                               _ptr(workspace, torch.uint8, "workspace"), workspace.numel(), _stream(stream))
    _check("dspark_sts_fit", st)


def verify(P: Problem, target, Z, E, Wt, anchor, draft_tok, draft_logq, draft_lse, n_sched,
           out_tok, n_accepted, next_anchor, logp, resid_mass, workspace, stream=None) -> None:
    lt, wt = _TORCH_DT[P.logits_dtype], _TORCH_DT[P.weight_dtype]
    st = load().dspark_verify(
        ctypes.byref(P), _ptr(target, lt, "target"), _ptr(Z, lt, "Z"), _ptr(E, wt, "E"), _ptr(Wt, wt, "Wt"),
        _ptr(anchor, torch.int32, "anchor"), _ptr(draft_tok, torch.int32, "draft_tok"),
        _ptr(draft_logq, torch.float32, "draft_logq"), _ptr(draft_lse, torch.float32, "draft_lse"),
        _ptr(n_sched, torch.int32, "n_sched"), _ptr(out_tok, torch.int32, "out_tok"),
        _ptr(n_accepted, torch.int32, "n_accepted"), _ptr(next_anchor, torch.int32, "next_anchor"),
        _ptr(logp, torch.float32, "logp"), _ptr(resid_mass, torch.float32, "resid_mass"),
        _ptr(workspace, None, "workspace"), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        _stream(stream))
    _check("dspark_verify", st)


def rnn_workspace_bytes(P: Problem) -> int:
    return int(load().dspark_rnn_workspace_bytes(ctypes.byref(P)))


def draft_rnn(P: Problem, Z, E, Wt, h, W_ih, b_ih, W_hh, b_hh, w_conf, b_conf: float, tau, anchor,
              draft_tok, draft_logq, draft_lse, conf, surv, state, workspace, stream=None) -> None:
    """dspark_draft with the RNN head; state [B][K][r] float32 receives s_k."""
    lt, wt, ht = _TORCH_DT[P.logits_dtype], _TORCH_DT[P.weight_dtype], _TORCH_DT[P.hidden_dtype]
    st = load().dspark_draft_rnn(
        ctypes.byref(P), _ptr(Z, lt, "Z"), _ptr(E, wt, "E"), _ptr(Wt, wt, "Wt"), _ptr(h, ht, "h"),
        _ptr(W_ih, wt, "W_ih"), _ptr(b_ih, torch.float32, "b_ih"), _ptr(W_hh, wt, "W_hh"),
        _ptr(b_hh, torch.float32, "b_hh"), _ptr(w_conf, torch.float32, "w_conf"), ctypes.c_float(b_conf),
        _ptr(tau, torch.float32, "tau"), _ptr(anchor, torch.int32, "anchor"),
        _ptr(draft_tok, torch.int32, "draft_tok"), _ptr(draft_logq, torch.float32, "draft_logq"),
        _ptr(draft_lse, torch.float32, "draft_lse"), _ptr(conf, torch.float32, "conf"),
        _ptr(surv, torch.float32, "surv"), _ptr(state, torch.float32, "state"),
        _ptr(workspace, None, "workspace"), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        _stream(stream))
    _check("dspark_draft_rnn", st)


def verify_rnn(P: Problem, target, Z, E, Wt, anchor, draft_tok, draft_logq, draft_lse, state, n_sched,
               out_tok, n_accepted, next_anchor, logp, resid_mass, workspace, stream=None) -> None:
    """dspark_verify with the RNN head's states as the projection operands."""
    lt, wt = _TORCH_DT[P.logits_dtype], _TORCH_DT[P.weight_dtype]
    st = load().dspark_verify_rnn(
        ctypes.byref(P), _ptr(target, lt, "target"), _ptr(Z, lt, "Z"), _ptr(E, wt, "E"), _ptr(Wt, wt, "Wt"),
        _ptr(anchor, torch.int32, "anchor"), _ptr(draft_tok, torch.int32, "draft_tok"),
        _ptr(draft_logq, torch.float32, "draft_logq"), _ptr(draft_lse, torch.float32, "draft_lse"),
        _ptr(state, torch.float32, "state"), _ptr(n_sched, torch.int32, "n_sched"),
        _ptr(out_tok, torch.int32, "out_tok"), _ptr(n_accepted, torch.int32, "n_accepted"),
        _ptr(next_anchor, torch.int32, "next_anchor"), _ptr(logp, torch.float32, "logp"),
        _ptr(resid_mass, torch.float32, "resid_mass"),
        _ptr(workspace, None, "workspace"), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
        _stream(stream))
    _check("dspark_verify_rnn", st)


def debug_flags(clear: bool = True) -> int:
    """dspark_debug_flags of libdspark_debug.so: the current device's flag word (synchronises)."""
    v = ctypes.c_uint32()
    _check("dspark_debug_flags", load(True).dspark_debug_flags(ctypes.byref(v), 1 if clear else 0))
    return v.value


def debug_check_inputs(P: Problem, Z=None, target=None, anchor=None, T_table=None, stream=None) -> None:
    """dspark_debug_check_inputs of libdspark_debug.so: the input scans alone (None: not scanned)."""
    lt = _TORCH_DT[P.logits_dtype]
    st = load(True).dspark_debug_check_inputs(
        ctypes.byref(P), None if Z is None else _ptr(Z, lt, "Z"), None if target is None else _ptr(target, lt, "target"),
        None if anchor is None else _ptr(anchor, torch.int32, "anchor"),
        None if T_table is None else _ptr(T_table, torch.float32, "T_table"), _stream(stream))
    _check("dspark_debug_check_inputs", st)


def debug_force_barrier_timeout(on: bool) -> None:
    """dspark_debug_force_barrier_timeout of libdspark_debug.so."""
    _check("dspark_debug_force_barrier_timeout", load(True).dspark_debug_force_barrier_timeout(1 if on else 0))
