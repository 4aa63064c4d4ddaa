"""Device buffers for one cycle and the three library calls in order.

Plumbing around the binding: uploads host arrays (bf16 given as raw uint16
bit patterns, fp32 as float32), allocates the caller-owned outputs and the
workspace with torch, and issues dspark_draft -> dspark_schedule ->
dspark_verify on the current stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import dspark


def to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload a host array; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    if a.dtype == np.float32:
        return torch.from_numpy(a).to(device)
    if a.dtype in (np.int32, np.int64):
        return torch.from_numpy(a.astype(np.int32)).to(device)
    raise TypeError(a.dtype)


@dataclass
class CycleInputs:
    Z: torch.Tensor
    Zt: torch.Tensor
    E: torch.Tensor
    Wt: torch.Tensor
    h: torch.Tensor
    w_c: torch.Tensor
    b_c: float
    tau: torch.Tensor
    anchor: torch.Tensor
    T: torch.Tensor

    @classmethod
    def upload(cls, inp: dict, device="cuda") -> "CycleInputs":
        return cls(Z=to_device(inp["Z"], device), Zt=to_device(inp["Zt"], device), E=to_device(inp["E"], device),
                   Wt=to_device(inp["Wt"], device), h=to_device(inp["h"], device), w_c=to_device(inp["w_c"], device),
                   b_c=float(inp["b_c"]), tau=to_device(inp["tau"], device), anchor=to_device(inp["anchor"], device),
                   T=to_device(inp["T"], device))


class CycleOutputs:
    """Caller-owned outputs of the three calls plus the shared workspace."""

    def __init__(self, P: dspark.Problem, device="cuda"):
        B, K = P.B, P.K
        f32, i32 = torch.float32, torch.int32
        self.tok = torch.empty((B, K), dtype=i32, device=device)
        self.logq = torch.empty((B, K), dtype=f32, device=device)
        self.lse = torch.empty((B, K), dtype=f32, device=device)
        self.conf = torch.empty((B, K), dtype=f32, device=device)
        self.surv = torch.empty((B, K), dtype=f32, device=device)
        self.n_sched = torch.empty((B,), dtype=i32, device=device)
        self.n_total = torch.empty((1,), dtype=i32, device=device)
        self.out_tok = torch.empty((B, K + 1), dtype=i32, device=device)
        self.n_acc = torch.empty((B,), dtype=i32, device=device)
        self.next_anchor = torch.empty((B,), dtype=i32, device=device)
        self.logp = torch.empty((B, K), dtype=f32, device=device)
        self.resid_mass = torch.empty((B,), dtype=f32, device=device)
        nbytes = dspark.workspace_bytes(P)
        if nbytes == 0:
            raise ValueError("invalid problem")
        self.workspace = torch.empty((nbytes,), dtype=torch.uint8, device=device)

    def host(self) -> dict:
        return {k: v.cpu().numpy() for k, v in vars(self).items() if k != "workspace"}


def draft(P, x: CycleInputs, o: CycleOutputs, stream=None, path: int = dspark.DRAFT_AUTO):
    if path == dspark.DRAFT_AUTO:
        dspark.draft(P, x.Z, x.E, x.Wt, x.h, x.w_c, x.b_c, x.tau, x.anchor,
                     o.tok, o.logq, o.lse, o.conf, o.surv, o.workspace, stream)
    else:
        dspark.draft_timed(P, x.Z, x.E, x.Wt, x.h, x.w_c, x.b_c, x.tau, x.anchor,
                           o.tok, o.logq, o.lse, o.conf, o.surv, o.workspace, None, stream, path=path)


def schedule(P, x: CycleInputs, o: CycleOutputs, stream=None):
    dspark.schedule(P, o.surv, x.T, o.n_sched, o.n_total, o.workspace, stream)


def verify(P, x: CycleInputs, o: CycleOutputs, stream=None):
    dspark.verify(P, x.Zt, x.Z, x.E, x.Wt, x.anchor, o.tok, o.logq, o.lse, o.n_sched,
                  o.out_tok, o.n_acc, o.next_anchor, o.logp, o.resid_mass, o.workspace, stream)


def run_cycle(P, x: CycleInputs, o: CycleOutputs, stream=None, path: int = dspark.DRAFT_AUTO):
    draft(P, x, o, stream, path)
    schedule(P, x, o, stream)
    verify(P, x, o, stream)
