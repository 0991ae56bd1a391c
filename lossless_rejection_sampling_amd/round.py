"""Device buffers for one round and the call sequence draft -> schedule -> verify.

Plumbing around the C entry points: allocation of outputs and workspace with
torch (device memory only) and the three calls in the pages' order (drafting,
confidence scoring, prefix scheduling, verification).
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import dspark as ds
from .workloads import Round


@dataclasses.dataclass
class Buffers:
    draft_tokens: torch.Tensor
    draft_logq: torch.Tensor
    draft_lse: torch.Tensor
    budget: Optional[torch.Tensor]
    out_tokens: torch.Tensor
    num_accepted: torch.Tensor
    num_emitted: torch.Tensor
    workspace: torch.Tensor
    sps_B: Optional[torch.Tensor] = None
    sps_val: Optional[torch.Tensor] = None
    debug_logp_logq: Optional[torch.Tensor] = None
    debug_residual: Optional[torch.Tensor] = None


def allocate(rnd: Round, debug: bool = False) -> Buffers:
    dev = rnd.base.device
    B, g, V, r = rnd.B, rnd.gamma, rnd.V, rnd.r
    i32 = dict(device=dev, dtype=torch.int32)
    buf = Buffers(
        draft_tokens=torch.empty((B, g), **i32),
        draft_logq=torch.empty((B, g), device=dev, dtype=torch.float32),
        draft_lse=torch.empty((B, g), device=dev, dtype=torch.float64),
        budget=(torch.empty((B,), **i32) if rnd.scheduled else rnd.budget),
        out_tokens=torch.empty((B, g + 1), **i32),
        num_accepted=torch.empty((B,), **i32),
        num_emitted=torch.empty((B,), **i32),
        workspace=torch.zeros((ds.dspark_workspace_bytes(B, g, V, r),), device=dev, dtype=torch.uint8),
    )
    if rnd.scheduled:
        buf.sps_B = torch.as_tensor(rnd.sps_B, dtype=torch.float64, device=dev)
        buf.sps_val = torch.as_tensor(rnd.sps_val, dtype=torch.float64, device=dev)
    if debug:
        buf.debug_logp_logq = torch.full((B, g, 2), float("nan"), device=dev, dtype=torch.float32)
        buf.debug_residual = torch.zeros((B, V), device=dev, dtype=torch.float32)
    return buf


def draft(rnd: Round, buf: Buffers, stream=None):
    ds.dspark_draft_round(rnd.base, rnd.U, rnd.Wt, rnd.prev0, rnd.temperature, rnd.seed, rnd.pos_offset,
                          buf.draft_tokens, buf.draft_logq, buf.draft_lse, buf.workspace, stream)


def draft_schedule(rnd: Round, buf: Buffers, stream=None):
    """The draft round and the scheduler in one call (scheduled rounds)."""
    ds.dspark_draft_schedule(rnd.base, rnd.U, rnd.Wt, rnd.prev0, rnd.temperature, rnd.seed, rnd.pos_offset,
                             buf.draft_tokens, buf.draft_logq, buf.draft_lse, rnd.conf, None, buf.sps_B,
                             buf.sps_val, "early_stop", 0.0, buf.budget, buf.workspace, stream)


def schedule(rnd: Round, buf: Buffers, stream=None):
    if rnd.scheduled:
        ds.dspark_schedule(rnd.conf, buf.sps_B, buf.sps_val, buf.budget, buf.workspace, stream)


def verify(rnd: Round, buf: Buffers, stream=None):
    ds.dspark_verify(rnd.target, rnd.base, rnd.U, rnd.Wt, rnd.prev0, buf.draft_tokens, buf.draft_logq,
                     buf.draft_lse, buf.budget, rnd.temperature, rnd.seed, rnd.pos_offset,
                     buf.out_tokens, buf.num_accepted, buf.num_emitted, buf.workspace,
                     buf.debug_logp_logq, buf.debug_residual, stream)


def run_round(rnd: Round, buf: Buffers, stream=None, side_stream=None, combined=True):
    """One round on ``stream`` (default: the current stream).  A scheduled round
    drafts and schedules in one call (``combined``: the scheduler runs in the
    launch of the last draw), or in two calls; with a ``side_stream`` the
    scheduler, which reads only the confidence scores, runs there concurrently
    with drafting instead, and verification waits for it."""
    main = torch.cuda.current_stream() if stream is None else stream
    if side_stream is not None and rnd.scheduled:
        side_stream.wait_stream(main)
        schedule(rnd, buf, side_stream)
        done = torch.cuda.Event()
        done.record(side_stream)
        draft(rnd, buf, main)
        main.wait_event(done)
    elif combined and rnd.scheduled:
        draft_schedule(rnd, buf, main)
    else:
        draft(rnd, buf, main)
        schedule(rnd, buf, main)
    verify(rnd, buf, main)
