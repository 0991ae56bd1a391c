"""Seeded synthetic inputs for one DSpark draft/verify round.

This module only *builds inputs*: logits tensors, Markov-head factors, previous
tokens, temperatures, confidence scores and a step-rate table.  It holds none
of the method's arithmetic (no softmax, no sampling, no acceptance rule), so the
HIP path and the CPU oracle can both consume what it produces without sharing
any code that computes a result.

The pages measure DSpark on real drafts over nine public benchmarks with trained
weights; neither is available here, so these generators stand in for them with
the shapes the pages give (blocks of 4-16 tokens, the deployed 5-token block,
batch sizes up to 1024 requests, vocabularies of the Qwen3 / DeepSeek-V3 / Gemma
families) and the distributions stated for each workload below.

Every generator is deterministic for a given ``device``: tensors are drawn with
a ``torch.Generator`` seeded from the workload's fixed seed.  The same tensor
object is then handed to both sides of a comparison.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch


@dataclasses.dataclass
class Round:
    """Inputs of one draft/verify round (device tensors unless noted)."""

    name: str
    target: torch.Tensor          # [B, gamma+1, V] bf16 or fp32 target logits
    base: torch.Tensor            # [B, gamma, V]   backbone draft logits, same dtype
    U: torch.Tensor               # [V, r] first low-rank factor W1 of the Markov head
    Wt: torch.Tensor              # [V, r] second factor W2 stored vocabulary-major (W2 = Wt^T)
    prev0: torch.Tensor           # [B] int32 last committed token of each request
    temperature: torch.Tensor     # [B] fp32, 0 = greedy
    seed: int                     # Philox key for this round
    pos_offset: Optional[torch.Tensor] = None   # [B] int32 absolute position of the block
    conf: Optional[torch.Tensor] = None         # [B, gamma] fp32 confidence scores in (0, 1)
    sps_B: Optional[np.ndarray] = None          # [n] float64 batch sizes (tokens), host
    sps_val: Optional[np.ndarray] = None        # [n] float64 steps per second, host
    budget: Optional[torch.Tensor] = None       # [B] int32 fixed verify budget, None = gamma

    @property
    def W(self) -> torch.Tensor:
        """The second factor W2 as an [r, V] view."""
        return self.Wt.t()

    @property
    def B(self) -> int:
        return int(self.base.shape[0])

    @property
    def gamma(self) -> int:
        return int(self.base.shape[1])

    @property
    def V(self) -> int:
        return int(self.base.shape[2])

    @property
    def r(self) -> int:
        return int(self.U.shape[1])

    @property
    def scheduled(self) -> bool:
        return self.conf is not None

    def subset(self, idx) -> "Round":
        """The same round restricted to the requests in ``idx``.  The Philox
        counter of a request uses its index in the full batch, so a caller that
        compares a subset passes ``idx`` on as the request ids."""
        idx_t = torch.as_tensor(idx, dtype=torch.long, device=self.base.device)
        pick = lambda t: None if t is None else t.index_select(0, idx_t)
        return dataclasses.replace(
            self,
            target=pick(self.target), base=pick(self.base), prev0=pick(self.prev0),
            temperature=pick(self.temperature), pos_offset=pick(self.pos_offset),
            conf=pick(self.conf), budget=pick(self.budget),
        )


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _randn(shape, g, device, std=1.0, dtype=torch.float32):
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).mul_(std).to(dtype)


def sps_table_linear(n_points: int = 16, t0_us: float = 20000.0, dt_us: float = 5.0):
    """Synthetic monotone step-rate table: batch sizes round(2**(10 i / 15)) for
    i = 0..15 (1 .. 1024 tokens) with step time t(B) = t0 + dt * B microseconds."""
    Bs = np.array([round(2.0 ** (10.0 * i / (n_points - 1))) for i in range(n_points)], dtype=np.float64)
    steps_per_s = 1.0e6 / (t0_us + dt_us * Bs)
    return Bs, steps_per_s


def confidence_scores(B: int, gamma: int, g, device):
    """c[b, j-1] = sigmoid(N(1.5 - 0.4 j, 1)) for block position j = 1..gamma."""
    j = torch.arange(1, gamma + 1, device=device, dtype=torch.float32)
    z = torch.randn((B, gamma), generator=g, device=device, dtype=torch.float32) + (1.5 - 0.4 * j)
    c = torch.sigmoid(z)
    # keep strictly inside (0, 1) in fp32
    return c.clamp_(min=1.0e-7, max=1.0 - 2.0 ** -24)


def tiny(device="cpu") -> Round:
    """B=4 requests, V=1024, gamma=4, T=1.  fp32 target N(0, 2^2); backbone logits =
    target[:, :4] + N(0, 0.5^2); Markov head rank 16 with fp32 factors N(0, 1/16);
    prev0 uniform; Philox seed 0; full verify."""
    B, gamma, V, r = 4, 4, 1024, 16
    g = _gen(device, 1234 + 1)
    target = _randn((B, gamma + 1, V), g, device, std=2.0)
    base = target[:, :gamma] + _randn((B, gamma, V), g, device, std=0.5)
    U = _randn((V, r), g, device, std=0.25)
    Wt = _randn((V, r), g, device, std=0.25)
    prev0 = torch.randint(0, V, (B,), generator=g, device=device, dtype=torch.int64).to(torch.int32)
    T = torch.ones(B, device=device, dtype=torch.float32)
    return Round("tiny", target.contiguous(), base.contiguous(), U, Wt, prev0, T, seed=0)


def _boosted_target(B, gamma, V, g, device, std=3.0, boost=6.0, frac=0.05):
    """bf16 target logits N(0, std^2) with one fixed seeded set of floor(frac*V)
    vocabulary ids raised by ``boost`` in every row (peaked distributions)."""
    t = torch.randn((B, gamma + 1, V), generator=g, device=device, dtype=torch.float32).mul_(std)
    ids = torch.randperm(V, generator=g, device=device)[: int(frac * V)]
    t[:, :, ids] += boost
    return t.to(torch.bfloat16)


def dspark5(B=64, V=151936, gamma=5, r=256, device="cpu", seed_base=1234 + 2, T=1.0,
            scheduled=False, name=None) -> Round:
    """Qwen3-4B-like DSpark-5 round.  bf16 target N(0, 3^2) with 5% of vocabulary
    ids boosted by +6; backbone logits = target + N(0, 1) (bf16); Markov factors
    bf16 N(0, 1/256); uniform previous tokens; T = 1.  With ``scheduled`` the
    round also carries confidence scores and the synthetic step-rate table."""
    g = _gen(device, seed_base)
    target = _boosted_target(B, gamma, V, g, device)
    base = (target[:, :gamma].float() + _randn((B, gamma, V), g, device)).to(torch.bfloat16)
    U = _randn((V, r), g, device, std=1.0 / 16.0, dtype=torch.bfloat16)
    Wt = _randn((V, r), g, device, std=1.0 / 16.0, dtype=torch.bfloat16)
    prev0 = torch.randint(0, V, (B,), generator=g, device=device, dtype=torch.int64).to(torch.int32)
    Tt = torch.full((B,), T, device=device, dtype=torch.float32)
    rnd = Round(name or f"dspark5_B{B}", target.contiguous(), base.contiguous(), U, Wt, prev0, Tt,
                seed=20260706)
    if scheduled:
        rnd.conf = confidence_scores(B, gamma, g, device)
        rnd.sps_B, rnd.sps_val = sps_table_linear()
    return rnd


def headline(device="cpu") -> Round:
    """B=256, gamma=5, V=151936, r=256: the DSpark-5 generator at B=256 with the
    confidence-scheduled verify (scores and step-rate table as in ``scheduled``)."""
    return dspark5(B=256, device=device, seed_base=1234 + 6, scheduled=True, name="headline_B256")


def block_length(gamma: int, B=256, V=151936, r=256, device="cpu") -> Round:
    """Block-length scaling at T = 0.8.  Each target row independently: 70% peaked
    (N(0, 2^2) with one uniform id +10), 30% flat N(0, 1).  Backbone row j =
    target row j-1 + N(0, sigma_j^2), sigma_j = 0.5 + 1.5 (j-1)/(gamma-1)."""
    g = _gen(device, 1234 + 3 + 100 * gamma)
    rows = B * (gamma + 1)
    t = torch.randn((rows, V), generator=g, device=device, dtype=torch.float32)
    peaked = torch.rand((rows,), generator=g, device=device) < 0.7
    scale = torch.where(peaked, torch.tensor(2.0, device=device), torch.tensor(1.0, device=device))
    t.mul_(scale[:, None])
    hot = torch.randint(0, V, (rows,), generator=g, device=device)
    t[torch.arange(rows, device=device), hot] += torch.where(peaked, 10.0, 0.0)
    target = t.view(B, gamma + 1, V).to(torch.bfloat16)
    sig = torch.tensor([0.5 + 1.5 * (j - 1) / max(gamma - 1, 1) for j in range(1, gamma + 1)],
                       device=device, dtype=torch.float32)
    noise = torch.randn((B, gamma, V), generator=g, device=device, dtype=torch.float32) * sig[None, :, None]
    base = (target[:, :gamma].float() + noise).to(torch.bfloat16)
    U = _randn((V, r), g, device, std=1.0 / 16.0, dtype=torch.bfloat16)
    Wt = _randn((V, r), g, device, std=1.0 / 16.0, dtype=torch.bfloat16)
    prev0 = torch.randint(0, V, (B,), generator=g, device=device, dtype=torch.int64).to(torch.int32)
    Tt = torch.full((B,), 0.8, device=device, dtype=torch.float32)
    return Round(f"block_length_g{gamma}", target.contiguous(), base.contiguous(), U, Wt, prev0, Tt,
                 seed=7000 + gamma)


def scheduled(B=512, V=129280, gamma=5, r=256, device="cpu") -> Round:
    """Confidence-scheduled verify: the DSpark-5 generator at B=512, V=129280, with
    c[b, j-1] = sigmoid(N(1.5 - 0.4 j, 1)) and the 16-point step-rate table."""
    return dspark5(B=B, V=V, gamma=gamma, r=r, device=device, seed_base=1234 + 4,
                   scheduled=True, name=f"scheduled_B{B}")


def stress(B=1024, V=262144, gamma=8, r=256, device="cpu") -> Round:
    """Stress round: fp32 target 8 N(0, 1) with exact ties injected on 0.1% of rows
    (the row maximum copied onto one other random id); backbone = target +
    N(0, 1.5^2) in fp32; bf16 factors; T = 0 for even requests and 1.3 for odd
    ones; verify budgets from the confidence scheduler with the 16-point table."""
    g = _gen(device, 1234 + 5)
    target = torch.randn((B, gamma + 1, V), generator=g, device=device, dtype=torch.float32).mul_(8.0)
    rows = target.view(-1, V)
    n_tie = max(1, int(math.ceil(0.001 * rows.shape[0])))
    tie_rows = torch.randperm(rows.shape[0], generator=g, device=device)[:n_tie]
    tie_cols = torch.randint(0, V, (n_tie,), generator=g, device=device)
    mx = rows[tie_rows].max(dim=1).values
    rows[tie_rows, tie_cols] = mx
    base = target[:, :gamma] + _randn((B, gamma, V), g, device, std=1.5)
    U = _randn((V, r), g, device, std=1.0 / 16.0, dtype=torch.bfloat16)
    Wt = _randn((V, r), g, device, std=1.0 / 16.0, dtype=torch.bfloat16)
    prev0 = torch.randint(0, V, (B,), generator=g, device=device, dtype=torch.int64).to(torch.int32)
    Tt = torch.where(torch.arange(B, device=device) % 2 == 0, 0.0, 1.3).to(torch.float32)
    rnd = Round(f"stress_B{B}", target.contiguous(), base.contiguous(), U, Wt, prev0, Tt, seed=99)
    rnd.conf = confidence_scores(B, gamma, g, device)
    rnd.sps_B, rnd.sps_val = sps_table_linear()
    return rnd


def small_random(B, gamma, V, r, device="cpu", seed=0, dtype=torch.float32, factor_dtype=None,
                 temps=(1.0,), std=2.0, noise=0.7, rank_std=None) -> Round:
    """Small generic round for property and edge-case tests."""
    g = _gen(device, 50000 + seed)
    target = _randn((B, gamma + 1, V), g, device, std=std)
    base = target[:, :gamma] + _randn((B, gamma, V), g, device, std=noise)
    fs = rank_std if rank_std is not None else 1.0 / math.sqrt(max(r, 1))
    fdt = factor_dtype or dtype
    U = _randn((V, r), g, device, std=math.sqrt(fs), dtype=fdt)
    Wt = _randn((V, r), g, device, std=math.sqrt(fs), dtype=fdt)
    prev0 = torch.randint(0, V, (B,), generator=g, device=device, dtype=torch.int64).to(torch.int32)
    tv = torch.tensor(temps, dtype=torch.float32, device=device)
    Tt = tv[torch.arange(B, device=device) % len(temps)]
    return Round(f"small_{B}x{gamma}x{V}", target.to(dtype).contiguous(), base.to(dtype).contiguous(),
                 U, Wt, prev0, Tt, seed=seed)


def to_host(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact host copy: bf16 is widened to fp32 (lossless) so numpy can hold it."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()
