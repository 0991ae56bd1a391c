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

The full-size workloads are drawn on the host (numpy PCG64, see
``host_normal``) and then moved to ``device``, so a run on any device and a
run of the CPU oracle see bit-identical inputs; the small generic rounds of
the edge-case tests (``small_random``) are drawn with a ``torch.Generator`` on
the device and handed, as the same tensor, to both sides of a comparison.
"""

from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor
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


# ---------------------------------------------------------------------------
# Host generation.  The full-size workloads are drawn on the host with numpy's
# PCG64 so that the CPU oracle can be run on exactly the inputs a GPU run sees:
# a tensor is filled in fixed chunks of 2^22 elements, chunk i from its own
# stream keyed by (seed, tag, i), so the values do not depend on how many threads
# fill it; small draws (permutations, token ids, row choices) come from one
# stream keyed by (seed, tag).
# ---------------------------------------------------------------------------
_CHUNK = 1 << 22
_THREADS = max(1, min(16, os.cpu_count() or 1))


def _stream(seed: int, tag: int, i: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag, i])))


def host_normal(shape, seed: int, tag: int, std: float = 1.0) -> np.ndarray:
    """float32 array of `shape` with N(0, std^2) entries (std applied in fp32)."""
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    n = out.size
    chunks = range((n + _CHUNK - 1) // _CHUNK)

    def fill(i):
        seg = out[i * _CHUNK:min(n, (i + 1) * _CHUNK)]
        _stream(seed, tag, i).standard_normal(seg.size, dtype=np.float32, out=seg)
        if std != 1.0:
            seg *= np.float32(std)

    with ThreadPoolExecutor(_THREADS) as ex:
        list(ex.map(fill, chunks))
    return out.reshape(shape)


def _t(a: np.ndarray, device, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(device)


def sps_table_linear(n_points: int = 16, t0_us: float = 20000.0, dt_us: float = 5.0):
    """Synthetic monotone step-rate table: batch sizes round(2**(10 i / 15)) for
    i = 0..15 (1 .. 1024 tokens) with step time t(B) = t0 + dt * B microseconds."""
    Bs = np.array([round(2.0 ** (10.0 * i / (n_points - 1))) for i in range(n_points)], dtype=np.float64)
    steps_per_s = 1.0e6 / (t0_us + dt_us * Bs)
    return Bs, steps_per_s


def sps_table_curved():
    """A step-rate table whose step time is not linear in the batch: 8 points
    from 1 to 512 tokens with t(B) = 20000 + 40 sqrt(B) + 0.02 B^2 microseconds
    (a flat launch-bound start, then a compute-bound rise).  Verify batches of a
    few hundred requests reach past its last point, where the scheduler extends
    the last segment."""
    Bs = np.array([1.0, 4.0, 16.0, 48.0, 96.0, 192.0, 320.0, 512.0])
    t_us = 20000.0 + 40.0 * np.sqrt(Bs) + 0.02 * Bs ** 2
    return Bs, 1.0e6 / t_us


def confidence_scores(B: int, gamma: int, g, device):
    """c[b, j-1] = sigmoid(N(1.5 - 0.4 j, 1)) for block position j = 1..gamma.
    `g` is a torch.Generator (drawn with torch) or an int seed (drawn on the host)."""
    j = np.arange(1, gamma + 1, dtype=np.float64)
    if isinstance(g, torch.Generator):
        z = torch.randn((B, gamma), generator=g, device=g.device, dtype=torch.float32).double().cpu().numpy()
    else:
        z = _stream(int(g), 90).standard_normal((B, gamma))
    c = (1.0 / (1.0 + np.exp(-(z + (1.5 - 0.4 * j))))).astype(np.float32)
    # keep strictly inside (0, 1) in fp32
    c = np.clip(c, np.float32(1.0e-7), np.float32(1.0 - 2.0 ** -24))
    return torch.from_numpy(c).to(device)


def tiny(device="cpu") -> Round:
    """B=4 requests, V=1024, gamma=4, T=1.  fp32 target N(0, 2^2); backbone logits =
    target[:, :4] + N(0, 0.5^2); Markov head rank 16 with fp32 factors N(0, 1/16);
    prev0 uniform; Philox seed 0; full verify."""
    B, gamma, V, r = 4, 4, 1024, 16
    seed = 1234 + 1
    target = host_normal((B, gamma + 1, V), seed, 1, std=2.0)
    base = target[:, :gamma] + host_normal((B, gamma, V), seed, 2, std=0.5)
    U = host_normal((V, r), seed, 3, std=0.25)
    Wt = host_normal((V, r), seed, 4, std=0.25)
    prev0 = _stream(seed, 5).integers(0, V, B).astype(np.int32)
    T = np.ones(B, dtype=np.float32)
    return Round("tiny", _t(target, device), _t(base, device), _t(U, device), _t(Wt, device),
                 _t(prev0, device), _t(T, device), seed=0)


def _boosted_target(B, gamma, V, seed, std=3.0, boost=6.0, frac=0.05):
    """fp32 target logits N(0, std^2) with one fixed seeded set of floor(frac*V)
    vocabulary ids raised by ``boost`` in every row (peaked distributions)."""
    t = host_normal((B, gamma + 1, V), seed, 1, std=std)
    ids = _stream(seed, 2).permutation(V)[: int(frac * V)]
    t[:, :, ids] += np.float32(boost)
    return t


def _bf16_sum(a: np.ndarray, b: np.ndarray, device) -> torch.Tensor:
    """bf16(a + b) with a + b formed in fp32, on the device."""
    return (_t(a, device) + _t(b, device)).to(torch.bfloat16)


def dspark5(B=64, V=151936, gamma=5, r=256, device="cpu", seed_base=1234 + 2, T=1.0,
            scheduled=False, name=None) -> Round:
    """Qwen3-4B-like DSpark-5 round.  bf16 target N(0, 3^2) with 5% of vocabulary
    ids boosted by +6; backbone logits = target + N(0, 1) (bf16); Markov factors
    bf16 N(0, 1/256); uniform previous tokens; T = 1.  With ``scheduled`` the
    round also carries confidence scores and the synthetic step-rate table."""
    seed = seed_base
    target = _t(_boosted_target(B, gamma, V, seed), device, torch.bfloat16)
    noise = host_normal((B, gamma, V), seed, 3)
    base = (target[:, :gamma].float() + _t(noise, device)).to(torch.bfloat16)
    del noise
    U = _t(host_normal((V, r), seed, 4, std=1.0 / 16.0), device, torch.bfloat16)
    Wt = _t(host_normal((V, r), seed, 5, std=1.0 / 16.0), device, torch.bfloat16)
    prev0 = _t(_stream(seed, 6).integers(0, V, B).astype(np.int32), device)
    Tt = torch.full((B,), T, device=device, dtype=torch.float32)
    rnd = Round(name or f"dspark5_B{B}", target.contiguous(), base.contiguous(), U, Wt, prev0, Tt,
                seed=20260706)
    if scheduled:
        rnd.conf = confidence_scores(B, gamma, seed, device)
        rnd.sps_B, rnd.sps_val = sps_table_linear()
    return rnd


def headline(device="cpu", scheduled=True) -> Round:
    """B=256, gamma=5, V=151936, r=256: the DSpark-5 generator at B=256 with the
    confidence-scheduled verify (scores and step-rate table as in ``scheduled``);
    ``scheduled=False``: the same inputs verified at the full budget L = gamma."""
    rnd = dspark5(B=256, device=device, seed_base=1234 + 6, scheduled=True, name="headline_B256")
    if not scheduled:
        rnd.conf = None
        rnd.name = "headline_B256_full"
    return rnd


def block_length(gamma: int, B=256, V=151936, r=256, device="cpu") -> Round:
    """Block-length scaling at T = 0.8.  Each target row independently: 70% peaked
    (N(0, 2^2) with one uniform id +10), 30% flat N(0, 1).  Backbone row j =
    target row j-1 + N(0, sigma_j^2), sigma_j = 0.5 + 1.5 (j-1)/(gamma-1)."""
    seed = 1234 + 3 + 100 * gamma
    rows = B * (gamma + 1)
    t = host_normal((rows, V), seed, 1)
    rs = _stream(seed, 2)
    peaked = rs.random(rows) < 0.7
    hot = rs.integers(0, V, rows)
    t *= np.where(peaked, np.float32(2.0), np.float32(1.0))[:, None]
    t[np.arange(rows), hot] += np.where(peaked, np.float32(10.0), np.float32(0.0))
    target = _t(t.reshape(B, gamma + 1, V), device, torch.bfloat16)
    del t
    sig = np.array([0.5 + 1.5 * (j - 1) / max(gamma - 1, 1) for j in range(1, gamma + 1)], dtype=np.float32)
    noise = host_normal((B, gamma, V), seed, 3)
    noise *= sig[None, :, None]
    base = (target[:, :gamma].float() + _t(noise, device)).to(torch.bfloat16)
    del noise
    U = _t(host_normal((V, r), seed, 4, std=1.0 / 16.0), device, torch.bfloat16)
    Wt = _t(host_normal((V, r), seed, 5, std=1.0 / 16.0), device, torch.bfloat16)
    prev0 = _t(_stream(seed, 6).integers(0, V, B).astype(np.int32), device)
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
    seed = 1234 + 5
    target = host_normal((B, gamma + 1, V), seed, 1, std=8.0)
    rows = target.reshape(-1, V)
    rs = _stream(seed, 2)
    n_tie = max(1, int(math.ceil(0.001 * rows.shape[0])))
    tie_rows = rs.permutation(rows.shape[0])[:n_tie]
    tie_cols = rs.integers(0, V, n_tie)
    rows[tie_rows, tie_cols] = rows[tie_rows].max(axis=1)
    base = host_normal((B, gamma, V), seed, 3, std=1.5)
    base += target[:, :gamma]
    target_t = _t(target, device)
    del target, rows
    base_t = _t(base, device)
    del base
    U = _t(host_normal((V, r), seed, 4, std=1.0 / 16.0), device, torch.bfloat16)
    Wt = _t(host_normal((V, r), seed, 5, std=1.0 / 16.0), device, torch.bfloat16)
    prev0 = _t(_stream(seed, 6).integers(0, V, B).astype(np.int32), device)
    Tt = torch.where(torch.arange(B, device=device) % 2 == 0, 0.0, 1.3).to(torch.float32)
    rnd = Round(f"stress_B{B}", target_t, base_t, U, Wt, prev0, Tt, seed=99)
    rnd.conf = confidence_scores(B, gamma, seed, device)
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


def input_fingerprint(rnd: Round) -> np.ndarray:
    """Weighted float64 sums over strided samples of every input tensor: a cheap
    check that two runs (on any device) drew the same inputs."""

    def f(t, step):
        if t is None:
            return 0.0
        x = t.detach().reshape(-1)[::step].to(torch.float64)
        w = torch.arange(1, x.numel() + 1, dtype=torch.float64, device=x.device).remainder(97)
        return float((x * w).sum())

    return np.array([f(rnd.target, 4099), f(rnd.base, 4097), f(rnd.U, 1031), f(rnd.Wt, 1033),
                     f(rnd.prev0, 1), f(rnd.temperature, 1), f(rnd.conf, 1)])


def to_host(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact host copy: bf16 is widened to fp32 (lossless) so numpy can hold it."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()
