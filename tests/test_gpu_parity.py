"""GPU round (through the C ABI) against the CPU oracle on the same seeded inputs.

Small rounds are compared request by request in full against the oracle run
here.  The full-size workloads (DSpark-5 at B=64, the B=256 round at its
scheduled and at its full budget, block lengths 4/8/16 at B=256, the scheduled
round at B=512 and the stress round at B=1024, V=262144) run the whole batch on
the GPU in the configuration the benchmark times; every request is compared
with the oracle's whole-batch expectations in tests/golden/rounds (written by
tests/golden/make_round_goldens.py from the same host-drawn inputs), the
residual rows of a few requests with the numpy oracle run here, and, up to the
B=512 round, every request again with the C oracle run here (oracle/dspark_ref.c,
pinned to the numpy oracle on the CPU), residual rows included.
"""

import os

import numpy as np
import pytest
import torch

from lossless_rejection_sampling_amd import dspark as ds
from lossless_rejection_sampling_amd import round as rd
from lossless_rejection_sampling_amd import workloads as wl
from oracle import dspark as od
from oracle import ref

from parity import check, compare, compare_golden, load_golden, run_c_oracle, run_gpu, run_oracle, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

DEV = "cuda"


def _full(rnd, name, debug=True):
    say(f"[{name}] B={rnd.B} gamma={rnd.gamma} V={rnd.V} r={rnd.r} dtype={rnd.base.dtype}")
    buf = run_gpu(rnd, debug=debug)
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
    idx = np.arange(rnd.B)
    rep = compare(rnd, buf, run_oracle(rnd, idx), idx)
    check(rep, name)
    return buf


def test_tiny_round():
    _full(wl.tiny(DEV), "tiny")


@pytest.mark.parametrize("case", [
    dict(B=24, gamma=5, V=1000, r=32, dtype=torch.float32, fdt=torch.bfloat16, temps=(1.0, 0.7, 1.5, 0.0)),
    dict(B=24, gamma=5, V=1000, r=32, dtype=torch.bfloat16, fdt=torch.bfloat16, temps=(1.0, 0.0)),
    dict(B=16, gamma=4, V=9000, r=16, dtype=torch.float32, fdt=torch.float32, temps=(1.0, 0.8)),
    dict(B=16, gamma=3, V=4097, r=48, dtype=torch.bfloat16, fdt=torch.bfloat16, temps=(1.3,)),
    dict(B=8, gamma=2, V=8, r=16, dtype=torch.float32, fdt=torch.bfloat16, temps=(1.0, 0.0)),
    dict(B=8, gamma=6, V=65, r=20, dtype=torch.float32, fdt=torch.bfloat16, temps=(0.9,)),
    dict(B=1, gamma=16, V=2048, r=64, dtype=torch.bfloat16, fdt=torch.bfloat16, temps=(1.0,)),
    dict(B=300, gamma=2, V=700, r=16, dtype=torch.float32, fdt=torch.bfloat16, temps=(1.0, 0.0, 2.0)),
    dict(B=300, gamma=3, V=5000, r=64, dtype=torch.bfloat16, fdt=torch.bfloat16, temps=(1.0, 0.0, 0.7)),
    dict(B=40, gamma=4, V=12345, r=128, dtype=torch.float32, fdt=torch.bfloat16, temps=(1.0, 1.2)),
    dict(B=70, gamma=3, V=9000, r=256, dtype=torch.bfloat16, fdt=torch.bfloat16, temps=(1.0, 0.0)),
    dict(B=520, gamma=2, V=3001, r=256, dtype=torch.float32, fdt=torch.bfloat16, temps=(0.9,)),
    # more tiles than workgroups: a partial last round of tiles
    dict(B=24, gamma=4, V=20000, r=256, dtype=torch.bfloat16, fdt=torch.bfloat16, temps=(1.0, 0.0, 0.8)),
    dict(B=40, gamma=3, V=24000, r=128, dtype=torch.bfloat16, fdt=torch.bfloat16, temps=(1.3, 0.0)),
    # more than 4096 tiles (the general draw) over bf16 streams: 4219 tiles, 123 in a partial last round
    dict(B=4, gamma=2, V=270000, r=128, dtype=torch.bfloat16, fdt=torch.bfloat16, temps=(1.0, 0.0)),
    # the general draw over fp32 logits (16-byte records with the tile-maximum shift): 4110 tiles
    dict(B=4, gamma=2, V=263000, r=16, dtype=torch.float32, fdt=torch.bfloat16, temps=(1.0, 0.0, 0.5)),
])
def test_small_rounds(case):
    rnd = wl.small_random(case["B"], case["gamma"], case["V"], case["r"], device=DEV, seed=case["B"] + case["V"],
                          dtype=case["dtype"], factor_dtype=case["fdt"], temps=case["temps"])
    g = torch.Generator(device="cpu").manual_seed(5)
    rnd.budget = torch.randint(0, rnd.gamma + 1, (rnd.B,), generator=g, dtype=torch.int32).to(DEV)
    rnd.pos_offset = torch.randint(0, 1 << 20, (rnd.B,), generator=g, dtype=torch.int32).to(DEV)
    _full(rnd, f"small_{case['B']}x{case['gamma']}x{case['V']}_r{case['r']}")


def test_identical_draft_always_accepts():
    rnd = wl.small_random(32, 4, 3000, 16, device=DEV, seed=3, temps=(1.0, 0.6))
    rnd.base = rnd.target[:, :4].contiguous()
    rnd.Wt = torch.zeros_like(rnd.Wt)
    buf = _full(rnd, "identical_draft")
    assert torch.all(buf.num_accepted == 4)


def test_zero_budget_is_plain_decode():
    rnd = wl.small_random(16, 4, 5000, 32, device=DEV, seed=4, factor_dtype=torch.bfloat16,
                          temps=(1.0, 0.0))
    rnd.budget = torch.zeros(16, dtype=torch.int32, device=DEV)
    buf = _full(rnd, "zero_budget")
    assert torch.all(buf.num_accepted == 0) and torch.all(buf.num_emitted == 1)


def test_deterministic_and_position_offsets():
    rnd = wl.small_random(16, 5, 5000, 32, device=DEV, seed=9, factor_dtype=torch.bfloat16)
    a = run_gpu(rnd)
    b = run_gpu(rnd)
    assert torch.equal(a.out_tokens, b.out_tokens) and torch.equal(a.draft_tokens, b.draft_tokens)
    rnd.pos_offset = torch.full((16,), 1000, dtype=torch.int32, device=DEV)
    c = run_gpu(rnd)
    assert not torch.equal(a.draft_tokens, c.draft_tokens)


def test_rounds_reuse_one_workspace():
    # every call leaves the verification counters at zero for the next one
    rnd = wl.small_random(40, 5, 9000, 32, device=DEV, seed=11, factor_dtype=torch.bfloat16, temps=(1.0, 0.0, 0.8))
    g = torch.Generator(device="cpu").manual_seed(2)
    rnd.budget = torch.randint(0, rnd.gamma + 1, (rnd.B,), generator=g, dtype=torch.int32).to(DEV)
    buf = rd.allocate(rnd, debug=True)
    outs = []
    for _ in range(3):
        rd.run_round(rnd, buf)
        torch.cuda.synchronize()
        assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
        outs.append((buf.out_tokens.clone(), buf.num_accepted.clone(), buf.draft_tokens.clone()))
    for o in outs[1:]:
        assert all(torch.equal(x, y) for x, y in zip(o, outs[0]))
    idx = np.arange(rnd.B)
    check(compare(rnd, buf, run_oracle(rnd, idx), idx), "reused_workspace")


@pytest.mark.parametrize("case", [
    # the scheduler in the launch of the last draw
    dict(B=64, gamma=5, V=20000, r=256, dtype=torch.bfloat16, temps=(1.0, 0.0)),
    dict(B=300, gamma=4, V=5000, r=128, dtype=torch.bfloat16, temps=(0.8,)),
    # rows of more than 4096 tiles: the general draw kernel, the scheduler after it
    dict(B=6, gamma=3, V=270000, r=64, dtype=torch.float32, temps=(1.0, 0.0)),
])
def test_draft_schedule_matches_two_calls(case):
    rnd = wl.small_random(case["B"], case["gamma"], case["V"], case["r"], device=DEV, seed=case["V"] % 97,
                          dtype=case["dtype"], factor_dtype=torch.bfloat16, temps=case["temps"])
    g = torch.Generator(device=DEV).manual_seed(case["B"])
    rnd.conf = wl.confidence_scores(rnd.B, rnd.gamma, g, DEV)
    rnd.sps_B, rnd.sps_val = wl.sps_table_linear()
    say(f"[draft_schedule] B={rnd.B} gamma={rnd.gamma} V={rnd.V} r={rnd.r}")
    bufs = []
    for combined in (False, True):
        buf = rd.allocate(rnd, debug=True)
        rd.run_round(rnd, buf, combined=combined)
        torch.cuda.synchronize()
        assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
        bufs.append(buf)
    for name in ("draft_tokens", "draft_logq", "draft_lse", "budget", "out_tokens", "num_accepted", "num_emitted"):
        assert torch.equal(getattr(bufs[0], name), getattr(bufs[1], name)), name
    idx = np.arange(min(rnd.B, 24))
    check(compare(rnd, bufs[1], run_oracle(rnd, idx), idx), "draft_schedule")


def test_bad_data_is_reported_not_faulted():
    rnd = wl.small_random(8, 3, 500, 16, device=DEV, seed=1)
    rnd.prev0 = rnd.prev0.clone()
    rnd.prev0[3] = 10 ** 6          # out of range: clamped on the device, reported
    rnd.budget = torch.tensor([3, 3, 9, 3, -1, 3, 3, 3], dtype=torch.int32, device=DEV)
    buf = run_gpu(rnd)
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_EDATA
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK   # cleared
    n = buf.num_accepted.cpu().numpy()
    assert n.min() >= 0 and n.max() <= 3


def _tie_round(B=64, gamma=3, V=40000, r=16, seed=21):
    """Greedy requests whose target rows carry exact ties at the row maximum, at
    two columns c1 < c2 placed (by row) within one 64-column tile, across the
    lanes of one 4096-column block, across two blocks of one verification work
    item, and across work items (block 1 vs the ragged last block 9); every
    fifth row has a third tied column.  The draft is the target row (W = 0)
    with the maximum moved to c2 for even requests (the draft then disagrees
    with the lowest-index target argmax: a rejection) and left at c1 for odd
    ones (acceptances up to the bonus, whose greedy token is again the tie)."""
    rnd = wl.small_random(B, gamma, V, r, device="cpu", seed=seed, temps=(0.0,))
    t = rnd.target.clone()
    base = t[:, :gamma].clone()
    rng = np.random.default_rng(seed)
    for b in range(B):
        for j in range(gamma + 1):
            kind = (b + j) % 4
            if kind == 0:
                c1 = int(rng.integers(0, V // 64)) * 64 + int(rng.integers(0, 32))
                c2 = c1 + int(rng.integers(1, 32))
            elif kind == 1:
                c1 = int(rng.integers(0, 4096 - 64 * 8))
                c2 = c1 + 64 * int(rng.integers(1, 8))
            elif kind == 2:
                c1, c2 = int(rng.integers(0, 4096)), 2 * 4096 + int(rng.integers(0, 4096))
            else:
                c1, c2 = 4096 + int(rng.integers(0, 4096)), 9 * 4096 + int(rng.integers(0, V - 9 * 4096))
            top = float(t[b, j].max()) + 1.0
            t[b, j, c1] = top
            t[b, j, c2] = top
            if (b * (gamma + 1) + j) % 5 == 0:
                t[b, j, min(V - 1, c2 + 7)] = top
            if j < gamma:
                base[b, j] = t[b, j]
                base[b, j, c2 if b % 2 == 0 else c1] += 0.5
    rnd.target = t.contiguous().to(DEV)
    rnd.base = base.contiguous().to(DEV)
    rnd.U, rnd.prev0, rnd.temperature = rnd.U.to(DEV), rnd.prev0.to(DEV), rnd.temperature.to(DEV)
    rnd.Wt = torch.zeros_like(rnd.U)
    return rnd


def test_greedy_target_ties_lowest_index():
    rnd = _tie_round()
    buf = _full(rnd, "greedy_ties")
    n = buf.num_accepted.cpu().numpy()
    # even requests reject at the first position, odd ones accept every position
    assert np.all(n[0::2] == 0) and np.all(n[1::2] == rnd.gamma)


@pytest.mark.parametrize("case", [
    dict(B=4, gamma=3, V=1, r=1, dtype=torch.float32, fdt=torch.bfloat16, temps=(1.0, 0.0)),
    dict(B=3, gamma=2, V=3, r=1, dtype=torch.bfloat16, fdt=torch.bfloat16, temps=(1.0, 0.5, 0.0)),
    dict(B=1, gamma=1, V=64, r=5, dtype=torch.bfloat16, fdt=torch.float32, temps=(1.0,)),
    dict(B=2, gamma=16, V=7, r=2, dtype=torch.float32, fdt=torch.float32, temps=(0.9, 0.0)),
], ids=["V1_r1", "V3_r1", "B1_gamma1", "gamma16_V7"])
def test_degenerate_sizes(case):
    # the smallest sizes the ABI allows: a one-token vocabulary (p = q = 1: every
    # position accepted, the bonus token 0), rank 1, one request of one position,
    # the longest block over a vocabulary smaller than one tile
    rnd = wl.small_random(case["B"], case["gamma"], case["V"], case["r"], device=DEV, seed=5, dtype=case["dtype"],
                          factor_dtype=case["fdt"], temps=case["temps"])
    buf = _full(rnd, f"degenerate_{case['V']}x{case['r']}")
    if rnd.V == 1:
        assert torch.all(buf.num_accepted == rnd.gamma)
        assert torch.all(buf.out_tokens == 0)


def test_low_temperature_round():
    # T = 0.05 on fp32 logits of scale 8 (|z| / T up to ~700): block sums and
    # residual masses must carry no error proportional to the row maximum over T.
    # Draft and target rows are close (noise 0.1 against scale 8), so some accept
    # tests fall within the oracle's 1e-6 margin: those requests are excused, and
    # the rate bar of the full-size workloads does not apply to this edge case.
    rnd = wl.small_random(48, 4, 20000, 64, device=DEV, seed=31, dtype=torch.float32,
                          factor_dtype=torch.bfloat16, temps=(0.05, 0.1, 1.0), std=8.0, noise=0.1)
    say(f"[low_temperature] B={rnd.B} gamma={rnd.gamma} V={rnd.V} r={rnd.r}")
    buf = run_gpu(rnd)
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
    idx = np.arange(rnd.B)
    rep = compare(rnd, buf, run_oracle(rnd, idx), idx)
    check(rep, "low_temperature", max_flag_frac=0.05)
    assert rep.requests - rep.flagged_requests >= 36


@pytest.mark.parametrize("temps", [(0.1, 0.25, 0.5), (0.05,)], ids=["T0.1-0.5", "T0.05"])
def test_low_temperature_bf16_round(temps):
    # bf16 logits of scale 3 through the streaming draft GEMM (r = 128): t = x + bias
    # carries one fp32 rounding at |t|'s scale, which 1/T magnifies in the tile
    # records; the draw takes the chosen tile's share of the row's mass from its
    # fp64 recompute, so ln q stays within the log tolerance (and q exceeds 1 by
    # no more than the probability tolerance, 1e-6).
    rnd = wl.small_random(48, 4, 30000, 128, device=DEV, seed=37, dtype=torch.bfloat16,
                          factor_dtype=torch.bfloat16, temps=temps, std=3.0, noise=0.5)
    say(f"[low_temperature_bf16] temps={temps} B={rnd.B} gamma={rnd.gamma} V={rnd.V} r={rnd.r}")
    buf = run_gpu(rnd)
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
    assert float(buf.draft_logq.max()) <= 1e-6
    idx = np.arange(rnd.B)
    rep = compare(rnd, buf, run_oracle(rnd, idx), idx)
    check(rep, "low_temperature_bf16", max_flag_frac=0.05)


def test_data_error_bits_are_reported():
    base = wl.small_random(8, 3, 500, 16, device=DEV, seed=2)
    cases = []
    for name, T in [("nan_temperature", float("nan")), ("negative_temperature", -0.5)]:
        rnd = wl.small_random(8, 3, 500, 16, device=DEV, seed=2)
        rnd.temperature = rnd.temperature.clone()
        rnd.temperature[5] = T
        cases.append((name, rnd))
    for name, rnd in cases:
        say(f"[data_error] {name}")
        buf = run_gpu(rnd)
        assert ds.dspark_status(buf.workspace) == ds.DSPARK_EDATA, name
        assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK, name
    B, gamma = 16, 4
    Bs, sps = wl.sps_table_linear()
    good = wl.confidence_scores(B, gamma, 4, DEV)
    budget = torch.empty(B, dtype=torch.int32, device=DEV)
    ws = torch.zeros(ds.dspark_schedule_workspace_bytes(B, gamma), dtype=torch.uint8, device=DEV)
    tB, tS = torch.tensor(Bs, device=DEV), torch.tensor(sps, device=DEV)
    for name, conf, tb, ts in [
            ("conf_one", good.clone().index_fill_(0, torch.tensor([3], device=DEV), 1.0), tB, tS),
            ("conf_zero", good.clone().index_fill_(0, torch.tensor([7], device=DEV), 0.0), tB, tS),
            ("conf_nan", good.clone().index_fill_(0, torch.tensor([1], device=DEV), float("nan")), tB, tS),
            ("table_not_increasing", good, tB.flip(0).contiguous(), tS),
            ("table_repeated_point", good, torch.cat([tB[:3], tB[2:3], tB[4:]]).contiguous(), tS),
            ("table_zero_rate", good, tB, tS.clone().index_fill_(0, torch.tensor([5], device=DEV), 0.0)),
            ("table_negative_rate", good, tB, -tS)]:
        say(f"[data_error] {name}")
        ds.dspark_schedule(conf, tb, ts, budget, ws)
        assert ds.dspark_status(ws) == ds.DSPARK_EDATA, name
        b = budget.cpu().numpy()
        assert np.all((b >= 0) & (b <= gamma)), name
        assert ds.dspark_status(ws) == ds.DSPARK_OK, name
    ds.dspark_schedule(good, tB, tS, budget, ws)
    assert ds.dspark_status(ws) == ds.DSPARK_OK


def test_pack_w2_and_layout_argument():
    rnd = wl.small_random(12, 3, 5000, 64, device=DEV, seed=12, factor_dtype=torch.bfloat16, temps=(1.0, 0.0))
    for W in (rnd.Wt.t().contiguous(), rnd.Wt.float().t().contiguous()):
        packed = torch.empty(W.shape[1], W.shape[0], dtype=W.dtype, device=DEV)
        ds.dspark_pack_w2(W, packed)
        torch.cuda.synchronize()
        assert torch.equal(packed, W.t().contiguous())
    # the round reads only the packed layout: W2 passed as [r, V] is refused before any launch
    buf = rd.allocate(rnd)
    with pytest.raises(ds.DsparkError) as e:
        ds.dspark_draft_round(rnd.base, rnd.U, rnd.Wt.t().contiguous(), rnd.prev0, rnd.temperature, rnd.seed,
                              None, buf.draft_tokens, buf.draft_logq, buf.draft_lse, buf.workspace)
    assert e.value.code == ds.DSPARK_EINVAL
    # a W2 held as [r, V], packed on the device, gives the round of the vocabulary-major copy
    a = run_gpu(rnd)
    W = rnd.Wt.t().contiguous()
    packed = torch.empty_like(rnd.Wt)
    ds.dspark_pack_w2(W, packed)
    rnd.Wt = packed
    b = run_gpu(rnd)
    for name in ("draft_tokens", "draft_lse", "out_tokens", "num_accepted"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def test_scheduler_beyond_the_last_table_point():
    # a curved step-time table ending at 512 tokens: verify batches of 256 and
    # 512 requests run past its last point, on its extended last segment
    Bs, sps = wl.sps_table_curved()
    crossed = 0
    for B, gamma, seed in [(256, 5, 11), (512, 5, 12), (100, 8, 13), (1024, 8, 14)]:
        say(f"[schedule curved] B={B} gamma={gamma}")
        conf = wl.confidence_scores(B, gamma, 1000 + seed, DEV)
        budget = torch.empty(B, dtype=torch.int32, device=DEV)
        ws = torch.zeros(ds.dspark_schedule_workspace_bytes(B, gamma), dtype=torch.uint8, device=DEV)
        ds.dspark_schedule(conf, torch.tensor(Bs, device=DEV), torch.tensor(sps, device=DEV), budget, ws)
        assert ds.dspark_status(ws) == ds.DSPARK_OK
        ref = od.schedule(conf.cpu().numpy(), Bs, sps)
        assert ref.min_gap > od.SCHED_FLAG
        got = budget.cpu().numpy()
        assert np.array_equal(got, ref.budget), (B, gamma)
        crossed += B + int(got.sum()) > Bs[-1]
    assert crossed >= 2


def test_scheduler_bit_exact():
    Bs, sps = wl.sps_table_linear()
    for B, gamma, seed in [(7, 3, 0), (256, 5, 1), (512, 5, 2), (1024, 8, 3), (64, 16, 4)]:
        say(f"[schedule] B={B} gamma={gamma}")
        g = torch.Generator(device=DEV).manual_seed(seed)
        conf = wl.confidence_scores(B, gamma, g, DEV)
        budget = torch.empty(B, dtype=torch.int32, device=DEV)
        ws = torch.zeros(ds.dspark_schedule_workspace_bytes(B, gamma), dtype=torch.uint8, device=DEV)
        ds.dspark_schedule(conf, torch.tensor(Bs, device=DEV), torch.tensor(sps, device=DEV), budget, ws)
        ref = od.schedule(conf.cpu().numpy(), Bs, sps)
        assert ref.min_gap > od.SCHED_FLAG
        assert np.array_equal(budget.cpu().numpy(), ref.budget)
    # special tables: constant rate admits every candidate with Q > 0; t ~ N admits none
    conf = torch.full((64, 4), 0.5, device=DEV)
    budget = torch.empty(64, dtype=torch.int32, device=DEV)
    ws = torch.zeros(ds.dspark_schedule_workspace_bytes(64, 4), dtype=torch.uint8, device=DEV)
    ds.dspark_schedule(conf, torch.tensor([1.0, 1024.0], device=DEV, dtype=torch.float64),
                       torch.tensor([50.0, 50.0], device=DEV, dtype=torch.float64), budget, ws)
    assert torch.all(budget == 4)
    pts = torch.tensor([1.0, 8.0, 64.0, 1024.0], device=DEV, dtype=torch.float64)
    ds.dspark_schedule(conf, pts, 1.0 / pts, budget, ws)
    assert torch.all(budget == 0)


# ---------------------------------------------------------------------------
# Full-size workloads: the whole batch on the GPU, a sample through the oracle.
# ---------------------------------------------------------------------------

def _sampled(rnd, name, n_sample, seed=0, whole=True):
    """The whole batch on the GPU in the benchmark's launch configuration; every
    request against the oracle's whole-batch expectations, the residual rows of
    a few sampled requests against the numpy oracle run here, and (``whole``)
    every request again, residual rows included, against the C oracle run
    here."""
    say(f"[{name}] B={rnd.B} gamma={rnd.gamma} V={rnd.V} r={rnd.r} dtype={rnd.base.dtype}")
    buf = run_gpu(rnd, debug=True)
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
    n = buf.num_accepted.cpu().numpy()
    L = buf.budget.cpu().numpy() if buf.budget is not None else np.full(rnd.B, rnd.gamma)
    assert np.all((0 <= n) & (n <= L)) and np.all(L <= rnd.gamma)
    out = buf.out_tokens.cpu().numpy()
    assert np.all(out[np.arange(rnd.B), n] >= 0) and np.all(out < rnd.V)
    compare_golden(rnd, buf, load_golden(name), name)
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.choice(rnd.B, size=min(n_sample, rnd.B), replace=False))
    check(compare(rnd, buf, run_oracle(rnd, idx), idx), name + "_residual_sample")
    if whole and os.path.exists(ref.LIB):
        want = run_c_oracle(rnd, keep_residual=True)
        n_res = sum(1 for b in range(rnd.B) if b in want.verify.residual)
        say(f"[{name}] C oracle, whole batch: {n_res} residual rows")
        check(compare(rnd, buf, want, np.arange(rnd.B)), name + "_c_oracle_whole")
    return buf


def test_dspark5_b64():
    _sampled(wl.dspark5(device=DEV), "dspark5_B64", 4)


def test_headline_b256():
    _sampled(wl.headline(device=DEV), "headline_B256", 4)


def test_headline_b256_full_budget():
    _sampled(wl.headline(device=DEV, scheduled=False), "headline_B256_full", 4)


@pytest.mark.parametrize("gamma", [4, 8, 16])
def test_block_length(gamma):
    _sampled(wl.block_length(gamma, device=DEV), f"block_length_g{gamma}", 3)


def test_scheduled_b512():
    _sampled(wl.scheduled(device=DEV), "scheduled_B512", 3)


def test_stress_b1024():
    rnd = wl.stress(device=DEV)
    _sampled(rnd, "stress_B1024", 3, whole=False)  # the C oracle's whole batch here would take minutes
    del rnd
    torch.cuda.empty_cache()
