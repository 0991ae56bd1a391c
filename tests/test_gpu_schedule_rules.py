"""GPU scheduler variants (dspark_schedule_ex through the C ABI) against the
oracle: every rule, with and without Sequential Temperature Scaling, budgets bit
for bit on seeded scores.  Scores the oracle marks as lying on an fp32 rounding
boundary after scaling, and schedules whose closest comparison is a tie to
1e-12, would be excused; the seeded cases below contain neither (asserted)."""

import numpy as np
import pytest
import torch

from lossless_rejection_sampling_amd import dspark as ds
from lossless_rejection_sampling_amd import workloads as wl
from oracle import dspark as od

from parity import say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

DEV = "cuda"
CASES = [(7, 3, 0), (256, 5, 1), (512, 5, 2), (1024, 8, 3), (64, 16, 4)]


def _run(conf, tau, rule, param, Bs=None, sps=None):
    B, gamma = conf.shape
    budget = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    ws = torch.zeros(ds.dspark_schedule_workspace_bytes(B, gamma), dtype=torch.uint8, device=DEV)
    tB = torch.tensor(Bs, device=DEV, dtype=torch.float64) if Bs is not None else None
    tS = torch.tensor(sps, device=DEV, dtype=torch.float64) if sps is not None else None
    ds.dspark_schedule_ex(conf, tau, tB, tS, rule, param, budget, ws)
    torch.cuda.synchronize()
    assert ds.dspark_status(ws) == ds.DSPARK_OK
    return budget.cpu().numpy()


def _tau(gamma, seed):
    return torch.tensor(np.random.default_rng(seed).uniform(0.6, 2.5, gamma), dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("rule,param", [("early_stop", 0.0), ("argmax", 0.0), ("fixed", 1), ("fixed", 3),
                                        ("threshold", 0.7), ("threshold", 0.45)])
@pytest.mark.parametrize("scaled", [False, True])
def test_rules_bit_exact(rule, param, scaled):
    Bs, sps = wl.sps_table_linear()
    for B, gamma, seed in CASES:
        say(f"[schedule_ex {rule} {param} scaled={scaled}] B={B} gamma={gamma}")
        g = torch.Generator(device=DEV).manual_seed(seed)
        conf = wl.confidence_scores(B, gamma, g, DEV)
        tau = _tau(gamma, seed) if scaled else None
        got = _run(conf, tau, rule, param, Bs, sps)
        c = conf.cpu().numpy()
        t = tau.cpu().numpy() if scaled else None
        if scaled:
            _, near = od.calibrate_scores(c, t)
            assert not near.any()
        ref = od.schedule_rule(c, Bs, sps, rule, param, tau=t)
        assert ref.min_gap > od.SCHED_FLAG
        assert np.array_equal(got, ref.budget), (rule, param, B, gamma)


def test_best_cut_on_a_stepped_capacity_curve():
    # the step makes Theta dip; the production rule looks past it, the
    # early-stop rule halts there (oracle pin of the same case)
    conf = torch.full((8, 3), 0.95, device=DEV)
    Bs = np.array([1.0, 9.0, 10.0, 14.0, 40.0])
    sps = 1.0 / np.array([1.0, 1.0, 1.6, 1.6, 3.0])
    early = _run(conf, None, "early_stop", 0.0, Bs, sps)
    best = _run(conf, None, "argmax", 0.0, Bs, sps)
    c = conf.cpu().numpy()
    assert np.array_equal(early, od.schedule_rule(c, Bs, sps, "early_stop").budget)
    assert np.array_equal(best, od.schedule_rule(c, Bs, sps, "argmax").budget)
    assert best.sum() > early.sum()


def test_lagged_scores_feed_the_production_rule():
    # the production scheduler decides round t from the scores of round t - 2:
    # a three-slot ring of past scores on the device, the rule applied to the
    # slot written two rounds earlier
    Bs, sps = wl.sps_table_linear()
    B, gamma = 256, 5
    g = torch.Generator(device=DEV).manual_seed(11)
    ring = [wl.confidence_scores(B, gamma, g, DEV) for _ in range(3)]
    for t in range(2, 6):
        cur = wl.confidence_scores(B, gamma, g, DEV)
        ring[t % 3].copy_(cur)
        lagged = ring[(t - 2) % 3]
        got = _run(lagged, None, "argmax", 0.0, Bs, sps)
        ref = od.schedule_rule(lagged.cpu().numpy(), Bs, sps, "argmax")
        assert np.array_equal(got, ref.budget)
