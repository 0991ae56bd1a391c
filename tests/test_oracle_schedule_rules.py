"""Pins of the oracle's scheduler variants against what the pages state
("DSpark, la bozza ...", sections "Verificare meglio, non di più" and "Che cosa
resta da verificare"; "DSpark : le pari de DeepSeek ...", section "Vérifier
seulement ce qui compte"):
  * Sequential Temperature Scaling changes the magnitude of the scores, never
    their order, and undoes a logit-scale overconfidence;
  * the production rule takes the cut with the largest Theta = tau SPS(B) over
    the sorted candidates (no early stop) -- checked by brute force -- and on a
    stepped capacity curve it admits tokens the early-stop rule refuses;
  * the fixed-length (MTP-k) and fixed-threshold baselines;
  * the expected throughput Theta the schedulers are compared by.
"""

import math

import numpy as np
import pytest

from lossless_rejection_sampling_amd import workloads as wl
from oracle import dspark as od


def _conf(B, gamma, seed, lo=0.05, hi=0.98):
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=(B, gamma)).astype(np.float32)


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def test_sts_unit_temperature_is_the_identity():
    c = _conf(30, 6, 1)
    out, near = od.calibrate_scores(c, np.ones(6, np.float32))
    assert np.array_equal(out, c) and not near.any()


def test_sts_keeps_the_order_and_moves_towards_one_half():
    c = np.sort(_conf(1, 400, 2)[0])[None, :]
    for t in (0.5, 2.0, 7.0):
        out, _ = od.calibrate_scores(c, np.full(400, t, np.float32))
        assert np.all(np.diff(out[0].astype(np.float64)) >= 0)          # order kept
        d_in, d_out = np.abs(c[0] - 0.5), np.abs(out[0] - 0.5)
        assert np.all(d_out <= d_in + 1e-7) if t > 1 else np.all(d_out >= d_in - 1e-7)
    out, _ = od.calibrate_scores(c, np.full(400, 1e6, np.float32))
    assert np.allclose(out, 0.5, atol=1e-5)


@pytest.mark.parametrize("kappa", [1.5, 3.0])
def test_sts_undoes_a_logit_scale_overconfidence(kappa):
    # raw = sigma(kappa * logit(c)); temperature kappa maps it back to c
    c = _conf(50, 4, 3, lo=0.1, hi=0.9).astype(np.float64)
    raw = _sigmoid(kappa * (np.log(c) - np.log1p(-c))).astype(np.float32)
    out, _ = od.calibrate_scores(raw, np.full(4, kappa, np.float32))
    assert np.allclose(out, c, rtol=2e-6, atol=1e-7)


def _brute_force_best_cut(c, Bs, sps):
    """Independent Theta along the sorted candidates: keys by numpy lexsort,
    step time by numpy's own interpolation of 1/SPS, every cut enumerated."""
    a = od.prefix_survival(c).astype(np.float64)
    B, gamma = a.shape
    Q = np.floor(a * 2.0 ** 32)
    b_idx, j_idx = np.meshgrid(np.arange(B), np.arange(gamma), indexing="ij")
    order = np.lexsort((j_idx.ravel(), b_idx.ravel(), -Q.ravel()))
    t = lambda N: np.interp(N, Bs, 1.0 / sps)
    tau = B * 2.0 ** 32 + np.concatenate([[0.0], np.cumsum(Q.ravel()[order])])
    theta = tau / t(B + np.arange(len(tau)))
    m = int(np.argmax(theta))
    budget = np.zeros(B, np.int32)
    for k in order[:m]:
        budget[k // gamma] = max(budget[k // gamma], k % gamma + 1)
    top2 = np.sort(theta)[-2:]
    return budget, m, (top2[1] - top2[0]) / top2[1]


@pytest.mark.parametrize("seed", range(6))
def test_best_cut_rule_matches_brute_force(seed):
    B, gamma = 24, 5
    c = _conf(B, gamma, 20 + seed, lo=0.2, hi=0.99)
    Bs, sps = wl.sps_table_linear()
    res = od.schedule_rule(c, Bs, sps, "argmax")
    want, m, gap = _brute_force_best_cut(c, Bs, sps)
    if gap < 1e-9:
        pytest.skip("two cuts tie to rounding")
    assert res.admitted == m
    assert np.array_equal(res.budget, want)


def test_best_cut_goes_past_a_dip_the_early_stop_halts_at():
    # a capacity curve with a step: the batch of 10 tokens costs as much as 14,
    # so Theta drops at the step and rises again after it
    c = np.full((8, 3), 0.95, np.float32)
    Bs = np.array([1.0, 9.0, 10.0, 14.0, 40.0])
    t = np.array([1.0, 1.0, 1.6, 1.6, 3.0])
    sps = 1.0 / t
    early = od.schedule_rule(c, Bs, sps, "early_stop")
    best = od.schedule_rule(c, Bs, sps, "argmax")
    assert early.admitted == 1          # the second candidate crosses the step
    assert best.admitted > early.admitted
    th = lambda r: od.expected_theta(c, r.budget, Bs, sps)[2]
    assert th(best) > th(early)


@pytest.mark.parametrize("seed", range(4))
def test_rules_agree_when_theta_is_unimodal(seed):
    # linear step time and scores sorted high-to-low along each request: Theta
    # rises then falls once, so the first drop is also the best cut
    c = np.sort(_conf(32, 5, 40 + seed, lo=0.3, hi=0.99), axis=1)[:, ::-1].copy()
    Bs, sps = np.array([1.0, 2048.0]), 1.0 / np.array([100.0, 100.0 + 2047.0 * 0.5])
    early = od.schedule_rule(c, Bs, sps, "early_stop")
    best = od.schedule_rule(c, Bs, sps, "argmax")
    assert np.array_equal(early.budget, best.budget)


def test_fixed_and_threshold_baselines():
    c = np.array([[0.9, 0.8, 0.6, 0.95],
                  [0.5, 0.99, 0.99, 0.99],
                  [0.71, 0.7, 0.9, 0.9]], np.float32)
    for k, want in [(1, 1), (3, 3), (9, 4), (-2, 0)]:
        assert np.array_equal(od.schedule_rule(c, None, None, "fixed", k).budget, [want] * 3)
    thr = od.schedule_rule(c, None, None, "threshold", 0.7)
    assert np.array_equal(thr.budget, [2, 0, 1])      # strictly above 0.7, leading run only


def test_expected_theta_by_hand():
    c = np.array([[0.5, 0.5], [0.9, 0.1]], np.float32)
    Bs, sps = np.array([1.0, 11.0]), np.array([1.0, 0.5])     # t(N) = 1 + (N - 1) / 10
    tok, N, theta = od.expected_theta(c, [1, 2], Bs, sps)
    a01 = float(np.float32(np.float32(0.9) * np.float32(0.1)))
    assert tok == pytest.approx(2.0 + 0.5 + 0.9 + a01, abs=1e-7)
    assert N == 5.0
    assert theta == pytest.approx(tok / 1.4, rel=1e-12)


def test_scheduled_rules_on_the_scheduled_workload():
    # the fixed-threshold and MTP baselines against the early-stop scheduler on
    # the synthetic scheduled workload's scores (Theta comparison, no GPU)
    rng = np.random.default_rng(7)
    B, gamma = 128, 5
    j = np.arange(1, gamma + 1)
    c = _sigmoid(rng.normal(1.5 - 0.4 * j, 1.0, size=(B, gamma))).astype(np.float32)
    Bs, sps = wl.sps_table_linear()
    th = {}
    for rule, p in [("early_stop", 0), ("argmax", 0), ("fixed", 1), ("fixed", 5), ("threshold", 0.7)]:
        r = od.schedule_rule(c, Bs, sps, rule, p)
        th[(rule, p)] = od.expected_theta(c, r.budget, Bs, sps)[2]
    # the best cut is by definition at least as good as any prefix cut of the
    # same order, the early stop included
    assert th[("argmax", 0)] >= th[("early_stop", 0)]
    assert all(math.isfinite(v) and v > 0 for v in th.values())
