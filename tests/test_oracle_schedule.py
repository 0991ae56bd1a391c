"""Pins of the oracle's hardware-aware prefix scheduler against its statement on
"DSpark, la bozza ..." (section "Verificare meglio, non di più"): a_j is the
product of the confidences, candidates of all requests are queued by a_{r,j} and
admitted one at a time while Theta = tau SPS(B) grows, stopping at the first
candidate that does not raise it; SPS takes the verify batch in tokens.  The
load-aware behaviour (budgets shrink as concurrency grows) is the one the live
telemetry shows on the same page, section "I numeri, sul traffico vero".
"""

import numpy as np
import pytest

from lossless_rejection_sampling_amd import workloads as wl
from oracle import dspark as od


def _conf(B, gamma, seed, lo=0.05, hi=0.98):
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=(B, gamma)).astype(np.float32)


def test_prefix_survival_is_sequential_fp32_product():
    c = np.array([[0.9, 0.8, 0.7]], dtype=np.float32)
    a = od.prefix_survival(c)
    assert a[0, 0] == np.float32(0.9)
    assert a[0, 1] == np.float32(np.float32(0.9) * np.float32(0.8))
    assert a[0, 2] == np.float32(a[0, 1] * np.float32(0.7))
    with pytest.raises(ValueError):
        od.prefix_survival(np.array([[0.5, 1.0]], dtype=np.float32))


def test_constant_rate_admits_every_nonzero_candidate():
    c = _conf(12, 4, 1)
    c[3, 1] = 1e-6          # a[3, 1:] < 2^-32 -> Q = 0
    c[3, 0] = 1e-4
    Bs = np.array([1.0, 1024.0])
    res = od.schedule(c, Bs, np.array([50.0, 50.0]))
    want = np.full(12, 4)
    want[3] = 1
    assert np.array_equal(res.budget, want)


def test_rate_inverse_to_batch_admits_nothing():
    # t(N) proportional to N: Theta = tau / N starts at 2^32 per token, which no
    # candidate (a < 1) can raise
    Bs = np.array([1.0, 8.0, 64.0, 1024.0])
    res = od.schedule(_conf(16, 5, 2), Bs, 1.0 / Bs)
    assert np.all(res.budget == 0) and res.admitted == 0


def _theta(tau, N, Bs, sps):
    return tau * np.interp(N, Bs, sps)   # library interpolation of the rate table


@pytest.mark.parametrize("seed", range(5))
def test_admission_follows_the_greedy_early_stop_rule(seed):
    B, gamma = 40, 5
    c = _conf(B, gamma, 10 + seed, lo=0.2, hi=0.99)
    Bs, sps = wl.sps_table_linear()
    # step time (not the rate) is linear between table points
    res = od.schedule(c, Bs, sps)
    a = od.prefix_survival(c)
    Q = np.floor(a.astype(np.float64) * 2.0 ** 32)
    order = sorted(((-Q[b, j], b, j) for b in range(B) for j in range(gamma)))
    m = res.admitted
    admitted = {(b, j) for _, b, j in order[:m]}
    # admitted sets are prefixes and match the budgets
    for b in range(B):
        assert {(b, j) for j in range(res.budget[b])} == {x for x in admitted if x[0] == b}
    # Theta strictly increases along the admitted candidates and the next one fails
    t_pts = 1.0 / sps

    def t_of(N):
        return np.interp(N, Bs, t_pts)

    tau, N = float(B), float(B)
    th = tau / t_of(N)
    for k in range(m + 1):
        if k == len(order):
            break
        q = -order[k][0] / 2.0 ** 32
        nxt = (tau + q) / t_of(N + 1)
        if k < m:
            assert nxt > th * (1 - 1e-12)
            tau, N, th = tau + q, N + 1, nxt
        else:
            assert nxt <= th * (1 + 1e-12)
    assert res.min_gap > 1e-12


def test_budgets_shrink_as_concurrency_grows():
    Bs, sps = wl.sps_table_linear()
    rng = np.random.default_rng(3)
    big = (1.0 / (1.0 + np.exp(-rng.normal(1.5 - 0.4 * np.arange(1, 6), 1.0, size=(400, 5))))).astype(np.float32)
    prev = None
    for B in (10, 50, 100, 200, 400):
        res = od.schedule(big[:B], Bs, sps)
        if prev is not None:
            assert np.all(res.budget[:len(prev)] <= prev)
        prev = res.budget
    # at light load the budget reaches several positions, under load it shrinks
    light = od.schedule(big[:10], Bs, sps).budget.mean()
    heavy = od.schedule(big[:400], Bs, sps).budget.mean()
    assert light > heavy


def test_rejects_bad_tables():
    with pytest.raises(ValueError):
        od.schedule(_conf(2, 2, 0), np.array([4.0, 2.0]), np.array([1.0, 1.0]))
    with pytest.raises(ValueError):
        od.schedule(_conf(2, 2, 0), np.array([4.0]), np.array([1.0]))


def test_step_time_hand_computed_non_linear_table():
    # t = 1/SPS at B = 2, 6, 10 is 1, 3, 11 (slopes 1/2 then 2 per token): below
    # the first point the first value, linear inside each segment, and beyond the
    # last point the last segment extended.  Every value below is exact in fp64.
    Bs = [2.0, 6.0, 10.0]
    t_tab = [1.0, 3.0, 11.0]
    want = {0.0: 1.0, 1.0: 1.0, 2.0: 1.0, 4.0: 2.0, 6.0: 3.0, 7.0: 5.0, 8.0: 7.0, 10.0: 11.0,
            12.0: 15.0, 20.0: 31.0, 1000.0: 1991.0}
    for N, t in want.items():
        assert od.step_time(N, Bs, t_tab) == t, N
    # a plain clamp beyond the table or the first segment's slope would give
    # 11 / 7 at N = 12; the interpolation inside the table agrees with numpy's
    for N in np.linspace(2.0, 10.0, 33):
        assert od.step_time(float(N), Bs, t_tab) == pytest.approx(float(np.interp(N, Bs, t_tab)), rel=1e-15)


def test_scheduler_admission_crossing_the_last_table_point():
    # Two requests, two positions; the table ends at 3 tokens: t(1) = t(2) = 10,
    # t(3) = 12, so beyond it t(N) = 12 + 2 (N - 3).  Prefix survivals
    # a = (0.9, 0.72) and (0.5, 0.25), in units of 2^32 of tau:
    #   tau = 2,    N = 2: (2 + 0.9) t(2) = 29     > 2 t(3) = 24         admit
    #   tau = 2.9,  N = 3: (2.9 + 0.72) t(3) = 43.44 > 2.9 t(4) = 40.6   admit
    #   tau = 3.62, N = 4: (3.62 + 0.5) t(4) = 57.68 > 3.62 t(5) = 57.92 fails: stop
    # (a table clamped at its last value would admit all four candidates).
    conf = np.array([[0.9, 0.8], [0.5, 0.5]], dtype=np.float32)
    Bs = np.array([1.0, 2.0, 3.0])
    sps = 1.0 / np.array([10.0, 10.0, 12.0])
    res = od.schedule(conf, Bs, sps)
    assert res.budget.tolist() == [2, 0]
    assert res.admitted == 2
    flat = od.schedule(conf, Bs, 1.0 / np.array([10.0, 10.0, 10.0]))
    assert flat.budget.tolist() == [2, 2]
