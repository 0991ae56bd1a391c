"""Pins of the oracle's analytic acceptance c*_k = sum_v min(p_k, q_k) =
1 - TV(p_k, q_k) ("DSpark, la bozza ...", section "Verificare meglio, non di
più", eq. c*_k), the label of the confidence head and the quantity the
acceptance pass computes on the GPU:
  * by enumeration at V = 8 it is the probability that position k's accept test
    passes given the drafted prefix was accepted, computed from the exact
    acceptance rule min(1, p/q) (a different formula from sum min(p, q));
  * sampled rounds of the oracle's own verify accept position k at the mean of
    c* over the drafts that reach it;
  * identical distributions give 1, disjoint supports 0, greedy the indicator
    of the target argmax.
"""

import itertools
import math

import numpy as np
import pytest

from oracle import dspark as od
from test_oracle_round import V8, Problem, _run


@pytest.mark.parametrize("T", [0.7, 1.0, 1.5])
def test_c_star_is_the_conditional_accept_probability_by_enumeration(T):
    pb = Problem(3, T, seed=31 + int(10 * T))
    for xs in itertools.product(range(V8), repeat=3):
        drafts = np.array([xs], dtype=np.int32)
        base, prev0, Tv = pb.batch(1)
        tgt = pb.target_for(drafts)
        c = od.analytic_acceptance(tgt, base, pb.U, pb.W, prev0, drafts, Tv)[0]
        prev = pb.prev0
        for k in range(1, 4):
            p, q = pb.p(xs[:k - 1]), pb.q(k, prev)
            # E_{x ~ q} min(1, p(x)/q(x)): the accept rule averaged over the draw
            want = sum(q[x] * min(1.0, p[x] / q[x]) for x in range(V8) if q[x] > 0)
            assert c[k - 1] == pytest.approx(want, abs=1e-13)
            prev = xs[k - 1]


def test_sampled_accept_rate_matches_mean_c_star():
    pb = Problem(3, 1.0, seed=77)
    B = 6000
    dr, tgt, vr = _run(pb, B, seed=9, L=3)
    base, prev0, T = pb.batch(B)
    c = od.analytic_acceptance(tgt, base, pb.U, pb.W, prev0, dr.tokens, T)
    n = vr.num_accepted
    for k in range(1, 4):
        reach = n >= k - 1                     # positions 1..k-1 accepted
        acc = (n[reach] >= k).astype(float)    # position k accepted too
        m = reach.sum()
        mean_c = c[reach, k - 1].mean()
        assert abs(acc.mean() - mean_c) < 4 * math.sqrt(mean_c * (1 - mean_c) / m) + 1e-3


def test_identical_disjoint_and_greedy_cases():
    rng = np.random.default_rng(3)
    B, gamma, V, r = 4, 3, 50, 4
    tgt = rng.normal(0, 2, size=(B, gamma + 1, V))
    U, W = np.zeros((V, r)), np.zeros((r, V))
    prev0 = rng.integers(0, V, size=B).astype(np.int32)
    drafts = rng.integers(0, V, size=(B, gamma)).astype(np.int32)
    T = np.ones(B)
    same = od.analytic_acceptance(tgt, tgt[:, :gamma], U, W, prev0, drafts, T)
    assert np.allclose(same, 1.0, atol=1e-14)
    # disjoint supports: the target lives on even ids, the draft on odd ones
    far = np.where(np.arange(V) % 2 == 0, 0.0, -1e4)
    t2 = tgt + far
    b2 = tgt[:, :gamma] + (-1e4 - far)
    assert np.allclose(od.analytic_acceptance(t2, b2, U, W, prev0, drafts, T), 0.0, atol=1e-12)
    # greedy: 1 exactly where the draft token is the target's lowest-index maximum
    T0 = np.zeros(B)
    drafts[0, 0] = int(np.argmax(tgt[0, 0]))
    c0 = od.analytic_acceptance(tgt, tgt[:, :gamma], U, W, prev0, drafts, T0)
    want = np.array([[1.0 if drafts[b, k] == np.argmax(tgt[b, k]) else 0.0 for k in range(gamma)]
                     for b in range(B)])
    assert np.array_equal(c0, want) and c0[0, 0] == 1.0
