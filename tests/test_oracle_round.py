"""Pins of the oracle's draft round and verify against what the pages fix.

* Losslessness ("Les mathématiques ...", section "La garantie de
  l'échantillonnage par rejet": the output is statistically identical to plain
  autoregressive decoding): exact enumeration of the rule at V = 8, and a
  chi-square test of the oracle's sampled rounds against the target's own
  autoregressive distribution.
* Expected tokens per pass (same page, section "Rendement attendu ..."): the
  closed form and its worked value at gamma = 4, alpha = 0.7.
* Analytic acceptance ("DSpark, la bozza ...", section "Verificare meglio, non di
  più", eq. c*): P(accept) = 1 - TV(p, q) = sum_v min(p_v, q_v), at the first
  position and, given the drafted token, at the second.
* The draft's Markov conditioning ("DSpark, la bozza ...", eq. p_k): the drafted
  pairs (x_1, x_2) follow q_1(x_1 | prev0) q_2(x_2 | x_1).
* Special cases: greedy = longest matching prefix, q = p always accepts,
  disjoint supports always reject; structural invariants.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
from scipy import stats

from oracle import dspark as od

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
V8 = 8


def softmax(s):
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - s.max())
    return e / e.sum()


class Problem:
    """A tiny round: prefix-dependent target table, fixed backbone logits, rank-2
    Markov head, one previous token shared by every request."""

    def __init__(self, gamma, T, seed, r=2, prefix_dependent=True):
        rng = np.random.default_rng(seed)
        self.gamma, self.T = gamma, T
        self.base = rng.normal(0, 1.2, size=(gamma, V8))
        self.U = rng.normal(0, 0.8, size=(V8, r))
        self.W = rng.normal(0, 0.8, size=(r, V8))
        self.prev0 = 3
        self.table = {}
        shared = rng.normal(0, 1.5, size=V8)
        for m in range(gamma + 2):
            for pre in itertools.product(range(V8), repeat=m):
                self.table[pre] = rng.normal(0, 1.5, size=V8) if prefix_dependent else shared

    def p(self, prefix):
        return softmax(self.table[tuple(prefix)] / self.T)

    def q(self, k, prev):
        return softmax((self.base[k - 1] + self.U[prev] @ self.W) / self.T)

    def target_seq_prob(self, seq):
        pr = 1.0
        for i, s in enumerate(seq):
            pr *= self.p(seq[:i])[s]
        return pr

    def batch(self, B):
        base = np.broadcast_to(self.base, (B, self.gamma, V8)).copy()
        prev0 = np.full(B, self.prev0, dtype=np.int32)
        T = np.full(B, self.T)
        return base, prev0, T

    def target_for(self, drafts):
        B = drafts.shape[0]
        tgt = np.zeros((B, self.gamma + 1, V8))
        for b in range(B):
            for j in range(self.gamma + 1):
                tgt[b, j] = self.table[tuple(int(t) for t in drafts[b, :j])]
        return tgt


def exact_emitted_distribution(pb: Problem, L):
    """Probability of every length-(L+1) sequence produced by one round with
    budget L (emitted tokens, extended with target draws), by enumeration of
    the acceptance / residual / bonus rule."""
    dist = {}

    def extend(prefix, pr):
        if len(prefix) == L + 1:
            dist[prefix] = dist.get(prefix, 0.0) + pr
            return
        for v, pv in enumerate(pb.p(prefix)):
            if pv > 0:
                extend(prefix + (v,), pr * pv)

    for xs in itertools.product(range(V8), repeat=L):
        w, prev = 1.0, pb.prev0
        for k, x in enumerate(xs, 1):
            w *= pb.q(k, prev)[x]
            prev = x
        if w == 0:
            continue
        reach = w
        prev = pb.prev0
        for k in range(1, L + 1):
            x = xs[k - 1]
            p, q = pb.p(xs[:k - 1]), pb.q(k, prev)
            acc = min(1.0, p[x] / q[x])
            rej = reach * (1.0 - acc)
            if rej > 0:
                r = np.maximum(0.0, p - q)
                r = r / r.sum() if r.sum() > 0 else p
                for y in range(V8):
                    if r[y] > 0:
                        extend(tuple(xs[:k - 1]) + (y,), rej * r[y])
            reach *= acc
            prev = x
        p_bonus = pb.p(xs)
        for y in range(V8):
            if p_bonus[y] > 0:
                extend(tuple(xs) + (y,), reach * p_bonus[y])
    return dist


@pytest.mark.parametrize("gamma", [1, 2, 3])
@pytest.mark.parametrize("T", [0.7, 1.0, 1.5])
def test_rule_is_lossless_by_enumeration(gamma, T):
    pb = Problem(gamma, T, seed=10 * gamma + int(10 * T))
    for L in range(0, gamma + 1):
        dist = exact_emitted_distribution(pb, L)
        assert sum(dist.values()) == pytest.approx(1.0, abs=1e-12)
        for seq in itertools.product(range(V8), repeat=L + 1):
            assert dist.get(seq, 0.0) == pytest.approx(pb.target_seq_prob(seq), abs=1e-12)


def _run(pb: Problem, B, seed, L=None):
    base, prev0, T = pb.batch(B)
    dr = od.draft_round(base, pb.U, pb.W, prev0, T, seed)
    tgt = pb.target_for(dr.tokens)
    budget = None if L is None else np.full(B, L)
    vr = od.verify(tgt, base, pb.U, pb.W, prev0, dr.tokens, T, seed, budget)
    return dr, tgt, vr


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_sampled_rounds_follow_target_distribution(T):
    pb = Problem(2, T, seed=42)
    B, L = 6000, 2
    dr, tgt, vr = _run(pb, B, seed=1000 + int(T * 10), L=L)
    rng = np.random.default_rng(0)
    seqs = []
    for b in range(B):
        s = tuple(int(t) for t in vr.out_tokens[b, :vr.num_emitted[b]])
        while len(s) < L + 1:
            s = s + (int(rng.choice(V8, p=pb.p(s))),)
        seqs.append(s[0] * 64 + s[1] * 8 + s[2])
    p = np.array([pb.target_seq_prob((i // 64, (i // 8) % 8, i % 8)) for i in range(512)])
    counts = np.bincount(seqs, minlength=512).astype(float)
    big = p * B >= 5
    o = np.append(counts[big], counts[~big].sum())
    e = np.append(p[big], p[~big].sum()) * B
    assert stats.chisquare(o, e).pvalue > 1e-4
    # first emitted token alone
    first = vr.out_tokens[:, 0]
    assert stats.chisquare(np.bincount(first, minlength=8), pb.p(()) * B).pvalue > 1e-4


def _alpha_problem(gamma, alpha_target, seed=3):
    """Prefix-independent target and draft with sum_v min(p, q) = alpha_target,
    built by bisecting a shift of the draft logits (no Markov bias: W = 0)."""
    pb = Problem(gamma, 1.0, seed=seed, prefix_dependent=False)
    pb.W[:] = 0.0
    p_log = pb.table[()]
    direction = np.linspace(-1.0, 1.0, V8)

    def alpha(lmb):
        q = softmax(p_log + lmb * direction)
        return np.minimum(softmax(p_log), q).sum()

    lo, hi = 0.0, 1.0
    while alpha(hi) > alpha_target:
        hi *= 2
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        (lo, hi) = (mid, hi) if alpha(mid) > alpha_target else (lo, mid)
    lmb = 0.5 * (lo + hi)
    pb.base[:] = p_log + lmb * direction
    return pb, alpha(lmb)


def test_expected_tokens_per_pass_closed_form():
    with open(os.path.join(GOLDEN, "expected_tokens_per_pass.json")) as f:
        gold = json.load(f)
    for case in gold["cases"]:
        g, a = case["gamma"], case["alpha"]
        closed = (1 - a ** (g + 1)) / (1 - a)
        assert abs(closed - case["printed"]) <= case["printed_precision"]
        pb, alpha = _alpha_problem(g, a)
        assert alpha == pytest.approx(a, abs=1e-14)
        B = 5000
        dr, tgt, vr = _run(pb, B, seed=77)
        mean = vr.num_emitted.mean()
        se = vr.num_emitted.std() / math.sqrt(B)
        assert abs(mean - closed) < 4 * se, (mean, closed, se)
        # per-position survival P(n >= j) = alpha^j
        for j in range(1, g + 1):
            frac = (vr.num_accepted >= j).mean()
            assert abs(frac - a ** j) < 4 * math.sqrt(a ** j * (1 - a ** j) / B) + 1e-3


def test_yield_approaches_block_plus_one_at_high_alpha():
    # the page notes the yield nears gamma + 1 at alpha = 0.9
    g = 4
    assert (1 - 0.9 ** (g + 1)) / (1 - 0.9) > 0.8 * (g + 1)


def draft_conditional_pvalue(m=od, T=1.0, B=4000, seed=31):
    """p-value of the drafted pairs (x_1, x_2) of B rounds against the joint
    q_1(x_1 | prev0) q_2(x_2 | x_1) of the draft definition ("DSpark, la bozza
    ...", eq. p_k: the Markov bias of position k is that of the token drawn at
    k - 1)."""
    pb = Problem(2, T, seed=17)
    base, prev0, temps = pb.batch(B)
    dr = m.draft_round(base, pb.U, pb.W, prev0, temps, seed)
    x1, x2 = dr.tokens[:, 0].astype(int), dr.tokens[:, 1].astype(int)
    q1 = pb.q(1, pb.prev0)
    exp = np.array([q1[a] * pb.q(2, a)[c] for a in range(V8) for c in range(V8)]) * B
    obs = np.bincount(x1 * V8 + x2, minlength=V8 * V8).astype(float)
    big = exp >= 5
    return stats.chisquare(np.append(obs[big], obs[~big].sum()), np.append(exp[big], exp[~big].sum())).pvalue


def accept_rate_pvalue(m=od, T=1.0, B=6000, seed=37):
    """p-value of the accept counts of B rounds at position 1 and, grouped by
    the drafted x_1, at position 2, against sum_v min(p_k, q_k) of the
    problem's own distributions (the probability that u < min(1, p/q) when
    x ~ q; "Les mathématiques ...", section "La garantie de l'échantillonnage
    par rejet")."""
    pb = Problem(2, T, seed=19)
    base, prev0, temps = pb.batch(B)
    dr = m.draft_round(base, pb.U, pb.W, prev0, temps, seed)
    tgt = pb.target_for(dr.tokens)
    vr = m.verify(tgt, base, pb.U, pb.W, prev0, dr.tokens, temps, seed, np.full(B, 2))
    n = np.asarray(vr.num_accepted)
    c1 = np.minimum(pb.p(()), pb.q(1, pb.prev0)).sum()
    k1 = int((n >= 1).sum())
    chi2, df = (k1 - B * c1) ** 2 / (B * c1 * (1 - c1)), 1
    x1 = dr.tokens[:, 0]
    for a in range(V8):
        sel = (n >= 1) & (x1 == a)
        N = int(sel.sum())
        c2 = np.minimum(pb.p((a,)), pb.q(2, a)).sum()
        if N < 30 or not 0 < c2 < 1:
            continue
        k = int((n[sel] >= 2).sum())
        chi2 += (k - N * c2) ** 2 / (N * c2 * (1 - c2))
        df += 1
    return stats.chi2.sf(chi2, df)


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_draft_tokens_follow_the_markov_conditionals(T):
    assert draft_conditional_pvalue(T=T) > 1e-4


@pytest.mark.parametrize("T", [1.0, 0.7])
def test_accept_rates_given_the_prefix(T):
    assert accept_rate_pvalue(T=T) > 1e-4


def test_single_position_acceptance_equals_one_minus_tv():
    pb = Problem(1, 1.0, seed=8, prefix_dependent=False)
    B = 8000
    dr, tgt, vr = _run(pb, B, seed=5)
    p, q = pb.p(()), pb.q(1, pb.prev0)
    c_star = 1 - 0.5 * np.abs(p - q).sum()
    assert c_star == pytest.approx(np.minimum(p, q).sum(), abs=1e-15)
    rate = vr.num_accepted.mean()
    assert abs(rate - c_star) < 4 * math.sqrt(c_star * (1 - c_star) / B)


def test_greedy_is_longest_matching_prefix():
    rng = np.random.default_rng(2)
    for trial in range(30):
        gamma, V, B = 4, 16, 12
        tgt = rng.normal(0, 1, size=(B, gamma + 1, V))
        base = rng.normal(0, 1, size=(B, gamma, V))
        # make the draft agree with the target argmax on a random prefix
        for b in range(B):
            agree = rng.integers(0, gamma + 1)
            for k in range(agree):
                base[b, k] = tgt[b, k] * 3
        U, W = np.zeros((V, 2)), np.zeros((2, V))
        prev0 = rng.integers(0, V, size=B).astype(np.int32)
        T = np.zeros(B)
        budget = rng.integers(0, gamma + 1, size=B)
        dr = od.draft_round(base, U, W, prev0, T, 1)
        vr = od.verify(tgt, base, U, W, prev0, dr.tokens, T, 1, budget)
        for b in range(B):
            n = vr.num_accepted[b]
            for k in range(n):
                assert dr.tokens[b, k] == np.argmax(tgt[b, k])
            if n < budget[b]:
                assert dr.tokens[b, n] != np.argmax(tgt[b, n])
            assert vr.out_tokens[b, n] == np.argmax(tgt[b, n])
            assert np.all(dr.tokens[b] == np.argmax(base[b], axis=1))


def test_greedy_ties_go_to_lowest_index():
    tgt = np.zeros((1, 2, 8))
    tgt[0, 0, [2, 5]] = 4.0
    base = np.zeros((1, 1, 8))
    base[0, 0, [5, 2]] = 3.0
    U, W = np.zeros((8, 1)), np.zeros((1, 8))
    dr = od.draft_round(base, U, W, [0], [0.0], 0)
    assert dr.tokens[0, 0] == 2
    vr = od.verify(tgt, base, U, W, [0], dr.tokens, [0.0], 0)
    assert vr.num_accepted[0] == 1 and vr.out_tokens[0, 1] == 0


def test_identical_draft_always_accepted():
    pb = Problem(3, 1.0, seed=12, prefix_dependent=False)
    pb.W[:] = 0.0
    pb.base[:] = pb.table[()]
    B = 2500
    dr, tgt, vr = _run(pb, B, seed=9)
    assert np.all(vr.num_accepted == 3)
    bonus = vr.out_tokens[:, 3]
    assert stats.chisquare(np.bincount(bonus, minlength=8), pb.p(()) * B).pvalue > 1e-4


def test_disjoint_supports_always_reject():
    pb = Problem(3, 1.0, seed=13, prefix_dependent=False)
    pb.W[:] = 0.0
    t = np.array([0.5, -0.3, 1.0, 0.0, -1e4, -1e4, -1e4, -1e4])
    for key in pb.table:
        pb.table[key] = t
    pb.base[:] = np.array([-1e4] * 4 + [0.2, 0.1, -0.4, 0.9])
    B = 2500
    dr, tgt, vr = _run(pb, B, seed=4)
    assert np.all(vr.num_accepted == 0)
    y = vr.out_tokens[:, 0]
    p = softmax(t)
    assert np.all(y < 4)
    assert stats.chisquare(np.bincount(y, minlength=8)[:4], p[:4] * B).pvalue > 1e-4


@pytest.mark.parametrize("seed", range(4))
def test_structural_invariants(seed):
    rng = np.random.default_rng(100 + seed)
    B, gamma, V, r = 24, 5, 300, 4
    tgt = rng.normal(0, 2, size=(B, gamma + 1, V))
    base = tgt[:, :gamma] + rng.normal(0, 0.8, size=(B, gamma, V))
    U, W = rng.normal(0, 0.5, size=(V, r)), rng.normal(0, 0.5, size=(r, V))
    prev0 = rng.integers(0, V, size=B)
    T = rng.choice([0.0, 0.7, 1.0, 1.5], size=B)
    budget = rng.integers(0, gamma + 1, size=B)
    dr = od.draft_round(base, U, W, prev0, T, seed)
    vr = od.verify(tgt, base, U, W, prev0, dr.tokens, T, seed, budget)
    for b in range(B):
        n = vr.num_accepted[b]
        assert 0 <= n <= budget[b] <= gamma
        assert vr.num_emitted[b] == n + 1 <= gamma + 1
        row = vr.out_tokens[b]
        assert np.all(row[:n] == dr.tokens[b, :n])
        assert 0 <= row[n] < V
        assert np.all(row[n + 1:] == -1)
    assert np.all((dr.tokens >= 0) & (dr.tokens < V))
    # log q of greedy positions is 0; otherwise it is a log-probability
    assert np.all(dr.logq[T == 0] == 0)
    assert np.all(dr.logq[T > 0] <= 0)
