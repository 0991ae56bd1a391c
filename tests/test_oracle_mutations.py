"""The oracle's pins are not vacuous: plausible mistakes planted in copies of
the oracle (on the CPU; the oracle itself is untouched) make a pin fail.

Each case replaces one line of `oracle/dspark.py` or `oracle/sampler.py` in a
copy that is loaded as a separate module, then runs pins' checks against that
copy:
  * the round pins of test_oracle_round.py (the drafted pairs against the
    draft's Markov conditionals, the emitted sequences against the target's own
    autoregressive distribution, the accept rates given the prefix against
    sum min(p, q)), at least one of which must fail: a residual with the wrong
    sign, the accept ratio inverted, the target's temperature dropped, the
    wrong target row for a test or for the final token, the wrong previous
    token in the verifier's or the drafter's Markov bias;
  * the hand-computed step times of a non-linear table (test_oracle_schedule.py):
    a table clamped at its last point, the first segment's slope everywhere;
  * the sequential fp32 prefix product (test_oracle_schedule.py): the product
    taken in fp64;
  * the scheduler pins (test_oracle_schedule.py): candidates in ascending
    order, tau started without the final tokens, the batch started empty;
  * the sampler's draws against softmax (test_oracle_sampler.py): tile masses
    taken as the tile's maximum, the leaf's Gumbel noise with the wrong sign;
    and the same sampler mistake seen through the round's pin.
The unmodified oracle passes the same checks (in their own test files, and
here for the cheap ones)."""

import os
import sys
import types

import numpy as np
import pytest
from scipy import stats

from oracle import dspark as od
from oracle import philox as px
from oracle import sampler as osampler

from test_oracle_round import V8, Problem, accept_rate_pvalue, draft_conditional_pvalue

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


def _mutant(fname, old, new, tag, sampler=None):
    """A copy of oracle/<fname> with `old` (which must occur once) replaced by
    `new` (old = None: an unchanged copy), loaded as its own module.
    `sampler`: a (mutated) sampler module the copy imports in place of
    oracle.sampler."""
    src = open(os.path.join(ORACLE, fname)).read()
    if old is not None:
        assert src.count(old) == 1, (fname, old)
        src = src.replace(old, new)
    name = f"oracle._mutant_{tag}"
    mod = types.ModuleType(name)
    mod.__package__ = "oracle"
    mod.__file__ = f"<mutant {tag} of {fname}>"
    sys.modules[name] = mod  # dataclasses look their module up
    saved = sys.modules.get("oracle.sampler")
    try:
        if sampler is not None:
            sys.modules["oracle.sampler"] = sampler
        exec(compile(src, mod.__file__, "exec"), mod.__dict__)
    finally:
        if sampler is not None:
            sys.modules["oracle.sampler"] = saved
    return mod


def _emitted_pvalue(m, T, B=2500, seed=7):
    """p-value of the chi-square test of the emitted 3-token sequences of B
    sampled rounds (gamma = 2, budget 2) against the target distribution."""
    pb = Problem(2, T, seed=42)
    base, prev0, temps = pb.batch(B)
    dr = m.draft_round(base, pb.U, pb.W, prev0, temps, seed)
    tgt = pb.target_for(dr.tokens)
    vr = m.verify(tgt, base, pb.U, pb.W, prev0, dr.tokens, temps, seed, np.full(B, 2))
    rng = np.random.default_rng(0)
    seqs = []
    for b in range(B):
        s = tuple(int(t) for t in vr.out_tokens[b, :vr.num_emitted[b]])
        while len(s) < 3:
            s = s + (int(rng.choice(V8, p=pb.p(s))),)
        seqs.append(s[0] * 64 + s[1] * 8 + s[2])
    p = np.array([pb.target_seq_prob((i // 64, (i // 8) % 8, i % 8)) for i in range(512)])
    counts = np.bincount(seqs, minlength=512).astype(float)
    big = p * B >= 5
    o = np.append(counts[big], counts[~big].sum())
    e = np.append(p[big], p[~big].sum()) * B
    return stats.chisquare(o, e).pvalue


VERIFY_MUTANTS = [
    ("residual_sign", "r = np.maximum(0.0, p - q)", "r = np.maximum(0.0, q - p)", 1.0),
    ("accept_ratio_inverted", "ok = ln_u < lp - lq ", "ok = ln_u < lq - lp ", 1.0),
    ("target_temperature_dropped", "lp = z[x] / T - logsumexp(z / T)", "lp = z[x] - logsumexp(z)", 0.7),
    ("test_on_next_target_row", "            z = target[b, k - 1]\n            x = xs[k]",
     "            z = target[b, k]\n            x = xs[k]", 1.0),
    ("final_token_from_previous_row", "        z = target[b, n]\n", "        z = target[b, max(n - 1, 0)]\n", 1.0),
    ("verifier_bias_of_wrong_token", "dq = draft_logits(base[b, k - 1], U, W, xs[k - 1]) / T",
     "dq = draft_logits(base[b, k - 1], U, W, xs[k]) / T", 1.0),
    ("drafter_bias_of_first_token", "prev = tokens[:, k - 1].astype(np.int64)",
     "prev = np.asarray(prev0, dtype=np.int64)", 1.0),
]


def _round_pin_fails(m, T):
    """True when one of the round pins rejects module m (p below the pins'
    1e-4), cheapest first."""
    return (draft_conditional_pvalue(m, T=T) < 1e-4 or _emitted_pvalue(m, T) < 1e-4
            or accept_rate_pvalue(m, T=T) < 1e-4)


@pytest.mark.parametrize("tag,old,new,T", VERIFY_MUTANTS, ids=[c[0] for c in VERIFY_MUTANTS])
def test_round_pins_catch(tag, old, new, T):
    assert _round_pin_fails(_mutant("dspark.py", old, new, tag), T)


def _step_time_matches_hand_values(m):
    Bs, t_tab = [2.0, 6.0, 10.0], [1.0, 3.0, 11.0]
    want = {0.0: 1.0, 4.0: 2.0, 7.0: 5.0, 10.0: 11.0, 12.0: 15.0, 1000.0: 1991.0}
    return all(m.step_time(N, Bs, t_tab) == t for N, t in want.items())


@pytest.mark.parametrize("tag,old,new", [
    ("clamped_beyond_the_table", "    if N <= sps_B[0]:\n        return t_tab[0]\n",
     "    if N <= sps_B[0]:\n        return t_tab[0]\n    if N >= sps_B[-1]:\n        return t_tab[-1]\n"),
    ("first_segment_everywhere", "    while i + 1 < n - 1 and sps_B[i + 1] <= N:", "    while False:"),
])
def test_step_time_pin_catches(tag, old, new):
    assert _step_time_matches_hand_values(od)
    assert not _step_time_matches_hand_values(_mutant("dspark.py", old, new, tag))


def _prefix_is_sequential_fp32(m):
    conf = np.random.default_rng(5).uniform(0.05, 0.95, size=(4, 16)).astype(np.float32)
    a = m.prefix_survival(conf)
    for b in range(conf.shape[0]):
        acc = np.float32(1.0)
        for j in range(conf.shape[1]):
            acc = np.float32(acc * conf[b, j])
            if a[b, j] != acc:
                return False
    return True


def test_prefix_product_pin_catches_fp64():
    # the product kept in fp64 and rounded only when stored
    assert _prefix_is_sequential_fp32(od)
    m = _mutant("dspark.py", "acc = np.float32(acc * c[b, j])", "acc = np.float64(acc) * np.float64(c[b, j])",
                "fp64_product")
    assert not _prefix_is_sequential_fp32(m)


def _sampler_pvalue(s_mod, n=6000):
    s = np.random.default_rng(11).normal(0.0, 1.5, size=160)  # one block of three tiles, the last ragged
    streams = (px.DRAFT_TOP, px.DRAFT_MID, px.DRAFT_LEAF)
    x = np.array([s_mod.tree_sample(s, 3, streams, b, 1)[0] for b in range(n)])
    p = np.exp(s - s.max())
    p /= p.sum()
    counts = np.bincount(x, minlength=s.size).astype(float)
    big = p * n >= 5
    o = np.append(counts[big], counts[~big].sum())
    e = np.append(p[big], p[~big].sum()) * n
    return stats.chisquare(o, e).pvalue


SAMPLER_MUTANTS = [
    ("tile_mass_as_tile_max",
     "t_lam = np.array([logsumexp(s[lo + t * TILE:min(lo + (t + 1) * TILE, hi)]) for t in range(nt)])",
     "t_lam = np.array([np.max(s[lo + t * TILE:min(lo + (t + 1) * TILE, hi)]) for t in range(nt)])"),
    ("leaf_gumbel_sign", "e, m_leaf = pick(s[tl:th] - t_lam[t] + g, cond)", "e, m_leaf = pick(s[tl:th] - t_lam[t] - g, cond)"),
]


def test_sampler_pin_passes_on_the_oracle():
    assert _sampler_pvalue(osampler) > 1e-4


@pytest.mark.parametrize("tag,old,new", SAMPLER_MUTANTS, ids=[c[0] for c in SAMPLER_MUTANTS])
def test_sampler_pin_catches(tag, old, new):
    assert _sampler_pvalue(_mutant("sampler.py", old, new, tag)) < 1e-6


def test_a_sampler_mistake_reaches_the_round():
    # the round's pin sees a sampler mistake too: the drafter and verifier built
    # on the mutated sampler (its draws no longer follow q)
    s_mod = _mutant("sampler.py", SAMPLER_MUTANTS[1][1], SAMPLER_MUTANTS[1][2], "leaf_gumbel_sign_round")
    m = _mutant("dspark.py", None, None, "round_on_mutant_sampler", sampler=s_mod)
    assert _round_pin_fails(m, 1.0)


# (Skipping a failed candidate instead of stopping is no mistake in this rule:
# a failure leaves tau and N unchanged and the test is monotone in Q, so every
# later candidate, whose Q is no larger, fails too.)
SCHEDULE_MUTANTS = [
    ("ascending_order", "cand = sorted((-int(Q[b, j]), b, j) for b in range(B) for j in range(gamma))",
     "cand = sorted((int(Q[b, j]), b, j) for b in range(B) for j in range(gamma))"),
    ("no_final_tokens_in_tau", "    tau = B << 32\n", "    tau = 0\n"),
    ("empty_initial_batch", "    N = B\n    budget = np.zeros(B, dtype=np.int32)\n",
     "    N = 0\n    budget = np.zeros(B, dtype=np.int32)\n"),
]


def _schedule_pins_fail(m, monkeypatch):
    """True when one of the scheduler pins of test_oracle_schedule.py fails
    (raises) with module m in place of the oracle."""
    import test_oracle_schedule as ts
    monkeypatch.setattr(ts, "od", m)
    pins = [lambda: ts.test_admission_follows_the_greedy_early_stop_rule(s) for s in range(3)]
    pins += [ts.test_scheduler_admission_crossing_the_last_table_point, ts.test_constant_rate_admits_every_nonzero_candidate,
             ts.test_budgets_shrink_as_concurrency_grows]
    for pin in pins:
        try:
            pin()
        except Exception:
            return True
    return False


def test_schedule_pins_pass_on_the_oracle(monkeypatch):
    assert not _schedule_pins_fail(od, monkeypatch)


@pytest.mark.parametrize("tag,old,new", SCHEDULE_MUTANTS, ids=[c[0] for c in SCHEDULE_MUTANTS])
def test_schedule_pins_catch(tag, old, new, monkeypatch):
    assert _schedule_pins_fail(_mutant("dspark.py", old, new, tag), monkeypatch)
