"""Pins of the oracle's three-level Gumbel-max sampler.

What the method fixes is the distribution of a draw: P(v) = softmax(s)_v.  The
sampler is checked against it by chi-square tests over many independent
(request, position) streams, at sizes with one tile, one ragged block, and
several blocks with a ragged tail; plus the structural properties a categorical
sampler must have (excluded entries never drawn, ties to the lowest index).
"""

import math

import numpy as np
import pytest
from scipy import stats

from oracle import philox as px
from oracle.sampler import BLOCK, TILE, logsumexp, pick, tree_sample

STREAMS = (px.DRAFT_TOP, px.DRAFT_MID, px.DRAFT_LEAF)


def _draws(s, n, seed=3):
    return np.array([tree_sample(s, seed, STREAMS, b, 1)[0] for b in range(n)])


def _chisq(obs_idx, p, min_expected=5.0):
    n = obs_idx.size
    counts = np.bincount(obs_idx, minlength=p.size).astype(float)
    exp = p * n
    big = exp >= min_expected
    o = np.append(counts[big], counts[~big].sum())
    e = np.append(exp[big], exp[~big].sum())
    if e[-1] == 0:
        o, e = o[:-1], e[:-1]
    return stats.chisquare(o, e).pvalue


def softmax(s):
    return np.exp(s - logsumexp(s))


def test_single_tile_matches_softmax():
    s = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.4, 0.7, 1.9])
    assert _chisq(_draws(s, 8000), softmax(s)) > 1e-4


def test_one_ragged_block_matches_softmax():
    rng = np.random.default_rng(0)
    s = rng.normal(0, 1.5, size=1000)           # 16 tiles, last one has 40 elements
    x = _draws(s, 6000)
    p = softmax(s)
    # per tile and for the 30 most likely single tokens
    tile = x // TILE
    pt = np.array([p[t * TILE:(t + 1) * TILE].sum() for t in range(-(-s.size // TILE))])
    assert _chisq(tile, pt) > 1e-4
    top = np.argsort(-p)[:30]
    counts = np.array([(x == v).sum() for v in top])
    assert stats.chisquare(np.append(counts, x.size - counts.sum()),
                           np.append(p[top], 1 - p[top].sum()) * x.size).pvalue > 1e-4


def test_several_blocks_with_ragged_tail():
    rng = np.random.default_rng(1)
    V = 2 * BLOCK + 700                       # 3 blocks, the last has 11 tiles, ragged
    s = rng.normal(0, 1.0, size=V)
    s[2 * BLOCK + 650] += 6.0                 # a hot token in the ragged tail
    s[100] += 5.0
    x = _draws(s, 4000)
    p = softmax(s)
    pb = np.array([p[k * BLOCK:(k + 1) * BLOCK].sum() for k in range(3)])
    assert _chisq(x // BLOCK, pb) > 1e-4
    hot = np.array([(x == 2 * BLOCK + 650).sum(), (x == 100).sum()])
    e = np.array([p[2 * BLOCK + 650], p[100]]) * x.size
    assert np.all(np.abs(hot - e) < 5 * np.sqrt(e) + 1)


def test_excluded_entries_never_drawn():
    s = np.full(300, -math.inf)
    s[[3, 77, 299]] = [0.0, 1.0, -0.5]
    x = _draws(s, 3000)
    assert set(np.unique(x)) <= {3, 77, 299}
    assert _chisq(np.searchsorted([3, 77, 299], x), softmax(s[[3, 77, 299]])) > 1e-4


def test_single_candidate_is_certain():
    s = np.full(9000, -math.inf)
    s[8999] = 0.0
    i, m = tree_sample(s, 0, STREAMS, 0, 0)
    assert i == 8999 and m == math.inf


def test_pick_breaks_ties_to_lowest_index_with_zero_margin():
    i, m = pick(np.array([1.0, 3.0, 3.0, -2.0]))
    assert i == 1 and m == 0.0
    i, m = pick(np.array([0.0, -0.5]))
    assert i == 0 and m == pytest.approx(0.5)


def test_margin_is_shift_invariant():
    rng = np.random.default_rng(5)
    s = rng.normal(0, 2, size=5000)
    a = tree_sample(s, 9, STREAMS, 4, 2)
    b = tree_sample(s + 1234.5, 9, STREAMS, 4, 2)
    assert a[0] == b[0] and a[1] == pytest.approx(b[1], rel=1e-6)
