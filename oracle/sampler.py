"""Three-level Gumbel-max categorical sampler, in fp64.

Test infrastructure only (see the package docstring).

The pages fix *what* is sampled (each draft position from its softmax, the
rejected position from the normalised residual, the bonus token from the
target) but not *how* a categorical draw is made.  The reading adopted here is
an exact hierarchical Gumbel-max over a fixed partition of the vocabulary:

    element v lies in tile t = v div 64 and block k = v div 4096
    (64 elements per tile, 64 tiles per block; the last tile and block may be
    shorter).  With log-weights s_v (minus infinity = excluded):

    1. block   k* = argmax_k  (Lambda_k - Lambda_row + G(u_top[k]))
    2. tile    t* = argmax_t  (Lambda_t - Lambda_k*  + G(u_mid[t]))   over the tiles of k*
    3. element v* = argmax_v  (s_v      - Lambda_t*  + G(u_leaf[e]))  over the elements of t*

where Lambda_X = ln sum_{v in X} exp(s_v), G(u) = -ln(-ln u), u_top[k] is draw
k of the "top" stream, u_mid[t] draw t (t counted inside the block) of the
"mid" stream, u_leaf[e] draw e (e counted inside the tile) of the "leaf"
stream, and ties go to the lowest index.  Each level is an exact Gumbel-max
draw from the conditional distribution of its children, so
P(v* = v) = exp(s_v - Lambda_row) exactly; the block and tile sizes change
which sample a given set of uniforms yields, not its distribution.

Every decision also reports its *margin*: the gap between the winning and the
runner-up perturbed value, divided by max(1, |winner|, |runner-up|) (plus, for
residual draws, the condition number of the candidate's log-mass).  Values are
log conditional probabilities plus a Gumbel, so they are invariant to shifting
the logits.  A margin below 1e-6 marks a decision that fp32 arithmetic on the
GPU may legitimately resolve the other way.
"""

from __future__ import annotations

import math

import numpy as np

from .philox import gumbel, uniforms

TILE = 64
TILES_PER_BLOCK = 64
BLOCK = TILE * TILES_PER_BLOCK


def logsumexp(x) -> float:
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return -math.inf
    m = float(np.max(x))
    if m == -math.inf:
        return -math.inf
    return m + math.log(float(np.sum(np.exp(x - m))))


def pick(vals, cond=None):
    """Index of the largest entry (lowest index among equal ones) and its
    relative margin over the runner-up.  ``cond`` optionally gives, per entry,
    an extra scale added to the denominator (the condition number of that
    entry's value)."""
    vals = np.asarray(vals, dtype=np.float64)
    i = int(np.argmax(vals))
    v1 = float(vals[i])
    if vals.size == 1:
        return i, math.inf
    rest = vals.copy()
    rest[i] = -math.inf
    j = int(np.argmax(rest))
    v2 = float(rest[j])
    if v2 == -math.inf:
        return i, math.inf
    scale = max(1.0, abs(v1), abs(v2))
    if cond is not None:
        scale += max(float(cond[i]), float(cond[j]))
    return i, (v1 - v2) / scale


def tree_sample(scores, seed, streams, request, position, cond_mass=None):
    """Draw one index from the distribution proportional to exp(scores).

    ``streams`` = (top, mid, leaf) Philox stream ids; ``request`` and
    ``position`` complete the counter.  ``cond_mass`` (optional, per element)
    is the mass whose cancellation produced exp(scores) (p + q for a residual):
    a candidate's condition number is sum(cond_mass) / sum(exp(scores)).

    Returns (index, smallest margin over the three levels)."""
    s = np.asarray(scores, dtype=np.float64)
    V = s.size
    nblk = -(-V // BLOCK)

    def kappa(lo, hi, lam):
        if cond_mass is None or lam == -math.inf:
            return 0.0
        return float(np.sum(cond_mass[lo:hi])) / math.exp(lam)

    blk_lam = np.array([logsumexp(s[k * BLOCK:(k + 1) * BLOCK]) for k in range(nblk)])
    row_lam = logsumexp(blk_lam)
    g = gumbel(uniforms(seed, streams[0], request, position, nblk))
    cond = None if cond_mass is None else [kappa(k * BLOCK, (k + 1) * BLOCK, blk_lam[k]) for k in range(nblk)]
    k, m_top = pick(blk_lam - row_lam + g, cond)

    lo, hi = k * BLOCK, min((k + 1) * BLOCK, V)
    nt = -(-(hi - lo) // TILE)
    t_lam = np.array([logsumexp(s[lo + t * TILE:min(lo + (t + 1) * TILE, hi)]) for t in range(nt)])
    g = gumbel(uniforms(seed, streams[1], request, position, nt))
    cond = None if cond_mass is None else [
        kappa(lo + t * TILE, min(lo + (t + 1) * TILE, hi), t_lam[t]) for t in range(nt)]
    t, m_mid = pick(t_lam - blk_lam[k] + g, cond)

    tl, th = lo + t * TILE, min(lo + (t + 1) * TILE, hi)
    g = gumbel(uniforms(seed, streams[2], request, position, th - tl))
    cond = None
    if cond_mass is not None:
        with np.errstate(divide="ignore", over="ignore", invalid="ignore"):
            cond = np.where(np.isfinite(s[tl:th]), cond_mass[tl:th] / np.exp(s[tl:th]), 0.0)
    e, m_leaf = pick(s[tl:th] - t_lam[t] + g, cond)
    return tl + e, min(m_top, m_mid, m_leaf)
