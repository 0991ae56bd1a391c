"""Sequential Temperature Scaling: fitting the per-position temperatures and
measuring calibration (host-side analysis, run once on a validation set).

"DSpark, la bozza ..." (section "Verificare meglio, non di più") and "DSpark :
le pari de DeepSeek ..." (section "Vérifier seulement ce qui compte"): the raw
scores of the confidence head rank tokens well but are overconfident; a
temperature per block position, fitted left to right on a small validation
set, fixes their magnitude without changing their order, and the expected
calibration error falls from 3-8% to about 1%.

Reading used here: position k's temperature tau_k minimises the binary
cross-entropy between sigma(logit(c_k) / tau_k) and the label y_k (a
probability: the analytic acceptance c*_k of the acceptance pass, or a 0/1
outcome), each validation row weighted by the probability that its positions
1..k-1 survived, prod_{i<k} y_i -- the score is defined conditionally on the
earlier positions having been accepted, which is what makes the fit go left
to right.  The temperatures are applied on the GPU by dspark_schedule_ex.
"""

from __future__ import annotations

import math

import numpy as np

TAU_RANGE = (0.05, 20.0)


def scale_scores(scores, tau) -> np.ndarray:
    """sigma(logit(c) / tau_k) per position, in fp64 (for analysis; the
    scheduler applies the same map on the device)."""
    c = np.clip(np.asarray(scores, dtype=np.float64), 1e-12, 1 - 1e-12)
    z = np.log(c) - np.log1p(-c)
    return 1.0 / (1.0 + np.exp(-z / np.asarray(tau, dtype=np.float64)))


def ece(scores, labels, n_bins: int = 15, weights=None) -> float:
    """Expected calibration error: equal-width score bins, sum over bins of the
    bin's weight share times |mean score - mean label|."""
    s = np.asarray(scores, dtype=np.float64).ravel()
    y = np.asarray(labels, dtype=np.float64).ravel()
    w = np.ones_like(s) if weights is None else np.asarray(weights, dtype=np.float64).ravel()
    idx = np.minimum((s * n_bins).astype(np.int64), n_bins - 1)
    tot = w.sum()
    err = 0.0
    for k in range(n_bins):
        m = idx == k
        wk = w[m].sum()
        if wk > 0:
            err += wk / tot * abs(np.dot(w[m], s[m]) / wk - np.dot(w[m], y[m]) / wk)
    return float(err)


def _nll(z, y, w, tau):
    p = 1.0 / (1.0 + np.exp(-z / tau))
    p = np.clip(p, 1e-15, 1 - 1e-15)
    return float(-(w * (y * np.log(p) + (1 - y) * np.log1p(-p))).sum() / max(w.sum(), 1e-300))


def fit_sts(scores, labels, iters: int = 100) -> np.ndarray:
    """Per-position temperatures [gamma] (float32) fitted left to right; each
    is a golden-section minimisation of the weighted cross-entropy over
    log tau in TAU_RANGE (the loss is unimodal in log tau for a fixed set)."""
    c = np.clip(np.asarray(scores, dtype=np.float64), 1e-12, 1 - 1e-12)
    y = np.asarray(labels, dtype=np.float64)
    n, gamma = c.shape
    z = np.log(c) - np.log1p(-c)
    tau = np.ones(gamma)
    surv = np.ones(n)  # prod of the labels of the earlier positions
    g = (math.sqrt(5.0) - 1.0) / 2.0
    for k in range(gamma):
        lo, hi = math.log(TAU_RANGE[0]), math.log(TAU_RANGE[1])
        f = lambda lt: _nll(z[:, k], y[:, k], surv, math.exp(lt))
        a, b = hi - g * (hi - lo), lo + g * (hi - lo)
        fa, fb = f(a), f(b)
        for _ in range(iters):
            if fa < fb:
                hi, b, fb = b, a, fa
                a = hi - g * (hi - lo)
                fa = f(a)
            else:
                lo, a, fa = a, b, fb
                b = lo + g * (hi - lo)
                fb = f(b)
        tau[k] = math.exp(0.5 * (lo + hi))
        surv = surv * y[:, k]
    return tau.astype(np.float32)


def sequential_ece(scores, labels, n_bins: int = 15) -> float:
    """ECE over all positions, each row's position k weighted by the survival
    of its earlier positions (the population the score describes)."""
    y = np.asarray(labels, dtype=np.float64)
    w = np.cumprod(np.concatenate([np.ones((y.shape[0], 1)), y[:, :-1]], axis=1), axis=1)
    return ece(scores, y, n_bins, w)
