"""One DSpark draft-and-verify round, written out plainly in fp64.

Test infrastructure only (see the package docstring).

Readings of the pages used here (each is also listed with its reason in the
design notes of the repository):
  * Temperature: every logit row is divided by the request's temperature T
    before the softmax (base + Markov bias for the draft, the target row for the
    target); T = 0 means greedy decoding (argmax, lowest index on ties).
  * Markov head: the bias added at block position k is row x_{k-1} of the
    low-rank product U W, with x_0 the last committed token; the same factors
    serve every position ("DSpark, la bozza ...", section "Un po' di
    autoregressione basta", eq. p_k and the rank-256 factorisation B = W1 W2;
    U here is W1 [V x r] and W is W2 [r x V]).
  * Residual: the rejected position is resampled from max(0, p - q) normalised
    (the pages name "the residual distribution" without printing it; this is
    the residual that makes the output distribution equal p).  If the residual
    has zero mass the draw falls back to p.
  * Budget L_b in [0, gamma] counts verified draft tokens; the final token comes
    from target row n (rejection at position n+1) or row L_b (bonus).
  * Scheduler: verify batch size counts tokens, one per request plus every
    admitted draft token; candidates are admitted in order of decreasing prefix
    survival while Theta = tau * SPS(N) strictly grows, and admission stops at
    the first candidate that does not raise it.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

from . import philox as px
from .sampler import logsumexp, pick, tree_sample

MARGIN_FLAG = 1.0e-6        # decisions closer than this may flip under fp32 arithmetic
SCHED_FLAG = 1.0e-12        # relative gap of a scheduler comparison treated as a tie


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def effective_temperature(T) -> float:
    """Greedy decoding is the T -> 0 limit; temperatures below 2^-64 are taken
    as that limit (T = 0)."""
    T = float(T)
    return T if T >= 2.0 ** -64 else 0.0


def softmax(s):
    s = _f64(s)
    return np.exp(s - logsumexp(s))


def draft_logits(base_row, U, W, prev: int):
    """Draft logits at one block position: U_k + B(x_{k-1}, .), with the Markov
    bias B(x, .) = row x of U W ("DSpark, la bozza ...", eq. p_k)."""
    return _f64(base_row) + _f64(U)[int(prev)] @ _f64(W)


def argmax_first(x) -> int:
    return int(np.argmax(_f64(x)))


@dataclass
class DraftResult:
    tokens: np.ndarray          # [B, gamma] int32
    logq: np.ndarray            # [B, gamma] log q_k(x_k) (0 for greedy requests)
    lse: np.ndarray             # [B, gamma] ln sum exp(d / T) (max d for greedy requests)
    margin: np.ndarray          # [B, gamma] smallest decision margin at each position


def draft_round(base, U, W, prev0, temperature, seed: int, pos_offset=None, req_ids=None) -> DraftResult:
    """Semi-autoregressive drafting of one block ("DSpark, la bozza ...",
    section "Un po' di autoregressione basta"): for k = 1..gamma the Markov bias
    of the previous token is added to the backbone logits of position k, the
    result is softmaxed and x_k is sampled; x_k then conditions position k+1."""
    base = _f64(base)
    B, gamma, V = base.shape
    U, W = _f64(U), _f64(W)
    req_ids = np.arange(B) if req_ids is None else np.asarray(req_ids)
    off = np.zeros(B, dtype=np.int64) if pos_offset is None else np.asarray(pos_offset, dtype=np.int64)
    tokens = np.zeros((B, gamma), dtype=np.int32)
    logq = np.zeros((B, gamma))
    lse = np.zeros((B, gamma))
    margin = np.full((B, gamma), math.inf)
    prev = np.asarray(prev0, dtype=np.int64).copy()
    for k in range(1, gamma + 1):
        d_all = base[:, k - 1, :] + U[prev] @ W
        for b in range(B):
            d = d_all[b]
            T = effective_temperature(temperature[b])
            if T == 0.0:
                x = argmax_first(d)
                _, m = pick(d - d[x])
                logq[b, k - 1] = 0.0
                lse[b, k - 1] = float(d[x])
            else:
                s = d / T
                lse_s = logsumexp(s)
                x, m = tree_sample(s, seed, (px.DRAFT_TOP, px.DRAFT_MID, px.DRAFT_LEAF),
                                   int(req_ids[b]), k + int(off[b]))
                logq[b, k - 1] = s[x] - lse_s
                lse[b, k - 1] = lse_s
            tokens[b, k - 1] = x
            margin[b, k - 1] = m
        prev = tokens[:, k - 1].astype(np.int64)
    return DraftResult(tokens, logq, lse, margin)


@dataclass
class VerifyResult:
    out_tokens: np.ndarray      # [B, gamma+1] int32, -1 padded
    num_accepted: np.ndarray    # [B] int32
    num_emitted: np.ndarray     # [B] int32
    logp: np.ndarray            # [B, gamma] log p_k(x_k) at verified positions (nan elsewhere)
    logq: np.ndarray            # [B, gamma] log q_k(x_k) at verified positions (nan elsewhere)
    residual: dict = field(default_factory=dict)   # b -> normalised residual row (rejected, T > 0)
    margin: np.ndarray = None   # [B] smallest decision margin of the request's verify
    rows_flagged: np.ndarray = None  # [B] number of target rows with a flagged decision


def verify(target, base, U, W, prev0, draft_tokens, temperature, seed: int, budget=None,
           pos_offset=None, req_ids=None, keep_residual=False) -> VerifyResult:
    """Lossless verification of one drafted block per request
    ("Les mathématiques derrière l'accélération ...", section "La garantie de
    l'échantillonnage par rejet"; "DeepSeek发布DSpark", section "DSpark 是什么？"):

      for k = 1..L: accept x_k with probability min(1, p_k(x_k) / q_k(x_k));
      stop at the first rejection (position n+1) and draw its replacement from
      max(0, p_{n+1} - q_{n+1}) normalised; if all L are accepted, draw a bonus
      token from p_{L+1}.  Greedy requests (T = 0) accept x_k iff it is the
      target argmax and emit the target argmax.

    p_k is the softmax of target row k-1 divided by T; q_k is recomputed from
    the draft definition with previous token x_{k-1}."""
    target, base = _f64(target), _f64(base)
    B, gamma, V = base.shape
    U, W = _f64(U), _f64(W)
    req_ids = np.arange(B) if req_ids is None else np.asarray(req_ids)
    off = np.zeros(B, dtype=np.int64) if pos_offset is None else np.asarray(pos_offset, dtype=np.int64)
    L_all = np.full(B, gamma, dtype=np.int64) if budget is None else np.asarray(budget, dtype=np.int64)

    out = np.full((B, gamma + 1), -1, dtype=np.int32)
    n_acc = np.zeros(B, dtype=np.int32)
    logp_out = np.full((B, gamma), np.nan)
    logq_out = np.full((B, gamma), np.nan)
    margin = np.full(B, math.inf)
    rows_flagged = np.zeros(B, dtype=np.int32)
    residual = {}

    for b in range(B):
        L = int(L_all[b])
        if not 0 <= L <= gamma:
            raise ValueError(f"budget {L} outside [0, {gamma}]")
        T = effective_temperature(temperature[b])
        rq, pos0 = int(req_ids[b]), int(off[b])
        xs = [int(prev0[b])] + [int(t) for t in draft_tokens[b]]
        n = 0
        for k in range(1, L + 1):
            z = target[b, k - 1]
            x = xs[k]
            if T == 0.0:
                ok = x == argmax_first(z)
            else:
                lp = z[x] / T - logsumexp(z / T)
                dq = draft_logits(base[b, k - 1], U, W, xs[k - 1]) / T
                lq = dq[x] - logsumexp(dq)
                ln_u = math.log(px.uniforms(seed, px.ACCEPT, rq, k + pos0, 1)[0])
                ok = ln_u < lp - lq      # u < min(1, p/q), since ln u < 0
                m = abs(ln_u - (lp - lq)) / max(1.0, abs(ln_u), abs(lp) + abs(lq))
                margin[b] = min(margin[b], m)
                rows_flagged[b] += m < MARGIN_FLAG
                logp_out[b, k - 1], logq_out[b, k - 1] = lp, lq
            if not ok:
                break
            n += 1
        z = target[b, n]
        if T == 0.0:
            y = argmax_first(z)
        elif n < L:
            p = softmax(z / T)
            q = softmax(draft_logits(base[b, n], U, W, xs[n]) / T)
            r = np.maximum(0.0, p - q)
            if float(np.sum(r)) > 0.0:
                with np.errstate(divide="ignore"):
                    scores = np.log(r)
                y, m = tree_sample(scores, seed, (px.FINAL_TOP, px.FINAL_MID, px.FINAL_LEAF),
                                   rq, n + 1 + pos0, cond_mass=p + q)
                if keep_residual:
                    residual[b] = r / np.sum(r)
            else:
                y, m = tree_sample(z / T, seed, (px.FINAL_TOP, px.FINAL_MID, px.FINAL_LEAF),
                                   rq, n + 1 + pos0)
                if keep_residual:
                    residual[b] = p
            margin[b] = min(margin[b], m)
            rows_flagged[b] += m < MARGIN_FLAG
        else:
            y, m = tree_sample(z / T, seed, (px.FINAL_TOP, px.FINAL_MID, px.FINAL_LEAF),
                               rq, n + 1 + pos0)
            margin[b] = min(margin[b], m)
            rows_flagged[b] += m < MARGIN_FLAG
        out[b, :n] = xs[1:n + 1]
        out[b, n] = y
        n_acc[b] = n
    return VerifyResult(out, n_acc, n_acc + 1, logp_out, logq_out, residual, margin, rows_flagged)


# ----------------------------------------------------------------------------
# Hardware-aware prefix scheduler ("DSpark, la bozza ...", section "Verificare
# meglio, non di più": a_j = prod_{i<=j} c_i, Theta = tau SPS(B), greedy
# admission in decreasing a_{r,j} that stops when Theta stops growing).
# ----------------------------------------------------------------------------

def prefix_survival(conf) -> np.ndarray:
    """a[b, j] = fl32(a[b, j-1] * c[b, j]) with a[b, -1] = 1: the product taken
    left to right in fp32, one rounding per factor."""
    c = np.asarray(conf, dtype=np.float32)
    if not np.all((c > 0) & (c < 1)):
        raise ValueError("confidence scores must lie strictly inside (0, 1)")
    a = np.empty_like(c)
    for b in range(c.shape[0]):
        acc = np.float32(1.0)
        for j in range(c.shape[1]):
            acc = np.float32(acc * c[b, j])
            a[b, j] = acc
    return a


def step_time(N: float, sps_B, t_tab) -> float:
    """1/SPS at a verify batch of N tokens: linear between the table points,
    the first value below the first point, the last segment extended beyond
    the last point.  t = t_i + (t_{i+1} - t_i) * ((N - B_i) / (B_{i+1} - B_i))
    with segment i the last one whose left end B_i <= N."""
    n = len(sps_B)
    if N <= sps_B[0]:
        return t_tab[0]
    i = 0
    while i + 1 < n - 1 and sps_B[i + 1] <= N:
        i += 1
    frac = (N - sps_B[i]) / (sps_B[i + 1] - sps_B[i])
    return t_tab[i] + (t_tab[i + 1] - t_tab[i]) * frac


@dataclass
class ScheduleResult:
    budget: np.ndarray          # [B] int32 verify budgets
    admitted: int               # number of admitted candidates
    min_gap: float              # smallest relative gap of any comparison made


def schedule(conf, sps_B, sps_val) -> ScheduleResult:
    """Budgets L_b from the greedy early-stop prefix rule.

    Candidates (b, j) carry Q = floor(a[b, j] 2^32) (exact integers).  They are
    taken in order of decreasing Q (ties: lower request, then lower position,
    so every request's admitted set is a prefix).  Starting from tau_0 = B 2^32
    expected tokens (every request emits at least its final token) and N_0 = B
    tokens in the verify batch, candidate m is admitted iff
        (tau_m + Q_m) * t(N_m) > tau_m * t(N_m + 1)
    i.e. iff Theta = tau / t(N) strictly grows; the first failure stops the scan."""
    sps_B = [float(v) for v in sps_B]
    if len(sps_B) < 2 or any(sps_B[i + 1] <= sps_B[i] for i in range(len(sps_B) - 1)):
        raise ValueError("step-rate table needs >= 2 points with increasing batch sizes")
    t_tab = [1.0 / float(v) for v in sps_val]
    a = prefix_survival(conf)
    B, gamma = a.shape
    Q = np.floor(a.astype(np.float64) * 2.0 ** 32).astype(np.int64)
    cand = sorted((-int(Q[b, j]), b, j) for b in range(B) for j in range(gamma))
    tau = B << 32
    N = B
    budget = np.zeros(B, dtype=np.int32)
    admitted = 0
    min_gap = math.inf
    for negq, b, j in cand:
        q = -negq
        lhs = float(tau + q) * step_time(float(N), sps_B, t_tab)
        rhs = float(tau) * step_time(float(N + 1), sps_B, t_tab)
        den = max(abs(lhs), abs(rhs))
        if den > 0:
            min_gap = min(min_gap, abs(lhs - rhs) / den)
        if not lhs > rhs:
            break
        tau += q
        N += 1
        budget[b] = j + 1
        admitted += 1
    return ScheduleResult(budget, admitted, min_gap)


def analytic_acceptance(target, base, U, W, prev0, draft_tokens, temperature) -> np.ndarray:
    """c*[b, k-1] = sum_v min(p_k(v), q_k(v)) = 1 - (1/2) ||p_k - q_k||_1 for
    k = 1..gamma ("DSpark, la bozza ...", section "Verificare meglio, non di
    più", eq. c*_k): the probability that position k's accept test passes
    given the drafted prefix x_1..x_{k-1} was accepted.  p_k = softmax(target
    row k-1 / T); q_k = softmax(draft logits of position k with previous token
    x_{k-1} / T).  Greedy requests: both are one-hot at their lowest-index
    maximum, so c* is 1 when the draft token is the target argmax, else 0."""
    target, base = _f64(target), _f64(base)
    B, gamma, V = base.shape
    U, W = _f64(U), _f64(W)
    out = np.zeros((B, gamma))
    for b in range(B):
        T = effective_temperature(temperature[b])
        xs = [int(prev0[b])] + [int(t) for t in draft_tokens[b]]
        for k in range(1, gamma + 1):
            z = target[b, k - 1]
            if T == 0.0:
                out[b, k - 1] = 1.0 if xs[k] == argmax_first(z) else 0.0
                continue
            p = softmax(z / T)
            q = softmax(draft_logits(base[b, k - 1], U, W, xs[k - 1]) / T)
            out[b, k - 1] = float(np.minimum(p, q).sum())
    return out


# ----------------------------------------------------------------------------
# Variants of the verify-budget rule ("DSpark, la bozza ...", sections
# "Verificare meglio, non di più" and "Che cosa resta da verificare"; "DSpark :
# le pari de DeepSeek ...", section "Vérifier seulement ce qui compte"):
#   * Sequential Temperature Scaling rescales each position's score,
#     c' = sigma(logit(c) / tau_k), before the products;
#   * the production scheduler takes the cut with the largest Theta over the
#     whole sorted list (no early stop), on scores two steps old;
#   * the baselines the pages compare against: a fixed draft length (MTP-1,
#     MTP-3, MTP-5) and a fixed confidence threshold ("verify while the
#     confidence exceeds 0.7").
# ----------------------------------------------------------------------------

RULES = ("early_stop", "argmax", "fixed", "threshold")
_F32_LO, _F32_HI = float(np.float32(2.0 ** -126)), float(np.nextafter(np.float32(1.0), np.float32(0.0)))


def calibrate_scores(conf, tau):
    """Sequential Temperature Scaling applied to raw scores: for position k,
    c' = 1 / (1 + exp(-z / tau_k)), z = ln c - ln(1 - c), evaluated in fp64 from
    the fp32 score and rounded once to fp32, then kept strictly inside (0, 1).
    Returns (c', near) where `near` marks values whose fp64 result lies within
    1e-12 (relative) of an fp32 rounding boundary: another correctly rounded
    evaluation of the same formula may round those the other way."""
    c = np.asarray(conf, dtype=np.float32)
    tau = np.asarray(tau, dtype=np.float32)
    out = np.empty_like(c)
    near = np.zeros(c.shape, dtype=bool)
    for b in range(c.shape[0]):
        for k in range(c.shape[1]):
            x = float(c[b, k])
            z = math.log(x) - math.log1p(-x)
            y = 1.0 / (1.0 + math.exp(-z / float(tau[k])))
            y = min(max(y, _F32_LO), _F32_HI)
            f = np.float32(y)
            out[b, k] = f
            lo, hi = sorted((float(f), float(np.nextafter(f, np.float32(2.0) if float(f) < y else np.float32(0.0)))))
            mid = 0.5 * (lo + hi)
            near[b, k] = abs(y - mid) <= 1e-12 * y
    return out, near


def _sorted_candidates(a):
    B, gamma = a.shape
    Q = np.floor(a.astype(np.float64) * 2.0 ** 32).astype(np.int64)
    return Q, sorted((-int(Q[b, j]), b, j) for b in range(B) for j in range(gamma))


def schedule_rule(conf, sps_B, sps_val, rule: str = "early_stop", param: float = 0.0, tau=None) -> ScheduleResult:
    """Budgets under one of RULES, optionally after Sequential Temperature
    Scaling with per-position temperatures `tau`.
      early_stop  the greedy prefix scheduler with its first-failure stop
      argmax      the cut m* maximising Theta_m = tau_m / t(N_m) over m = 0..B gamma
                  along the same sorted list (tau_m = B 2^32 + the first m Q,
                  N_m = B + m; Theta as one correctly rounded fp64 division;
                  ties go to the smaller m)
      fixed       L_b = min(param, gamma) for every request
      threshold   L_b = number of leading positions whose score exceeds param
    """
    if rule not in RULES:
        raise ValueError(f"unknown rule {rule}")
    c = np.asarray(conf, dtype=np.float32)
    if tau is not None:
        c, _ = calibrate_scores(c, tau)
    B, gamma = c.shape
    if rule == "early_stop":
        return schedule(c, sps_B, sps_val)
    if rule == "fixed":
        L = int(min(max(int(param), 0), gamma))
        return ScheduleResult(np.full(B, L, dtype=np.int32), B * L, math.inf)
    if rule == "threshold":
        thr = np.float32(param)
        budget = np.zeros(B, dtype=np.int32)
        for b in range(B):
            n = 0
            while n < gamma and c[b, n] > thr:
                n += 1
            budget[b] = n
        return ScheduleResult(budget, int(budget.sum()), math.inf)
    # argmax
    sps_B = [float(v) for v in sps_B]
    t_tab = [1.0 / float(v) for v in sps_val]
    a = prefix_survival(c)
    Q, cand = _sorted_candidates(a)
    tau_m = B << 32
    best, best_m = float(tau_m) / step_time(float(B), sps_B, t_tab), 0
    thetas = [best]
    for m, (negq, b, j) in enumerate(cand, start=1):
        tau_m += -negq
        th = float(tau_m) / step_time(float(B + m), sps_B, t_tab)
        thetas.append(th)
        if th > best:
            best, best_m = th, m
    budget = np.zeros(B, dtype=np.int32)
    for negq, b, j in cand[:best_m]:
        budget[b] = max(budget[b], j + 1)
    # the closest call: the best Theta against every other cut's
    others = [t for i, t in enumerate(thetas) if i != best_m]
    gap = min((abs(best - t) / best for t in others), default=math.inf)
    return ScheduleResult(budget, best_m, gap)


def expected_theta(conf, budget, sps_B, sps_val, tau=None):
    """Expected tokens per round tau = sum_b (1 + sum_{j <= L_b} a_{b,j}), verify
    batch N = sum_b (1 + L_b) tokens and Theta = tau / t(N) in fp64: the measure
    the pages compare schedulers by (Theta = tau SPS(B))."""
    c = np.asarray(conf, dtype=np.float32)
    if tau is not None:
        c, _ = calibrate_scores(c, tau)
    a = prefix_survival(c).astype(np.float64)
    budget = np.asarray(budget)
    B = a.shape[0]
    tok = float(B) + sum(float(a[b, :int(budget[b])].sum()) for b in range(B))
    N = float(B + int(budget.sum()))
    t = step_time(N, [float(v) for v in sps_B], [1.0 / float(v) for v in sps_val])
    return tok, N, tok / t


# ----------------------------------------------------------------------------
# A whole round and its flags.
# ----------------------------------------------------------------------------

@dataclass
class RoundResult:
    draft: DraftResult
    budget: np.ndarray
    sched: Optional[ScheduleResult]
    verify: VerifyResult

    def request_flagged(self, threshold=MARGIN_FLAG) -> np.ndarray:
        """Requests with any decision closer than ``threshold`` (draft or verify)."""
        return (self.draft.margin.min(axis=1) < threshold) | (self.verify.margin < threshold)

    def rows_flagged(self, threshold=MARGIN_FLAG) -> int:
        return int((self.draft.margin < threshold).sum() + self.verify.rows_flagged.sum())


def run_round(target, base, U, W, prev0, temperature, seed, pos_offset=None, conf=None,
              sps_B=None, sps_val=None, budget=None, req_ids=None, keep_residual=False) -> RoundResult:
    """draft -> schedule -> verify, the order of the pages (drafting, confidence
    scoring, prefix scheduling, verification)."""
    dr = draft_round(base, U, W, prev0, temperature, seed, pos_offset, req_ids)
    sched = None
    if conf is not None:
        sched = schedule(conf, sps_B, sps_val)
        budget = sched.budget
    vr = verify(target, base, U, W, prev0, dr.tokens, temperature, seed, budget, pos_offset,
                req_ids, keep_residual)
    return RoundResult(dr, budget if budget is not None else np.full(base.shape[0], base.shape[1]),
                       sched, vr)
