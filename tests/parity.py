"""Comparison of one GPU round with the CPU oracle on the same seeded inputs.

Bar (per request-round, for requests the oracle does not flag):
  * draft tokens, verify budgets, accepted counts and emitted tokens: bit-exact;
  * probabilities: exp(ln q) and exp(ln p) at the drafted / verified positions and
    the normalised residual row within 1e-6 absolute / 1e-4 relative; the
    logarithms themselves within 1e-5 absolute + 1e-6 relative (fp32 rounding of
    values up to ~20 in magnitude);
  * draft ln-sum-exp (fp64 output) within 1e-6 relative.
A request is flagged when any of its decisions (sampling level, accept test,
greedy argmax of a draft row) is closer than 1e-6 in the oracle's
shift-invariant decision value; flagged rows must stay under 0.01% of the rows
of a large sample.
"""

from __future__ import annotations

import os
import sys
from dataclasses import dataclass

import numpy as np
import torch

from lossless_rejection_sampling_amd import round as rd
from lossless_rejection_sampling_amd import workloads as wl
from oracle import dspark as od

ATOL_P, RTOL_P = 1e-6, 1e-4


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(rnd: wl.Round, debug=True) -> rd.Buffers:
    buf = rd.allocate(rnd, debug=debug)
    rd.run_round(rnd, buf)
    torch.cuda.synchronize()
    return buf


def run_c_oracle(rnd: wl.Round, keep_residual=False) -> od.RoundResult:
    """The C oracle (oracle/dspark_ref.c) on the whole batch: the scheduler (or
    the round's own budgets), the draft round and the verification, with the
    residual rows of every rejected sampled request when ``keep_residual``."""
    from oracle import ref

    h = wl.to_host
    target, base, U, W = h(rnd.target), h(rnd.base), h(rnd.U), h(rnd.W)
    prev0, T = h(rnd.prev0), h(rnd.temperature)
    off = None if rnd.pos_offset is None else h(rnd.pos_offset)
    sched = None
    if rnd.scheduled:
        sched = ref.schedule(h(rnd.conf), rnd.sps_B, rnd.sps_val)
        budget = sched.budget
    elif rnd.budget is not None:
        budget = h(rnd.budget).astype(np.int32)
    else:
        budget = np.full(rnd.B, rnd.gamma, dtype=np.int32)
    dr = ref.draft_round(base, U, W, prev0, T, rnd.seed, off)
    vr = ref.verify(target, base, U, W, prev0, dr.tokens, T, rnd.seed, budget, off, keep_residual=keep_residual)
    return od.RoundResult(dr, budget, sched, vr)


def run_oracle(rnd: wl.Round, idx, budget_full=None) -> od.RoundResult:
    """Oracle on requests ``idx`` of the round; budgets come from the oracle's
    scheduler over the whole batch (the scheduler is global)."""
    h = wl.to_host
    t = torch.as_tensor(idx, dtype=torch.long, device=rnd.base.device)
    pick = lambda x: None if x is None else h(x.index_select(0, t))
    base, target = pick(rnd.base), pick(rnd.target)
    prev0, T, off = pick(rnd.prev0), pick(rnd.temperature), pick(rnd.pos_offset)
    U, W = h(rnd.U), h(rnd.W)
    sched = None
    if rnd.scheduled:
        sched = od.schedule(h(rnd.conf), rnd.sps_B, rnd.sps_val)
        budget = sched.budget[np.asarray(idx)]
    elif rnd.budget is not None:
        budget = pick(rnd.budget)
    else:
        budget = None
    dr = od.draft_round(base, U, W, prev0, T, rnd.seed, off, req_ids=idx)
    vr = od.verify(target, base, U, W, prev0, dr.tokens, T, rnd.seed, budget, off, req_ids=idx,
                   keep_residual=True)
    B = len(idx)
    return od.RoundResult(dr, budget if budget is not None else np.full(B, rnd.gamma), sched, vr)


@dataclass
class Report:
    requests: int
    flagged_requests: int
    rows: int
    flagged_rows: int
    mismatches: list


def compare(rnd: wl.Round, buf: rd.Buffers, ref: od.RoundResult, idx, check_probs=True) -> Report:
    idx = np.asarray(idx)
    g = rnd.gamma
    h = lambda x: x.detach().cpu().numpy()
    draft = h(buf.draft_tokens)[idx]
    logq = h(buf.draft_logq)[idx].astype(np.float64)
    lse = h(buf.draft_lse)[idx]
    out = h(buf.out_tokens)[idx]
    nacc = h(buf.num_accepted)[idx]
    nemit = h(buf.num_emitted)[idx]
    T = h(rnd.temperature)[idx]
    budget = h(buf.budget)[idx] if buf.budget is not None else np.full(len(idx), g)
    flagged = ref.request_flagged()
    bad = []
    rows = 0
    for i, b in enumerate(idx):
        L = int(ref.budget[i])
        rows += g + int(ref.verify.num_emitted[i])
        if int(budget[i]) != L and not (ref.sched is not None and ref.sched.min_gap < od.SCHED_FLAG):
            bad.append((int(b), "budget", int(budget[i]), L))
        if flagged[i]:
            continue
        if not np.array_equal(draft[i], ref.draft.tokens[i]):
            bad.append((int(b), "draft", draft[i].tolist(), ref.draft.tokens[i].tolist()))
            continue
        if not np.array_equal(out[i], ref.verify.out_tokens[i]) or nacc[i] != ref.verify.num_accepted[i] \
                or nemit[i] != ref.verify.num_emitted[i]:
            bad.append((int(b), "verify", out[i].tolist(), ref.verify.out_tokens[i].tolist()))
            continue
        if not check_probs:
            continue
        if T[i] > 0:
            lq_ref = ref.draft.logq[i]
            if not np.allclose(logq[i], lq_ref, atol=1e-5, rtol=1e-6) or \
                    not np.allclose(np.exp(logq[i]), np.exp(lq_ref), atol=ATOL_P, rtol=RTOL_P):
                bad.append((int(b), "logq", logq[i].tolist(), lq_ref.tolist()))
            if not np.allclose(lse[i], ref.draft.lse[i], rtol=1e-6, atol=0):
                bad.append((int(b), "lse", lse[i].tolist(), ref.draft.lse[i].tolist()))
            if buf.debug_logp_logq is not None:
                dbg = h(buf.debug_logp_logq)[b]
                n_ver = min(int(ref.verify.num_accepted[i]) + 1, L)
                lp_ref = ref.verify.logp[i, :n_ver]
                lq_v = ref.verify.logq[i, :n_ver]
                if not (np.allclose(dbg[:n_ver, 0], lp_ref, atol=1e-5, rtol=1e-6)
                        and np.allclose(np.exp(dbg[:n_ver, 0]), np.exp(lp_ref), atol=ATOL_P, rtol=RTOL_P)
                        and np.allclose(dbg[:n_ver, 1], lq_v, atol=1e-5, rtol=1e-6)):
                    bad.append((int(b), "logp", dbg[:n_ver].tolist(), list(zip(lp_ref, lq_v))))
            if buf.debug_residual is not None and i in ref.verify.residual:
                res = h(buf.debug_residual[b])
                want = ref.verify.residual[i]
                if not np.allclose(res, want, atol=ATOL_P, rtol=RTOL_P):
                    k = int(np.argmax(np.abs(res - want)))
                    bad.append((int(b), "residual", float(res[k]), float(want[k]), k))
    return Report(len(idx), int(flagged.sum()), rows, ref.rows_flagged(), bad)


def check(rep: Report, name: str, max_flag_frac=1e-4):
    say(f"[{name}] requests={rep.requests} flagged_requests={rep.flagged_requests} "
        f"rows={rep.rows} flagged_rows={rep.flagged_rows} mismatches={len(rep.mismatches)}")
    assert not rep.mismatches, rep.mismatches[:5]
    # a single flagged row is allowed in a small sample; beyond that the rate bar applies
    assert rep.flagged_rows <= max(1, max_flag_frac * rep.rows), rep


GOLDEN_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rounds")


def load_golden(name: str):
    """Whole-batch oracle expectations written by tests/golden/make_round_goldens.py."""
    path = os.path.join(GOLDEN_DIR, f"{name}.npz")
    with np.load(path, allow_pickle=False) as z:
        return {k: z[k] for k in z.files}


def _close(what, got, want, atol, rtol):
    got, want = np.asarray(got, dtype=np.float64), np.asarray(want, dtype=np.float64)
    err = np.abs(got - want) - (atol + rtol * np.abs(want))
    if err.size and not np.all(err <= 0):
        k = int(np.argmax(err))
        raise AssertionError(f"{what}: {int((err > 0).sum())} of {err.size} outside atol {atol} rtol {rtol}; "
                             f"worst got {got.flat[k]!r} want {want.flat[k]!r}")


def compare_golden(rnd: wl.Round, buf: rd.Buffers, gold: dict, name: str):
    """Every request of a GPU round against the oracle's whole-batch expectations
    (same bar as ``compare``; requests the oracle flags are excused)."""
    fp = wl.input_fingerprint(rnd)
    assert np.allclose(fp, gold["fingerprint"], rtol=1e-9, atol=0), f"{name}: inputs differ from the golden's"
    h = lambda x: x.detach().cpu().numpy()
    B, g = rnd.B, rnd.gamma
    budget = h(buf.budget) if buf.budget is not None else np.full(B, g)
    if float(gold["sched_min_gap"]) > od.SCHED_FLAG:
        assert np.array_equal(budget, gold["budget"]), f"{name}: budgets differ"
    ok = ~gold["flagged"]
    bad = []
    draft = h(buf.draft_tokens)
    out, nacc, nemit = h(buf.out_tokens), h(buf.num_accepted), h(buf.num_emitted)
    for b in np.nonzero(ok)[0]:
        if not np.array_equal(draft[b], gold["draft_tokens"][b]):
            bad.append((int(b), "draft", draft[b].tolist(), gold["draft_tokens"][b].tolist()))
        elif not np.array_equal(out[b], gold["out_tokens"][b]) or nacc[b] != gold["num_accepted"][b] \
                or nemit[b] != gold["num_accepted"][b] + 1:
            bad.append((int(b), "verify", out[b].tolist(), gold["out_tokens"][b].tolist()))
    assert not bad, f"{name}: {len(bad)} requests differ: {bad[:4]}"
    T = h(rnd.temperature)
    s = ok & (T > 0)
    logq = h(buf.draft_logq).astype(np.float64)[s]
    lq_ref = gold["draft_logq"][s]
    _close(f"{name}: ln q", logq, lq_ref, 1e-5, 1e-6)
    _close(f"{name}: q", np.exp(logq), np.exp(lq_ref), ATOL_P, RTOL_P)
    _close(f"{name}: draft lse", h(buf.draft_lse)[s], gold["draft_lse"][s], 0.0, 1e-6)
    if buf.debug_logp_logq is not None:
        dbg = h(buf.debug_logp_logq)[s].astype(np.float64)
        want_p, want_q = gold["logp"][s], gold["logq"][s]
        tested = ~np.isnan(want_p)   # positions whose accept test ran
        _close(f"{name}: ln p", dbg[..., 0][tested], want_p[tested], 1e-5, 1e-6)
        _close(f"{name}: p", np.exp(dbg[..., 0][tested]), np.exp(want_p[tested]), ATOL_P, RTOL_P)
        _close(f"{name}: ln q at verify", dbg[..., 1][tested], want_q[tested], 1e-5, 1e-6)
    rows, fl = int(gold["rows"]), int(gold["rows_flagged"])
    say(f"[{name}] whole batch: requests={B} compared={int(ok.sum())} rows={rows} flagged_rows={fl} "
        f"verified={int(budget.sum())} accepted={int(nacc.sum())}")
    assert fl < 1e-4 * rows + 1, f"{name}: flagged rows {fl} of {rows}"
