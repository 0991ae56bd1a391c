"""Whole-batch expectations of the full-size rounds, computed by the CPU oracle.

For every full-size workload (the DSpark-5 round at B=64, the B=256 round at
its scheduled and at its full budget, block lengths 4/8/16, the scheduled
B=512 round and the B=1024 stress round) this script draws the inputs on the
host with the seeded generators, runs the oracle over every request (draft,
scheduler over the whole batch, verify) and writes what a GPU run must
reproduce to ``tests/golden/rounds/<name>.npz``: draft tokens, ln q, ln-sum-exp,
budgets, emitted tokens, accepted counts, ln p / ln q at the verified
positions, and which requests and rows the oracle flags (decision margin
below 1e-6).  For the B=256 round and block length 8 it also writes the
analytic acceptance c*_k of every drafted position (``acceptance_<name>.npz``).  It also records a fingerprint of the inputs, so a GPU test can
check that it regenerated the same tensors.

Only the oracle (``oracle/``) computes anything here; the inputs come from
``workloads``, which holds none of the method's arithmetic.  Requests are
independent given their budgets, so they are computed in chunks by worker
processes forked after the inputs exist.

    python tests/golden/make_round_goldens.py [name ...] [--workers N]
"""

from __future__ import annotations

import argparse
import multiprocessing as mp
import os
import sys
import time

# one BLAS / OpenMP thread per process: the requests are spread over worker processes
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ[_v] = "1"

import numpy as np  # noqa: E402

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)
OUT = os.path.join(HERE, "rounds")

CHUNK = 8

# name -> generator call (host tensors)
CONFIGS = {
    "dspark5_B64": lambda wl: wl.dspark5(device="cpu"),
    "headline_B256": lambda wl: wl.headline(device="cpu"),
    "headline_B256_full": lambda wl: wl.headline(device="cpu", scheduled=False),
    "block_length_g4": lambda wl: wl.block_length(4, device="cpu"),
    "block_length_g8": lambda wl: wl.block_length(8, device="cpu"),
    "block_length_g16": lambda wl: wl.block_length(16, device="cpu"),
    "scheduled_B512": lambda wl: wl.scheduled(device="cpu"),
    "stress_B1024": lambda wl: wl.stress(device="cpu"),
}

# analytic acceptance c*_k of every drafted position (the oracle's own drafts)
ACCEPTANCE = {
    "acceptance_headline_B256": lambda wl: wl.headline(device="cpu"),
    "acceptance_block_length_g8": lambda wl: wl.block_length(8, device="cpu"),
}

_G = {}  # inputs shared with forked workers


def _chunk(idx):
    from oracle import dspark as od
    g = _G
    idx = np.asarray(idx)
    base, target = g["base"][idx], g["target"][idx]
    prev0, T = g["prev0"][idx], g["T"][idx]
    budget = g["budget"][idx]
    dr = od.draft_round(base, g["U"], g["W"], prev0, T, g["seed"], None, req_ids=idx)
    vr = od.verify(target, base, g["U"], g["W"], prev0, dr.tokens, T, g["seed"], budget, None, req_ids=idx)
    return idx, dr, vr


def _acc_chunk(idx):
    from oracle import dspark as od
    g = _G
    idx = np.asarray(idx)
    base, target = g["base"][idx], g["target"][idx]
    prev0, T = g["prev0"][idx], g["T"][idx]
    dr = od.draft_round(base, g["U"], g["W"], prev0, T, g["seed"], None, req_ids=idx)
    c = od.analytic_acceptance(target, base, g["U"], g["W"], prev0, dr.tokens, T)
    return idx, dr, c


def make_acceptance(name: str, workers: int):
    from lossless_rejection_sampling_amd import workloads as wl

    t0 = time.time()
    rnd = ACCEPTANCE[name](wl)
    B, gamma = rnd.B, rnd.gamma
    h = wl.to_host
    _G.clear()
    _G.update(target=h(rnd.target), base=h(rnd.base), U=h(rnd.U), W=h(rnd.W), prev0=h(rnd.prev0),
              T=h(rnd.temperature), seed=rnd.seed)
    tokens = np.zeros((B, gamma), np.int32)
    margin = np.zeros((B, gamma))
    c_star = np.zeros((B, gamma))
    chunks = [list(range(i, min(B, i + CHUNK))) for i in range(0, B, CHUNK)]
    with mp.get_context("fork").Pool(workers) as pool:
        for idx, dr, c in pool.imap_unordered(_acc_chunk, chunks):
            tokens[idx], margin[idx], c_star[idx] = dr.tokens, dr.margin, c
    path = os.path.join(OUT, f"{name}.npz")
    np.savez_compressed(path, draft_tokens=tokens, draft_margin=margin, c_star=c_star,
                        fingerprint=wl.input_fingerprint(rnd))
    print(f"[{name}] wrote {path}: mean c* {c_star.mean():.4f} ({time.time() - t0:.0f} s)", flush=True)
    _G.clear()


def make(name: str, workers: int):
    import torch
    from lossless_rejection_sampling_amd import workloads as wl
    from oracle import dspark as od

    t0 = time.time()
    rnd = CONFIGS[name](wl)
    B, gamma = rnd.B, rnd.gamma
    print(f"[{name}] inputs drawn in {time.time() - t0:.1f} s: B={B} gamma={gamma} V={rnd.V} r={rnd.r}", flush=True)
    h = wl.to_host
    _G.clear()
    _G.update(target=h(rnd.target), base=h(rnd.base), U=h(rnd.U), W=h(rnd.W), prev0=h(rnd.prev0),
              T=h(rnd.temperature), seed=rnd.seed)
    sched_gap = np.inf
    if rnd.scheduled:
        sc = od.schedule(h(rnd.conf), rnd.sps_B, rnd.sps_val)
        budget = sc.budget.astype(np.int32)
        sched_gap = sc.min_gap
    else:
        budget = np.full(B, gamma, dtype=np.int32)
    _G["budget"] = budget

    out = dict(
        draft_tokens=np.zeros((B, gamma), np.int32), draft_logq=np.zeros((B, gamma)), draft_lse=np.zeros((B, gamma)),
        draft_margin=np.zeros((B, gamma)), out_tokens=np.zeros((B, gamma + 1), np.int32),
        num_accepted=np.zeros(B, np.int32), logp=np.full((B, gamma), np.nan), logq=np.full((B, gamma), np.nan),
        verify_margin=np.zeros(B), verify_rows_flagged=np.zeros(B, np.int32))
    chunks = [list(range(i, min(B, i + CHUNK))) for i in range(0, B, CHUNK)]
    t1 = time.time()
    done = 0
    with mp.get_context("fork").Pool(workers) as pool:
        for idx, dr, vr in pool.imap_unordered(_chunk, chunks):
            out["draft_tokens"][idx] = dr.tokens
            out["draft_logq"][idx] = dr.logq
            out["draft_lse"][idx] = dr.lse
            out["draft_margin"][idx] = dr.margin
            out["out_tokens"][idx] = vr.out_tokens
            out["num_accepted"][idx] = vr.num_accepted
            out["logp"][idx] = vr.logp
            out["logq"][idx] = vr.logq
            out["verify_margin"][idx] = vr.margin
            out["verify_rows_flagged"][idx] = vr.rows_flagged
            done += len(idx)
            if done % (CHUNK * 16) == 0 or done == B:
                print(f"[{name}] {done}/{B} requests ({time.time() - t1:.0f} s)", flush=True)
    flagged = (out["draft_margin"].min(axis=1) < od.MARGIN_FLAG) | (out["verify_margin"] < od.MARGIN_FLAG)
    rows = gamma * B + int(out["num_accepted"].sum()) + B   # draft rows + target rows 0..n
    rows_flagged = int((out["draft_margin"] < od.MARGIN_FLAG).sum() + out["verify_rows_flagged"].sum())
    os.makedirs(OUT, exist_ok=True)
    path = os.path.join(OUT, f"{name}.npz")
    np.savez_compressed(path, budget=budget, flagged=flagged, rows=np.int64(rows),
                        rows_flagged=np.int64(rows_flagged), sched_min_gap=np.float64(sched_gap),
                        fingerprint=wl.input_fingerprint(rnd), **out)
    print(f"[{name}] wrote {path}: rows={rows} flagged_rows={rows_flagged} flagged_requests={int(flagged.sum())} "
          f"verified={int(budget.sum())} ({time.time() - t0:.0f} s)", flush=True)
    _G.clear()
    del rnd
    torch.cuda.empty_cache() if torch.cuda.is_available() else None


def main():
    p = argparse.ArgumentParser()
    p.add_argument("names", nargs="*", default=list(CONFIGS) + list(ACCEPTANCE))
    p.add_argument("--workers", type=int, default=max(1, (os.cpu_count() or 2) - 1))
    args = p.parse_args()
    for n in args.names:
        if n in ACCEPTANCE:
            make_acceptance(n, args.workers)
        else:
            make(n, args.workers)


if __name__ == "__main__":
    main()
