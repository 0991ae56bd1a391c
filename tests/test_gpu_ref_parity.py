"""Whole batches of moderate-size rounds against the C oracle
(oracle/dspark_ref.c), run in the test: every request compared, with the bar of
the other parity tests (tokens, accepted counts and budgets exact except where
the oracle flags a decision margin below 1e-6; ln q, ln p and the row
log-sum-exp within their tolerances).

The C oracle (plain fp64 loops, OpenMP over requests) is pinned against the
numpy oracle by tests/test_oracle_ref.py and is fast enough that whole batches
with tens of thousands of vocabulary entries are compared request by request
here.  The sizes select every kernel path of the round: the streaming draft
GEMM (bf16 logits and factors, V a multiple of 8, r = 128 or 256; one slot
group, and two with the second partly filled at B = 300), the
LDS-staged GEMM (r = 64), the generic paths (V not a multiple of 8, fp32
logits, fp32 factors), scheduler budgets, random budgets with position
offsets, and the full budget; and a round whose logits exceed 4 GiB (the
64-bit addressed paths), compared on requests sampled across the batch.
"""

import os

import numpy as np
import pytest
import torch

from lossless_rejection_sampling_amd import dspark as ds
from lossless_rejection_sampling_amd import workloads as wl
from oracle import dspark as od
from oracle import ref

from parity import check, compare, run_c_oracle, run_gpu, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
    pytest.mark.skipif(not os.path.exists(ref.LIB), reason="C oracle not built (oracle/build.py)"),
]

DEV = "cuda"
BF16, F32 = torch.bfloat16, torch.float32

# name, B, gamma, V, r, logits dtype, factor dtype, temperatures, budgets
CASES = [
    ("streaming r256 scheduled", 192, 6, 98344, 256, BF16, BF16, (1.0, 0.7, 0.0, 1.3), "scheduled"),
    ("streaming r128 random budgets offsets", 160, 8, 65536, 128, BF16, BF16, (0.9, 0.0, 1.1), "random"),
    ("V not a multiple of 8", 100, 5, 70001, 256, BF16, BF16, (1.0, 0.0), "full"),
    ("fp32 logits", 64, 5, 50000, 256, F32, BF16, (1.0, 0.5, 0.0), "scheduled"),
    ("fp32 factors r64", 48, 4, 40000, 64, BF16, F32, (1.2, 0.0), "random"),
    ("LDS-staged r64", 128, 4, 60000, 64, BF16, BF16, (1.0,), "full"),
    ("streaming two slot groups the second partial", 300, 3, 50000, 256, BF16, BF16, (1.0, 0.0, 0.6), "random"),
]


def _round(case, seed):
    _, B, gamma, V, r, dt, fdt, temps, budgets = case
    rnd = wl.small_random(B, gamma, V, r, device=DEV, seed=seed, dtype=dt, factor_dtype=fdt, temps=temps)
    rng = np.random.default_rng(seed)
    if budgets == "scheduled":
        rnd.conf = wl.confidence_scores(B, gamma, seed, DEV)
        rnd.sps_B, rnd.sps_val = wl.sps_table_linear()
    elif budgets == "random":
        rnd.budget = torch.tensor(rng.integers(0, gamma + 1, B), dtype=torch.int32, device=DEV)
        rnd.pos_offset = torch.tensor(rng.integers(0, 4000, B), dtype=torch.int32, device=DEV)
    return rnd


def _c_oracle(rnd) -> od.RoundResult:
    return run_c_oracle(rnd)


@pytest.mark.parametrize("k", range(len(CASES)), ids=[c[0].replace(" ", "_") for c in CASES])
def test_whole_batch_against_the_c_oracle(k):
    case = CASES[k]
    rnd = _round(case, seed=600 + k)
    say(f"[c oracle {case[0]}] B={rnd.B} gamma={rnd.gamma} V={rnd.V} r={rnd.r} budgets={case[8]}")
    buf = run_gpu(rnd)
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
    want = _c_oracle(rnd)
    idx = np.arange(rnd.B)
    rep = compare(rnd, buf, want, idx)
    check(rep, f"c_oracle_{k}")
    # the round exercises both outcomes of the accept test
    n = buf.num_accepted.cpu().numpy()
    assert (n < want.budget).any() and (n == want.budget).any()


def test_logits_beyond_4_gib():
    # B = 1024, gamma = 16, V = 151936 in bf16: target and backbone logits of
    # 5.3 and 5.0 GB, beyond the 32-bit byte offsets of the coalesced kernels, so
    # the round runs on the 64-bit addressed paths.  Requests sampled across the
    # batch (the last ones past the 4 GiB mark) against the C oracle with their
    # own request ids.
    B, gamma, V, r = 1024, 16, 151936, 256
    rnd = wl.small_random(B, gamma, V, r, device=DEV, seed=77, dtype=BF16, factor_dtype=BF16, temps=(1.0, 0.0, 0.8))
    rng = np.random.default_rng(77)
    rnd.budget = torch.tensor(rng.integers(0, gamma + 1, B), dtype=torch.int32, device=DEV)
    assert B * (gamma + 1) * V * 2 > 1 << 32
    say(f"[c oracle beyond 4 GiB] B={B} gamma={gamma} V={V} r={r}")
    buf = run_gpu(rnd)
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
    idx = np.array([0, 1, 257, 511, 600, 777, 1000, 1021, 1022, 1023])
    h = wl.to_host
    t = torch.as_tensor(idx, dtype=torch.long, device=DEV)
    pick = lambda x: h(x.index_select(0, t))
    target, base, prev0, T = pick(rnd.target), pick(rnd.base), pick(rnd.prev0), pick(rnd.temperature)
    U, W = h(rnd.U), h(rnd.W)
    budget = h(rnd.budget)[idx].astype(np.int32)
    ids = idx.astype(np.int32)
    dr = ref.draft_round(base, U, W, prev0, T, rnd.seed, None, ids)
    vr = ref.verify(target, base, U, W, prev0, dr.tokens, T, rnd.seed, budget, None, ids)
    rep = compare(rnd, buf, od.RoundResult(dr, budget, None, vr), idx)
    check(rep, "beyond_4gib")
