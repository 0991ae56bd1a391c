"""The resident draft round (one cooperative launch for every block position,
W2 held on chip) against the per-position launches, bit for bit.

Both implementations compute the tile statistics with the same arithmetic and
draw with the same code, so tokens, ln q and the row log-sum-exp must agree
exactly; the per-position path is itself compared with the oracle by the other
parity tests.  Each resident case runs twice on one workspace (the second call
relies on the first leaving its phase flags at zero) and checks, through the
kernel-class timer, that the resident kernel really ran.  The shapes cover a
ragged last tile, a last tile of 8 columns (its second stage wholly beyond V),
fewer tiles than workgroups (empty wavefronts and tiles split across them),
more requests than workgroups (several draws per workgroup), a single request,
the largest batch, the largest vocabulary that fits (10 tiles per CU) and the
first one that does not (which falls back to the per-position launches).
"""

import pytest
import torch

from lossless_rejection_sampling_amd import dspark as ds
from lossless_rejection_sampling_amd import round as rd
from lossless_rejection_sampling_amd import workloads as wl

from parity import say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

DEV = "cuda"
CLS_ROUND = ds.KERNEL_CLASSES["draft_round"]


def _draft(rnd, buf, path):
    prev = ds.dspark_set_draft_path(path)
    try:
        rd.draft(rnd, buf)
        torch.cuda.synchronize()
    finally:
        ds.dspark_set_draft_path(prev)
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
    return buf.draft_tokens.clone(), buf.draft_logq.clone(), buf.draft_lse.clone()


def _same(a, b, what):
    for name, x, y in zip(("tokens", "ln q", "lse"), a, b):
        if not torch.equal(x, y):
            bad = (x != y).nonzero()
            raise AssertionError(f"{what}: {name} differs at {bad.shape[0]} places, first {bad[:4].tolist()}")


def _resident_launches(rnd, buf):
    ds.dspark_profile_enable(CLS_ROUND, 1)
    try:
        _draft(rnd, buf, ds.DSPARK_DRAFT_RESIDENT)
        n, _ = ds.dspark_profile_read(CLS_ROUND)
    finally:
        ds.dspark_profile_enable(CLS_ROUND, 0)
    return n


CASES = [
    ("headline shape", dict(B=256, gamma=5, V=151936, temps=(1.0, 0.0, 0.7, 1.3))),
    ("ragged last tile", dict(B=37, gamma=4, V=20000, temps=(1.0, 0.0, 0.8))),
    ("8-column last tile", dict(B=70, gamma=3, V=64 * 300 + 8, temps=(0.9, 0.0))),
    ("fewer tiles than workgroups", dict(B=300, gamma=2, V=9000, temps=(1.0, 0.0, 2.0))),
    ("one request", dict(B=1, gamma=16, V=2048, temps=(1.0,))),
    ("largest batch", dict(B=2048, gamma=1, V=4096, temps=(1.0, 0.0))),
    ("largest vocabulary", dict(B=64, gamma=2, V=163840, temps=(1.0, 0.5))),
]


@pytest.mark.parametrize("name,case", CASES, ids=[c[0] for c in CASES])
def test_resident_matches_per_position(name, case):
    say(f"[resident {name}] {case}")
    rnd = wl.small_random(case["B"], case["gamma"], case["V"], 256, DEV, seed=7, dtype=torch.bfloat16,
                          factor_dtype=torch.bfloat16, temps=case["temps"])
    rnd.pos_offset = torch.arange(rnd.B, device=DEV, dtype=torch.int32) * 3
    buf = rd.allocate(rnd)
    ref = _draft(rnd, buf, ds.DSPARK_DRAFT_PER_POSITION)
    assert _resident_launches(rnd, buf) == 1, "the resident kernel did not run"
    _same(ref, (buf.draft_tokens, buf.draft_logq, buf.draft_lse), f"{name}, first call")
    again = _draft(rnd, buf, ds.DSPARK_DRAFT_RESIDENT)
    _same(ref, again, f"{name}, second call")


def test_vocabulary_beyond_the_resident_capacity_falls_back():
    # 2561 tiles: 11 on some CU of 256, one more than W2's register budget holds
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    V = 64 * (10 * cus + 1)
    rnd = wl.small_random(16, 2, V, 256, DEV, seed=8, dtype=torch.bfloat16, factor_dtype=torch.bfloat16)
    buf = rd.allocate(rnd)
    ref = _draft(rnd, buf, ds.DSPARK_DRAFT_PER_POSITION)
    assert _resident_launches(rnd, buf) == 0
    _same(ref, (buf.draft_tokens, buf.draft_logq, buf.draft_lse), "fallback")


def test_per_position_is_the_default():
    prev = ds.dspark_set_draft_path(ds.DSPARK_DRAFT_PER_POSITION)
    ds.dspark_set_draft_path(prev)
    assert prev == ds.DSPARK_DRAFT_PER_POSITION


def test_draft_schedule_resident_budgets():
    # the combined call: the resident round, then the scheduler
    rnd = wl.headline(DEV)
    buf = rd.allocate(rnd)
    prev = ds.dspark_set_draft_path(ds.DSPARK_DRAFT_PER_POSITION)
    try:
        rd.draft_schedule(rnd, buf)
        torch.cuda.synchronize()
        ref = (buf.draft_tokens.clone(), buf.draft_logq.clone(), buf.draft_lse.clone(), buf.budget.clone())
        ds.dspark_set_draft_path(ds.DSPARK_DRAFT_RESIDENT)
        rd.draft_schedule(rnd, buf)
        torch.cuda.synchronize()
    finally:
        ds.dspark_set_draft_path(prev)
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
    _same(ref[:3], (buf.draft_tokens, buf.draft_logq, buf.draft_lse), "draft_schedule")
    assert torch.equal(ref[3], buf.budget)


def test_set_draft_path_rejects_unknown_values():
    assert ds.lib().dspark_set_draft_path(7) == ds.DSPARK_EINVAL
