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



def test_forced_stall_is_reported_and_the_workspace_recovers():
    # the waits' bound forced to zero from the host: workgroups pass their
    # device-wide waits early, the kernel completes (every index it reads across
    # workgroups is clamped), the status word carries the stall bit, and the
    # workspace then serves both paths with the results of a fresh one
    say("[resident stall] wait bound 0, B=64 gamma=4 V=30000")
    rnd = wl.small_random(64, 4, 30000, 256, DEV, seed=9, dtype=torch.bfloat16, factor_dtype=torch.bfloat16,
                          temps=(1.0, 0.0, 0.7))
    fresh = rd.allocate(rnd)
    ref = _draft(rnd, fresh, ds.DSPARK_DRAFT_PER_POSITION)
    buf = rd.allocate(rnd)
    prev_bound = ds.dspark_set_resident_wait_bound(0.0)
    prev_path = ds.dspark_set_draft_path(ds.DSPARK_DRAFT_RESIDENT)
    ds.dspark_profile_enable(CLS_ROUND, 1)
    try:
        rd.draft(rnd, buf)
        torch.cuda.synchronize()
        launches, _ = ds.dspark_profile_read(CLS_ROUND)
    finally:
        ds.dspark_profile_enable(CLS_ROUND, 0)
        ds.dspark_set_draft_path(prev_path)
        ds.dspark_set_resident_wait_bound(prev_bound)
    assert prev_bound == pytest.approx(0.2)
    assert launches == 1, "the resident kernel did not run"
    word = int(buf.workspace[:4].view(torch.int32).item())
    assert word & 64, f"status word {word:#x}: no stall reported"
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_EDATA
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK  # read and cleared
    _same(ref, _draft(rnd, buf, ds.DSPARK_DRAFT_PER_POSITION), "per-position after the stall")
    _same(ref, _draft(rnd, buf, ds.DSPARK_DRAFT_RESIDENT), "resident after the stall")


COOP_CHILD = r"""
import sys
sys.path.insert(0, ROOT)
import torch
from lossless_rejection_sampling_amd import dspark as ds, round as rd, workloads as wl
cls = ds.KERNEL_CLASSES["draft_round"]
rnd = wl.small_random(64, 4, 30000, 256, "cuda", seed=9, dtype=torch.bfloat16, factor_dtype=torch.bfloat16,
                      temps=(1.0, 0.0, 0.7))
ref_buf, buf = rd.allocate(rnd), rd.allocate(rnd)
rd.draft(rnd, ref_buf)
ds.dspark_set_draft_path(ds.DSPARK_DRAFT_RESIDENT)
ds.dspark_profile_enable(cls, 1)
rd.draft(rnd, buf)
torch.cuda.synchronize()
n = ds.dspark_profile_read(cls)[0]
ds.dspark_profile_enable(cls, 0)
ds.dspark_set_draft_path(ds.DSPARK_DRAFT_PER_POSITION)
rd.draft(rnd, buf)  # and the next call on this thread sees no stale error
torch.cuda.synchronize()
assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
for k in ("draft_tokens", "draft_logq", "draft_lse"):
    assert torch.equal(getattr(buf, k), getattr(ref_buf, k)), k
print("coop ok: resident launches", n, flush=True)
"""


def test_second_process_falls_back_when_cooperative_launch_is_refused():
    # this process has made cooperative launches (the tests above), which the
    # HIP runtime lets only one process on the device hold: a second process
    # asking for the resident round gets the per-position launches, with the
    # same results and no error left behind
    import os
    import subprocess
    import sys

    rnd = wl.small_random(8, 2, 4096, 256, DEV, seed=3, dtype=torch.bfloat16, factor_dtype=torch.bfloat16)
    assert _resident_launches(rnd, rd.allocate(rnd)) == 1
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    say("[resident coop] second process, B=64 gamma=4 V=30000")
    res = subprocess.run([sys.executable, "-c", COOP_CHILD.replace("ROOT", repr(root), 1)], capture_output=True,
                         text=True, timeout=300, cwd=root)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "coop ok" in res.stdout, res.stdout
    say(res.stdout.strip())
