"""dspark_schedule_static (the scheduler on the library's own scratch, no
workspace and no allocation) against dspark_schedule on a caller workspace:
budgets bit for bit on two calls in a row, the second with a smaller batch,
then data-error reporting through the status word and the size limit."""

import numpy as np
import pytest
import torch

from lossless_rejection_sampling_amd import dspark as ds
from lossless_rejection_sampling_amd import workloads as wl

from parity import say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

DEV = "cuda"


def _with_workspace(conf, tB, tS):
    B, gamma = conf.shape
    budget = torch.full((B,), -5, dtype=torch.int32, device=DEV)
    ws = torch.zeros(ds.dspark_schedule_workspace_bytes(B, gamma), dtype=torch.uint8, device=DEV)
    ds.dspark_schedule(conf, tB, tS, budget, ws)
    torch.cuda.synchronize()
    assert ds.dspark_status(ws) == ds.DSPARK_OK
    return budget.cpu().numpy()


def test_static_scratch_matches_workspace_call():
    Bs, sps = wl.sps_table_linear()
    tB, tS = torch.tensor(Bs, device=DEV), torch.tensor(sps, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    # two calls in a row, the second smaller; then the largest size the scratch holds
    for B, gamma, seed in [(1024, 8, 1), (256, 5, 2), (7, 3, 3), (2048, 4, 4)]:
        say(f"[schedule_static] B={B} gamma={gamma}")
        conf = wl.confidence_scores(B, gamma, 700 + seed, DEV)
        budget = torch.full((B,), -3, dtype=torch.int32, device=DEV)
        ds.dspark_schedule_static(conf, tB, tS, budget, status)
        torch.cuda.synchronize()
        got = budget.cpu().numpy()
        assert int(status.item()) == 0
        assert np.array_equal(got, _with_workspace(conf, tB, tS)), (B, gamma)
        assert got.sum() > 0


def test_static_scratch_reports_data_errors_and_limits():
    Bs, sps = wl.sps_table_linear()
    tB, tS = torch.tensor(Bs, device=DEV), torch.tensor(sps, device=DEV)
    conf = wl.confidence_scores(64, 4, 9, DEV)
    bad = conf.clone()
    bad[3, 1] = 1.5
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    budget = torch.empty(64, dtype=torch.int32, device=DEV)
    ds.dspark_schedule_static(bad, tB, tS, budget, status)
    torch.cuda.synchronize()
    assert int(status.item()) != 0
    # without a status word the bits are dropped; the next good call is exact again
    ds.dspark_schedule_static(bad, tB, tS, budget, None)
    status.zero_()
    ds.dspark_schedule_static(conf, tB, tS, budget, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert np.array_equal(budget.cpu().numpy(), _with_workspace(conf, tB, tS))
    # beyond the scratch's size: refused on the host, nothing enqueued
    big = torch.full((1025, 8), 0.5, device=DEV)
    with pytest.raises(ds.DsparkError) as e:
        ds.dspark_schedule_static(big, tB, tS, torch.empty(1025, dtype=torch.int32, device=DEV))
    assert e.value.code == ds.DSPARK_EINVAL
