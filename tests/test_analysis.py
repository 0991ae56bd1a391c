"""Host-side Theta of a set of verify budgets agrees with the oracle's
expected throughput (the measure "DSpark, la bozza ..." compares schedulers
by, section "Verificare meglio, non di più"), including batches beyond the
last point of the step-rate table."""

import numpy as np
import pytest

from lossless_rejection_sampling_amd import analysis
from lossless_rejection_sampling_amd import workloads as wl
from oracle import dspark as od


@pytest.mark.parametrize("B,gamma,seed", [(8, 3, 0), (256, 5, 1), (512, 5, 2)])
def test_theta_matches_the_oracle(B, gamma, seed):
    rng = np.random.default_rng(seed)
    c = rng.uniform(0.05, 0.99, size=(B, gamma)).astype(np.float32)
    Bs, sps = wl.sps_table_linear()
    for budget in [np.zeros(B, int), np.full(B, gamma), rng.integers(0, gamma + 1, B)]:
        got = analysis.expected_theta(c, budget, Bs, sps)
        want = od.expected_theta(c, budget, Bs, sps)
        assert got == pytest.approx(want, rel=1e-9)
