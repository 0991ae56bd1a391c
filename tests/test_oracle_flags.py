"""How often the oracle flags a decision as too close to call (margin below
1e-6, where fp32 arithmetic on the GPU may legitimately decide the other way),
measured on the full-size workloads.

The whole-batch expectations in tests/golden/rounds were written by
tests/golden/make_round_goldens.py from the oracle over every request of every
full-size workload; each records the decisions it made (one per draft row, one
per target row up to the first rejection, the final draw) and how many of them
the oracle flagged.  The bar on flagged rows is 0.01% of all rows, counted here
without a one-row allowance, over more than 2 x 10^4 rows."""

import os

import numpy as np
import pytest

from oracle import dspark as od

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rounds")
NAMES = ["dspark5_B64", "headline_B256", "headline_B256_full", "block_length_g4", "block_length_g8",
         "block_length_g16", "scheduled_B512", "stress_B1024"]


def _load(name):
    with np.load(os.path.join(GOLDEN, f"{name}.npz"), allow_pickle=False) as z:
        return {k: z[k] for k in z.files}


@pytest.mark.parametrize("name", NAMES)
def test_golden_is_consistent(name):
    g = _load(name)
    B, gamma = g["draft_tokens"].shape
    n = g["num_accepted"]
    assert np.all((0 <= n) & (n <= g["budget"])) and np.all(g["budget"] <= gamma)
    # x_1..x_n, the final token, then -1
    for b in range(B):
        assert np.array_equal(g["out_tokens"][b, :n[b]], g["draft_tokens"][b, :n[b]])
        assert g["out_tokens"][b, n[b]] >= 0 and np.all(g["out_tokens"][b, n[b] + 1:] == -1)
    # the flags follow from the recorded margins
    flagged = (g["draft_margin"].min(axis=1) < od.MARGIN_FLAG) | (g["verify_margin"] < od.MARGIN_FLAG)
    assert np.array_equal(flagged, g["flagged"])
    assert int(g["rows"]) == B * gamma + int(n.sum()) + B
    assert float(g["sched_min_gap"]) > od.SCHED_FLAG


def test_flagged_rows_below_one_in_ten_thousand():
    rows = flagged = 0
    for name in NAMES:
        g = _load(name)
        rows += int(g["rows"])
        flagged += int(g["rows_flagged"])
    assert rows >= 20000, rows
    assert flagged < 1e-4 * rows, (flagged, rows)


def test_flag_fires_on_a_tie():
    # a greedy draft row with two equal maxima: the oracle must flag it (margin 0)
    V, r = 64, 2
    base = np.zeros((1, 1, V))
    base[0, 0, 5] = base[0, 0, 9] = 3.0
    U = np.zeros((V, r))
    W = np.zeros((r, V))
    dr = od.draft_round(base, U, W, np.array([0]), np.array([0.0]), 1)
    assert dr.tokens[0, 0] == 5 and dr.margin[0, 0] == 0.0
