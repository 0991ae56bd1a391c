"""A CPU model of the lazy verification pass's cross-workgroup protocol
(`verify_lazy_kernel` in csrc/verify.hip), run under random interleavings.

The kernel's items (target row j of request b, one chunk of blocks) never wait
for one another.  Per request, one 32-bit progress word changes only by atomic
read-modify-writes: bit j = "row j complete", a counter m = "positions 1..m
accepted", and a done bit.  A per-row counter finds the row's last item.  The
test of position j + 1 needs row j complete and positions 1..j accepted, and
whichever of the two atomic updates that establish these comes second runs it:
the row's last item (OR of bit j, seeing m == j) or the tester of position j
(ADD to m, seeing bit j).  Items of rows 2 and later first read the word and
skip their row once the request is decided.

The model runs the same steps as indivisible operations on shared state and
interleaves the items at random (each item's steps in program order).  It
checks:
  * every test runs exactly once, in position order, and only when its row is
    complete (all of the row's chunks counted);
  * each request is finalised exactly once, with the accepted count that the
    sequence of accept decisions fixes;
  * no needed row is skipped.
The model checks the protocol's logic; the memory ordering that makes the
row's statistics visible to the tester (stores completed before the counter
is raised, coherent loads) is the kernel's and is covered by the GPU parity
tests.
"""

import random

import pytest

DONE = 1 << 31
PROG_ONE = 1 << 20


def prog_of(w):
    return (w >> 20) & 31


class Request:
    def __init__(self, budget, n_acc, nch):
        self.L, self.n_acc, self.nch = budget, n_acc, nch
        self.word = 0
        self.rowcnt = [0] * (budget + 1)
        self.tests = []       # positions tested, in order
        self.finals = []      # accepted counts at finalisation
        self.skipped = set()  # rows whose items skipped after the check

    def accept(self, k):      # position k passes its test
        return k <= self.n_acc


def item_steps(req, j, bug=None):
    """The steps of one item of row j as a generator: each yield ends one
    indivisible operation on shared state.  `bug` plants a mistake (the
    checks must catch each one)."""
    if j > 1:
        seen = req.word              # relaxed load of the progress word
        yield
        if seen & DONE:
            req.skipped.add(j)
            return
    # block statistics stored and completed, then the row counter
    before = req.rowcnt[j]
    req.rowcnt[j] += 1
    yield
    if before != req.nch - 1:
        return
    old = req.word                   # fetch-or of the row bit
    req.word |= 1 << j
    yield
    if bug != "test_regardless" and ((old & DONE) or prog_of(old) != j):
        return
    n = j
    while True:
        if n == req.L:
            break                    # every drafted position accepted: the bonus
        k = n + 1
        assert req.rowcnt[n] == req.nch, "test run on an incomplete row"
        req.tests.append(k)
        if not req.accept(k):
            break
        old = req.word               # fetch-add of the accepted count
        req.word += PROG_ONE
        yield
        if bug == "drop_handoff":
            return                   # never goes on, even with row k complete
        if bug != "ignore_row_bit" and not (old & (1 << k)):
            return                   # row k not complete: its last item goes on
        n = k
    req.finals.append(n)
    req.word |= DONE                 # fetch-or of the done bit
    yield


def run(budget, n_acc, nch, seed, order="random", bug=None):
    rng = random.Random(seed)
    req = Request(budget, n_acc, nch)
    items = [item_steps(req, j, bug) for j in range(budget + 1) for _ in range(nch)]
    if order == "reverse":
        items.reverse()
    live = list(items)
    while live:
        g = rng.choice(live) if order == "random" else live[0]
        try:
            next(g)
        except StopIteration:
            live.remove(g)
    return req


def check(req):
    n = req.n_acc
    assert req.finals == [n], req.finals
    want = list(range(1, min(n + 1, req.L) + 1))
    assert req.tests == want, (req.tests, want)
    for j in req.skipped:
        assert j > n, f"row {j} skipped but needed (accepted {n})"


@pytest.mark.parametrize("budget", [0, 1, 2, 3, 5, 8])
@pytest.mark.parametrize("nch", [1, 2, 10])
def test_progress_word_random_interleavings(budget, nch):
    for n_acc in range(budget + 1):
        for seed in range(40):
            check(run(budget, n_acc, nch, seed))


@pytest.mark.parametrize("order", ["in_order", "reverse"])
def test_progress_word_extreme_orders(order):
    # every item to completion in dispatch order (position-major), and the
    # deepest rows first: both parties of every test are exercised
    for budget in range(0, 7):
        for n_acc in range(budget + 1):
            check(run(budget, n_acc, 4, 0, order))


@pytest.mark.parametrize("bug", ["drop_handoff", "ignore_row_bit", "test_regardless"])
def test_model_catches_planted_mistakes(bug):
    # the checks are not vacuous: a tester that never hands over, a tester that
    # runs the next test on a row not yet complete, and a row's last item that
    # tests without its turn each fail them under some interleaving
    caught = 0
    for seed in range(200):
        try:
            check(run(4, 4, 3, seed, bug=bug))
        except AssertionError:
            caught += 1
    assert caught > 0
