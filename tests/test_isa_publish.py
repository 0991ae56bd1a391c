"""The cross-workgroup publications keep their order through compilation.

The lazy verification pass and the scheduler pass data between workgroups
with relaxed agent-scope atomics: a workgroup stores its data with coherent
(sc1) stores, waits for them to complete (an explicit `s_waitcnt vmcnt(0)`),
meets its other wavefronts at a barrier and only then takes the atomic that
tells other workgroups the data is there (the row counter of the verification
pass, the scheduler's ticket).  The order is what the source writes, but the
language's memory model does not oblige the compiler to keep relaxed atomics
in it, so this test reads the gfx950 assembly of the built sources and checks,
at each publication point (marked in the source by an assembly comment):

  * the first global atomic after the marker is a returning atomic add;
  * no global store or atomic comes between the marker and it;
  * the nearest `s_barrier` before the marker comes after the last global store
    or atomic before the marker, with an `s_waitcnt vmcnt(0)` between them.

Text order stands for program order here: the checked stretch is straight-line
code (a barrier every wavefront reaches, then the atomic).  CPU only: hipcc
cross-compiles the device code; no GPU is used.
"""

import os
import re
import subprocess

import pytest

from lossless_rejection_sampling_amd import build

STORE = re.compile(r"^\s*(global_store|global_atomic|buffer_store|buffer_atomic|flat_store|flat_atomic)\w*\s")
ATOMIC = re.compile(r"^\s*(global|flat|buffer)_atomic\w*\s")
WAIT_ALL = re.compile(r"^\s*s_waitcnt\s+vmcnt\(0\)(\s|$)")
BARRIER = re.compile(r"^\s*s_barrier(\s|$)")


def _hipcc():
    try:
        return build.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    cc = _hipcc()
    out = {}
    d = tmp_path_factory.mktemp("isa")
    for src in ("verify.hip", "schedule.hip", "draft.hip"):
        s = str(d / (src + ".s"))
        cmd = [cc, *build.HIPCC_FLAGS, *build.SOURCE_FLAGS.get(src, []), "-I", build.INCLUDE, "-I", build.CSRC,
               "--cuda-device-only", "-S", os.path.join(build.CSRC, src), "-o", s]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert res.returncode == 0, res.stderr[-3000:]
        out[src] = open(s).read().splitlines()
    return out


def _functions(lines):
    """(name, body lines) of every function in an assembly listing."""
    funcs, name, body = [], None, []
    for ln in lines:
        m = re.match(r"^(_Z\w+):", ln)
        if m:
            name, body = m.group(1), []
            continue
        if name is not None:
            if ln.startswith("\t.size") or ln.startswith(".Lfunc_end"):
                funcs.append((name, body))
                name = None
            else:
                body.append(ln)
    return funcs


def _check_point(body, at):
    # the atomic that publishes
    i = next((k for k in range(at + 1, len(body)) if ATOMIC.match(body[k]) or STORE.match(body[k])), None)
    assert i is not None, "no atomic after the marker"
    assert ATOMIC.match(body[i]) and "_add" in body[i].split()[0], body[i]
    assert re.search(r"\bsc0\b", body[i]), f"not a returning atomic: {body[i].strip()}"
    # the barrier before the marker, and the data stores before it
    b = max((k for k in range(at) if BARRIER.match(body[k])), default=None)
    assert b is not None, "no barrier before the marker"
    assert not any(STORE.match(body[k]) for k in range(b + 1, at)), "a store between the barrier and the marker"
    s = max((k for k in range(b) if STORE.match(body[k])), default=None)
    assert s is not None, "no published store before the barrier"
    assert any(WAIT_ALL.match(body[k]) for k in range(s + 1, b)), (
        f"no s_waitcnt vmcnt(0) between the last store ({body[s].strip()}) and the barrier")
    return i


@pytest.mark.parametrize("src,marker,kernels", [
    ("verify.hip", "dspark publish: row counter", ["verify_lazy_kernel"]),
    ("schedule.hip", "dspark publish: scheduler ticket", ["schedule_kernel"]),
    ("draft.hip", "dspark publish: scheduler ticket", ["draft_select_schedule"]),
])
def test_publication_order_survives_compilation(asm, src, marker, kernels):
    seen = 0
    for name, body in _functions(asm[src]):
        if not any(k in name for k in kernels):
            continue
        points = [k for k, ln in enumerate(body) if marker in ln]
        assert points, f"{name}: marker not found"
        for at in points:
            _check_point(body, at)
        seen += 1
    assert seen >= 1, f"no {kernels} in {src}"


def test_checker_catches_a_missing_wait():
    # the rule itself, on hand-written listings: with the wait, and without it
    good = ["\tglobal_store_dwordx2 v[2:3], v[0:1], off sc1", "\ts_waitcnt vmcnt(0)", "\ts_barrier",
            "\t;; dspark publish: row counter", "\tv_mov_b32 v1, 0", "\tglobal_atomic_add v1, v1, v2, s[10:11] sc0"]
    assert _check_point(good, 3) == 5
    bad = [good[0], good[2], good[3], good[4], good[5]]
    with pytest.raises(AssertionError, match="s_waitcnt"):
        _check_point(bad, 2)
    late = [good[0], good[1], good[2], good[3], "\tglobal_store_dword v1, v2, off sc1", good[5]]
    with pytest.raises(AssertionError):
        _check_point(late, 3)
