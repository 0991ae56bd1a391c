"""Host threads calling the library concurrently, each with its own stream and
workspace (the ABI's contract: calls that share no workspace need no ordering),
from a fresh process so that every kernel's one-time launch set-up (LDS
attributes, occupancy-derived grids) is raced for: the rounds equal the same
rounds run one after another, bit for bit.

The rounds differ in shape so that several kernels are set up at once: the
streaming draft GEMM (bf16, r = 256), the generic paths (V not a multiple of 8,
r = 128), the LDS-staged GEMM (r = 64), and the scheduler beside the last draw."""

import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

CHILD = r"""
import sys, threading
sys.path.insert(0, ROOT)
import numpy as np, torch
from lossless_rejection_sampling_amd import dspark as ds, round as rd, workloads as wl

shapes = [dict(B=32, V=30000, gamma=4, r=256), dict(B=48, V=20001, gamma=3, r=128),
          dict(B=16, V=40000, gamma=5, r=64), dict(B=24, V=12000, gamma=4, r=256)]
rounds = [wl.dspark5(device="cuda", seed_base=500 + i, scheduled=True, name=f"thread{i}", **s)
          for i, s in enumerate(shapes)]
torch.cuda.synchronize()
OUT = ("draft_tokens", "draft_logq", "draft_lse", "budget", "out_tokens", "num_accepted", "num_emitted")
results, errors = {}, []
start = threading.Barrier(len(rounds))

def work(i):
    try:
        s = torch.cuda.Stream()  # default priority
        with torch.cuda.stream(s):
            buf = rd.allocate(rounds[i])
            start.wait()
            for _ in range(3):
                rd.run_round(rounds[i], buf, stream=s)
            s.synchronize()
            if ds.dspark_status(buf.workspace, s) != ds.DSPARK_OK:
                raise RuntimeError(f"status of round {i}")
            results[i] = {k: getattr(buf, k).cpu().numpy().copy() for k in OUT}
    except Exception as e:  # reported by the main thread
        errors.append(f"{i}: {e!r}")

threads = [threading.Thread(target=work, args=(i,)) for i in range(len(rounds))]
for t in threads: t.start()
for t in threads: t.join(timeout=120)
assert not errors, errors
assert len(results) == len(rounds), "a thread did not finish"
for i, rnd in enumerate(rounds):
    buf = rd.allocate(rnd)
    rd.run_round(rnd, buf)
    torch.cuda.synchronize()
    assert ds.dspark_status(buf.workspace) == ds.DSPARK_OK
    for k in OUT:
        a, b = results[i][k], getattr(buf, k).cpu().numpy()
        assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (i, k)
print("threads ok:", [int(results[i]["num_emitted"].sum()) for i in range(len(rounds))], flush=True)
"""


def test_concurrent_host_threads_match_sequential_rounds():
    print("[threads] 4 host threads, own streams and workspaces, fresh process", flush=True)
    res = subprocess.run([sys.executable, "-c", CHILD.replace("ROOT", repr(ROOT), 1)], capture_output=True,
                         text=True, timeout=300, cwd=ROOT)
    assert res.returncode == 0, res.stdout[-2000:] + res.stderr[-4000:]
    assert "threads ok" in res.stdout, res.stdout
