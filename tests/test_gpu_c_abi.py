"""The C ABI from a plain C program (tests/c/abi_round.c: HIP runtime buffers,
no Python or PyTorch in its process) gives the round the Python binding gives on
the same inputs, bit for bit: draft tokens, ln q, ln-sum-exp, budgets, emitted
tokens and counts.

The program draws its inputs from a counter-based integer hash (lowbias32 over
(index * 0x9E3779B9 + stream), uint32 arithmetic); this test regenerates them
with numpy, runs dspark_draft_schedule and dspark_verify through the binding,
and compares with the file the program wrote.  The program is built by the
entry script's build() (tests/c/build.py)."""

import os
import subprocess

import numpy as np
import pytest
import torch

from lossless_rejection_sampling_amd import dspark as ds

HERE = os.path.dirname(os.path.abspath(__file__))
BIN = os.path.join(HERE, "c", "_bin", "abi_round")
B, GAMMA, V, R = 64, 4, 12392, 128
SEED = 12345

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
    pytest.mark.skipif(not os.path.exists(BIN), reason="C program not built (tests/c/build.py)"),
]


def _mix(x):
    x = x ^ (x >> np.uint32(16))
    x = x * np.uint32(0x7FEB352D)
    x = x ^ (x >> np.uint32(15))
    x = x * np.uint32(0x846CA68B)
    return x ^ (x >> np.uint32(16))


def _hash(salt, n):
    i = np.arange(n, dtype=np.uint32)
    with np.errstate(over="ignore"):
        return _mix(i * np.uint32(0x9E3779B9) + np.uint32(salt))


def _bf16_bits(h, e0):
    s, m, e = h >> np.uint32(31), h & np.uint32(127), np.uint32(e0 + 127) + ((h >> np.uint32(7)) & np.uint32(3))
    return ((s << np.uint32(15)) | (e << np.uint32(7)) | m).astype(np.uint16)


def _inputs():
    target = _bf16_bits(_hash(1, B * (GAMMA + 1) * V), -2).reshape(B, GAMMA + 1, V)
    flips = (_hash(2, B * GAMMA * V) & np.uint32(3)).astype(np.uint16).reshape(B, GAMMA, V)
    base = target[:, :GAMMA, :] ^ flips
    U = _bf16_bits(_hash(3, V * R), -7).reshape(V, R)
    W = _bf16_bits(_hash(4, V * R), -7).reshape(V, R)
    prev0 = (_hash(5, B) % np.uint32(V)).astype(np.int32)
    b = np.arange(B)
    temperature = np.where(b % 4 == 3, np.float32(0.0), np.where(b % 2 == 1, np.float32(0.7), np.float32(1.0)))
    conf = ((np.uint32(1) + _hash(6, B * GAMMA) % np.uint32(998)).astype(np.float32) / np.float32(1000.0))
    sps_B = np.array([1.0, 8.0, 64.0, 512.0])
    sps_val = 1e6 / (20000.0 + 5.0 * sps_B)
    return target, base, U, W, prev0, temperature.astype(np.float32), conf.reshape(B, GAMMA), sps_B, sps_val


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def test_c_program_matches_the_binding(tmp_path):
    out = tmp_path / "round.bin"
    print(f"[c abi] {BIN} B={B} gamma={GAMMA} V={V} r={R}", flush=True)
    res = subprocess.run([BIN, str(out)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert res.stdout.startswith("abi_round ok"), res.stdout

    target, base, U, W, prev0, temperature, conf, sps_B, sps_val = _inputs()
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    t_target, t_base, t_U, t_W = _bf16_dev(target), _bf16_dev(base), _bf16_dev(U), _bf16_dev(W)
    t_prev0, t_T, t_conf, t_sB, t_sV = dev(prev0), dev(temperature), dev(conf), dev(sps_B), dev(sps_val)
    ws = torch.zeros(ds.dspark_workspace_bytes(B, GAMMA, V, R), dtype=torch.uint8, device="cuda")
    draft = torch.empty(B, GAMMA, dtype=torch.int32, device="cuda")
    logq = torch.empty(B, GAMMA, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, GAMMA, dtype=torch.float64, device="cuda")
    budget = torch.empty(B, dtype=torch.int32, device="cuda")
    tokens = torch.empty(B, GAMMA + 1, dtype=torch.int32, device="cuda")
    nacc = torch.empty(B, dtype=torch.int32, device="cuda")
    nem = torch.empty(B, dtype=torch.int32, device="cuda")
    ds.dspark_draft_schedule(t_base, t_U, t_W, t_prev0, t_T, SEED, None, draft, logq, lse, t_conf, None, t_sB, t_sV,
                             "early_stop", 0.0, budget, ws)
    ds.dspark_verify(t_target, t_base, t_U, t_W, t_prev0, draft, logq, lse, budget, t_T, SEED, None, tokens, nacc, nem,
                     ws)
    assert ds.dspark_status(ws) == ds.DSPARK_OK

    raw = out.read_bytes()
    parts, at = [], 0
    for dt, n in [(np.int32, B * GAMMA), (np.float32, B * GAMMA), (np.float64, B * GAMMA), (np.int32, B),
                  (np.int32, B * (GAMMA + 1)), (np.int32, B), (np.int32, B)]:
        parts.append(np.frombuffer(raw, dtype=dt, count=n, offset=at))
        at += n * np.dtype(dt).itemsize
    assert at == len(raw)
    mine = [draft, logq, lse, budget, tokens, nacc, nem]
    for name, c, t in zip(["draft", "logq", "lse", "budget", "tokens", "accepted", "emitted"], parts, mine):
        t = t.cpu().numpy().reshape(-1)
        assert np.array_equal(c.view(np.uint8), t.view(np.uint8)), name
    # the round exercises both outcomes of the accept test and a spread of budgets
    n, L = parts[5], parts[3]
    assert (n < L).any() and (n == L).any() and len(set(L.tolist())) > 1
