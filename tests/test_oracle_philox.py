"""Pins of the oracle's Philox4x32-10 and its uniform / Gumbel maps.

The exact output bits are pinned against an independent implementation of the
same published generator: PyTorch ships a header-only Philox4x32-10 engine
(ATen/core/PhiloxRNGEngine.h); a small program compiled here from that header
(a library routine, not code of this repository) is run on the same counters.
The statistical properties the method needs (uniform, independent draws) are
pinned by chi-square and correlation tests.
"""

import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest
from scipy import stats

from oracle import philox as px

_PROGRAM = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
int main() {
  unsigned long long seed, subseq, offset;
  while (std::scanf("%llu %llu %llu", &seed, &subseq, &offset) == 3) {
    at::philox_engine e(seed, subseq, offset);
    unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
"""


def _torch_include():
    try:
        import torch
    except Exception:
        return None
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    return inc if os.path.exists(os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")) else None


@pytest.fixture(scope="module")
def torch_philox():
    inc = _torch_include()
    if inc is None or shutil.which("g++") is None:
        pytest.skip("torch Philox header or g++ unavailable")
    d = tempfile.mkdtemp()
    src, exe = os.path.join(d, "drv.cpp"), os.path.join(d, "drv")
    with open(src, "w") as f:
        f.write(_PROGRAM)
    subprocess.run(["g++", "-std=c++17", "-O1", "-I", inc, src, "-o", exe], check=True)

    def run(triples):
        inp = "".join(f"{s} {q} {o}\n" for s, q, o in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [tuple(int(x) for x in line.split()) for line in out.strip().splitlines()]

    return run


def test_philox_matches_independent_implementation(torch_philox):
    # The library engine maps (seed, subsequence, offset) to key = seed and
    # counter = (offset lo, offset hi, subsequence lo, subsequence hi).
    rng = np.random.default_rng(7)
    cases = [(0, 0, 0), (2 ** 64 - 1, 2 ** 64 - 1, 2 ** 64 - 1), (20260706, 3 << 32 | 17, 5 << 32 | 9)]
    for _ in range(200):
        cases.append(tuple(int(x) for x in rng.integers(0, 2 ** 63, size=3, dtype=np.uint64)))
    want = torch_philox(cases)
    for (seed, sub, off), w in zip(cases, want):
        got = px.philox4x32_10(off & 0xFFFFFFFF, off >> 32, sub & 0xFFFFFFFF, sub >> 32,
                               seed & 0xFFFFFFFF, seed >> 32)
        assert tuple(int(g) for g in got) == w, (seed, sub, off)


def test_counter_layout_matches_library_engine(torch_philox):
    # words(seed, stream, request, position, n): counter = (n div 4, position, request, stream)
    seed, stream, req, pos = 99, 4, 513, 7
    w = px.words(seed, stream, req, pos, 12)
    sub = req | (stream << 32)
    want = torch_philox([(seed, sub, pos << 32 | i) for i in range(3)])
    assert [int(x) for x in w] == [v for quad in want for v in quad]


def test_uniform_map_is_open_interval_and_fp32_exact():
    w = np.array([0, 511, 512, 2 ** 32 - 1, 2 ** 31, 2 ** 31 + 512], dtype=np.uint32)
    u = px.to_uniform(w)
    assert u.min() > 0.0 and u.max() < 1.0
    assert u[0] == 2.0 ** -24 and u[1] == u[0] and u[3] == 1.0 - 2.0 ** -24
    assert u[4] == 0.5 + 2.0 ** -24 and u[5] == 0.5 + 3 * 2.0 ** -24
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_uniforms_are_uniform_and_independent():
    u = np.concatenate([px.uniforms(5, s, b, 3, 4096) for s in range(4) for b in range(64)])
    counts, _ = np.histogram(u, bins=256, range=(0.0, 1.0))
    assert stats.chisquare(counts).pvalue > 1e-4
    assert abs(np.corrcoef(u[:-1], u[1:])[0, 1]) < 5.0 / np.sqrt(u.size)
    a = px.uniforms(5, 0, 0, 3, 100000)
    b = px.uniforms(5, 1, 0, 3, 100000)
    assert abs(np.corrcoef(a, b)[0, 1]) < 5.0 / np.sqrt(a.size)
    # different seeds, positions and requests give different streams
    assert not np.array_equal(px.words(1, 0, 0, 0, 8), px.words(2, 0, 0, 0, 8))
    assert not np.array_equal(px.words(1, 0, 0, 0, 8), px.words(1, 0, 0, 1, 8))
    assert not np.array_equal(px.words(1, 0, 0, 0, 8), px.words(1, 0, 1, 0, 8))


def test_gumbel_distribution():
    g = px.gumbel(px.uniforms(11, 2, 0, 0, 200000))
    assert stats.kstest(g, stats.gumbel_r.cdf).pvalue > 1e-4
    assert abs(g.mean() - np.euler_gamma) < 0.02
