"""The counter summaries behind the bench line's `roofline.traffic` (CPU):
rocprofv3 counter CSVs are parsed, scaled by the copy calibration, written as
a summary whose machine-readable line the benchmark reads back, and the
figure is reported only while the kernel sources still hash to the recorded
value.  Synthetic CSVs with known values stand in for the profiler's output."""

import csv
import os
import re

import pytest

import bench
from lossless_rejection_sampling_amd import counters

GEMM = "void dspark::(anonymous namespace)::gemm_draft_stream<256>(dspark::GemmArgs)"
DRAW = "void dspark::(anonymous namespace)::draft_select_fast<unsigned short, unsigned short>(dspark::DraftSelectArgs)"
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def _write(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, counter, value, ns) in enumerate(rows):
            w.writerow(dict(Dispatch_Id=i, Kernel_Name=kernel, Counter_Name=counter, Counter_Value=value,
                            Start_Timestamp=1000 * i, End_Timestamp=1000 * i + ns))
    return str(path)


@pytest.fixture
def runs(tmp_path):
    copy_kib = counters.COPY_BYTES / 1024
    # the copy reads half of its bytes in FETCH_SIZE units and all of them in WRITE_SIZE units;
    # a small copy (below a quarter of the size) is left out of the calibration
    copy_fetch = _write(tmp_path / "cf.csv", [(counters.COPY_KERNEL, "FETCH_SIZE", copy_kib / 2, 50000)] * 5
                        + [(counters.COPY_KERNEL, "FETCH_SIZE", 10.0, 100)])
    copy_write = _write(tmp_path / "cw.csv", [(counters.COPY_KERNEL, "WRITE_SIZE", copy_kib, 50000)] * 5)
    bench_fetch = _write(tmp_path / "bf.csv", [(GEMM, "FETCH_SIZE", 70000.0, 40000), (GEMM, "FETCH_SIZE", 80000.0, 42000),
                                               (DRAW, "FETCH_SIZE", 6000.0, 10000)])
    bench_write = _write(tmp_path / "bw.csv", [(GEMM, "WRITE_SIZE", 5000.0, 41000), (GEMM, "WRITE_SIZE", 7000.0, 41000),
                                               (DRAW, "WRITE_SIZE", 100.0, 10000)])
    return bench_fetch, bench_write, copy_fetch, copy_write


def test_summarize_and_calibration(runs):
    bench_fetch, _, copy_fetch, copy_write = runs
    s = counters.summarize(bench_fetch, "gemm_draft_stream", "FETCH_SIZE")
    assert s["dispatches"] == 2 and s["mean_kib"] == 75000.0
    assert counters.calibration(copy_fetch, "FETCH_SIZE") == 2048.0   # bytes per counter unit
    assert counters.calibration(copy_write, "WRITE_SIZE") == 1024.0
    with pytest.raises(SystemExit):
        counters.summarize(bench_fetch, "no_such_kernel", "FETCH_SIZE")


def test_calibration_needs_every_copy(tmp_path):
    few = _write(tmp_path / "few.csv", [(counters.COPY_KERNEL, "FETCH_SIZE", counters.COPY_BYTES / 2048, 1)] * 3)
    with pytest.raises(SystemExit):
        counters.calibration(few, "FETCH_SIZE")


def test_report_line_round_trip(runs, tmp_path):
    md = counters.report(*runs, "gemm_draft_stream", "draft_gemm")
    want = 75000.0 * 2048 + 6000.0 * 1024   # mean FETCH x its scale + mean WRITE x its scale
    path = tmp_path / "summary.md"
    path.write_text(md)
    rec = counters.read_summary(str(path))
    assert rec == dict(kernel="draft_gemm", bytes=round(want), source=counters.source_hash())
    assert f"{want / 1e6:.2f}" in md


def test_kernel_table(runs):
    table = counters.kernel_table(*runs)
    rows = {m.group(1): m for m in re.finditer(r"\| `([^`]+)` \| (\d+) \| ([\d.]+) \| ([\d.]+) \| ([\d.]+) \|", table)}
    g = rows["gemm_draft_stream<256>"]
    assert g.group(2) == "2"
    assert float(g.group(3)) == pytest.approx(75000 * 2048 / 1e6, abs=0.01)
    assert float(g.group(4)) == pytest.approx(6000 * 1024 / 1e6, abs=0.01)
    assert "draft_select_fast<unsigned short, unsigned short>" in rows
    # largest traffic first
    assert table.index("gemm_draft_stream") < table.index("draft_select_fast")


def test_source_hash_gates_the_bench_figure(runs, tmp_path, monkeypatch):
    h = counters.source_hash()
    assert re.fullmatch(r"[0-9a-f]{16}", h) and h == counters.source_hash()
    path = tmp_path / "traffic.md"
    path.write_text(counters.report(*runs, "gemm_draft_stream", "draft_gemm"))
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(path))
    assert bench.measured_traffic("draft_gemm") == 75000.0 * 2048 + 6000.0 * 1024
    assert bench.measured_traffic("verify") is None            # another kernel's summary
    path.write_text(path.read_text().replace(f"source={h}", "source=0123456789abcdef"))
    assert bench.measured_traffic("draft_gemm") is None        # the sources changed since
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("draft_gemm") is None


def test_committed_summary_is_readable():
    rec = counters.read_summary(os.path.join(os.path.dirname(bench.__file__), "profiles", "draft_gemm_B256_traffic.md"))
    assert rec is not None and rec["kernel"] == "draft_gemm" and rec["bytes"] > 0


def test_algorithmic_bytes_of_the_headline_round():
    # the per-launch algorithmic work of the bench line, hand-computed for the
    # DSpark-5 round at B = 256, gamma = 5, V = 151936, r = 256 in bf16
    import torch
    from types import SimpleNamespace

    bf = torch.empty(0, dtype=torch.bfloat16)
    rnd = SimpleNamespace(B=256, gamma=5, V=151936, r=256, base=bf, U=bf)
    a = bench.algorithmic(rnd, budgets=None, emitted=[583], rejected=196)
    # draft step: backbone rows 256 x 151936 x 2 B = 77 791 232, W2 once per
    # round 151936 x 256 x 2 B / 5 = 15 558 246.4, U rows 256 x 256 x 2 B = 131 072
    assert a["draft_gemm"]["bytes"] == pytest.approx(93_480_550.4, abs=1e-3)
    assert a["draft_gemm"]["flops"] == 19_914_555_392.0          # 2 B r V
    assert a["draft_gemm"]["overhead_bytes"] == 256 * 2374 * 8   # 8-byte tile records
    # verification: the 583 target rows up to the first rejection
    assert a["row_stats"]["bytes"] == 583 * 151936 * 2 == 177_157_376
    # residual: one target and one backbone row for each of 196 rejected requests, W2 once
    assert a["residual_gemm"]["bytes"] == 196 * 2 * 151936 * 2 + 151936 * 256 * 2 == 196_909_056
    # resident round: five steps' rows and W2 once
    assert a["draft_round"]["bytes"] == 5 * (77_791_232 + 131_072) + 77_791_232
    # fp32 logits keep a 16-byte record (shift, max, exp-sum)
    f32 = torch.empty(0, dtype=torch.float32)
    a32 = bench.algorithmic(SimpleNamespace(B=256, gamma=5, V=151936, r=256, base=f32, U=bf), None, [583], 196)
    assert a32["draft_gemm"]["overhead_bytes"] == 256 * 2374 * 16
