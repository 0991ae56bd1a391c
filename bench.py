"""Benchmark of one DSpark draft-and-verify round on one MI355X.

A step is one whole round over the batch: dspark_draft_round (Markov-bias GEMM
+ softmax statistics and a draw per block position), dspark_schedule (verify
budgets from the confidence scores) and dspark_verify (target row statistics,
accept tests, residual or bonus draw), in that order on one stream.  Workload: B = 256 requests, gamma = 5,
V = 151936, Markov rank r = 256, bf16 logits and factors (the DSpark-5 generator
at B = 256), confidence scores sigmoid(N(1.5 - 0.4 j, 1)) and the synthetic
16-point step-rate table; inputs are seeded synthetic tensors resident in HBM.

Metric: verified draft tokens per second = sum_b L_b (the budgets the scheduler
grants) per round / seconds per round.  Three copies of the inputs are used in
rotation so that no round finds the previous round's data in the 256 MB
Infinity Cache.

Prints one JSON line.  With --gpus N > 1 it exits: the library runs on one GPU.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16
N_SETS = 3


TIMING_PERIOD = 7
ROUND_REPS = 60


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--minimal", action="store_true",
                   help="the timed rounds only (no reference rates, extras, per-round distribution or CPU "
                        "baseline): for profiler runs")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain device copy of known size (counter calibration) and exit")
    return p.parse_args()


def calibrate_copy():
    """A plain device-to-device copy of counters.COPY_BYTES, COPY_REPS times:
    the reference that scales the FETCH_SIZE / WRITE_SIZE counters to bytes."""
    import torch

    from lossless_rejection_sampling_amd import counters

    n = counters.COPY_BYTES // 4
    src = torch.arange(n, device="cuda", dtype=torch.int32)
    dst = torch.empty_like(src)
    for _ in range(counters.COPY_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    print(json.dumps({"calibration_copy_bytes": counters.COPY_BYTES, "reps": counters.COPY_REPS}))


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "draft_gemm_B256_traffic.md")


def measured_traffic(kernel_name):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None when there is none or the kernel source has changed since."""
    from lossless_rejection_sampling_amd import counters

    rec = counters.read_summary(TRAFFIC_SUMMARY)
    if rec is None or rec["kernel"] != kernel_name or rec["source"] != counters.source_hash():
        return None
    return rec["bytes"]


def algorithmic(rnd, budgets, emitted, rejected):
    """Bytes and flops each kernel class must move / perform per launch (what
    the method needs, not what the kernels happen to do), counted as the
    measurement plan of the hot path counts them:
      draft step   the backbone row of every request (B V), W2 once per round
                   (V r / gamma per step: the factor is the same at every block
                   position), the U rows of the previous tokens (B r); the
                   kernel's own tile records are overhead, reported apart;
      draft round  the resident kernel (every position in one launch): gamma
                   draft steps' rows and W2 once;
      verification target rows 0..n_b of request b (sum_b (n_b + 1) rows = the
                   emitted count: the rows up to the first rejection);
      residual     for every rejected request one target and one backbone row,
                   plus W2 once."""
    B, g, V, r = rnd.B, rnd.gamma, rnd.V, rnd.r
    es = rnd.base.element_size()
    fs = rnd.U.element_size()
    n_tiles = -(-V // 64)
    rec = 8 if es == 2 else 16  # bytes of a tile record: (max, exp-sum), plus the shift for fp32 logits
    rows = int(sum(int(e) for e in emitted))
    return {
        "draft_gemm": dict(bytes=B * V * es + V * r * fs / g + B * r * fs,
                           overhead_bytes=B * n_tiles * rec, flops=2.0 * B * r * V, per="draft step"),
        "draft_round": dict(bytes=g * (B * V * es + B * r * fs) + V * r * fs,
                            overhead_bytes=g * B * n_tiles * rec, flops=2.0 * B * r * V * g, per="draft round"),
        "row_stats": dict(bytes=rows * V * es, flops=0.0, per="verify"),
        "residual_gemm": dict(bytes=rejected * 2 * V * es + V * r * fs, flops=2.0 * rejected * r * V,
                              per="verify"),
    }


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from lossless_rejection_sampling_amd import dspark as ds
    from lossless_rejection_sampling_amd import round as rd
    from lossless_rejection_sampling_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    ds.lib()
    dev = "cuda"
    base_round = wl.headline(device=dev)
    rounds, bufs = [], []
    for i in range(N_SETS):
        r_i = base_round if i == 0 else wl.Round(
            base_round.name, base_round.target.clone(), base_round.base.clone(), base_round.U.clone(),
            base_round.Wt.clone(), base_round.prev0.clone(), base_round.temperature.clone(),
            base_round.seed, None, base_round.conf.clone(), base_round.sps_B, base_round.sps_val)
        rounds.append(r_i)
        bufs.append(rd.allocate(r_i))
    torch.cuda.synchronize()

    def step(i):
        rd.run_round(rounds[i % N_SETS], bufs[i % N_SETS])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    assert ds.dspark_status(bufs[0].workspace) == ds.DSPARK_OK

    # per-kernel classes, untimed pass: which kernel dominates the round
    for c in ds.KERNEL_CLASSES.values():
        ds.dspark_profile_enable(c, True)
    for i in range(N_SETS * 2):
        step(i)
    torch.cuda.synchronize()
    per_class = {}
    for name, c in ds.KERNEL_CLASSES.items():
        n, ms = ds.dspark_profile_read(c)
        ds.dspark_profile_enable(c, False)
        per_class[name] = dict(launches=n, ms=ms)
    dominant = max(per_class, key=lambda k: per_class[k]["ms"])

    # timed region: K whole rounds; HIP events carried in the dispatch time every
    # 7th launch of the dominant kernel (7 is prime to the 5 draft steps of a
    # round, so the sample covers every position; timing every launch would add
    # ~20 us of dispatch time per round to the timed region)
    ds.dspark_profile_enable(ds.KERNEL_CLASSES[dominant], TIMING_PERIOD)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    dom_n, dom_ms = ds.dspark_profile_read(ds.KERNEL_CLASSES[dominant])
    ds.dspark_profile_enable(ds.KERNEL_CLASSES[dominant], False)
    assert ds.dspark_status(bufs[0].workspace) == ds.DSPARK_OK

    # per-round distribution, after the timed region: ROUND_REPS rounds, each
    # between HIP events on the stream the rounds run on
    round_ms = None if args.minimal else round_distribution(step, args.steps)

    budgets = bufs[0].budget.cpu().numpy()
    verified = int(budgets.sum())
    n_acc = bufs[0].num_accepted.cpu().numpy()
    emitted = int(bufs[0].num_emitted.sum().item())
    rejected = int((n_acc < budgets).sum())
    sec_per_step = (t1 - t0) / args.steps
    value = verified / sec_per_step

    alg = algorithmic(base_round, budgets, bufs[0].num_emitted.cpu().numpy(), rejected)
    kernels = {}
    for name, st in per_class.items():
        if st["launches"]:
            kernels[name] = dict(avg_us=1e3 * st["ms"] / st["launches"], launches_per_round=st["launches"] / (N_SETS * 2))
    for name, a in alg.items():
        if name in kernels:
            us = kernels[name]["avg_us"]
            kernels[name]["algorithmic_bytes"] = a["bytes"]
            kernels[name]["GB_s"] = a["bytes"] / (us * 1e-6) / 1e9
            kernels[name]["frac_hbm"] = kernels[name]["GB_s"] / HBM_PEAK_GBS
            if a["flops"]:
                kernels[name]["TFLOP_s"] = a["flops"] / (us * 1e-6) / 1e12
                kernels[name]["frac_mfma_bf16"] = kernels[name]["TFLOP_s"] / MFMA_BF16_PEAK_TFLOPS

    dom_avg_s = dom_ms / max(dom_n, 1) / 1e3
    a = alg.get(dominant, dict(bytes=0.0, flops=0.0))
    ach_bw = a["bytes"] / dom_avg_s / 1e9
    ach_fl = a["flops"] / dom_avg_s / 1e12
    # bound set by the launch's arithmetic intensity against the ridge of the peaks
    if a["flops"] and a["flops"] / a["bytes"] > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
        roof = dict(bound="mfma", achieved=ach_fl, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s")
    else:
        roof = dict(bound="hbm", achieved=ach_bw, peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    traffic = measured_traffic(dominant)
    roof["traffic"] = traffic
    roof["algorithmic_bytes"] = a["bytes"]
    roof["traffic_over_algorithmic"] = traffic / a["bytes"] if traffic else None
    roof["kernel"] = dominant
    roof["avg_us"] = dom_avg_s * 1e6
    roof["timed_launches"] = dom_n
    if a["flops"]:
        roof["mfma"] = dict(achieved=ach_fl, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s",
                            frac=ach_fl / MFMA_BF16_PEAK_TFLOPS, flops=a["flops"])
    if "overhead_bytes" in a:
        roof["overhead_bytes"] = a["overhead_bytes"]
    # the same achieved rate against what this device reaches in plain kernels
    if not args.minimal:
        peaks = measure_peaks()
        roof["measured_peak"] = peaks
        roof["frac_of_measured"] = roof["achieved"] / (peaks["stream_read_GB_s"] if roof["unit"] == "GB/s"
                                                       else peaks["mfma_bf16_TFLOP_s"])

    extras = None
    if not args.minimal:
        extras = measure_extras(rounds[0], bufs[0])
        extras["full_budget"] = full_budget_round(rounds, args.steps)
        extras["resident_draft"] = resident_draft_round(rounds, bufs, args.steps)

    cpu = None
    if not args.no_cpu_baseline and not args.minimal:
        cpu = cpu_baseline(base_round, budgets, args.cpu_seconds)

    line = {
        "metric": "verified draft tokens/sec + HBM GB/s vs peak, B=256 gamma=5 V=151,936",
        "value": value,
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "DSpark-5 round, B=256 gamma=5 V=151936 r=256, bf16 logits and factors, "
                               "T=1, confidence-scheduled budgets",
                   "B": base_round.B, "gamma": base_round.gamma, "V": base_round.V, "r": base_round.r,
                   "verified_per_round": verified, "emitted_per_round": emitted,
                   "rejected_per_round": rejected,
                   "emitted_tokens_per_s": emitted / sec_per_step},
        "round_ms": round_ms,
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


def resident_draft_round(rounds, bufs, steps):
    """The same headline rounds with the draft round as one resident launch (W2
    held on chip across the positions; dspark_set_draft_path): ms per round and
    the resident kernel's time (events recorded around its cooperative launch,
    so they include its dispatch), beside the per-position default."""
    import torch

    from lossless_rejection_sampling_amd import dspark as ds
    from lossless_rejection_sampling_amd import round as rd

    prev = ds.dspark_set_draft_path(ds.DSPARK_DRAFT_RESIDENT)
    try:
        step = lambda i: rd.run_round(rounds[i % N_SETS], bufs[i % N_SETS])
        for i in range(3):
            step(i)
        torch.cuda.synchronize()
        cls = ds.KERNEL_CLASSES["draft_round"]
        ds.dspark_profile_enable(cls, True)
        for i in range(N_SETS * 2):
            step(i)
        torch.cuda.synchronize()
        n, kms = ds.dspark_profile_read(cls)
        ds.dspark_profile_enable(cls, False)
        t0 = time.perf_counter()
        for i in range(steps):
            step(i)
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / steps
        assert ds.dspark_status(bufs[0].workspace) == ds.DSPARK_OK
    finally:
        ds.dspark_set_draft_path(prev)
    return {"ms_per_step": sec * 1e3, "draft_round_us": 1e3 * kms / max(n, 1), "launches_timed": n}


def full_budget_round(rounds, steps):
    """The same inputs verified at the full budget L = gamma (no scheduler):
    verified tokens/s and per-kernel times, timed as the headline (three input
    sets in rotation, K rounds between synchronisations)."""
    import dataclasses

    import torch

    from lossless_rejection_sampling_amd import dspark as ds
    from lossless_rejection_sampling_amd import round as rd

    full = [dataclasses.replace(r, conf=None, budget=None) for r in rounds]
    bufs = [rd.allocate(r) for r in full]
    step = lambda i: rd.run_round(full[i % N_SETS], bufs[i % N_SETS])
    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    for c in ds.KERNEL_CLASSES.values():
        ds.dspark_profile_enable(c, True)
    for i in range(N_SETS * 2):
        step(i)
    torch.cuda.synchronize()
    per = {}
    for name, c in ds.KERNEL_CLASSES.items():
        n, ms = ds.dspark_profile_read(c)
        ds.dspark_profile_enable(c, False)
        if n:
            per[name] = dict(avg_us=1e3 * ms / n, launches_per_round=n / (N_SETS * 2))
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    assert ds.dspark_status(bufs[0].workspace) == ds.DSPARK_OK
    B, g = full[0].B, full[0].gamma
    n_acc = bufs[0].num_accepted.cpu().numpy()
    emitted = int(bufs[0].num_emitted.sum().item())
    alg = algorithmic(full[0], None, bufs[0].num_emitted.cpu().numpy(), int((n_acc < g).sum()))
    for name, a in alg.items():
        if name in per:
            us = per[name]["avg_us"]
            per[name]["GB_s"] = a["bytes"] / (us * 1e-6) / 1e9
            per[name]["frac_hbm"] = per[name]["GB_s"] / HBM_PEAK_GBS
    out = {"verified_per_round": B * g, "emitted_per_round": emitted, "ms_per_step": sec * 1e3,
           "verified_tokens_per_s": B * g / sec, "emitted_tokens_per_s": emitted / sec, "kernels": per}
    del bufs
    torch.cuda.empty_cache()
    return out


def round_distribution(step, start, reps=None):
    """Median, 10th and 90th percentile of single-round times (ms), each round
    between two HIP events recorded on the current stream."""
    import numpy as np
    import torch

    reps = reps or ROUND_REPS
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (e0, e1) in enumerate(evs):
        e0.record()
        step(start + i)
        e1.record()
    torch.cuda.synchronize()
    t = np.array([e0.elapsed_time(e1) for e0, e1 in evs])
    return dict(reps=reps, median=float(np.median(t)), p10=float(np.percentile(t, 10)),
                p90=float(np.percentile(t, 90)))


def measure_peaks(reps=3):
    """Reference rates of this device, timed with events around one kernel each:
    a streaming read of a 2 GiB buffer (8x the Infinity Cache) and a dense bf16
    MFMA loop.  Median of `reps`."""
    import torch
    from lossless_rejection_sampling_amd import dspark as ds
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    buf = torch.ones(2 << 30, dtype=torch.uint8, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e-3)
        return sorted(out)[len(out) // 2]

    t_read = timed(lambda: ds.dspark_peak_stream_read(buf, sink))
    del buf
    blocks, iters = 1024, 4096
    t_mfma = timed(lambda: ds.dspark_peak_mfma_bf16(blocks, iters, sink))
    flops = blocks * 4 * iters * 4 * 32768
    torch.cuda.empty_cache()
    return {"stream_read_GB_s": (2 << 30) / t_read / 1e9, "mfma_bf16_TFLOP_s": flops / t_mfma / 1e12,
            "how": "streaming read of 2 GiB (one contiguous 8 KB chunk per wavefront, 8 x 16-byte "
                   "non-temporal loads in flight per lane); "
                   "1024 WGs x 4 waves x 4096 rounds of 4 independent v_mfma_f32_32x32x16_bf16 chains"}


def measure_extras(rnd, buf, reps=5):
    """Outside the timed round: (1) the analytic-acceptance pass (c*_k of every
    drafted position) on the same inputs, its GEMM launch timed with HIP events
    and priced against HBM; (2) Theta = tau SPS(B) of the verify budgets each
    scheduler rule grants for the round's scores (budgets computed on the GPU);
    (3) Sequential Temperature Scaling on synthetic overconfident scores whose
    labels are the acceptance pass's c*: ECE before and after, temperatures
    fitted on half of the requests and scored on the other half."""
    import numpy as np
    import torch

    from lossless_rejection_sampling_amd import analysis, calibration
    from lossless_rejection_sampling_amd import dspark as ds

    B, g, V, r = rnd.B, rnd.gamma, rnd.V, rnd.r
    c = torch.empty((B, g), dtype=torch.float64, device="cuda")
    run = lambda: ds.dspark_acceptance(rnd.target, rnd.base, rnd.U, rnd.Wt, rnd.prev0, buf.draft_tokens,
                                       buf.draft_lse, rnd.temperature, c, buf.workspace)
    run()
    torch.cuda.synchronize()
    cls = ds.KERNEL_CLASSES["acceptance"]
    ds.dspark_profile_enable(cls, True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    n, ms = ds.dspark_profile_read(cls)
    ds.dspark_profile_enable(cls, False)
    es = rnd.base.element_size()
    n_tiles = -(-V // 64)
    # target rows 0..gamma-1 and backbone rows once, W2 once, tile masses written
    alg = 2 * B * g * V * es + V * r * rnd.U.element_size() + B * g * n_tiles * 4
    gemm_us = 1e3 * ms / max(n, 1)
    acc = {"call_us": 1e3 * e0.elapsed_time(e1) / reps, "gemm_us": gemm_us,
           "gemm_algorithmic_bytes": alg, "gemm_GB_s": alg / gemm_us / 1e3,
           "gemm_frac_hbm": alg / gemm_us / 1e3 / HBM_PEAK_GBS,
           "mean_c_star": float(c.mean().item())}

    conf = rnd.conf
    tB = torch.as_tensor(rnd.sps_B, dtype=torch.float64, device="cuda")
    tS = torch.as_tensor(rnd.sps_val, dtype=torch.float64, device="cuda")
    ws = torch.zeros(ds.dspark_schedule_workspace_bytes(B, g), dtype=torch.uint8, device="cuda")
    budget = torch.empty(B, dtype=torch.int32, device="cuda")
    sched = {}
    for name, rule, p in [("dspark_early_stop", "early_stop", 0), ("production_best_cut", "argmax", 0),
                          ("mtp1", "fixed", 1), ("mtp3", "fixed", 3), ("mtp5", "fixed", 5),
                          ("threshold_0.7", "threshold", 0.7)]:
        ds.dspark_schedule_ex(conf, None, tB, tS, rule, p, budget, ws)
        L = budget.cpu().numpy()
        tau, N, theta = analysis.expected_theta(conf.cpu().numpy(), L, rnd.sps_B, rnd.sps_val)
        sched[name] = {"verified_per_round": int(L.sum()), "expected_tokens": tau, "batch_tokens": N,
                       "theta_tokens_per_s": theta}

    cs = c.cpu().numpy()
    rng = np.random.default_rng(17)
    z = np.log(np.clip(cs, 1e-9, 1 - 1e-9)) - np.log1p(-np.clip(cs, 1e-9, 1 - 1e-9))
    raw = 1 / (1 + np.exp(-(2.5 * z + rng.normal(0, 0.3, size=z.shape))))
    half = B // 2
    tau_k = calibration.fit_sts(raw[:half], cs[:half])
    sts = {"temperatures": [float(t) for t in tau_k],
           "ece_before": calibration.sequential_ece(raw[half:], cs[half:]),
           "ece_after": calibration.sequential_ece(calibration.scale_scores(raw[half:], tau_k), cs[half:]),
           "scores": "sigmoid(2.5 logit(c*) + N(0, 0.3^2)), c* from the acceptance pass"}
    return {"acceptance_pass": acc, "schedulers": sched, "sequential_temperature_scaling": sts}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(rnd, budgets, seconds, threads=None):
    """The C oracle (plain fp64 loops, OpenMP over requests), as it stands, on a
    bounded sample of the same round: chunks of whole requests (draft of every
    position, then verification with the GPU-granted budgets), one request per
    thread, until about ``seconds`` of wall time; the scheduler runs over the
    full batch once.  Reported as verified draft tokens per second,
    extrapolated per request to the batch; the same at one thread beside it."""
    import numpy as np

    from lossless_rejection_sampling_amd import workloads as wl
    from oracle import ref

    if not os.path.exists(ref.LIB):
        from oracle import build as ob
        ob.build()
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = threads or max(1, min(16, avail))
    h = wl.to_host
    U, W = np.ascontiguousarray(h(rnd.U), np.float32), np.ascontiguousarray(h(rnd.W), np.float32)
    base, target = h(rnd.base), h(rnd.target)
    prev0, T = h(rnd.prev0), h(rnd.temperature)
    budgets = np.asarray(budgets, dtype=np.int32)
    before = ref.threads()
    t0 = time.perf_counter()
    if rnd.scheduled:
        ref.schedule(h(rnd.conf), rnd.sps_B, rnd.sps_val)
    t_sched = time.perf_counter() - t0

    def run(n_threads, budget_s):
        ref.threads(n_threads)
        done, t0 = 0, time.perf_counter()
        while done < rnd.B and (done == 0 or time.perf_counter() - t0 < budget_s):
            idx = np.arange(done, min(rnd.B, done + n_threads), dtype=np.int32)
            sl = slice(int(idx[0]), int(idx[-1]) + 1)
            dr = ref.draft_round(base[sl], U, W, prev0[sl], T[sl], rnd.seed, req_ids=idx)
            ref.verify(target[sl], base[sl], U, W, prev0[sl], dr.tokens, T[sl], rnd.seed, budgets[sl], req_ids=idx)
            done += len(idx)
        return done, time.perf_counter() - t0

    try:
        done, wall = run(threads, seconds)
        d1, w1 = run(1, seconds / 4)
    finally:
        ref.threads(before)
    verified = float(np.sum(budgets))
    round_s = wall / done * rnd.B + t_sched
    single = {"value": verified / (w1 / d1 * rnd.B + t_sched), "cores": 1,
              "sample": f"{d1} requests ({w1:.1f} s) on one thread, same extrapolation"}
    return {
        "value": verified / round_s,
        "unit": "verified draft tokens/s",
        "cores": threads,
        "kind": "oracle",
        "implementation": "C oracle (oracle/dspark_ref.c), fp64, OpenMP over requests",
        "cpu_model": _cpu_model(),
        "host_cpus_visible": os.cpu_count(),
        "sample": f"{done} of {rnd.B} requests timed whole (draft + verify) in chunks of {threads}, one request "
                  f"per thread, in {wall:.1f} s, plus the scheduler over all {rnd.B} ({t_sched:.2f} s), "
                  f"extrapolated per request to the batch",
        "single_thread": single,
    }


if __name__ == "__main__":
    main()
