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

Prints one JSON line.  With --gpus N > 1 it exits: this build runs on one GPU.
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


def algorithmic(rnd, budgets, emitted):
    """Bytes and flops each kernel class must move / perform per launch (what
    the method needs, not what the kernels happen to do).  Verification needs
    the target rows up to the first rejection only: rows 0..n_b of request b,
    sum_b (n_b + 1) = sum of the emitted counts."""
    B, g, V, r = rnd.B, rnd.gamma, rnd.V, rnd.r
    es = rnd.base.element_size()
    fs = rnd.U.element_size()
    n_tiles = -(-V // 64)
    rows = int(sum(int(e) for e in emitted))
    return {
        # one draft step: backbone row of every request, W2 once, U rows gathered,
        # tile statistics written
        "draft_gemm": dict(bytes=B * V * es + V * r * fs + B * r * fs + B * n_tiles * 16,
                           flops=2.0 * B * r * V, per="draft step"),
        # target rows 0..n_b of every request read once (statistics, tests, final tokens)
        "row_stats": dict(bytes=rows * V * es, flops=0.0, per="verify"),
    }


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU layout is "
              "a design note, not part of this build", file=sys.stderr)
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
    round_ms = round_distribution(step, args.steps)

    budgets = bufs[0].budget.cpu().numpy()
    verified = int(budgets.sum())
    emitted = int(bufs[0].num_emitted.sum().item())
    sec_per_step = (t1 - t0) / args.steps
    value = verified / sec_per_step

    alg = algorithmic(base_round, budgets, bufs[0].num_emitted.cpu().numpy())
    kernels = {}
    for name, st in per_class.items():
        if st["launches"]:
            kernels[name] = dict(avg_us=1e3 * st["ms"] / st["launches"], launches_per_round=st["launches"] / (N_SETS * 2))
    for name, a in alg.items():
        if name in kernels:
            us = kernels[name]["avg_us"]
            kernels[name]["GB_s"] = a["bytes"] / (us * 1e-6) / 1e9
            if a["flops"]:
                kernels[name]["TFLOP_s"] = a["flops"] / (us * 1e-6) / 1e12

    dom_avg_s = dom_ms / max(dom_n, 1) / 1e3
    if dominant in alg and alg[dominant]["flops"] and dominant == "draft_gemm":
        a = alg[dominant]
        ach_bw = a["bytes"] / dom_avg_s / 1e9
        ach_fl = a["flops"] / dom_avg_s / 1e12
        # bound set by the arithmetic intensity of this launch against the ridge
        if a["flops"] / a["bytes"] > MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9):
            roof = dict(bound="mfma", achieved=ach_fl, peak=MFMA_BF16_PEAK_TFLOPS, unit="TFLOP/s")
        else:
            roof = dict(bound="hbm", achieved=ach_bw, peak=HBM_PEAK_GBS, unit="GB/s")
    else:
        a = alg.get(dominant, dict(bytes=0.0))
        roof = dict(bound="hbm", achieved=a["bytes"] / dom_avg_s / 1e9, peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(dominant)
    roof["kernel"] = dominant
    roof["avg_us"] = dom_avg_s * 1e6
    roof["timed_launches"] = dom_n
    # the same achieved rate against what this device reaches in plain kernels
    peaks = measure_peaks()
    roof["measured_peak"] = peaks
    roof["frac_of_measured"] = roof["achieved"] / (peaks["stream_read_GB_s"] if roof["unit"] == "GB/s"
                                                   else peaks["mfma_bf16_TFLOP_s"])

    extras = measure_extras(rounds[0], bufs[0])

    cpu = None
    if not args.no_cpu_baseline:
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
                   "emitted_tokens_per_s": emitted / sec_per_step},
        "round_ms": round_ms,
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


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


def cpu_baseline(rnd, budgets, seconds):
    """The oracle, as it stands, on a bounded sample of the same round: whole
    requests (draft of every position, verify with the GPU-granted budgets)
    until about ``seconds`` of CPU time; the scheduler runs over the full batch
    once.  Reported as verified draft tokens per second."""
    import numpy as np
    import torch

    from lossless_rejection_sampling_amd import workloads as wl
    from oracle import dspark as od

    try:
        from threadpoolctl import threadpool_info
        threads = max([t.get("num_threads", 1) for t in threadpool_info()] or [1])
    except Exception:
        threads = 1
    h = wl.to_host
    U, W = h(rnd.U), h(rnd.W)
    conf = h(rnd.conf)
    t_start = time.perf_counter()
    sched = od.schedule(conf, rnd.sps_B, rnd.sps_val)
    t_sched = time.perf_counter() - t_start
    done, verified, t_work = 0, 0, 0.0
    while t_work < seconds and done < rnd.B:
        idx = [done]
        t = torch.as_tensor(idx, device=rnd.base.device)
        base, target = h(rnd.base.index_select(0, t)), h(rnd.target.index_select(0, t))
        prev0, T = h(rnd.prev0.index_select(0, t)), h(rnd.temperature.index_select(0, t))
        c0 = time.perf_counter()
        dr = od.draft_round(base, U, W, prev0, T, rnd.seed, req_ids=idx)
        od.verify(target, base, U, W, prev0, dr.tokens, T, rnd.seed, sched.budget[idx], req_ids=idx)
        t_work += time.perf_counter() - c0
        verified += int(sched.budget[done])
        done += 1
    per_req = t_work / done
    round_s = per_req * rnd.B + t_sched
    # the same at one thread, on the first requests of the sample
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            n1, t1 = 0, 0.0
            while t1 < seconds / 4 and n1 < done:
                idx = [n1]
                t = torch.as_tensor(idx, device=rnd.base.device)
                base, target = h(rnd.base.index_select(0, t)), h(rnd.target.index_select(0, t))
                prev0, T = h(rnd.prev0.index_select(0, t)), h(rnd.temperature.index_select(0, t))
                c0 = time.perf_counter()
                dr = od.draft_round(base, U, W, prev0, T, rnd.seed, req_ids=idx)
                od.verify(target, base, U, W, prev0, dr.tokens, T, rnd.seed, sched.budget[idx], req_ids=idx)
                t1 += time.perf_counter() - c0
                n1 += 1
            single = {"value": float(np.sum(budgets)) / (t1 / n1 * rnd.B + t_sched), "cores": 1,
                      "sample": f"{n1} requests ({t1:.1f} s), same extrapolation"}
    except Exception:
        single = None
    return {
        "value": float(np.sum(budgets)) / round_s,
        "unit": "verified draft tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {rnd.B} requests timed whole (draft + verify, {t_work:.1f} s) plus the "
                  f"scheduler over all {rnd.B} ({t_sched:.2f} s), extrapolated per request to the batch",
        "single_thread": single,
    }


if __name__ == "__main__":
    main()
