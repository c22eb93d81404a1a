#!/usr/bin/env python3
"""Benchmark: HSTU jagged masked attention, forward + backward, on one MI355X.

Workload (the production HSTU layer shape): B = 1024 sequences of 2663 rows
(2,726,912 tokens), H = 4 heads, D = 128, bf16, causal func encoded with
nfunc = 5 (two pad intervals), alpha = 1/sqrt(128), max_len = 2663.  Inputs
are synthetic N(0, 1) drawn on the device with torch's seeded generator and
are resident in HBM before timing starts.  One step = hstu_attn_fwd followed by
hstu_attn_bwd over the whole batch.

Reported ("value"): effective TFLOP/s = 14 * D * H * sum_i |V_i| / step time,
counting 4*D (forward) + 10*D (backward) flops per visible (query, key) pair and
head, over unmasked pairs only.  Also reported: per-step median and minimum
over 3 further runs and the spread of their medians (step_stats), the
targets-only mode (one candidate row per sequence against full-length K/V),
the backward alone with each dQ path (stored P, recompute, fp32 atomics:
dq_variants),
per-kernel times measured with HIP events on the launch stream during the
timed steps, the roofline of the dominant kernel, the other workloads at their
full sizes (per_workload: SLA 1k / 2k, three-interval, OneRank, ragged, L=4086,
each with its effective TFLOP/s and its fractions of the MFMA and HBM peaks),
and the fp64 CPU oracle: its rate on a sample of the headline workload
(cpu_baseline) and, under cpu_baseline.runs, timed in full on the small
workloads and on samples of the others, with the host it ran on.

Usage: python bench.py [--steps K] [--warmup W] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "HSTU attn fwd+bwd ms + effective TFLOP/s (% bf16 MFMA peak), B=1024 L=2663"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# algorithmic flops per visible pair and head, as multiples of D
KERNEL_FLOPS_PER_PAIR = {"k_fwd_bf16": 4, "k_bwd_kv": 8, "k_bwd_kv_p": 8, "k_bwd_q": 2,
                         "k_bwd_dq": 2}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def measured_traffic(kernel: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE / WRITE_SIZE scaled by a copy-kernel calibration), if it was
    taken on the current source of that kernel; else None."""
    from hstu_jagged_masked_amd import profiling

    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(kernel)
    if not rec or rec.get("source_sha256") != profiling.source_digest(kernel):
        return None
    return round(rec["bytes_per_launch"])


def make_inputs(cfg, device, targets=False):
    import torch

    lengths = cfg["lengths"]
    off = wl.offsets_from_lengths(lengths)
    T = int(off[-1])
    B, H, D = len(lengths), cfg["H"], cfg["D"]
    seed = cfg["seed"]
    rows_q = B if targets else T
    dt = torch.bfloat16
    t = {
        "off": torch.from_numpy(off).to(device),
        "func": torch.from_numpy(cfg["func"](lengths, cfg["nfunc"])).to(device),
        "k": wl.normal_device((T, H, D), seed * 10 + 1, dt, device),
        "v": wl.normal_device((T, H, D), seed * 10 + 2, dt, device),
        "q": wl.normal_device((rows_q, H, D), seed * 10 + (5 if targets else 0), dt, device),
        "do": wl.normal_device((rows_q, H, D), seed * 10 + (6 if targets else 3), dt, device),
    }
    if targets:
        t["tr"] = torch.from_numpy(wl.targets_last(lengths)).to(device)
    return t, off


def run_steps(hj, t, cfg, n, targets=False, pstore=None, host_offsets=None):
    tr = t.get("tr") if targets else None
    for _ in range(n):
        hj.attn_fwd(t["q"], t["k"], t["v"], t["off"], t["func"], cfg["alpha"], cfg["max_len"], tr)
        hj.attn_bwd(t["q"], t["k"], t["v"], t["do"], t["off"], t["func"], cfg["alpha"],
                    cfg["max_len"], tr, pstore=pstore, host_offsets=host_offsets)


def pstore_runs(lengths, H, budget):
    """Runs the bounded stored-P backward cuts a batch into (consecutive
    sequences, each run as long as the buffer holds its stored P)."""
    runs, need = 1, 0
    for L in lengths:
        one = -(-int(L) // 128) * -(-int(L) // 32) * 8192 * H
        if need + one > budget:
            runs, need = runs + 1, 0
        need += one
    return runs


def timed(hj, torch, t, cfg, steps, targets=False, pstore=None, host_offsets=None):
    """ms per step over `steps` steps (a HIP event pair around them, nothing
    else recorded), then the same steps again with the library's per-kernel
    event pairs on, for the per-kernel times (those events add small gaps
    between kernels, so the step time is not taken from that pass)."""
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    run_steps(hj, t, cfg, steps, targets, pstore, host_offsets)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    hj.profile_reset()
    hj.profile_enable(True)
    run_steps(hj, t, cfg, steps, targets, pstore, host_offsets)
    torch.cuda.synchronize()
    hj.profile_enable(False)
    prof = hj.profile_read()
    return e0.elapsed_time(e1) / steps, wall, prof


def split_ms(hj, torch, t, cfg, steps, pstore):
    """Forward alone and backward alone, `steps` calls each (after the timed
    region; HIP events on the current stream)."""
    out = {}
    for name in ("fwd", "bwd"):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(steps):
            if name == "fwd":
                hj.attn_fwd(t["q"], t["k"], t["v"], t["off"], t["func"], cfg["alpha"],
                            cfg["max_len"])
            else:
                hj.attn_bwd(t["q"], t["k"], t["v"], t["do"], t["off"], t["func"], cfg["alpha"],
                            cfg["max_len"], pstore=pstore)
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(e0.elapsed_time(e1) / steps, 4)
    return out


def dq_variants(hj, torch, t, cfg, steps, stored_p_bwd_ms):
    """The backward alone with each dQ path on the same inputs: stored P (its
    time from split_ms), recompute (a query-owner pass that recomputes the
    scores) and atomic (fp32 atomics from the key-owner pass; dq not bitwise
    repeatable).  ms per backward and per-kernel ms."""
    acc = torch.empty(t["k"].shape, dtype=torch.float32, device=t["k"].device)
    a = (t["q"], t["k"], t["v"], t["do"], t["off"], t["func"], cfg["alpha"], cfg["max_len"])
    calls = {"recompute": lambda: hj.attn_bwd(*a),
             "atomic": lambda: hj.attn_bwd_atomic(*a, dq_accum=acc)}
    out = {"stored_p": {"bwd_ms": stored_p_bwd_ms}}
    for name, fn in calls.items():
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        hj.profile_reset()
        hj.profile_enable(True)
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        hj.profile_enable(False)
        prof = hj.profile_read()
        out[name] = {"bwd_ms": round(e0.elapsed_time(e1) / steps, 4),
                     "kernels_ms": {k: round(v[1] / steps, 4) for k, v in sorted(prof.items())}}
    del acc
    torch.cuda.empty_cache()
    return out


def step_stats(hj, torch, t, cfg, steps, runs, pstore):
    """Per-step fwd+bwd times (a HIP event pair around each step), `runs`
    runs of `steps` steps after the timed region: median and min of each run
    and the spread of the run medians."""
    per_run = []
    for _ in range(runs):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(steps):
            run_steps(hj, t, cfg, 1, pstore=pstore)
            ev[i + 1].record()
        torch.cuda.synchronize()
        per_run.append([ev[i].elapsed_time(ev[i + 1]) for i in range(steps)])
    med = [float(np.median(r)) for r in per_run]
    return {"runs": runs, "steps_per_run": steps,
            "median_ms": [round(m, 4) for m in med],
            "min_ms": [round(min(r), 4) for r in per_run],
            "spread_pct": round(100.0 * (max(med) - min(med)) / min(med), 2)}


# workloads measured beside the headline one (each at its own full size, same
# entry points and backward path as the headline run)
EXTRA_WORKLOADS = ("sla_1k", "sla_2k", "three_interval", "onerank", "hstu_ragged", "hstu_4086")


def tensor_bytes(T, H, D):
    """Algorithmic HBM bytes of one fwd+bwd: the forward reads q, k, v and
    writes o; the backward reads q, k, v, dO and writes dq, dk, dv (bf16)."""
    return 11.0 * T * H * D * 2


def measure_workload(hj, torch, name, device, steps, dq_path):
    """fwd+bwd of one named workload at full size: ms per step (HIP events),
    fwd / bwd split, effective TFLOP/s (14 D per visible pair), fraction of
    the bf16 MFMA peak and of HBM bandwidth (algorithmic bytes), per-kernel
    times."""
    cfg = wl.workload(name)
    H, D = cfg["H"], cfg["D"]
    t, off = make_inputs(cfg, device)
    T = int(off[-1])
    _, pairs_t = hj.visible_counts(t["off"], t["func"], T)
    pairs = int(pairs_t.item())
    pstore = None
    if dq_path == "stored_p":
        pstore = torch.empty(hj.pstore_bytes(t["off"], H), dtype=torch.uint8, device=device)
    run_steps(hj, t, cfg, 2, pstore=pstore)
    ms, _, prof = timed(hj, torch, t, cfg, steps, pstore=pstore)
    split = split_ms(hj, torch, t, cfg, steps, pstore)
    flops = 14.0 * D * H * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = tensor_bytes(T, H, D) / (ms * 1e-3) / 1e9
    out = {"batch": len(cfg["lengths"]), "tokens": T, "heads": H, "head_dim": D,
           "max_len": int(cfg["max_len"]), "visible_pairs_per_head": pairs,
           "dq_path": dq_path, "ms_per_step": round(ms, 4), "split_ms": split,
           "tflops_effective": round(tflops, 2),
           "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
           "algorithmic_gb": round(tensor_bytes(T, H, D) / 1e9, 3),
           "gbs_algorithmic": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
           "kernels_ms": {k: round(m / max(c, 1), 4) for k, (c, m) in sorted(prof.items())}}
    del t, pstore
    torch.cuda.empty_cache()
    return out


def host_info():
    """The host the CPU baseline ran on: logical CPUs, CPUs this process may
    use, the CPU model and the OpenMP thread count the oracle runs with."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    omp = None
    try:
        import ctypes

        omp = int(ctypes.CDLL("libgomp.so.1").omp_get_max_threads())
    except (OSError, AttributeError):
        pass
    return {"nproc": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
            "cpu_model": model, "omp_threads": omp,
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def oracle_time(torch, cfg, t, off, seqs, targets=None):
    """fwd+bwd of the fp64 oracle on the sequences `seqs` (all of them when
    None): seconds and the effective flops (14 D per visible pair) it did."""
    import oracle

    if seqs is None:
        seqs = list(range(len(cfg["lengths"])))
    rows, sub_off = oracle.subset(off, seqs)
    rows_t = torch.from_numpy(rows).to(t["k"].device)
    to64 = lambda x: x.index_select(0, rows_t).float().cpu().numpy().astype(np.float64)  # noqa: E731
    k, v = to64(t["k"]), to64(t["v"])
    if targets is not None:
        sel = torch.tensor(seqs, device=t["k"].device)
        q = t["q"].index_select(0, sel).float().cpu().numpy().astype(np.float64)
        do = t["do"].index_select(0, sel).float().cpu().numpy().astype(np.float64)
        tr = targets[seqs]
    else:
        q, do, tr = to64(t["q"]), to64(t["do"]), None
    func = np.ascontiguousarray(t["func"].cpu().numpy()[:, rows])
    orc = oracle.default()
    _, pairs = orc.visible_counts(sub_off, func, tr)
    t0 = time.perf_counter()
    orc.fwd(q, k, v, sub_off, func, cfg["alpha"], cfg["max_len"], tr)
    orc.bwd(q, k, v, do, sub_off, func, cfg["alpha"], cfg["max_len"], tr)
    dt = time.perf_counter() - t0
    return dt, 14.0 * cfg["D"] * cfg["H"] * pairs


def cpu_record(torch, device):
    """The oracle timed in full on the small workloads and on samples of the
    large ones (scaled by visible pairs, which the oracle's work is
    proportional to): seconds, effective TFLOP/s, and for samples the
    extrapolated full time."""
    runs = {}
    for name, sample in (("tiny_fp32", None), ("sla_1k", None), ("sla_2k", None),
                         ("hstu_2663_targets_only", None), ("three_interval", 8)):
        base = "hstu_2663" if name.startswith("hstu_2663") else name
        cfg = wl.workload(base)
        targets = name.endswith("targets_only")
        if cfg["dtype"] == "fp32":
            lengths = cfg["lengths"]
            off = wl.offsets_from_lengths(lengths)
            T = int(off[-1])
            mk = lambda sh, sd: torch.from_numpy(wl.normal_f32(sh, sd)).to(device)  # noqa: E731
            sh = (T, cfg["H"], cfg["D"])
            t = {"q": mk(sh, 11), "k": mk(sh, 12), "v": mk(sh, 13), "do": mk(sh, 14),
                 "func": torch.from_numpy(cfg["func"](lengths, cfg["nfunc"])).to(device)}
        else:
            t, off = make_inputs(cfg, device, targets=targets)
        lengths = cfg["lengths"]
        seqs = None
        if sample:
            seqs = [int(i) for i in np.linspace(0, len(lengths) - 1, sample)]
        dt, flops = oracle_time(torch, cfg, t, off, seqs,
                                wl.targets_last(lengths) if targets else None)
        rec = {"seconds": round(dt, 3), "tflops_effective": round(flops / dt / 1e12, 6),
               "sequences": len(seqs) if seqs else len(lengths), "of": len(lengths)}
        if seqs:
            import hstu_jagged_masked_amd as hj

            f_all = torch.from_numpy(cfg["func"](lengths, cfg["nfunc"])).to(device)
            _, tot = hj.visible_counts(torch.from_numpy(off).to(device), f_all, int(off[-1]))
            full_flops = 14.0 * cfg["D"] * cfg["H"] * int(tot.item())
            rec["extrapolated_full_seconds"] = round(dt * full_flops / flops, 1)
        runs[name] = rec
        log(f"[bench] cpu oracle {name}: {rec}")
        del t
    torch.cuda.empty_cache()
    return runs


def cpu_baseline(cfg, t, off, nseq):
    """The fp64 oracle on the first `nseq` sequences (fwd + bwd), host cores."""
    import oracle

    rows, sub_off = oracle.subset(off, list(range(nseq)))
    lo, hi = int(rows[0]), int(rows[-1]) + 1
    to64 = lambda x: x[lo:hi].float().cpu().numpy().astype(np.float64)  # noqa: E731
    q, k, v, do = (to64(t[n]) for n in ("q", "k", "v", "do"))
    func = t["func"][:, lo:hi].cpu().numpy()
    orc = oracle.default()
    counts, pairs = orc.visible_counts(sub_off, func)
    t0 = time.perf_counter()
    orc.fwd(q, k, v, sub_off, func, cfg["alpha"], cfg["max_len"])
    orc.bwd(q, k, v, do, sub_off, func, cfg["alpha"], cfg["max_len"])
    dt = time.perf_counter() - t0
    flops = 14.0 * cfg["D"] * cfg["H"] * pairs
    info = host_info()
    threads = info["omp_threads"] or int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    full_flops = 14.0 * cfg["D"] * cfg["H"] * float(np.sum(cfg["lengths"] * (cfg["lengths"] + 1) // 2))
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s",
            # the oracle runs one OpenMP thread per (sequence, head) unit at most
            "cores": min(threads, nseq * cfg["H"]),
            "kind": "oracle",
            "sample": f"fp64 oracle fwd+bwd on {nseq} of {len(cfg['lengths'])} sequences "
                      f"(L={int(cfg['lengths'][0])}, all {cfg['H']} heads), {dt:.2f} s, "
                      f"effective flops 14*D per visible pair",
            "extrapolated_full_seconds": round(dt * full_flops / flops, 1),
            **info}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="hstu_2663", choices=wl.WORKLOADS)
    ap.add_argument("--targets-steps", type=int, default=20)
    ap.add_argument("--cpu-seqs", type=int, default=12,
                    help="sequences in the CPU oracle sample (0 disables it)")
    ap.add_argument("--dq", choices=("stored-p", "recompute"), default="stored-p",
                    help="dQ path of the backward: from stored P (needs ~2 bytes per (row, "
                         "column) pair of each sequence per head of HBM) or recomputing the "
                         "scores; the run fails rather than switch paths when memory is short")
    ap.add_argument("--pstore-budget-gb", type=float, default=4.0,
                    help="also time the stored-P backward over a buffer of this many GiB, in "
                         "runs of sequences (0: skip)")
    ap.add_argument("--no-dq-variants", dest="dq_variants", action="store_false",
                    help="skip timing the backward with the recompute and atomic dQ paths")
    ap.add_argument("--no-extra", dest="extra", action="store_false",
                    help="skip the other workloads (SLA, three-interval, OneRank, ragged, "
                         "L=4086) and the full CPU record")
    ap.add_argument("--calib-copy-mib", type=int, default=1024,
                    help="size of a plain device-to-device copy run once before timing; "
                         "counter runs scale HBM byte counters by it (0 disables it)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE={world}): "
              "the operator has no cross-GPU step; several GPUs each run their own slice of "
              "the sequences",
              file=sys.stderr)
        return 2

    import torch

    import hstu_jagged_masked_amd as hj

    hj.library()
    device = torch.device("cuda:0")
    cfg = wl.workload(args.workload)
    if cfg["dtype"] != "bf16":
        raise SystemExit("bench.py times the bf16 workloads")
    H, D = cfg["H"], cfg["D"]
    log(f"[bench] workload {args.workload}: B={len(cfg['lengths'])} H={H} D={D}")
    t, off = make_inputs(cfg, device)
    _, pairs_t = hj.visible_counts(t["off"], t["func"], int(off[-1]))
    pairs = int(pairs_t.item())
    log(f"[bench] visible pairs per head: {pairs}")

    if args.calib_copy_mib > 0:
        nbytes = args.calib_copy_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=device).fill_(1)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    pstore = None
    p_bytes = hj.pstore_bytes(t["off"], H)
    use_p = args.dq == "stored-p"
    if use_p:
        pstore = torch.empty(p_bytes, dtype=torch.uint8, device=device)
    log(f"[bench] dQ path: {'stored P, %.1f GB' % (p_bytes / 1e9) if use_p else 'recompute'}")
    run_steps(hj, t, cfg, args.warmup, pstore=pstore)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")
    ms, wall, prof = timed(hj, torch, t, cfg, args.steps, pstore=pstore)
    log(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step")
    split = split_ms(hj, torch, t, cfg, args.steps, pstore)
    stats = step_stats(hj, torch, t, cfg, args.steps, 3, pstore)
    flops_eff = 14.0 * D * H * pairs
    value = flops_eff / (ms * 1e-3) / 1e12

    kernels = {}
    for name, (count, total_ms) in sorted(prof.items()):
        per = total_ms / max(count, 1)
        rec = {"launches": count, "avg_ms": round(per, 4), "ms_per_step": round(total_ms / args.steps, 4)}
        if name in KERNEL_FLOPS_PER_PAIR:
            fl = KERNEL_FLOPS_PER_PAIR[name] * D * H * pairs
            rec["algorithmic_tflop_per_launch"] = round(fl / 1e12, 4)
            rec["tflops"] = round(fl / (per * 1e-3) / 1e12, 1)
        kernels[name] = rec
    dom = max((k for k in kernels if k in KERNEL_FLOPS_PER_PAIR),
              key=lambda k: kernels[k]["ms_per_step"])
    ach = kernels[dom]["tflops"]
    roofline = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic(dom)}

    del pstore
    torch.cuda.empty_cache()
    # the stored-P backward over a bounded buffer, in runs of sequences
    chunked = None
    if use_p and args.pstore_budget_gb > 0:
        budget = int(args.pstore_budget_gb * (1 << 30)) // 256 * 256
        runs = pstore_runs(cfg["lengths"], H, budget)
        pb = torch.empty(budget, dtype=torch.uint8, device=device)
        run_steps(hj, t, cfg, 2, pstore=pb, host_offsets=off)
        c_ms, _, c_prof = timed(hj, torch, t, cfg, args.steps, pstore=pb, host_offsets=off)
        log(f"[bench] stored P in {runs} runs over {args.pstore_budget_gb} GiB: {c_ms:.3f} ms/step")
        chunked = {"budget_gib": args.pstore_budget_gb, "runs": runs,
                   "ms_per_step": round(c_ms, 4),
                   "effective_tflops": round(flops_eff / (c_ms * 1e-3) / 1e12, 2),
                   "vs_whole_batch_buffer": round(c_ms / ms, 4),
                   "kernels_ms_per_step": {k: round(v[1] / args.steps, 4)
                                           for k, v in sorted(c_prof.items())}}
        del pb
        torch.cuda.empty_cache()
    # targets-only mode on the same K/V
    tt, _ = make_inputs(cfg, device, targets=True)
    tt["k"], tt["v"] = t["k"], t["v"]
    run_steps(hj, tt, cfg, 2, targets=True)
    t_ms, _, t_prof = timed(hj, torch, tt, cfg, args.targets_steps, targets=True)
    log(f"[bench] targets-only: {t_ms:.3f} ms/step")
    T = int(off[-1])
    # fwd streams K, V; bwd streams K, V in and dK, dV out (bf16)
    t_bytes = 6.0 * T * H * D * 2
    targets = {"ms_per_step": round(t_ms, 4), "speedup_vs_full": round(ms / t_ms, 2),
               "traffic_bytes_per_launch": {k: measured_traffic(k)
                                            for k in ("k_targets_fwd", "k_targets_bwd")},
               "algorithmic_gb": round(t_bytes / 1e9, 3),
               "gbs": round(t_bytes / (t_ms * 1e-3) / 1e9, 1),
               "frac_hbm_peak": round(t_bytes / (t_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
               "kernels": {k: {"launches": c, "avg_ms": round(m / max(c, 1), 4)}
                           for k, (c, m) in sorted(t_prof.items())}}
    del tt

    # cost of padded empty intervals: the SLA 2k workload (B=16, S=2048, H=8)
    # with its two intervals encoded as nfunc=3 and padded to nfunc=5
    c3 = wl.workload("sla_2k")
    t3, _ = make_inputs(c3, device)
    pad = {"workload": "sla_2k"}
    for nf in (3, 5):
        t3["func"] = torch.from_numpy(c3["func"](c3["lengths"], nf)).to(device)
        run_steps(hj, t3, c3, 3)
        m3, _, _ = timed(hj, torch, t3, c3, 20)
        pad[f"ms_nfunc{nf}"] = round(m3, 4)
    pad["delta_pct"] = round(100.0 * (pad["ms_nfunc5"] / pad["ms_nfunc3"] - 1.0), 2)
    del t3
    log(f"[bench] sla_2k nfunc 3 vs 5: {pad}")

    variants = None
    if args.dq_variants:
        variants = dq_variants(hj, torch, t, cfg, min(args.steps, 5), split["bwd"])
        log(f"[bench] backward by dQ path: " +
            ", ".join(f"{k} {v['bwd_ms']} ms" for k, v in variants.items()))

    cpu = None
    if args.cpu_seqs > 0:
        log(f"[bench] cpu oracle baseline on {args.cpu_seqs} sequences ...")
        cpu = cpu_baseline(cfg, t, off, args.cpu_seqs)
        log(f"[bench] cpu oracle: {cpu['value']:.6f} TFLOP/s")
    del t
    torch.cuda.empty_cache()

    per_workload = {}
    if args.extra:
        for name in EXTRA_WORKLOADS:
            if name == args.workload:
                continue
            per_workload[name] = measure_workload(hj, torch, name, device,
                                                  min(args.steps, 10),
                                                  "stored_p" if use_p else "recompute")
            log(f"[bench] {name}: {per_workload[name]['ms_per_step']} ms/step, "
                f"{per_workload[name]['tflops_effective']} TFLOP/s")
        if cpu is not None:
            cpu["runs"] = cpu_record(torch, device)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": len(cfg["lengths"]),
                   "seq_len": int(cfg["lengths"].max()), "tokens": T, "heads": H, "head_dim": D,
                   "nfunc": cfg["nfunc"], "mask": "causal" if "hstu" in args.workload else
                   args.workload, "visible_pairs_per_head": pairs,
                   "dq_path": "stored_p" if use_p else "recompute",
                   "pstore_gb": round(p_bytes / 1e9, 2) if use_p else 0.0},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        # the same step counted at 12*D per pair (no recomputed products)
        "value_12d": round(12.0 * D * H * pairs / (ms * 1e-3) / 1e12, 2),
        "split_ms": split,
        "step_stats": stats,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "targets_only": targets,
        "pstore_bounded": chunked,
        "dq_variants": variants,
        "nfunc_pad_cost": pad,
        "per_workload": per_workload,
        "kernels": kernels,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
