"""Benchmark of the owner-side Muon step on one MI355X.

One step = dmuon_step over the whole owned set (momentum, Newton-Schulz,
update) with inputs resident in HBM.  Default workload: the 28-layer stack of
the 3B decoder shapes (196 matrices, 2.82 G elements, bf16 params and grads,
fp32 momentum, bf16 NS products, Gram backend).  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload 2] [--ns-backend gram]
                  [--ns-precision bf16] [--no-cpu-baseline] [--copy-probe]
  python bench.py --pmc-summary FETCH_DIR WRITE_DIR      (writes the traffic summary)
  python bench.py --clip [--steps K] [--warmup W]        (gradient clipping alone)
  python bench.py --tp 8 [--steps K] [--warmup W]        (NS on tensor-parallel shards)
  python bench.py --owners 8 [--steps K] [--warmup W]    (each owner's share of the step, timed)
  python bench.py --adamw [--steps K] [--warmup W]       (fused AdamW of the symmetric parameters)
  python bench.py --adamw --pmc-summary FETCH_DIR WRITE_DIR
  python bench.py --clip --pmc-summary FETCH_DIR WRITE_DIR

--tp K times dmuon_orthogonalize_sharded with every matrix of the workload
cut into K tensor-parallel shards as the usual layout cuts them (q, k, v,
gate, up by output rows; o, down by input columns), and the unsharded
dmuon_orthogonalize of the same matrices for comparison; one JSON line.

--owners N plans the workload's matrices over N owners with each cost model
of dmuon_assign_owners, runs every owner's share through dmuon_step on the
one GPU, and reports the measured step-time imbalance of each plan.

--adamw times dmuon_adamw_step over the AdamW group of a 3B-shaped model
(the 128256 x 3072 embedding and 57 RMSNorm weights, bf16 parameters and
gradients, fp32 moments); one JSON line, HBM-bound.

--clip times dmuon_clip_grad_norm over the same gradient set (one bucket,
p = 2, clipping active on every call: each call's max_norm is half the
gradients' current norm) and prints its own JSON line, HBM-bound.

HBM traffic of the GEMM kernel comes from two rocprofv3 counter runs of this
script (FETCH_SIZE, then WRITE_SIZE, with --copy-probe so that each run also
holds a plain 1 GiB device copy whose counter reading calibrates the
counter): --pmc-summary turns them into TRAFFIC_SUMMARY, which later runs read
while the GEMM source is unchanged (its SHA-256 is recorded there).
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_bf16_3b_stack_hbm_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "matrix_optimizer_step_owned_amd", "csrc", "gemm.hip")
CLIP_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "clip_scale_3b_stack_grads_hbm_traffic.md")
CLIP_SOURCE = os.path.join(ROOT, "matrix_optimizer_step_owned_amd", "csrc", "clip.hip")
ELEMENTWISE_SOURCE = os.path.join(ROOT, "matrix_optimizer_step_owned_amd", "csrc", "elementwise.hip")
ADAMW_TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "adamw_3b_symmetric_group_hbm_traffic.md")
ADAMW_SOURCE = os.path.join(ROOT, "matrix_optimizer_step_owned_amd", "csrc", "adamw.hip")
ADAMW_METRIC = "fused AdamW GB/s (bf16 params and grads, fp32 moments) for a 3B-shaped symmetric group"
ADAMW_SHAPES = [(128256, 3072)] + [(3072,)] * 57
CLIP_METRIC = "gradient clipping GB/s (per-bucket global 2-norm clip, in place) for a 3B-shaped gradient set"
COPY_PROBE_BYTES = 1 << 30

METRIC = "NS TFLOP/s and optimizer steps/s for a 3B-shaped owner set; % bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3       # MI355X fp32 matrix
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--ns-backend", default="gram", choices=["gram", "direct"])
    ap.add_argument("--ns-precision", default="bf16", choices=["bf16", "f32"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-standard-form", action="store_true",
                    help="time only the chosen form (the default run also times the standard form)")
    ap.add_argument("--cpu-sample", default="auto",
                    help="'auto' (one matrix of each distinct shape) or 'none'")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, copy 1 GiB device to device (counter calibration)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs into the traffic summary and exit")
    ap.add_argument("--pmc-kernel", default="gemm_bf16_kernel", choices=["gemm_bf16_kernel", "momentum_kernel"],
                    help="with --pmc-summary: the kernel to summarise")
    ap.add_argument("--mfma-summary", nargs=2, metavar=("PMC_DIR", "BENCH_JSON"),
                    help="summarise a rocprofv3 run of MFMA counters (one step) against a bench line and exit")
    ap.add_argument("--clip", action="store_true",
                    help="time gradient clipping of the workload's gradients instead of the step")
    ap.add_argument("--adamw", action="store_true",
                    help="time the fused AdamW step of a 3B-shaped symmetric group instead of the step")
    ap.add_argument("--owners", type=int, default=0,
                    help="time each owner's share of the step for this many owners")
    ap.add_argument("--tp", type=int, default=0,
                    help="time NS on this many tensor-parallel shards per matrix instead of the step")
    return ap.parse_args()


def source_sha256(path=GEMM_SOURCE):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _pmc_rows(d, counter):
    """(kernel name, dispatch id, value) of one counter from a rocprofv3 csv directory."""
    out = []
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith("counter_collection.csv"):
                with open(os.path.join(root, fn)) as f:
                    for r in csv.DictReader(f):
                        if r["Counter_Name"] == counter:
                            out.append((r["Kernel_Name"], int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    return out


def pmc_summary(fetch_dir, write_dir, steps, kernel="gemm_bf16_kernel", per_step=16):
    """Per-launch HBM bytes of one kernel over the last ``steps`` steps'
    launches (``per_step`` each), each counter scaled by its reading for the
    1 GiB copy."""
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = _pmc_rows(d, counter)
        gemm = sorted((di, v) for k, di, v in rows if kernel in k)
        copies = sorted((di, v) for k, di, v in rows if "dmuon" not in k)
        if not gemm or not copies:
            raise SystemExit(f"no {kernel} or copy dispatches in {d}")
        copy_kib = copies[-1][1]                 # the probe is the last dispatch
        factor = (COPY_PROBE_BYTES / 1024.0) / copy_kib
        last = [v for _, v in gemm[-per_step * steps:]]
        res[counter] = {"kib_per_launch": sum(last) / len(last), "copy_kib": copy_kib, "factor": factor,
                        "bytes_per_launch": sum(last) / len(last) * 1024.0 * factor, "launches": len(last)}
    return res


def mfma_summary(pmc_dir, bench_json, per_step=16):
    """Executed MFMA work of the GEMM launches of one step from
    SQ_INSTS_VALU_MFMA_MOPS_BF16 (x 512 flops), and the MFMA-busy and
    shader-busy cycle counters, against the algorithmic flops and the GEMM
    time of a bench line."""
    rows = {}
    for counter in ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES"):
        vals = sorted((di, v) for k, di, v in _pmc_rows(pmc_dir, counter) if "gemm_bf16_kernel" in k)
        rows[counter] = [v for _, v in vals[-per_step:]]
    with open(bench_json) as f:
        b = json.loads(f.read().strip().splitlines()[-1])
    exec_flops = sum(rows["SQ_INSTS_VALU_MFMA_MOPS_BF16"]) * 512
    alg_flops = (b["ns_algorithmic_tflop_per_step"] * 1e12 if "ns_algorithmic_tflop_per_step" in b
                 else b["kernels"]["gemm_bf16"]["tflops"] * 1e12 * b["ns_ms_per_step"] * 1e-3)
    t = b["ns_ms_per_step"] * 1e-3
    print("# Executed MFMA work of gemm_bf16_kernel, 3B 28-layer stack (workload 2), gram, bf16\n")
    print(f"- executed MFMA flops per step (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512, {per_step} launches): "
          f"{exec_flops / 1e12:.2f} TFLOP")
    print(f"- algorithmic flops per step (symmetric results counted once): {alg_flops / 1e12:.2f} TFLOP "
          f"(executed / algorithmic = {exec_flops / alg_flops:.3f})")
    print(f"- GEMM time per step (bench HIP events): {t * 1e3:.2f} ms -> executed MFMA rate "
          f"{exec_flops / t / 1e12:.1f} TFLOP/s = {exec_flops / t / 1e12 / PEAK_BF16_TFLOPS:.3f} of {PEAK_BF16_TFLOPS}")
    busy = sum(rows["SQ_VALU_MFMA_BUSY_CYCLES"])
    sq = sum(rows["SQ_BUSY_CYCLES"])
    print(f"- SQ_VALU_MFMA_BUSY_CYCLES summed: {busy:.4e}; SQ_BUSY_CYCLES summed: {sq:.4e}")
    print(f"- gemm_source_sha256: {source_sha256()}")


def read_traffic(summary=TRAFFIC_SUMMARY, source=GEMM_SOURCE):
    """Bytes per launch of the summarised kernel from the committed summary,
    if it was taken on the current source of that kernel; else None."""
    try:
        with open(summary) as f:
            text = f.read()
    except OSError:
        return None
    m_sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_val or m_sha.group(1) != source_sha256(source):
        return None
    return float(m_val.group(1))


MFMA_SUMMARY = os.path.join(ROOT, "profiles", "gemm_bf16_3b_stack_mfma_counters.md")


def read_mfma_counters(summary=MFMA_SUMMARY, source=GEMM_SOURCE):
    """Executed MFMA flops per step of the GEMM from the committed counter
    summary, if it was taken on the current GEMM source; else None."""
    try:
        with open(summary) as f:
            text = f.read()
    except OSError:
        return None
    m_sha = re.search(r"gemm_source_sha256:\s*([0-9a-f]{64})", text)
    m_val = re.search(r"executed MFMA flops per step[^:]*:\s*([0-9.]+)\s*TFLOP", text)
    if not m_sha or not m_val or m_sha.group(1) != source_sha256(source):
        return None
    return float(m_val.group(1)) * 1e12


def nominal_flops(shapes, ns_steps):
    tot = 0.0
    for r, c in shapes:
        m, n = min(r, c), max(r, c)
        tot += ns_steps * (4.0 * m * m * n + 2.0 * m ** 3)
    return tot


def step_roofline(w, gemm_flops, ms_step, peak_tflops):
    """The step rate against its roofline: the GEMM launches' algorithmic
    flops at the matrix-core peak and the elementwise passes' algorithmic
    bytes (grad in, fp32 momentum in and out, the NS input out, parameter in
    and out, O in: 12 + 6 bytes per element with bf16 parameters and
    gradients) at the HBM peak, overlapped (max) or in sequence (sum).
    Steps/s and matrices/s share these fractions."""
    pb = 2 if w.param_dtype == "bf16" else 4
    gb = 2 if w.grad_dtype == "bf16" else 4
    ew_bytes = w.numel * (gb + 8 + 2 + 2 * pb + 2)
    t_mfma = gemm_flops / (peak_tflops * 1e12) * 1e3
    t_hbm = ew_bytes / (PEAK_HBM_GBS * 1e9) * 1e3
    overlap, seq = max(t_mfma, t_hbm), t_mfma + t_hbm
    return {"gemm_ms_at_peak": t_mfma, "elementwise_ms_at_peak": t_hbm, "elementwise_bytes": ew_bytes,
            "overlap_bound_ms": overlap, "sequential_bound_ms": seq,
            "frac_of_overlap_bound": overlap / ms_step, "frac_of_sequential_bound": seq / ms_step}


def cpu_baseline(w, hp, budget_s=30.0, min_s=10.0):
    """The oracle timed on this host: one step of one matrix of each distinct
    shape (inputs from the seeded generator), repeated over further matrices
    of the same shapes until at least ``min_s`` seconds are timed, then
    extrapolated to the workload by shape counts."""
    import numpy as np
    import dmuon_inputs as di
    from oracle import muon as orc
    shapes = {}
    for i, m in enumerate(w.matrices):
        shapes.setdefault((m.rows, m.cols), []).append(i)
    times = {}
    t_start = time.time()
    sampled = 0
    timed = 0.0
    for rnd in range(64):
        for (r, c), idx in sorted(shapes.items(), key=lambda kv: kv[0][0] * kv[0][1]):
            if rnd >= len(idx):
                continue
            i = idx[rnd]
            _, wexact = di.param_init(w, i)
            _, g = di.grad_at(w, i, 0)
            t0 = time.perf_counter()
            orc.muon_step(wexact, g, np.zeros_like(g), lr=hp["lr"], momentum=hp["momentum"],
                          nesterov=hp["nesterov"], ns_steps=hp["ns_steps"],
                          weight_decay=hp["weight_decay"], ns_backend=hp["ns_backend"],
                          param_dtype=w.param_dtype)
            dt = time.perf_counter() - t0
            times.setdefault((r, c), []).append(dt)
            timed += dt
            sampled += 1
            if time.time() - t_start > budget_s:
                break
        if timed >= min_s or time.time() - t_start > budget_s:
            break
    per_shape = {s: sum(v) / len(v) for s, v in times.items()}
    if len(per_shape) < len(shapes):
        # extrapolate the unsampled shapes by nominal flops of the sampled ones
        rate = sum(nominal_flops([s], hp["ns_steps"]) for s in per_shape) / sum(per_shape.values())
        for s in shapes:
            per_shape.setdefault(s, nominal_flops([s], hp["ns_steps"]) / rate)
    t_step = sum(per_shape[s] * len(idx) for s, idx in shapes.items())
    flops = nominal_flops([(m.rows, m.cols) for m in w.matrices], hp["ns_steps"])
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {
        "value": flops / t_step / 1e12, "unit": "TFLOP/s", "cores": min(cores, threads),
        "kind": "oracle",
        "steps_per_s": 1.0 / t_step, "matrices_per_s": len(w.matrices) / t_step,
        "sample": (f"float64 numpy oracle, one step each of {sampled} matrices covering "
                   f"{len(times)} of the {len(shapes)} distinct shapes ({timed:.1f} s timed), "
                   f"mean time per shape extrapolated to {len(w.matrices)} matrices by shape counts"),
    }


def main():
    args = parse()
    if args.mfma_summary:
        return mfma_summary(*args.mfma_summary)
    if args.pmc_summary and args.adamw:
        r = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], 1, kernel="adamw_kernel", per_step=1)
        tot = r["FETCH_SIZE"]["bytes_per_launch"] + r["WRITE_SIZE"]["bytes_per_launch"]
        print("# HBM traffic of adamw_kernel, the AdamW group of a 3B-shaped model (bf16 params and grads)\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            x = r[c]
            print(f"- {c}: {x['kib_per_launch']:.6g} KiB per launch (the last timed call); "
                  f"1 GiB copy reads {x['copy_kib']:.6g} KiB -> factor {x['factor']:.4f}; "
                  f"{x['bytes_per_launch'] / 1e9:.4f} GB per launch")
        print(f"- hbm_bytes_per_launch: {tot:.6e}")
        print(f"- adamw_source_sha256: {source_sha256(ADAMW_SOURCE)}")
        return
    if args.pmc_summary and args.clip:
        r = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], 1, kernel="clip_scale_kernel", per_step=1)
        tot = r["FETCH_SIZE"]["bytes_per_launch"] + r["WRITE_SIZE"]["bytes_per_launch"]
        print(f"# HBM traffic of clip_scale_kernel, gradients of the 3B 28-layer stack (bf16), p = 2\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            x = r[c]
            print(f"- {c}: {x['kib_per_launch']:.6g} KiB per launch (the last timed call); "
                  f"1 GiB copy reads {x['copy_kib']:.6g} KiB -> factor {x['factor']:.4f}; "
                  f"{x['bytes_per_launch'] / 1e9:.4f} GB per launch")
        print(f"- hbm_bytes_per_launch: {tot:.6e}")
        print(f"- clip_source_sha256: {source_sha256(CLIP_SOURCE)}")
        return
    if args.pmc_summary and args.pmc_kernel == "momentum_kernel":
        r = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], 1, kernel="momentum_kernel", per_step=1)
        tot = r["FETCH_SIZE"]["bytes_per_launch"] + r["WRITE_SIZE"]["bytes_per_launch"]
        print("# HBM traffic of momentum_kernel, 3B 28-layer stack (workload 2), gram, bf16\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            x = r[c]
            print(f"- {c}: {x['kib_per_launch']:.6g} KiB per launch (the last step's launch); "
                  f"1 GiB copy reads {x['copy_kib']:.6g} KiB -> factor {x['factor']:.4f}; "
                  f"{x['bytes_per_launch'] / 1e9:.4f} GB per launch")
        print(f"- hbm_bytes_per_launch: {tot:.6e}")
        print(f"- elementwise_source_sha256: {source_sha256(ELEMENTWISE_SOURCE)}")
        return
    if args.pmc_summary:
        steps = 1
        r = pmc_summary(args.pmc_summary[0], args.pmc_summary[1], steps)
        tot = r["FETCH_SIZE"]["bytes_per_launch"] + r["WRITE_SIZE"]["bytes_per_launch"]
        print(f"# HBM traffic of gemm_bf16_kernel, 3B 28-layer stack (workload 2), gram, bf16\n")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            x = r[c]
            print(f"- {c}: {x['kib_per_launch']:.6g} KiB per launch (mean of {x['launches']} launches of one step); "
                  f"1 GiB copy reads {x['copy_kib']:.6g} KiB -> factor {x['factor']:.4f}; "
                  f"{x['bytes_per_launch'] / 1e9:.4f} GB per launch")
        print(f"- hbm_bytes_per_launch: {tot:.6e}")
        print(f"- gemm_source_sha256: {source_sha256()}")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the owner step runs on one device with no "
              f"collectives; --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import torch
    import dmuon_inputs as di
    import matrix_optimizer_step_owned_amd as dm

    dev = torch.device("cuda:0")
    if args.clip:
        return run_clip(args, dev)
    if args.tp:
        return run_tp(args, dev)
    if args.owners:
        return run_owners(args, dev)
    if args.adamw:
        return run_adamw(args, dev)
    w = di.workload(args.workload)
    hp = w.hparams(ns_backend=args.ns_backend, ns_precision=args.ns_precision)
    shapes = [(m.rows, m.cols) for m in w.matrices]
    pdt = torch.bfloat16 if w.param_dtype == "bf16" else torch.float32
    gdt = torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32

    # inputs resident in HBM: params, momenta, and one gradient set per step
    params = []
    for i, (r, c) in enumerate(shapes):
        t = torch.empty(r, c, dtype=pdt, device=dev)
        di.torch_normal_(t, w.param_std, seed=1000 + i)
        params.append(t)
    moms = [torch.zeros(r, c, dtype=torch.float32, device=dev) for r, c in shapes]
    n_grad_sets = min(args.steps + args.warmup, 4)
    grad_sets = []
    for s in range(n_grad_sets):
        gs = []
        for i, (r, c) in enumerate(shapes):
            t = torch.empty(r, c, dtype=gdt, device=dev)
            di.torch_normal_(t, w.grad_std, seed=100000 * (s + 1) + i)
            gs.append(t)
        grad_sets.append(gs)
    stream = torch.cuda.current_stream(dev)
    peak = PEAK_BF16_TFLOPS if args.ns_precision == "bf16" else PEAK_F32_TFLOPS
    flops_step = nominal_flops(shapes, hp["ns_steps"])

    power = PowerSampler()

    def timed_run(hp_run, copy_after=False):
        """Warm-up steps, then the timed steps of one configuration; returns
        (ms per step, per-kernel profile, wall seconds); the board power over
        the timed steps is left in timed_run.power."""
        ws_bytes = dm.dmuon_step_workspace_size(params, grad_sets[0], moms, **hp_run)
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        print(f"# workload {w.name} ({hp_run['ns_backend']}/{hp_run['ns_precision']}): {len(shapes)} matrices, "
              f"{w.numel / 1e9:.3f} G elements, workspace {ws_bytes / 2**30:.2f} GiB", file=sys.stderr, flush=True)
        for s in range(args.warmup):
            dm.dmuon_step(params, grad_sets[s % n_grad_sets], moms, workspace=workspace, **hp_run)
        torch.cuda.synchronize()
        print("# warmup done", file=sys.stderr, flush=True)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        dm.dmuon_profile_begin()
        torch.cuda.synchronize()
        power.start()
        t0 = time.perf_counter()
        start.record(stream)
        for s in range(args.steps):
            dm.dmuon_step(params, grad_sets[(args.warmup + s) % n_grad_sets], moms, workspace=workspace, **hp_run)
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        timed_run.power = power.stop()
        prof = dm.dmuon_profile_end()["kernels"]
        if copy_after:
            copy_probe(dev)
        ms_step = start.elapsed_time(end) / args.steps
        print(f"# timed {args.steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f})",
              file=sys.stderr, flush=True)
        del workspace
        torch.cuda.empty_cache()
        return ms_step, prof, wall

    def gemm_summary(prof):
        """GEMM time and algorithmic flops per step, and the dominant kernel."""
        gemm = {k: v for k, v in prof.items() if k.startswith("gemm")}
        # the GEMM phase's time: the union of the launches' intervals (the
        # summed durations when one stream runs them; less when a small
        # batch's two stream groups overlap)
        ns_ms = sum(v.get("wall_ms", v["ms"]) for v in gemm.values()) / args.steps
        alg_flops = sum(v["flops"] for v in gemm.values()) / args.steps
        dom_name, dom = max(gemm.items(), key=lambda kv: kv[1]["ms"])
        # algorithmic flops of the step's launches over their time: the summed
        # launch durations (the duration-weighted mean over launches of flops /
        # launch time), or, when two stream groups run launches side by side,
        # the union of their intervals (each launch's own duration then also
        # counts the time it shares the GPU with the other group's)
        achieved = dom["flops"] / (dom.get("wall_ms", dom["ms"]) * 1e-3) / 1e12
        return ns_ms, alg_flops, dom_name, dom, achieved

    ms_step, prof, wall = timed_run(hp, copy_after=args.copy_probe)
    power_main = timed_run.power
    value = flops_step / (ms_step * 1e-3) / 1e12
    ns_ms, alg_flops, dom_name, dom, achieved = gemm_summary(prof)
    # the committed counter summaries cover the default configuration only
    default_cfg = args.workload == 2 and args.ns_precision == "bf16" and args.ns_backend == "gram"
    traffic = read_traffic() if default_cfg else None
    counted = read_mfma_counters() if default_cfg else None
    kernels = {k: {"launches_per_step": v["launches"] / args.steps,
                   "ms_per_step": v["ms"] / args.steps,
                   "wall_ms_per_step": v.get("wall_ms", v["ms"]) / args.steps,
                   "tflops": (v["flops"] / (v["ms"] * 1e-3) / 1e12) if v["flops"] else None,
                   "gbs": v["bytes"] / (v["ms"] * 1e-3) / 1e9}
               for k, v in prof.items()}
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.ns_precision,
        "data": "synthetic (seeded normal params and grads, generated on device)",
        "config": {"workload": w.name, "matrices": len(shapes), "elements": w.numel,
                   "ns_backend": args.ns_backend, "ns_precision": args.ns_precision,
                   "ns_steps": hp["ns_steps"], "param_dtype": w.param_dtype,
                   "grad_dtype": w.grad_dtype, "momentum_dtype": "f32"},
        "steps_per_s": 1e3 / ms_step,
        "matrices_per_s": len(shapes) * 1e3 / ms_step,
        "step_roofline": step_roofline(w, alg_flops, ms_step, peak),
        # the metric's nominal count (4 m^2 n + 2 m^3 per iteration) over the NS launches' time:
        # a standard-form-equivalent rate, not a fraction of any peak
        "ns_tflops_nominal": flops_step / (ns_ms * 1e-3) / 1e12,
        # flops the planned products need (symmetric results counted once) over the same time
        "ns_algorithmic_tflops": alg_flops / (ns_ms * 1e-3) / 1e12,
        "ns_algorithmic_frac_of_peak": alg_flops / (ns_ms * 1e-3) / 1e12 / peak,
        "ns_algorithmic_tflop_per_step": alg_flops / 1e12,
        "ns_ms_per_step": ns_ms,
        "kernels": kernels,
        "roofline": {"bound": "mfma", "kernel": dom_name, "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch",
                     "launches": dom["launches"], "mean_launch_ms": dom["ms"] / dom["launches"],
                     "time_basis": ("union of overlapping launch intervals (two stream groups)"
                                    if dom.get("wall_ms", dom["ms"]) < 0.999 * dom["ms"] else "summed launch durations"),
                     "alg_flops_per_launch": dom["flops"] / dom["launches"],
                     "alg_bytes_per_launch": dom["bytes"] / dom["launches"]},
        # executed MFMA work from the committed rocprofv3 counter summary (same GEMM source only)
        "mfma_counters": None if counted is None else {
            "executed_tflop_per_step": counted / 1e12,
            "executed_tflops": counted / (ns_ms * 1e-3) / 1e12,
            "frac_of_peak": counted / (ns_ms * 1e-3) / 1e12 / peak,
            "summary": os.path.relpath(MFMA_SUMMARY, ROOT)},
        # board power and clock over the timed steps (the GEMMs run at the power cap)
        "power": power_main,
    }
    if default_cfg and not args.no_standard_form:
        # the headline configuration names both NS forms: time the standard form too
        hp_std = dict(hp, ns_backend="direct")
        ms_std, prof_std, _ = timed_run(hp_std)
        ns_ms_s, alg_s, dom_name_s, dom_s, ach_s = gemm_summary(prof_std)
        out["standard_form"] = {
            "ns_backend": "direct", "ms_per_step": ms_std, "value": flops_step / (ms_std * 1e-3) / 1e12,
            "unit": "TFLOP/s", "steps_per_s": 1e3 / ms_std, "matrices_per_s": len(shapes) * 1e3 / ms_std,
            "ns_ms_per_step": ns_ms_s, "ns_algorithmic_tflops": alg_s / (ns_ms_s * 1e-3) / 1e12,
            "step_roofline": step_roofline(w, alg_s, ms_std, peak),
            "roofline": {"bound": "mfma", "kernel": dom_name_s, "achieved": ach_s, "peak": peak,
                         "unit": "TFLOP/s", "frac": ach_s / peak,
                         "mean_launch_ms": dom_s["ms"] / dom_s["launches"]},
            "gram_speedup": ms_std / ms_step, "power": timed_run.power}
    if not args.no_cpu_baseline:
        print("# cpu baseline ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, hp)
    print(json.dumps(out), flush=True)


class PowerSampler:
    """Board power and graphics clock, read through amdsmi (read-only queries)
    every 50 ms on a thread of its own while the timed steps run; the summary
    is None where amdsmi is not available."""

    def __init__(self):
        self.handle = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            self.amdsmi = amdsmi
            self.handle = amdsmi.amdsmi_get_processor_handles()[0]
            self.cap_w = amdsmi.amdsmi_get_power_cap_info(self.handle)["power_cap"] / 1e6
        except Exception:
            self.handle = None

    def start(self):
        import threading
        self.samples = []
        if self.handle is None:
            return
        self.stop_flag = threading.Event()

        def run():
            while not self.stop_flag.is_set():
                try:
                    m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
                    self.samples.append((m.get("current_socket_power"), m.get("current_gfxclk")))
                except Exception:
                    pass
                time.sleep(0.05)

        self.thread = threading.Thread(target=run, daemon=True)
        self.thread.start()

    def stop(self):
        if self.handle is None:
            return None
        self.stop_flag.set()
        self.thread.join()
        pw = sorted(p for p, _ in self.samples if isinstance(p, (int, float)))
        ck = sorted(c for _, c in self.samples if isinstance(c, (int, float)))
        if not pw:
            return None
        return {"socket_w_median": pw[len(pw) // 2], "socket_w_max": pw[-1], "cap_w": self.cap_w,
                "gfxclk_mhz_median": ck[len(ck) // 2] if ck else None, "samples": len(pw),
                "source": "amdsmi gpu metrics, sampled every 50 ms over the timed steps"}


def copy_probe(dev):
    """A plain 1 GiB device-to-device copy (calibrates the HBM byte counters)."""
    import torch
    src = torch.ones(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def clip_cpu_baseline(w, budget_s=60.0, min_s=10.0):
    """The clipping oracle timed on this host over whole gradients of the
    workload (seeded, bf16-valued; one drawn per distinct shape and reused for
    the other matrices of that shape), one bucket per call, in the workload's
    order until ``min_s`` seconds are timed; reported as gradient bytes (bf16)
    per second."""
    import dmuon_inputs as di
    from oracle import clip as orc_clip
    t_start = time.time()
    timed, nbytes, done = 0.0, 0, 0
    by_shape = {}
    for i, m in enumerate(w.matrices):
        if (m.rows, m.cols) not in by_shape:
            by_shape[(m.rows, m.cols)] = di.grad_at(w, i, 0)[1]
        g = by_shape[(m.rows, m.cols)]
        t0 = time.perf_counter()
        _, tot, _ = orc_clip.clip_grad_norm([g], [0], [1e-4], 2.0)
        timed += time.perf_counter() - t0
        nbytes += g.size * 2
        done += 1
        if timed >= min_s or time.time() - t_start > budget_s:
            break
    # numpy's elementwise operations and reductions run on one thread
    return {"value": nbytes / timed / 1e9, "unit": "GB/s of bf16 gradient clipped", "cores": 1,
            "kind": "oracle",
            "sample": (f"float64 numpy oracle, norm and scale of the first {done} gradients of the "
                       f"workload, one call each ({nbytes / 1e9:.3f} GB as bf16, {timed:.1f} s timed)")}


def clip_then_step(w, grads, dev, stream, norm, reps=3):
    """Clipping followed by the step over the same matrices, two ways: the
    in-place clip then dmuon_step, and the clip's coefficients then
    dmuon_step with the gradients scaled as the momentum pass reads them.
    Every call clips (max_norm is half the gradients' current norm).
    Returns ms per (clip + step) for both."""
    import torch
    import dmuon_inputs as di
    import matrix_optimizer_step_owned_amd as dm
    hp = w.hparams()
    params, moms = [], []
    for i, m in enumerate(w.matrices):
        p = torch.empty(m.rows, m.cols, dtype=torch.bfloat16, device=dev)
        di.torch_normal_(p, w.param_std, seed=1000 + i)
        params.append(p)
        moms.append(torch.zeros(m.rows, m.cols, dtype=torch.float32, device=dev))
    ws = torch.empty(dm.dmuon_step_workspace_size(params, grads, moms, **hp), dtype=torch.uint8, device=dev)
    cws = torch.empty(max(1, dm._lib.dmuon_clip_workspace_size(*_clip_args(dm, grads), 1)), dtype=torch.uint8,
                      device=dev)
    coefs = torch.ones(1, dtype=torch.float64, device=dev)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    state = {"norm": norm}

    def unfused():
        state["norm"] *= 0.5
        dm.dmuon_clip_grad_norm(grads, state["norm"], workspace=cws)
        dm.dmuon_step(params, grads, moms, workspace=ws, **hp)

    def fused():
        dm.dmuon_clip_coefficients(grads, 0.5 * state["norm"], coefs=coefs, workspace=cws)
        dm.dmuon_step(params, grads, moms, workspace=ws, grad_scale=coefs, **hp)

    t_unfused = timed(unfused)
    t_fused = timed(fused)
    del ws
    return {"in_place_clip_then_step_ms": t_unfused, "coefficients_then_scaled_step_ms": t_fused,
            "saved_ms": t_unfused - t_fused}


def _clip_args(dm, grads):
    import ctypes
    arr = (dm.dmuon_grad_t * len(grads))()
    for i, g in enumerate(grads):
        arr[i].numel, arr[i].grad, arr[i].dtype, arr[i].bucket = g.numel(), g.data_ptr(), dm._dtype(g), 0
    return arr, len(grads)


def run_clip(args, dev):
    """Gradient clipping alone: dmuon_clip_grad_norm over the workload's
    gradient set; a step is one call (norm, finalize, scale)."""
    import torch
    import dmuon_inputs as di
    import matrix_optimizer_step_owned_amd as dm

    w = di.workload(args.workload)
    gdt = torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32
    esize = 2 if w.grad_dtype == "bf16" else 4
    grads = []
    for i, m in enumerate(w.matrices):
        t = torch.empty(m.rows, m.cols, dtype=gdt, device=dev)
        di.torch_normal_(t, w.grad_std, seed=100000 + i)
        grads.append(t)
    nbytes = w.numel * esize
    total = torch.empty(1, dtype=torch.float64, device=dev)
    # the current norm (nothing clipped: max_norm far above it)
    dm.dmuon_clip_grad_norm(grads, 1e30, total_norm=total)
    norm = float(total.cpu()[0])
    stream = torch.cuda.current_stream(dev)
    print(f"# clip of {len(grads)} gradients, {nbytes / 1e9:.3f} GB, norm {norm:.6g}", file=sys.stderr, flush=True)
    # each call halves the norm: the coefficient is about 0.5 on every call
    for s in range(args.warmup):
        norm *= 0.5
        dm.dmuon_clip_grad_norm(grads, norm, total_norm=total)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    dm.dmuon_profile_begin()
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(args.steps):
        norm *= 0.5
        dm.dmuon_clip_grad_norm(grads, norm, total_norm=total)
    end.record(stream)
    torch.cuda.synchronize()
    prof = dm.dmuon_profile_end()["kernels"]
    ms_step = start.elapsed_time(end) / args.steps
    if args.copy_probe:
        copy_probe(dev)
    fused = None if args.copy_probe else clip_then_step(w, grads, dev, stream, norm)
    # every call wrote: the scale kernel ran on every gradient
    alg_bytes = 3 * nbytes
    value = alg_bytes / (ms_step * 1e-3) / 1e9
    dom = prof["clip_scale"]
    achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
    kernels = {k: {"launches_per_step": v["launches"] / args.steps, "ms_per_step": v["ms"] / args.steps,
                   "gbs": v["bytes"] / (v["ms"] * 1e-3) / 1e9}
               for k, v in prof.items()}
    out = {
        "metric": CLIP_METRIC, "value": value, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f64 accumulation, " + w.grad_dtype + " gradients",
        "data": "synthetic (seeded normal gradients, generated on device)",
        "config": {"workload": w.name + " gradients", "tensors": len(grads), "elements": w.numel,
                   "grad_dtype": w.grad_dtype, "norm_type": 2, "buckets": 1,
                   "alg_bytes_per_call": alg_bytes},
        "kernels": kernels,
        "clip_then_step": fused,
        "roofline": {"bound": "hbm", "kernel": "clip_scale", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": read_traffic(CLIP_TRAFFIC_SUMMARY, CLIP_SOURCE),
                     "traffic_unit": "HBM bytes per launch", "launches": dom["launches"],
                     "mean_launch_ms": dom["ms"] / dom["launches"],
                     "alg_bytes_per_launch": dom["bytes"] / dom["launches"]},
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = clip_cpu_baseline(w)
    print(json.dumps(out), flush=True)


TP_SPLIT = {"q_proj": 0, "k_proj": 0, "v_proj": 0, "gate_proj": 0, "up_proj": 0, "o_proj": 1, "down_proj": 1}
TP_METRIC = ("NS TFLOP/s on tensor-parallel shards (Gram sums across shards) for a 3B-shaped owner set; "
             "% bf16 MFMA peak")


def tp_layout(w, k):
    """(split, shard sizes) of every matrix: the usual tensor-parallel cut."""
    out = []
    for m in w.matrices:
        split = TP_SPLIT[m.name.split(".")[-1]]
        along = m.rows if split == 0 else m.cols
        if along % k:
            raise SystemExit(f"{m.name}: {along} does not split into {k} shards")
        out.append((split, [along // k] * k))
    return out


def tp_cpu_baseline(w, k, hp, budget_s=60.0, min_s=10.0):
    """The sharded oracle timed on this host: one matrix of each distinct
    (shape, split), cheapest first, until ``min_s`` seconds are timed; the
    other kinds are extrapolated by nominal flops; scaled to the workload by
    counts."""
    import dmuon_inputs as di
    from oracle import tp_gram as otp
    layout = tp_layout(w, k)
    kinds = {}
    for i, m in enumerate(w.matrices):
        kinds.setdefault((m.rows, m.cols, layout[i][0]), []).append(i)
    times = {}
    t_start, timed = time.time(), 0.0
    for key, idx in sorted(kinds.items(), key=lambda kv: nominal_flops([kv[0][:2]], hp["ns_steps"])):
        i = idx[0]
        _, u = di.grad_at(w, i, 0)
        parts = otp.split_matrix(u, layout[i][0], layout[i][1])
        t0 = time.perf_counter()
        otp.orthogonalize_sharded(parts, layout[i][0], hp["ns_steps"], hp["ns_backend"])
        dt = time.perf_counter() - t0
        times[key] = dt
        timed += dt
        if timed >= min_s or time.time() - t_start > budget_s:
            break
    rate = sum(nominal_flops([s[:2]], hp["ns_steps"]) for s in times) / sum(times.values())
    t_all = sum((times[s] if s in times else nominal_flops([s[:2]], hp["ns_steps"]) / rate) * len(idx)
                for s, idx in kinds.items())
    flops = nominal_flops([(m.rows, m.cols) for m in w.matrices], hp["ns_steps"])
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    threads = int(os.environ.get("OMP_NUM_THREADS", cores))
    return {"value": flops / t_all / 1e12, "unit": "TFLOP/s", "cores": min(cores, threads), "kind": "oracle",
            "sample": (f"float64 numpy sharded oracle, one matrix of {len(times)} of the {len(kinds)} "
                       f"(shape, split) kinds ({timed:.1f} s timed), the rest extrapolated by nominal "
                       f"flops, scaled to {len(w.matrices)} matrices by counts")}


def run_tp(args, dev):
    """NS of the workload's matrices held as args.tp tensor-parallel shards,
    one dmuon_orthogonalize_sharded call per step; the unsharded
    dmuon_orthogonalize of the same matrices is timed alongside."""
    import torch
    import dmuon_inputs as di
    import matrix_optimizer_step_owned_amd as dm

    k = args.tp
    w = di.workload(args.workload)
    hp = w.hparams(ns_backend=args.ns_backend, ns_precision=args.ns_precision)
    nshp = {key: hp[key] for key in ("ns_steps", "ns_backend", "ns_precision")}
    layout = tp_layout(w, k)
    shapes = [(m.rows, m.cols) for m in w.matrices]
    whole, ins, outs, splits = [], [], [], []
    for i, (r, c) in enumerate(shapes):
        u = torch.empty(r, c, dtype=torch.bfloat16, device=dev)
        di.torch_normal_(u, 1.0, seed=300000 + i)
        whole.append(u)
        split, sizes = layout[i]
        ins.append([p.contiguous() for p in torch.split(u, sizes, dim=1 if split == 1 else 0)])
        outs.append([torch.empty_like(p) for p in ins[-1]])
        splits.append(split)
    ws_bytes = dm.dmuon_orthogonalize_sharded_workspace_size([[tuple(p.shape) for p in mat] for mat in ins],
                                                            splits, **nshp)
    ws_whole = dm.dmuon_orthogonalize_workspace_size(shapes, **nshp)
    workspace = torch.empty(max(ws_bytes, ws_whole), dtype=torch.uint8, device=dev)
    whole_out = [torch.empty_like(u) for u in whole]
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    print(f"# {w.name}: {len(shapes)} matrices in {k} shards each, workspace {ws_bytes / 2**30:.2f} GiB",
          file=sys.stderr, flush=True)

    def timed(fn, steps):
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / steps

    def sharded():
        dm.dmuon_orthogonalize_sharded(ins, outs, splits, workspace=workspace, **nshp)

    def unsharded():
        dm.dmuon_orthogonalize(whole, whole_out, workspace=workspace, **nshp)

    for _ in range(args.warmup):
        sharded()
        unsharded()
    torch.cuda.synchronize()
    ms_whole = timed(unsharded, max(1, args.steps // 2))
    dm.dmuon_profile_begin()
    ms_step = timed(sharded, args.steps)
    prof = dm.dmuon_profile_end()["kernels"]
    print(f"# sharded {ms_step:.3f} ms, unsharded {ms_whole:.3f} ms per call", file=sys.stderr, flush=True)

    flops = nominal_flops(shapes, hp["ns_steps"])
    peak = PEAK_BF16_TFLOPS if args.ns_precision == "bf16" else PEAK_F32_TFLOPS
    gemm = {key: v for key, v in prof.items() if key.startswith("gemm")}
    dom_name, dom = max(gemm.items(), key=lambda kv: kv[1]["ms"])
    achieved = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
    kernels = {key: {"launches_per_step": v["launches"] / args.steps, "ms_per_step": v["ms"] / args.steps,
                     "tflops": (v["flops"] / (v["ms"] * 1e-3) / 1e12) if v["flops"] else None,
                     "gbs": v["bytes"] / (v["ms"] * 1e-3) / 1e9}
               for key, v in prof.items()}
    out = {
        "metric": TP_METRIC, "value": flops / (ms_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": args.ns_precision,
        "data": "synthetic (seeded normal matrices, generated on device, cut into shards)",
        "config": {"workload": f"{w.name}, {k} tensor-parallel shards per matrix", "matrices": len(shapes),
                   "shards": k * len(shapes), "elements": w.numel, "ns_backend": args.ns_backend,
                   "ns_precision": args.ns_precision, "ns_steps": hp["ns_steps"],
                   "splits": "q, k, v, gate, up: row blocks; o, down: column blocks"},
        "unsharded_ms_per_call": ms_whole,
        "unsharded_tflops_nominal": flops / (ms_whole * 1e-3) / 1e12,
        "kernels": kernels,
        "roofline": {"bound": "mfma", "kernel": dom_name, "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None,
                     "traffic_unit": "HBM bytes per launch", "launches": dom["launches"],
                     "mean_launch_ms": dom["ms"] / dom["launches"],
                     "alg_bytes_per_launch": dom["bytes"] / dom["launches"]},
    }
    if not args.no_cpu_baseline:
        print("# cpu baseline ...", file=sys.stderr, flush=True)
        out["cpu_baseline"] = tp_cpu_baseline(w, k, hp)
    print(json.dumps(out), flush=True)


OWNERS_METRIC = "measured step-time imbalance of the owner shares (max / mean - 1) for a 3B-shaped model"


def run_owners(args, dev):
    """Plan the workload over args.owners owners with every cost model, run
    each owner's share through dmuon_step, and compare the measured share
    times: the imbalance the owners would see as waiting at the next
    collective."""
    import torch
    import dmuon_inputs as di
    import matrix_optimizer_step_owned_amd as dm
    from oracle import owners as oow

    N = args.owners
    w = di.workload(args.workload)
    hp = w.hparams(ns_backend=args.ns_backend, ns_precision=args.ns_precision)
    shapes = [(m.rows, m.cols) for m in w.matrices]
    pdt = torch.bfloat16 if w.param_dtype == "bf16" else torch.float32
    gdt = torch.bfloat16 if w.grad_dtype == "bf16" else torch.float32
    params, grads, moms = [], [], []
    for i, (r, c) in enumerate(shapes):
        p = torch.empty(r, c, dtype=pdt, device=dev)
        di.torch_normal_(p, w.param_std, seed=1000 + i)
        g = torch.empty(r, c, dtype=gdt, device=dev)
        di.torch_normal_(g, w.grad_std, seed=100000 + i)
        params.append(p)
        grads.append(g)
        moms.append(torch.zeros(r, c, dtype=torch.float32, device=dev))
    plans = {}
    t0 = time.perf_counter()
    reps = 200
    for _ in range(reps):
        for model in ("numel", "ns_nominal", "roofline"):
            plans[model] = dm.dmuon_assign_owners(shapes, N, model, ns_steps=hp["ns_steps"],
                                                  ns_backend=hp["ns_backend"])
    planner_us = (time.perf_counter() - t0) / (3 * reps) * 1e6
    ws_need = 0
    for model, pl in plans.items():
        for q in range(N):
            idx = [i for i, o in enumerate(pl["owner"]) if o == q]
            if idx:
                ws_need = max(ws_need, dm.dmuon_step_workspace_size([params[i] for i in idx], [grads[i] for i in idx],
                                                                   [moms[i] for i in idx], **hp))
    workspace = torch.empty(ws_need, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    print(f"# {w.name} over {N} owners; planner {planner_us:.1f} us per plan", file=sys.stderr, flush=True)

    def share_ms(idx):
        if not idx:
            return 0.0
        sub = ([params[i] for i in idx], [grads[i] for i in idx], [moms[i] for i in idx])
        for _ in range(args.warmup):
            dm.dmuon_step(*sub, workspace=workspace, **hp)
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for _ in range(args.steps):
            dm.dmuon_step(*sub, workspace=workspace, **hp)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / args.steps

    dm.dmuon_profile_begin()
    results = {}
    for model, pl in plans.items():
        ms = [share_ms([i for i, o in enumerate(pl["owner"]) if o == q]) for q in range(N)]
        mean = sum(ms) / N
        results[model] = {"predicted_imbalance": pl["imbalance"], "measured_imbalance": max(ms) / mean - 1,
                          "share_ms": ms, "matrices_per_owner": [pl["owner"].count(q) for q in range(N)]}
        print(f"# {model}: predicted {pl['imbalance']:.4f}, measured {max(ms) / mean - 1:.4f}, "
              f"max share {max(ms):.2f} ms", file=sys.stderr, flush=True)
    prof = dm.dmuon_profile_end()["kernels"]
    gemm = {key: v for key, v in prof.items() if key.startswith("gemm")}
    dom_name, dom = max(gemm.items(), key=lambda kv: kv[1]["ms"])
    peak = PEAK_BF16_TFLOPS if args.ns_precision == "bf16" else PEAK_F32_TFLOPS
    achieved = dom["flops"] / (dom["ms"] * 1e-3) / 1e12
    best = results["roofline"]
    out = {
        "metric": OWNERS_METRIC, "value": best["measured_imbalance"], "unit": "fraction",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": max(best["share_ms"]),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": args.ns_precision,
        "data": "synthetic (seeded normal params and grads, generated on device)",
        "config": {"workload": f"{w.name} over {N} owners", "matrices": len(shapes), "owners": N,
                   "cost_model": "roofline", "ns_backend": args.ns_backend, "ns_precision": args.ns_precision},
        "models": results, "planner_us_per_plan": planner_us,
        "roofline": {"bound": "mfma", "kernel": dom_name, "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": None, "traffic_unit": "HBM bytes per launch",
                     "launches": dom["launches"], "mean_launch_ms": dom["ms"] / dom["launches"],
                     "alg_bytes_per_launch": dom["bytes"] / dom["launches"]},
    }
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        n_plans = 0
        while time.perf_counter() - t0 < 10.0:
            oow.plan(shapes, N, "roofline", hp["ns_steps"], hp["ns_backend"])
            n_plans += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": n_plans / dt, "unit": "plans/s", "cores": 1, "kind": "oracle",
                               "sample": f"the pure-Python planner oracle on the {len(shapes)} shapes, "
                                         f"{n_plans} plans in {dt:.1f} s (the library's planner: "
                                         f"{1e6 / planner_us:.0f} plans/s)"}
    print(json.dumps(out), flush=True)


def adamw_cpu_baseline(budget_s=60.0, min_s=10.0):
    """The AdamW oracle timed on this host on 2^22-element slices of the
    group until ``min_s`` seconds are timed; parameter bytes (bf16) per
    second over the algorithmic 22 bytes per element."""
    import numpy as np
    from oracle import adamw as oad
    rng = np.random.default_rng(0)
    n = 1 << 22
    p = rng.standard_normal(n) * 0.02
    g = rng.standard_normal(n) * 1e-3
    m = np.zeros(n)
    v = np.zeros(n)
    t0 = time.time()
    timed, done, step = 0.0, 0, 1
    while timed < min_s and time.time() - t0 < budget_s:
        s0 = time.perf_counter()
        p_new, m, v = oad.adamw_step(p, g, m, v, step)
        oad.store(p_new, "bf16")
        timed += time.perf_counter() - s0
        done += n
        step += 1
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": done * 22 / timed / 1e9, "unit": "GB/s (22 bytes per element)", "cores": 1,
            "kind": "oracle",
            "sample": f"float64 numpy oracle, {step - 1} steps of a 2^22-element slice "
                      f"({done / 1e6:.0f} M elements, {timed:.1f} s timed; numpy elementwise, one thread of {cores})"}


def run_adamw(args, dev):
    """Fused AdamW over the symmetric group of a 3B-shaped model; a step is
    one dmuon_adamw_step call over every tensor."""
    import torch
    import dmuon_inputs as di
    import matrix_optimizer_step_owned_amd as dm

    params, grads, ms, vs = [], [], [], []
    for i, s in enumerate(ADAMW_SHAPES):
        p = torch.empty(s, dtype=torch.bfloat16, device=dev)
        di.torch_normal_(p, 0.02, seed=40000 + i)
        g = torch.empty(s, dtype=torch.bfloat16, device=dev)
        di.torch_normal_(g, 1e-3, seed=50000 + i)
        params.append(p)
        grads.append(g)
        ms.append(torch.zeros(s, dtype=torch.float32, device=dev))
        vs.append(torch.zeros(s, dtype=torch.float32, device=dev))
    numel = sum(p.numel() for p in params)
    alg_bytes = numel * 22
    workspace = torch.empty(dm.dmuon_adamw_workspace_size(len(params)), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    step = 1
    for _ in range(args.warmup):
        dm.dmuon_adamw_step(params, grads, ms, vs, step=step, workspace=workspace)
        step += 1
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    dm.dmuon_profile_begin()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(args.steps):
        dm.dmuon_adamw_step(params, grads, ms, vs, step=step, workspace=workspace)
        step += 1
    end.record(stream)
    torch.cuda.synchronize()
    prof = dm.dmuon_profile_end()["kernels"]
    ms_step = start.elapsed_time(end) / args.steps
    if args.copy_probe:
        copy_probe(dev)
    dom = prof["adamw"]
    achieved = dom["bytes"] / (dom["ms"] * 1e-3) / 1e9
    out = {
        "metric": ADAMW_METRIC, "value": alg_bytes / (ms_step * 1e-3) / 1e9, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32 (bf16 params and grads, fp32 moments)",
        "data": "synthetic (seeded normal params and grads, generated on device)",
        "config": {"workload": "3B AdamW group: 128256 x 3072 embedding + 57 RMSNorm weights of 3072",
                   "tensors": len(params), "elements": numel, "alg_bytes_per_step": alg_bytes,
                   "lr": 1e-3, "betas": [0.9, 0.999], "eps": 1e-8, "weight_decay": 0.01},
        "elements_per_s": numel / (ms_step * 1e-3),
        "roofline": {"bound": "hbm", "kernel": "adamw", "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                     "traffic": read_traffic(ADAMW_TRAFFIC_SUMMARY, ADAMW_SOURCE),
                     "traffic_unit": "HBM bytes per launch", "launches": dom["launches"],
                     "mean_launch_ms": dom["ms"] / dom["launches"],
                     "alg_bytes_per_launch": dom["bytes"] / dom["launches"]},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = adamw_cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
