#!/usr/bin/env python3
"""Benchmark of the batched gesv hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one batched gesv call (factor + forward + back substitution for
every matrix of the batch) on synthetic inputs already resident in HBM.  The
factorisation is in place, so every step gets its own pre-copied input set
(copies happen before the timed region).  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import lu_inputs  # noqa: E402

HBM_PEAK_GBS = 8000.0
FP32_ALU_PEAK_TFLOPS = 78.6     # 256 CU x 64 lanes x 2 flop x 2.4 GHz, no packed FP32
FP32_MFMA_PEAK_TFLOPS = 157.3
FP64_PEAK_TFLOPS = 78.6
METRIC = "batched gesv matrices/s + GFLOP/s (n=32 f32, n=256 f64), % of roofline"
# sources of the kernel whose HBM counters a workload's summary records
# (the summary is used only while these sources are unchanged)
_C = "dense_linear_algebra_amd/csrc/"
KERNEL_SOURCES = {
    "sgesv_n16_b1024": [_C + "register_lu_row16.h", _C + "device_ops.h"],
    "sgesv_n32_r8_b32768": [_C + "register_lu_row16.h", _C + "device_ops.h"],
    "cgesv_n64_r16_b8192": [_C + "register_lu_kernel.h", _C + "device_ops.h"],
    "dgesv_n256_b1024": [_C + "blocked_fused.hip", _C + "device_ops.h"],
}


def algorithmic_bytes(w) -> int:
    """A read and written, B read and X written, ipiv and info written."""
    es = np.dtype(w.dtype).itemsize
    return es * (2 * w.n * w.n + 2 * w.n * w.nrhs) + 4 * w.n + 4


def algorithmic_flops(w) -> float:
    """2/3 n^3 + 2 n^2 nrhs per matrix; complex counts 4 real flops per op."""
    f = 2.0 / 3.0 * w.n ** 3 + 2.0 * w.n ** 2 * w.nrhs
    return f * (4.0 if np.dtype(w.dtype).kind == "c" else 1.0)


def source_hash(workload: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES.get(workload, []):
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per launch of the workload's dominant kernel from the
    committed rocprofv3 counter summary, if it was taken on the current kernel
    source; else None."""
    if workload not in KERNEL_SOURCES:
        return None
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            d = json.load(f)
    except Exception:
        return None
    if d.get("source_hash") != source_hash(workload):
        return None
    return d.get("hbm_bytes_per_launch")


def _counter_rows(db: str):
    """(kernel name, dispatch id, counter value) rows of one rocprofv3 --pmc
    database, read through rocpd2csv."""
    import csv
    import subprocess
    import tempfile
    out = os.path.join(tempfile.mkdtemp(), "csv")
    subprocess.run(["/opt/rocm/bin/rocpd2csv", "-i", os.path.abspath(db), "-d", out], check=True,
                   capture_output=True, cwd="/tmp")
    rows = {}
    with open(os.path.join(out, "out_counter_collection_trace.csv")) as f:
        for r in csv.DictReader(f):
            key = int(r["Dispatch_Id"])
            name, val = r["Kernel_Name"], float(r["Counter_Value"])
            rows[key] = (name, rows.get(key, (name, 0.0))[1] + val)
    return rows


def write_counter_summary(workload: str, kernel: str, fetch_db: str, write_db: str, copy_mb: int, commands):
    """HBM bytes per launch of `kernel` from a FETCH_SIZE and a WRITE_SIZE run,
    each scaled by what the counter reads for the plain device copy of
    copy_mb MiB that the same run made first (bench.py --copy-probe-mb)."""
    w = lu_inputs.WORKLOADS[workload]
    res = {"kernel": kernel, "workload": workload, "source_hash": source_hash(workload), "commands": list(commands)}
    per = {}
    for tag, db in (("fetch", fetch_db), ("write", write_db)):
        rows = _counter_rows(db)
        copies = [v for n, v in rows.values() if n.startswith("__amd_rocclr_copyBuffer")]
        mine = [v for n, v in rows.values() if kernel in n]
        if not copies or not mine:
            raise SystemExit(f"{db}: no copy probe or no '{kernel}' dispatch")
        per[tag] = (sum(mine) / len(mine), max(copies))
    nbytes = copy_mb << 20
    fetch_scale = nbytes / (per["fetch"][1] * 1024.0)
    write_scale = nbytes / (per["write"][1] * 1024.0)
    rd = per["fetch"][0] * 1024.0 * fetch_scale
    wr = per["write"][0] * 1024.0 * write_scale
    alg = algorithmic_bytes(w) * w.batch
    res.update({
        "fetch_size_kib_per_dispatch": per["fetch"][0], "write_size_kib_per_dispatch": per["write"][0],
        "copy_probe": {"bytes_read": nbytes, "bytes_written": nbytes, "fetch_size_kib": per["fetch"][1],
                       "write_size_kib": per["write"][1], "fetch_scale": fetch_scale, "write_scale": write_scale},
        "hbm_bytes_read_per_launch": rd, "hbm_bytes_written_per_launch": wr, "hbm_bytes_per_launch": rd + wr,
        "algorithmic_bytes_per_launch": alg, "traffic_over_algorithmic": (rd + wr) / alg})
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    with open(path, "w") as f:
        json.dump(res, f, indent=1)
    print(path)


def cpu_baseline(w, A, B, budget_s: float = 10.0):
    """The oracle (as is) on host cores: whole-batch gesv repeated until about
    budget_s of wall time has elapsed."""
    import oracle
    reps, used, t_total, mats = 0, 0, 0.0, 0
    while t_total < budget_s and reps < 1000:
        a, b = A.copy(), B.copy()
        t0 = time.perf_counter()
        _, _, _, used = oracle.gesv(a, w.n, w.n, w.n * w.n, b, w.nrhs, w.n, w.n * w.nrhs, w.batch)
        t_total += time.perf_counter() - t0
        reps += 1
        mats += w.batch
    return {"value": mats / t_total, "unit": "matrices/s", "cores": int(used), "kind": "oracle",
            "sample": f"{reps} x the full batch of {w.batch} ({t_total:.1f} s wall)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="sgesv_n32_r8_b32768", choices=sorted(lu_inputs.WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one plain device copy of this size first (reference for HBM counters)")
    ap.add_argument("--counters-summary", nargs=3, metavar=("KERNEL", "FETCH_DB", "WRITE_DB"),
                    help="write the HBM-traffic summary of KERNEL from two rocprofv3 --pmc databases "
                         "(FETCH_SIZE, WRITE_SIZE) taken with --copy-probe-mb; no GPU needed")
    args = ap.parse_args()
    if args.counters_summary:
        kern, fdb, wdb = args.counters_summary
        mb = args.copy_probe_mb or 256
        base = f"python3 bench.py --workload {args.workload} --steps 3 --warmup 1 --no-cpu-baseline --copy-probe-mb {mb}"
        write_counter_summary(args.workload, kern, fdb, wdb, mb,
                              [f"rocprofv3 --pmc FETCH_SIZE -d <dir> -o f -- {base}",
                               f"rocprofv3 --pmc WRITE_SIZE -d <dir> -o w -- {base}"])
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: every matrix is independent, so more GPUs would each "
              f"take batch/{args.gpus} matrices with no communication; --gpus {args.gpus} is not run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import dense_linear_algebra_amd as lib

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    lib.load()
    w = lu_inputs.WORKLOADS[args.workload]
    A, B = lu_inputs.dense_problem(w)
    dev = torch.device("cuda:0")
    t = lib.dtype_code(A.dtype)
    hA = torch.from_numpy(A)
    hB = torch.from_numpy(B)
    nsets = args.warmup + args.steps
    sets = []
    for _ in range(nsets):
        sets.append((hA.to(dev), hB.to(dev)))
    ipiv = torch.empty(w.batch * w.n, dtype=torch.int32, device=dev)
    info = torch.empty(w.batch, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    tier = lib.batchlu_select_tier(t, 2, w.n, w.nrhs, w.batch)

    def step(i):
        dA, dB = sets[i]
        if w.op == "gesv":
            lib.batchlu_gesv(t, w.n, w.nrhs, dA, w.n, w.n * w.n, ipiv, w.n, dB, w.n, w.n * w.nrhs, info, w.batch,
                             stream=stream)
        else:
            lib.batchlu_getrf(t, w.n, dA, w.n, w.n * w.n, ipiv, w.n, info, w.batch, stream=stream)
            lib.batchlu_getrs(t, "N", w.n, w.nrhs, dA, w.n, w.n * w.n, ipiv, w.n, dB, w.n, w.n * w.nrhs, w.batch,
                              stream=stream)

    if args.copy_probe_mb > 0:
        src = torch.empty(args.copy_probe_mb << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # quick parity sample of the first warm-up output against the oracle
    parity = None
    if args.warmup > 0:
        import oracle
        k = min(16, w.batch)
        a0 = A[: k * w.n * w.n].copy()
        b0 = B[: k * w.n * w.nrhs].copy()
        oip, oinfo, _, _ = oracle.gesv(a0, w.n, w.n, w.n * w.n, b0, w.nrhs, w.n, w.n * w.nrhs, k,
                                       nthreads=0)
        gA0 = sets[0][0][: k * w.n * w.n].cpu().numpy()
        parity = {"sampled_matrices": k,
                  "lu_bitwise_equal": bool(np.array_equal(gA0.view(np.uint8), a0.view(np.uint8)))}

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.warmup, nsets):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = ev0.elapsed_time(ev1) / args.steps

    ms_per_step = wall * 1e3 / args.steps
    mats_per_s = w.batch / (ms_per_step * 1e-3)
    bytes_launch = algorithmic_bytes(w) * w.batch
    flops_launch = algorithmic_flops(w) * w.batch
    achieved_gbs = bytes_launch / (kernel_ms * 1e-3) / 1e9
    gflops = flops_launch / (ms_per_step * 1e-3) / 1e9
    kind = "register" if tier in (lib.TIER_TINY, lib.TIER_CTA) else "blocked"
    if kind == "register":
        roof = {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": traffic_from_profile(w.name),
                "kernel_ms": kernel_ms, "algorithmic_bytes_per_launch": bytes_launch}
    else:
        # blocked tier: the factorisation is the dominant part of the step;
        # it is timed on its own (HIP events on the launch stream, fresh
        # copies of the same inputs) against the FP roof, the whole step
        # beside it
        peak = FP64_PEAK_TFLOPS if np.dtype(w.dtype) in (np.float64, np.complex128) else FP32_MFMA_PEAK_TFLOPS
        getrf_ms = []
        for i in range(args.steps):
            dA = sets[i % nsets][0]
            dA.copy_(hA)
            torch.cuda.synchronize()
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            lib.batchlu_getrf(t, w.n, dA, w.n, w.n * w.n, ipiv, w.n, info, w.batch, stream=stream)
            g1.record(stream)
            torch.cuda.synchronize()
            getrf_ms.append(g0.elapsed_time(g1))
        gms = float(np.mean(getrf_ms))
        # the solve on the factors just made, NoTrans and Trans, each timed on
        # its own (fresh B, HIP events on the launch stream); algorithmic
        # bytes: the factors read once, B read and X written
        es = np.dtype(w.dtype).itemsize
        solve_bytes = es * (w.n * w.n + 2 * w.n * w.nrhs) * w.batch + 4 * w.n * w.batch
        solve = {"algorithmic_bytes_per_launch": solve_bytes}
        dA = sets[(args.steps - 1) % nsets][0]
        for tr in ("N", "T"):
            sms = []
            for i in range(args.steps):
                dB = sets[i % nsets][1]
                dB.copy_(hB)
                torch.cuda.synchronize()
                s0 = torch.cuda.Event(enable_timing=True)
                s1 = torch.cuda.Event(enable_timing=True)
                s0.record(stream)
                lib.batchlu_getrs(t, tr, w.n, w.nrhs, dA, w.n, w.n * w.n, ipiv, w.n, dB, w.n, w.n * w.nrhs,
                                  w.batch, stream=stream)
                s1.record(stream)
                torch.cuda.synchronize()
                sms.append(s0.elapsed_time(s1))
            ms = float(np.mean(sms))
            solve[tr] = {"ms": ms, "GB/s": solve_bytes / (ms * 1e-3) / 1e9}
        # getri on the same factors: algorithmic bytes = factors read once,
        # the n x n inverse written
        dC = torch.empty(w.batch * w.n * w.n, dtype=dA.dtype, device=dev)
        inv_bytes = 2 * es * w.n * w.n * w.batch + 4 * w.n * w.batch
        ims = []
        for i in range(args.steps):
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            lib.batchlu_getri(t, w.n, dA, w.n, w.n * w.n, ipiv, w.n, dC, w.n, w.n * w.n, w.batch, stream=stream)
            s1.record(stream)
            torch.cuda.synchronize()
            ims.append(s0.elapsed_time(s1))
        ms = float(np.mean(ims))
        getri = {"ms": ms, "algorithmic_bytes_per_launch": inv_bytes, "GB/s": inv_bytes / (ms * 1e-3) / 1e9,
                 "TFLOP/s": 4.0 / 3.0 * w.n ** 3 * (4.0 if np.dtype(w.dtype).kind == "c" else 1.0) * w.batch
                 / (ms * 1e-3) / 1e12}
        del dC
        getrf_flops = 2.0 / 3.0 * w.n ** 3 * (4.0 if np.dtype(w.dtype).kind == "c" else 1.0) * w.batch
        tf = getrf_flops / (gms * 1e-3) / 1e12
        fused = lib.batchlu_select_tier(t, 0, w.n, 0, w.batch) == lib.TIER_BLOCKED and w.n <= 256 and \
            np.dtype(w.dtype).kind == "f"
        roof = {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s", "frac": tf / peak,
                "traffic": traffic_from_profile(w.name) if fused else None,
                "kernel_ms": gms, "algorithmic_flops_per_launch": getrf_flops,
                "scope": ("batchlu_getrf = one lu_fused_kernel launch" if fused else
                          "batchlu_getrf = its panel, U12-solve, update and interchange launches"),
                "whole_step": {"ms": kernel_ms, "tflops": flops_launch / (kernel_ms * 1e-3) / 1e12},
                "getrs": solve, "getri": getri}
    line = {
        "metric": METRIC,
        "value": mats_per_s,
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"float32": "f32", "float64": "f64", "complex64": "c64", "complex128": "c128"}[np.dtype(w.dtype).name],
        "data": "synthetic",
        "config": {"workload": w.name, "op": w.op, "n": w.n, "nrhs": w.nrhs, "batch": w.batch,
                   "tier": lib.TIER_NAMES.get(tier, str(tier))},
        "gflops": gflops,
        "roofline": roof,
        "parity": parity,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, A, B, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
