#!/usr/bin/env python3
"""Benchmark of the batched gesv hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME|all]

A step is one batched gesv (factor + forward + back substitution of every
matrix of the batch; for the n = 1024 workload getrf then getrs) on synthetic
inputs already resident in HBM; the Cholesky workloads time one batched posv
(potrf + both triangular solves) the same way.  The factorisation is in place, so every step
runs on its own pre-copied input set, and the sets rotate through enough
bytes that they cannot all sit in the 256 MB last-level cache; copies happen
outside the timed regions.

One JSON line.  The headline (``value``) is sgesv n = 32, nrhs = 8,
batch 32768: K steps bracketed by a synchronisation on both sides, wall
clock.  ``workloads`` carries every workload of the metric, each with the
median per-step time over at least 7 event-timed steps, the back-to-back
rate, the roofline of its dominant kernel and the oracle's host rate on all
cores and on one core.
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
FP32_MFMA_PEAK_TFLOPS = 157.3
FP64_PEAK_TFLOPS = 78.6
METRIC = "batched gesv matrices/s + GFLOP/s (n=32 f32, n=256 f64), % of roofline"
HEADLINE = "sgesv_n32_r8_b32768"
ORDER = ["sgesv_n16_b1024", "sgesv_n32_r8_b32768", "cgesv_n64_r16_b8192", "dgesv_n256_b1024",
         "sgetrf_sgetrs_n1024_r32_b64", "sposv_n32_r8_b32768", "cposv_n64_r16_b8192", "dposv_n256_b1024",
         "sgetrf_m512_n128_b2048", "sgesv_vbatched_n16_256_r1_b4096"]
ALL_WORKLOADS = {**lu_inputs.WORKLOADS, **lu_inputs.CHOL_WORKLOADS, **lu_inputs.RECT_WORKLOADS,
                 **lu_inputs.VBATCH_WORKLOADS}
ROTATE_BYTES = 320 << 20          # in-place input bytes the rotating sets span at least
MAX_SETS = 600
# sources of the kernel whose HBM counters a workload's summary records
# (the summary is used only while these sources are unchanged)
_C = "dense_linear_algebra_amd/csrc/"
KERNEL_SOURCES = {
    "sgesv_n16_b1024": [_C + "register_lu_row16.h", _C + "device_ops.h"],
    "sgesv_n32_r8_b32768": [_C + "register_lu_row16.h", _C + "device_ops.h"],
    "cgesv_n64_r16_b8192": [_C + "register_lu_kernel.h", _C + "device_ops.h"],
    "dgesv_n256_b1024": [_C + "blocked_fused.hip", _C + "device_ops.h"],
    "sgetrf_sgetrs_n1024_r32_b64": [_C + "blocked_lu_impl.h", _C + "device_ops.h"],
    "sposv_n32_r8_b32768": [_C + "chol_kernels.h"],
    "cposv_n64_r16_b8192": [_C + "chol_kernels.h"],
    "dposv_n256_b1024": [_C + "chol_kernels.h"],
}


def is_chol(w) -> bool:
    return w.op == "posv"


def algorithmic_bytes(w) -> int:
    """LU: A read and written, B read and X written, ipiv and info written.
    Cholesky: the named triangle (n(n+1)/2 entries) read and written, B read
    and X written, info written."""
    es = np.dtype(w.dtype).itemsize
    if is_chol(w):
        return es * (w.n * (w.n + 1) + 2 * w.n * w.nrhs) + 4
    return es * (2 * w.n * w.n + 2 * w.n * w.nrhs) + 4 * w.n + 4


def algorithmic_flops(w) -> float:
    """LU 2/3 n^3 + 2 n^2 nrhs, Cholesky 1/3 n^3 + 2 n^2 nrhs per matrix;
    complex counts 4 real flops per operation."""
    f = (1.0 if is_chol(w) else 2.0) / 3.0 * w.n ** 3 + 2.0 * w.n ** 2 * w.nrhs
    return f * (4.0 if np.dtype(w.dtype).kind == "c" else 1.0)


def getrf_flops(w) -> float:
    """Flops of the factorisation alone (getrf 2/3 n^3, potrf 1/3 n^3)."""
    return (1.0 if is_chol(w) else 2.0) / 3.0 * w.n ** 3 * (4.0 if np.dtype(w.dtype).kind == "c" else 1.0)


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
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if workload not in KERNEL_SOURCES or not os.path.exists(path):
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
    """(kernel name, counter value) per dispatch of one rocprofv3 --pmc
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
    copy_mb MiB that the same run made first (bench.py --copy-probe-mb).
    For a workload whose step is several launches, `kernel` is the dominant
    one and the bytes are per launch of it."""
    w = ALL_WORKLOADS[workload]
    res = {"kernel": kernel, "workload": workload, "source_hash": source_hash(workload), "commands": list(commands)}
    # several kernels may be named, separated by '|': their bytes are summed
    # and divided by the dispatches of the first one (e.g. the launches of one
    # blocked getrf per dispatch of its final interchange kernel)
    names = kernel.split("|")
    per = {}
    for tag, db in (("fetch", fetch_db), ("write", write_db)):
        rows = _counter_rows(db)
        copies = [v for n, v in rows.values() if n.startswith("__amd_rocclr_copyBuffer")]
        mine = [v for n, v in rows.values() if any(k in n for k in names)]
        units = [v for n, v in rows.values() if names[0] in n]
        if not copies or not units:
            raise SystemExit(f"{db}: no copy probe or no '{names[0]}' dispatch")
        per[tag] = (sum(mine) / len(units), max(copies))
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


def kernel_counter_table(dbs):
    """Per kernel: dispatches and the mean of every counter per dispatch, from
    one or more rocprofv3 --pmc databases; with the SQ busy counters also the
    derived MFMA and VALU utilisation.  rocprofv3 reports a counter summed
    over the GPU's instances, so GRBM_GUI_ACTIVE (per XCD) is divided by the
    8 XCDs, as its 'max' reduction in the derived metrics assumes.  Printed
    as a markdown table."""
    import csv
    import subprocess
    import tempfile
    per = {}
    for db in dbs:
        out = os.path.join(tempfile.mkdtemp(), "csv")
        subprocess.run(["/opt/rocm/bin/rocpd2csv", "-i", os.path.abspath(db), "-d", out], check=True,
                       capture_output=True, cwd="/tmp")
        with open(os.path.join(out, "out_counter_collection_trace.csv")) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("batchlu::", "")
                name = name[5:] if name.startswith("void ") else name
                name = name.split("(")[0]
                d = per.setdefault(name, {})
                d.setdefault(r["Counter_Name"], {})[(db, r["Dispatch_Id"])] = float(r["Counter_Value"])
    cols = sorted({c for d in per.values() for c in d})
    derived = {"GRBM_GUI_ACTIVE", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU"} <= set(cols)
    head = ["kernel", "dispatches"] + cols + (["MFMA busy %", "VALU busy %"] if derived else [])
    print("| " + " | ".join(head) + " |")
    print("|" + "---|" * len(head))
    for name, d in sorted(per.items()):
        k = max(len(v) for v in d.values())
        mean = {c: (sum(d[c].values()) / len(d[c]) if c in d else float("nan")) for c in cols}
        row = [f"`{name}`", str(k)] + [f"{mean[c]:.4g}" for c in cols]
        if derived:
            g = mean["GRBM_GUI_ACTIVE"] / 8.0
            row += [f"{100.0 * mean['SQ_VALU_MFMA_BUSY_CYCLES'] / (g * 1024):.1f}",
                    f"{100.0 * mean['SQ_ACTIVE_INST_VALU'] / 256 / g:.1f}"]
        print("| " + " | ".join(row) + " |")


def kernel_trace_table(db):
    """Per kernel: calls, total ms, mean and median us and share of the
    kernel time in one rocprofv3 --kernel-trace database (markdown)."""
    import csv
    import subprocess
    import tempfile
    out = os.path.join(tempfile.mkdtemp(), "csv")
    subprocess.run(["/opt/rocm/bin/rocpd2csv", "-i", os.path.abspath(db), "-d", out], check=True,
                   capture_output=True, cwd="/tmp")
    per = {}
    with open(os.path.join(out, "out_kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").replace("batchlu::", "")
            name = name[5:] if name.startswith("void ") else name
            name = name.split("(")[0]
            per.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    total = sum(sum(v) for v in per.values())
    print("| kernel | calls | total ms | mean us | median us | % |")
    print("|---|---|---|---|---|---|")
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        print(f"| `{name}` | {len(v)} | {sum(v) * 1e-3:.3f} | {np.mean(v):.2f} | {np.median(v):.2f} | "
              f"{100.0 * sum(v) / total:.1f} |")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on host cores
# ---------------------------------------------------------------------------

def _oracle_step(w, A, B, m, nthreads):
    import oracle
    n, r = w.n, w.nrhs
    a = A[: m * n * n].copy()
    b = B[: m * n * r].copy()
    t0 = time.perf_counter()
    if is_chol(w):
        _, used = oracle.posv(a, n, n, n * n, b, r, n, n * r, m, nthreads=nthreads)
    elif w.op == "gesv":
        _, _, _, used = oracle.gesv(a, n, n, n * n, b, r, n, n * r, m, nthreads=nthreads)
    else:
        ipiv, _, _, used = oracle.getrf(a, n, n, n * n, m, nthreads=nthreads)
        oracle.getrs(a, n, n, n * n, ipiv, b, r, n, n * r, m, nthreads=nthreads)
    return time.perf_counter() - t0, int(used)


def _oracle_rate(w, A, B, nthreads, min_run_s):
    """Matrices/s of the oracle on the first m matrices (m doubled until one
    run takes min_run_s or the batch is used up), median of 3 runs."""
    m = 1 if nthreads == 1 else min(w.batch, os.cpu_count() or 1)
    while True:
        dt, used = _oracle_step(w, A, B, m, nthreads)
        if dt >= min_run_s or m >= w.batch:
            break
        m = min(w.batch, m * 2)
    times = sorted([dt] + [_oracle_step(w, A, B, m, nthreads)[0] for _ in range(2)])
    return m / times[1], used, m, times[1]


def cpu_baseline(w, A, B, min_run_s):
    all_rate, used, m_all, t_all = _oracle_rate(w, A, B, 0, min_run_s)
    one_rate, _, m_one, t_one = _oracle_rate(w, A, B, 1, min_run_s)
    return {"value": all_rate, "unit": "matrices/s", "cores": used, "kind": "oracle",
            "sample": f"median of 3 runs of the oracle's {w.op} on the first {m_all} matrices of the batch "
                      f"({t_all:.2f} s each, {used} threads)",
            "single_core": {"value": one_rate, "unit": "matrices/s", "cores": 1,
                            "sample": f"median of 3 runs on the first {m_one} matrices ({t_one:.2f} s each)"}}


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

class Runner:
    """Input sets of one workload on the device and the calls that time them."""

    def __init__(self, lib, torch, w, nsets):
        self.lib, self.torch, self.w = lib, torch, w
        dev = torch.device("cuda:0")
        A, B = lu_inputs.chol_problem(w) if is_chol(w) else lu_inputs.dense_problem(w)
        self.hA, self.hB = A, B
        self.pA = torch.from_numpy(A).to(dev)
        self.pB = torch.from_numpy(B).to(dev)
        self.sets = [(self.pA.clone(), self.pB.clone()) for _ in range(nsets)]
        self.ipiv = torch.empty(w.batch * w.n, dtype=torch.int32, device=dev)
        self.info = torch.empty(w.batch, dtype=torch.int32, device=dev)
        self.t = lib.dtype_code(A.dtype)
        self.stream = torch.cuda.current_stream()
        self.dev = dev

    def restore(self, k=None):
        for dA, dB in self.sets[: k]:
            dA.copy_(self.pA)
            dB.copy_(self.pB)
        self.torch.cuda.synchronize()

    def step(self, i):
        w, lib, t = self.w, self.lib, self.t
        dA, dB = self.sets[i % len(self.sets)]
        n, r = w.n, w.nrhs
        if is_chol(w):
            lib.batchlu_posv(t, "L", n, r, dA, n, n * n, dB, n, n * r, self.info, w.batch, stream=self.stream)
        elif w.op == "gesv":
            lib.batchlu_gesv(t, n, r, dA, n, n * n, self.ipiv, n, dB, n, n * r, self.info, w.batch,
                             stream=self.stream)
        else:
            lib.batchlu_getrf(t, n, dA, n, n * n, self.ipiv, n, self.info, w.batch, stream=self.stream)
            lib.batchlu_getrs(t, "N", n, r, dA, n, n * n, self.ipiv, n, dB, n, n * r, w.batch, stream=self.stream)

    def timed_each(self, fn, reps):
        """HIP events around each of `reps` calls of fn(i) on the launch
        stream; per-call milliseconds."""
        torch = self.torch
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for i, (e0, e1) in enumerate(evs):
            e0.record(self.stream)
            fn(i)
            e1.record(self.stream)
        torch.cuda.synchronize()
        return [e0.elapsed_time(e1) for e0, e1 in evs]

    def back_to_back(self, first, k):
        """k steps on sets first .. first+k-1 between two synchronisations:
        (wall ms per step, event ms per step)."""
        torch = self.torch
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(self.stream)
        for i in range(first, first + k):
            self.step(i)
        e1.record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall * 1e3 / k, e0.elapsed_time(e1) / k

    def free(self):
        del self.sets, self.pA, self.pB
        self.torch.cuda.empty_cache()


def nsets_for(w, k):
    per = np.dtype(w.dtype).itemsize * w.n * (w.n + w.nrhs) * w.batch
    return int(min(MAX_SETS, max(k, -(-ROTATE_BYTES // per))))


def parity_sample(r, k):
    """LU of the first k matrices of set 0 (just factorised) against the
    oracle, bit for bit."""
    import oracle
    w = r.w
    n = w.n
    a0 = r.hA[: k * n * n].copy()
    b0 = r.hB[: k * n * w.nrhs].copy()
    gA0 = r.sets[0][0][: k * n * n].cpu().numpy()
    if is_chol(w):
        oracle.posv(a0, n, n, n * n, b0, w.nrhs, n, n * w.nrhs, k)
        return {"sampled_matrices": k, "factor_bitwise_equal": bool(np.array_equal(gA0.view(np.uint8),
                                                                                   a0.view(np.uint8)))}
    oracle.gesv(a0, n, n, n * n, b0, w.nrhs, n, n * w.nrhs, k)
    return {"sampled_matrices": k, "lu_bitwise_equal": bool(np.array_equal(gA0.view(np.uint8), a0.view(np.uint8)))}


def measure(lib, torch, w, steps, warmup, cpu_s, with_cpu):
    """Every figure of one workload; the dict that goes into the line."""
    reps = max(7, steps)
    nsets = nsets_for(w, max(reps, warmup + steps))
    r = Runner(lib, torch, w, nsets)
    op = 4 if is_chol(w) else (2 if w.op == "gesv" else 0)
    tier = lib.batchlu_select_tier(r.t, op, w.n, w.nrhs, w.batch)
    for i in range(warmup):
        r.step(i)
    torch.cuda.synchronize()
    parity = parity_sample(r, 2 if w.n >= 512 else min(16, w.batch)) if warmup > 0 else None
    r.restore()
    wall_ms, b2b_ms = r.back_to_back(0, min(steps, nsets))
    r.restore()
    each = r.timed_each(r.step, reps)
    med = float(np.median(each))
    mean = float(np.mean(each))
    bytes_launch = algorithmic_bytes(w) * w.batch
    out = {"n": w.n, "nrhs": w.nrhs, "batch": w.batch, "dtype": np.dtype(w.dtype).name, "op": w.op,
           "tier": lib.TIER_NAMES.get(tier, str(tier)), "input_sets": nsets,
           "rotated_bytes": int(np.dtype(w.dtype).itemsize * w.n * (w.n + w.nrhs) * w.batch * nsets),
           "step_ms_median": med, "step_ms_mean": mean, "step_ms_back_to_back": b2b_ms,
           "wall_ms_per_step": wall_ms, "reps": reps,
           "matrices_per_s": w.batch / (med * 1e-3), "matrices_per_s_back_to_back": w.batch / (b2b_ms * 1e-3),
           "gflops": algorithmic_flops(w) * w.batch / (med * 1e-3) / 1e9, "parity": parity}
    if tier in (lib.TIER_TINY, lib.TIER_CTA):
        # one launch per step: the step is the dominant kernel
        gbs = bytes_launch / (mean * 1e-3) / 1e9
        out["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "traffic": traffic_from_profile(w.name),
                           "kernel_ms_mean": mean, "kernel_ms_median": med,
                           "algorithmic_bytes_per_launch": bytes_launch}
    else:
        # blocked tier: the factorisation is the dominant part; timed on its
        # own (fresh copies of the same inputs) against the FP roof
        peak = FP64_PEAK_TFLOPS if np.dtype(w.dtype) in (np.float64, np.complex128) else FP32_MFMA_PEAK_TFLOPS
        n = w.n
        r.restore()
        if is_chol(w):
            g = r.timed_each(lambda i: lib.batchlu_potrf(r.t, "L", n, r.sets[i % nsets][0], n, n * n, r.info,
                                                         w.batch, stream=r.stream), reps)
        else:
            g = r.timed_each(lambda i: lib.batchlu_getrf(r.t, n, r.sets[i % nsets][0], n, n * n, r.ipiv, n, r.info,
                                                         w.batch, stream=r.stream), reps)
        gmed, gmean = float(np.median(g)), float(np.mean(g))
        fl = getrf_flops(w) * w.batch
        tf = fl / (gmean * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": tf, "peak": peak, "unit": "TFLOP/s", "frac": tf / peak,
                           "traffic": traffic_from_profile(w.name), "kernel_ms_mean": gmean,
                           "kernel_ms_median": gmed, "algorithmic_flops_per_launch": fl,
                           "scope": ("batchlu_potrf" if is_chol(w) else "batchlu_getrf") + " (every launch it makes)"}
        if w.op == "getrf+getrs":
            # the solve and the inverse on the factors of the last getrf
            es = np.dtype(w.dtype).itemsize
            dA = r.sets[(reps - 1) % nsets][0].clone()   # the factors that r.ipiv belongs to
            solve_bytes = es * (n * n + 2 * n * w.nrhs) * w.batch + 4 * n * w.batch
            solve = {"algorithmic_bytes_per_launch": solve_bytes}
            for tr in ("N", "T"):
                for _, dB in r.sets:
                    dB.copy_(r.pB)
                ms = r.timed_each(lambda i: lib.batchlu_getrs(r.t, tr, n, w.nrhs, dA, n, n * n, r.ipiv, n,
                                                              r.sets[i % nsets][1], n, n * w.nrhs, w.batch,
                                                              stream=r.stream), reps)
                m = float(np.median(ms))
                solve[tr] = {"ms_median": m, "GB/s": solve_bytes / (m * 1e-3) / 1e9}
            out["getrs"] = solve
            dC = torch.empty(w.batch * n * n, dtype=dA.dtype, device=r.dev)
            inv_bytes = 2 * es * n * n * w.batch + 4 * n * w.batch
            ms = r.timed_each(lambda i: lib.batchlu_getri(r.t, n, dA, n, n * n, r.ipiv, n, dC, n, n * n, w.batch,
                                                          stream=r.stream), max(3, min(reps, 7)))
            m = float(np.median(ms))
            out["getri"] = {"ms_median": m, "algorithmic_bytes_per_launch": inv_bytes,
                            "GB/s": inv_bytes / (m * 1e-3) / 1e9,
                            "TFLOP/s": 4.0 / 3.0 * n ** 3 * w.batch / (m * 1e-3) / 1e12}
            del dC, dA
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(w, r.hA, r.hB, cpu_s)
    r.free()
    return out


# ---------------------------------------------------------------------------
# rectangular and variable-size LU (one work-group per matrix, VALU)
# ---------------------------------------------------------------------------

FP32_VALU_PEAK_TFLOPS = 157.3


def _timed(torch, fn, reps, stream):
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        fn(i)
        e1.record(stream)
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def rect_flops(m, n):
    """m n^2 - n^3/3 (m >= n), else n m^2 - m^3/3, less the lower-order terms."""
    k, big = min(m, n), max(m, n)
    return big * k * k - k ** 3 / 3.0


def measure_rect(lib, torch, w, steps, warmup, cpu_s, with_cpu):
    import oracle
    m, n = lu_inputs.RECT_ROWS[w.name], w.n
    rng = np.random.Generator(np.random.PCG64(w.seed))
    A = lu_inputs.draw(rng, w.dtype, w.batch * m * n)
    es = np.dtype(w.dtype).itemsize
    reps = max(7, steps)
    nsets = int(min(MAX_SETS, max(reps + warmup, -(-ROTATE_BYTES // (es * m * n * w.batch)))))
    dev = torch.device("cuda:0")
    pA = torch.from_numpy(A).to(dev)
    sets = [pA.clone() for _ in range(nsets)]
    k = min(m, n)
    ipiv = torch.empty(w.batch * k, dtype=torch.int32, device=dev)
    info = torch.empty(w.batch, dtype=torch.int32, device=dev)
    t = lib.dtype_code(A.dtype)
    stream = torch.cuda.current_stream()
    step = lambda i: lib.batchlu_getrf_rect(t, m, n, sets[i % nsets], m, m * n, ipiv, k, info, w.batch,  # noqa
                                            stream=stream)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    a0 = A[: 2 * m * n].copy()
    oracle.getrf_rect(a0, m, n, m, m * n, 2)
    parity = {"sampled_matrices": 2,
              "lu_bitwise_equal": bool(np.array_equal(sets[0][: 2 * m * n].cpu().numpy().view(np.uint8),
                                                      a0.view(np.uint8)))}
    for s_ in sets:
        s_.copy_(pA)
    ms = _timed(torch, step, reps, stream)
    med, mean = float(np.median(ms)), float(np.mean(ms))
    fl = rect_flops(m, n) * w.batch
    tf = fl / (mean * 1e-3) / 1e12
    out = {"m": m, "n": n, "batch": w.batch, "dtype": np.dtype(w.dtype).name, "op": "getrf_rect",
           "tier": "general", "input_sets": nsets, "step_ms_median": med, "step_ms_mean": mean, "reps": reps,
           "matrices_per_s": w.batch / (med * 1e-3), "gflops": fl / (med * 1e-3) / 1e9, "parity": parity,
           "roofline": {"bound": "alu", "achieved": tf, "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tf / FP32_VALU_PEAK_TFLOPS, "traffic": None, "kernel_ms_mean": mean,
                        "kernel_ms_median": med, "algorithmic_flops_per_launch": fl,
                        "scope": "batchlu_getrf_rect (one launch)"}}
    if with_cpu:
        def run(mm, nt):
            a = A[: mm * m * n].copy()
            t0 = time.perf_counter()
            _, _, _, used = oracle.getrf_rect(a, m, n, m, m * n, mm, nthreads=nt)
            return time.perf_counter() - t0, used
        out["cpu_baseline"] = _bounded_oracle_rate(run, w.batch, cpu_s, "getrf_rect")
    del sets, pA
    torch.cuda.empty_cache()
    return out


def _bounded_oracle_rate(run, batch, cpu_s, what):
    """Matrices/s of run(m, threads) on the first m matrices (m doubled until
    one run takes cpu_s), median of 3, on all cores and on one."""
    res = {}
    for nt in (0, 1):
        mm = 1 if nt == 1 else min(batch, os.cpu_count() or 1)
        while True:
            dt, used = run(mm, nt)
            if dt >= cpu_s or mm >= batch:
                break
            mm = min(batch, mm * 2)
        times = sorted([dt] + [run(mm, nt)[0] for _ in range(2)])
        res[nt] = (mm / times[1], used, mm, times[1])
    all_rate, used, m_all, t_all = res[0]
    one_rate, _, m_one, t_one = res[1]
    return {"value": all_rate, "unit": "matrices/s", "cores": used, "kind": "oracle",
            "sample": f"median of 3 runs of the oracle's {what} on the first {m_all} matrices ({t_all:.2f} s each)",
            "single_core": {"value": one_rate, "unit": "matrices/s", "cores": 1,
                            "sample": f"median of 3 runs on the first {m_one} matrices ({t_one:.2f} s each)"}}


def measure_vbatch(lib, torch, w, steps, warmup, cpu_s, with_cpu):
    import oracle
    orders, A, B, aoff, boff = lu_inputs.vbatch_problem(w)
    es = np.dtype(w.dtype).itemsize
    reps = max(7, steps)
    per_set = es * (A.size + B.size)
    nsets = int(min(MAX_SETS, max(reps + warmup, -(-ROTATE_BYTES // per_set))))
    dev = torch.device("cuda:0")
    pA, pB = torch.from_numpy(A).to(dev), torch.from_numpy(B).to(dev)
    sets = [(pA.clone(), pB.clone()) for _ in range(nsets)]
    dn = torch.from_numpy(orders).to(dev)
    dr = torch.full((w.batch,), w.nrhs, dtype=torch.int32, device=dev)
    maxn = int(orders.max())
    dpiv = torch.empty(w.batch * maxn, dtype=torch.int32, device=dev)
    pptr = torch.tensor(dpiv.data_ptr() + 4 * maxn * np.arange(w.batch, dtype=np.int64), device=dev)
    info = torch.empty(w.batch, dtype=torch.int32, device=dev)
    ptrs = [(torch.tensor(a.data_ptr() + es * aoff, device=dev), torch.tensor(b.data_ptr() + es * boff, device=dev))
            for a, b in sets]
    t = lib.dtype_code(A.dtype)
    stream = torch.cuda.current_stream()

    def step(i):
        pa, pb = ptrs[i % nsets]
        lib.batchlu_gesv_vbatched(t, dn, dr, pa, dn, pptr, pb, dn, info, maxn, w.batch, stream=stream)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    gA, gB = sets[0][0].cpu().numpy(), sets[0][1].cpu().numpy()
    ok = True
    for b in (0, w.batch // 2, w.batch - 1):
        nb_, sa, sb = int(orders[b]), int(aoff[b]), int(boff[b])
        a, bb = A[sa: sa + nb_ * nb_].copy(), B[sb: sb + nb_ * w.nrhs].copy()
        oracle.gesv(a, nb_, nb_, nb_ * nb_, bb, w.nrhs, nb_, nb_ * w.nrhs, 1)
        ok = ok and np.array_equal(gA[sa: sa + nb_ * nb_].view(np.uint8), a.view(np.uint8)) and \
            np.array_equal(gB[sb: sb + nb_ * w.nrhs].view(np.uint8), bb.view(np.uint8))
    parity = {"sampled_matrices": 3, "lu_and_x_bitwise_equal": bool(ok)}
    for a_, b_ in sets:
        a_.copy_(pA)
        b_.copy_(pB)
    ms = _timed(torch, step, reps, stream)
    med, mean = float(np.median(ms)), float(np.mean(ms))
    o = orders.astype(np.float64)
    fl = float(np.sum(2.0 / 3.0 * o ** 3 + 2.0 * o ** 2 * w.nrhs))
    tf = fl / (mean * 1e-3) / 1e12
    out = {"n_min": int(orders.min()), "n_max": maxn, "n_mean": float(o.mean()), "nrhs": w.nrhs, "batch": w.batch,
           "dtype": np.dtype(w.dtype).name, "op": "gesv_vbatched", "tier": "general", "input_sets": nsets,
           "step_ms_median": med, "step_ms_mean": mean, "reps": reps,
           "matrices_per_s": w.batch / (med * 1e-3), "gflops": fl / (med * 1e-3) / 1e9, "parity": parity,
           "roofline": {"bound": "alu", "achieved": tf, "peak": FP32_VALU_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": tf / FP32_VALU_PEAK_TFLOPS, "traffic": None, "kernel_ms_mean": mean,
                        "kernel_ms_median": med, "algorithmic_flops_per_launch": fl,
                        "scope": "batchlu_gesv_vbatched (factor and solve launches)"}}
    if with_cpu:
        def run(mm, nt):
            t0 = time.perf_counter()
            for b in range(mm):
                nb_, sa, sb = int(orders[b]), int(aoff[b]), int(boff[b])
                a, bb = A[sa: sa + nb_ * nb_].copy(), B[sb: sb + nb_ * w.nrhs].copy()
                oracle.gesv(a, nb_, nb_, nb_ * nb_, bb, w.nrhs, nb_, nb_ * w.nrhs, 1, nthreads=1)
            return time.perf_counter() - t0, 1
        cb = _bounded_oracle_rate(run, w.batch, cpu_s, "gesv, one matrix per call")
        cb["value"], cb["cores"] = cb["single_core"]["value"], 1
        cb["sample"] = cb["single_core"]["sample"] + " (one matrix per call, one host thread)"
        out["cpu_baseline"] = cb
    del sets, pA, pB
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# tier sweep: every tier that can run a shape, timed against the selector
# ---------------------------------------------------------------------------

SWEEP_NS = (8, 16, 32, 33, 48, 64, 96, 128, 256)
SWEEP_BATCHES = (1, 16, 64, 256, 1024, 8192)
SWEEP_NRHS = (1, 16)
TIER_CODES = {"tiny": 1, "cta": 2, "blocked": 3, "cta_lds": 4}


def _sweep_cells(only):
    for dt in (0, 1, 2, 3):
        for n in SWEEP_NS:
            for batch in SWEEP_BATCHES:
                if n * n * batch > 16 << 20:       # keep one input set at most 256 MiB
                    continue
                for nrhs in SWEEP_NRHS:
                    for op in ("gesv", "posv"):
                        if only and (dt, n, batch, nrhs, op) != only:
                            continue
                        yield dt, n, batch, nrhs, op


def tier_sweep(lib, torch, only=None, reps=5):
    """One JSON line per (dtype, n, batch, nrhs, op): the selector's tier and
    the median event time of every tier that can run the shape (pinned with
    batchlu_set_tier), on uniform[-1, 1] (gesv) or SPD (posv) inputs."""
    st = torch.cuda.current_stream()
    dts = {0: np.float32, 1: np.float64, 2: np.complex64, 3: np.complex128}
    for dt, n, batch, nrhs, op in _sweep_cells(only):
        if op == "gesv":
            A, B = lu_inputs.random_problem(n * 131 + batch, dts[dt], n, nrhs, batch)
        else:
            A, B = lu_inputs.dominant_spd_problem(n * 131 + batch, dts[dt], n, nrhs, batch)
        dA0, dB0 = torch.from_numpy(A).cuda(), torch.from_numpy(B).cuda()
        ip = torch.empty(batch * n, dtype=torch.int32, device="cuda")
        inf = torch.empty(batch, dtype=torch.int32, device="cuda")
        code = 2 if op == "gesv" else 4
        lib.batchlu_set_tier(0)
        auto = lib.batchlu_select_tier(dt, code, n, nrhs, batch)
        res = {"dtype": dt, "n": n, "batch": batch, "nrhs": nrhs, "op": op,
               "auto": {v: k for k, v in TIER_CODES.items()}.get(auto, str(auto))}
        for name, tc in TIER_CODES.items():
            lib.batchlu_set_tier(tc)
            if lib.batchlu_select_tier(dt, code, n, nrhs, batch) != tc:
                continue
            sets = [(dA0.clone(), dB0.clone()) for _ in range(reps + 1)]

            def call(i):
                a, b = sets[i]
                if op == "gesv":
                    lib.batchlu_gesv(dt, n, nrhs, a, n, n * n, ip, n, b, n, n * nrhs, inf, batch, stream=st)
                else:
                    lib.batchlu_posv(dt, "L", n, nrhs, a, n, n * n, b, n, n * nrhs, inf, batch, stream=st)
            call(reps)                           # warm-up on the spare set
            res[name + "_ms"] = float(np.median(_timed(torch, call, reps, st)))
            del sets
        lib.batchlu_set_tier(0)
        print(json.dumps(res), flush=True)


def sweep_summary(path, full=False):
    """A tier sweep rendered as markdown: per operation and type, a grid over
    n (rows) and batch (columns) of the selector's tier for nrhs 1 / 16, with
    its time over the fastest tier's where that is above 1.02; then the
    cells where another tier was faster, and the totals.  full=True prints
    every cell's times instead of the grids."""
    rows = [json.loads(line) for line in open(path) if line.startswith("{")]
    tn = {0: "f32", 1: "f64", 2: "c64", 3: "c128"}
    letter = {"tiny": "t", "cta": "c", "cta_lds": "l", "blocked": "b"}
    cells, worst = [], []
    for r in rows:
        t = {k[:-3]: v for k, v in r.items() if k.endswith("_ms")}
        if not t:
            continue
        best = min(t, key=t.get)
        ratio = t.get(r["auto"], float("nan")) / t[best]
        worst.append(ratio)
        cells.append((r, t, best, ratio))
    if full:
        print("| op | type | n | batch | nrhs | selector | fastest | times (ms) | selector / fastest |")
        print("|---|---|---|---|---|---|---|---|---|")
        for r, t, best, ratio in cells:
            print(f"| {r['op']} | {tn[r['dtype']]} | {r['n']} | {r['batch']} | {r['nrhs']} | {r['auto']} | {best} | "
                  + ", ".join(f"{k} {v:.4f}" for k, v in sorted(t.items())) + f" | {ratio:.2f} |")
    else:
        print("Tiers: t = tiny (register), c = cta (register), l = cta_lds (LDS-staged), b = blocked. "
              "Each entry is the selector's tier for nrhs 1 / nrhs 16, with (its time / the fastest "
              "tier's time) where above 1.02.\n")
        grid = {}
        for r, t, best, ratio in cells:
            mark = letter.get(r["auto"], r["auto"]) + (f" ({ratio:.2f})" if ratio > 1.02 else "")
            grid.setdefault((r["op"], r["dtype"]), {}).setdefault((r["n"], r["batch"]), {})[r["nrhs"]] = mark
        for (op, dt), g in grid.items():
            ns = sorted({k[0] for k in g})
            bs = sorted({k[1] for k in g})
            print(f"**{op} {tn[dt]}**\n")
            print("| n \\ batch | " + " | ".join(str(b) for b in bs) + " |")
            print("|---" * (len(bs) + 1) + "|")
            for n in ns:
                ent = []
                for b in bs:
                    c = g.get((n, b), {})
                    ent.append(" / ".join(c[k] for k in sorted(c)) if c else "")
                print(f"| {n} | " + " | ".join(ent) + " |")
            print()
        print("Cells where another tier was more than 2 % faster:\n")
        print("| op | type | n | batch | nrhs | selector | fastest | times (ms) | ratio |")
        print("|---|---|---|---|---|---|---|---|---|")
        for r, t, best, ratio in cells:
            if ratio > 1.02:
                print(f"| {r['op']} | {tn[r['dtype']]} | {r['n']} | {r['batch']} | {r['nrhs']} | {r['auto']} | "
                      f"{best} | " + ", ".join(f"{k} {v:.4f}" for k, v in sorted(t.items())) + f" | {ratio:.2f} |")
    w = np.array(worst)
    print(f"\n{len(w)} cells; selector within 5 % of the fastest tier in {int(np.sum(w <= 1.05))}, "
          f"within 10 % in {int(np.sum(w <= 1.10))}; worst {np.nanmax(w):.2f}, geometric mean "
          f"{float(np.exp(np.nanmean(np.log(w)))):.3f}.")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all", choices=["all"] + sorted(ALL_WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-run-s", type=float, default=0.4, help="least wall time of one timed oracle run")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one plain device copy of this size first (reference for HBM counters)")
    ap.add_argument("--counters-summary", nargs=3, metavar=("KERNEL", "FETCH_DB", "WRITE_DB"),
                    help="write the HBM-traffic summary of KERNEL from two rocprofv3 --pmc databases "
                         "(FETCH_SIZE, WRITE_SIZE) taken with --copy-probe-mb; no GPU needed")
    ap.add_argument("--kernel-counters", nargs="+", metavar="DB",
                    help="print per-kernel means of the counters in rocprofv3 --pmc databases; no GPU needed")
    ap.add_argument("--tier-sweep", action="store_true",
                    help="time every tier that can run each shape of a grid against the selector (JSON lines)")
    ap.add_argument("--sweep-cell", nargs=5, metavar=("DTYPE", "N", "BATCH", "NRHS", "OP"),
                    help="restrict --tier-sweep to one cell (dtype code 0..3, op gesv or posv)")
    ap.add_argument("--sweep-summary", metavar="JSONL", help="render a tier sweep as tables; no GPU needed")
    ap.add_argument("--sweep-full", action="store_true", help="with --sweep-summary: every cell's times")
    ap.add_argument("--trace-summary", metavar="DB",
                    help="print per-kernel times of a rocprofv3 --kernel-trace database; no GPU needed")
    args = ap.parse_args()
    if args.sweep_summary:
        sweep_summary(args.sweep_summary, args.sweep_full)
        return
    if args.trace_summary:
        kernel_trace_table(args.trace_summary)
        return
    if args.kernel_counters:
        kernel_counter_table(args.kernel_counters)
        return
    if args.counters_summary:
        kern, fdb, wdb = args.counters_summary
        mb = args.copy_probe_mb or 256
        base = (f"python3 bench.py --workload {args.workload} --steps 3 --warmup 1 --no-cpu-baseline "
                f"--copy-probe-mb {mb}")
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
    if args.copy_probe_mb > 0:
        src = torch.empty(args.copy_probe_mb << 18, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.tier_sweep:
        only = None
        if args.sweep_cell:
            d, nn, bb, rr, oo = args.sweep_cell
            only = (int(d), int(nn), int(bb), int(rr), oo)
        tier_sweep(lib, torch, only)
        return

    names = ORDER if args.workload == "all" else [args.workload]
    head = HEADLINE if args.workload == "all" else args.workload
    results = {}
    for name in names:
        print(f"# {name}", file=sys.stderr, flush=True)
        wl = ALL_WORKLOADS[name]
        fn = {"getrf_rect": measure_rect, "gesv_vbatched": measure_vbatch}.get(wl.op, measure)
        results[name] = fn(lib, torch, wl, args.steps, args.warmup, args.cpu_run_s, not args.no_cpu_baseline)
    h = results[head]
    w = ALL_WORKLOADS[head]
    ms_per_step = h.get("wall_ms_per_step", h["step_ms_median"])
    cfg = {"workload": head, "op": w.op}
    for key in ("m", "n", "n_min", "n_max", "nrhs", "batch", "tier"):
        if key in h:
            cfg[key] = h[key]
    line = {
        "metric": METRIC,
        "value": w.batch / (ms_per_step * 1e-3),
        "unit": "matrices/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"float32": "f32", "float64": "f64", "complex64": "c64", "complex128": "c128"}[h["dtype"]],
        "data": "synthetic",
        "config": cfg,
        "gflops": h["gflops"] * h["step_ms_median"] / ms_per_step,
        "roofline": h["roofline"],
        "parity": h["parity"],
    }
    if "cpu_baseline" in h:
        line["cpu_baseline"] = h["cpu_baseline"]
    line["workloads"] = results
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
