#!/usr/bin/env python3
"""Benchmark of the fused FP32 row reductions on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one call of every operator of the workload on one batch of seeded
synthetic input (the default workload: residual LayerNorm, RMSNorm and
softmax on 1024x4096 FP32, inputs U[-1, 1]).  Inputs and outputs are
resident in HBM before timing starts.  Each operator's K timed calls run on
its own rotation of >= 3 buffer sets totalling >= 2 GiB, so no call finds its
data in the 256 MB last-level cache; the K calls are captured in one HIP graph per
operator so the host's launch cost does not gate 5-10 us kernels.  HIP
events on the launch stream bracket each graph replay; an operator's average
call time is its replay time / K.

`value` is the whole step's algorithmic bytes (one read of each input and
one write of the output, 4 B per element each) divided by its time.  The
JSON line also carries the roofline of the dominant kernel, the FP64 CPU
oracle's throughput on host cores, and per-operator figures.

    python bench.py --pmc --all # counter pass: one dispatch of each kernel of
                                # workloads 1..7 on cold buffers, + a 256 MiB
                                # copy per workload for calibration
    python bench.py --all       # one JSON line per core workload (1..5)
    python bench.py --next      # plain and affine LayerNorm, row sum / min-max (6-8)
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import synthetic  # noqa: E402

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, 8 TB/s
METRIC = "HBM GB/s and % of peak, FP32 row LayerNorm/RMSNorm/softmax, µs per call"
POOL_BYTES = 2 * 2 ** 30  # >= 8x the 256 MB last-level cache

# The pages' Apple M1 Max numbers at 1024x4096 (context only, other hardware):
# "Immutable input reuse in Metal reductions", section "Fixed-width GPU and
# dispatch results" (cached-input variant).
M1MAX_CONTEXT_US = {"softmax": 53.949, "rmsnorm": 55.863}

WORKLOAD_NAMES = {
    1: "residual LayerNorm 17x257 + 1x127, U[-1,1]",
    2: "residual LayerNorm + RMSNorm + softmax, 1024x4096, U[-1,1]",
    3: "RMSNorm + softmax, 131072 x {127, 257, 1537}, N(0,1)",
    4: "residual LayerNorm + RMSNorm + softmax, 16384x8192, U[-1,1]",
    5: "softmax stress, 8192x32768, 8*N(0,1) + U[-80,80] row offsets, 1% -inf",
    6: "plain LayerNorm (no residual), 1024x4096 and 16384x8192, U[-1,1]",
    7: "affine LayerNorm (gamma, beta), 1024x4096 and 16384x8192, U[-1,1]",
    8: "row sum and row min/max, 16384x8192 U[-1,1] and 131072x257 N(0,1)",
}
CORE = (1, 2, 3, 4, 5)
NEXT = (6, 7, 8)
WORKLOADS = {**synthetic.CONFIGS, **synthetic.NEXT_CONFIGS}


def n_inputs(op):
    return 2 if op == "layernorm_residual" else 1


def algo_split(case):
    """(read, write) algorithmic bytes: one read of every input element, one
    write of every output element; affine LayerNorm also reads gamma and beta
    once; row sum writes one float per row, row min/max two."""
    rd = 4 * case.rows * case.width * n_inputs(case.op)
    if case.op == "layernorm_affine":
        rd += 8 * case.width
    if case.op in ("row_sum", "row_minmax"):
        return rd, 4 * case.rows * (1 if case.op == "row_sum" else 2)
    return rd, 4 * case.rows * case.width


def algo_bytes(case):
    return sum(algo_split(case))


def kernel_source_hash():
    h = hashlib.sha256()
    for p in ("row_wise_reduction_amd/csrc/rowred_kernels.hip", "row_wise_reduction_amd/csrc/rowred_api.cpp",
              "row_wise_reduction_amd/csrc/rowred_internal.h"):
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# device buffers
# ---------------------------------------------------------------------------

class CaseBuffers:
    """`sets` copies of one case's inputs and outputs, resident on the GPU."""

    def __init__(self, case, sets):
        import torch
        self.case = case
        x = synthetic.case_input(case, "x")
        r = synthetic.case_input(case, "r") if case.op == "layernorm_residual" else None
        self.host_x, self.host_r = x, r
        self.host_g = self.host_b = None
        self.g = self.b = None
        if case.op == "layernorm_affine":
            self.host_g, self.host_b = synthetic.affine_vectors(case)
            self.g = torch.from_numpy(self.host_g).cuda()
            self.b = torch.from_numpy(self.host_b).cuda()
        xd = torch.from_numpy(x).cuda()
        rd = torch.from_numpy(r).cuda() if r is not None else None
        self.x = [xd] + [xd.clone() for _ in range(sets - 1)]
        self.r = ([rd] + [rd.clone() for _ in range(sets - 1)]) if rd is not None else [None] * sets
        if case.op in ("row_sum", "row_minmax"):
            self.y = [torch.empty(case.rows, device="cuda") for _ in range(sets)]
            self.y2 = [torch.empty(case.rows, device="cuda") for _ in range(sets)]
        else:
            self.y = [torch.empty_like(xd) for _ in range(sets)]
        self.sets = sets

    def call(self, i):
        import row_wise_reduction_amd as R
        k = i % self.sets
        op = self.case.op
        if op in ("layernorm", "layernorm_affine"):
            R.rowred_layernorm(self.x[k], None, self.g, self.b, self.y[k], eps=self.case.eps)
        elif op == "row_sum":
            R.rowred_row_sum(self.x[k], self.y[k])
        elif op == "row_minmax":
            R.rowred_row_minmax(self.x[k], self.y[k], self.y2[k])
        else:
            R.run_op(op, self.x[k], self.r[k], self.y[k], eps=self.case.eps)


def rotation_sets(case):
    """Buffer sets for one case: >= 3 and >= 2 GiB of inputs + outputs, so a
    call never finds its operands in the 256 MB last-level cache."""
    return max(3, -(-POOL_BYTES // algo_bytes(case)))


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

def time_workload(cfg, steps, warmup):
    import torch
    cases = WORKLOADS[cfg]
    bufs = [CaseBuffers(c, rotation_sets(c)) for c in cases]
    sets = [b.sets for b in bufs]
    torch.cuda.synchronize()
    for w in range(warmup):
        for b in bufs:
            b.call(w)
    torch.cuda.synchronize()

    # One graph of `steps` calls per case, on rotating buffer sets.
    graphs = []
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        for b in bufs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    b.call(i)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(stream)
    for g in graphs:  # untimed replay: first-replay setup out of the timed region
        g.replay()
    torch.cuda.synchronize()

    # Timed region: replay each case's graph between HIP events on the stream
    # the kernels run on (torch's current stream).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in graphs]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for g, (a, b) in zip(graphs, evs):
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_case_ms = [a.elapsed_time(b) for a, b in evs]
    total_ms = evs[0][0].elapsed_time(evs[-1][1])
    return cases, bufs, sets, per_case_ms, total_ms, wall


def cpu_baseline(cases, bufs, seconds):
    """The FP64 oracle on host cores, on a bounded sample of each case."""
    import oracle
    threads = oracle.default_threads()
    done_bytes = 0
    elapsed = 0.0
    sample_desc = []
    budget = seconds / len(cases)
    for c, b in zip(cases, bufs):
        # probe on a small row block, then size the sample to the budget
        probe_rows = max(1, min(c.rows, (1 << 20) // c.width))
        t = time.perf_counter()
        oracle.run_op(c.op, b.host_x[:probe_rows], b.host_r[:probe_rows] if b.host_r is not None else None,
                      eps=c.eps, threads=threads, gamma=b.host_g, beta=b.host_b)
        dt = max(time.perf_counter() - t, 1e-6)
        rows = int(min(c.rows, max(probe_rows, probe_rows * budget / dt)))
        reps = 0
        t = time.perf_counter()
        while True:
            oracle.run_op(c.op, b.host_x[:rows], b.host_r[:rows] if b.host_r is not None else None,
                          eps=c.eps, threads=threads, gamma=b.host_g, beta=b.host_b)
            reps += 1
            if time.perf_counter() - t >= budget or reps >= 1000:
                break
        elapsed += time.perf_counter() - t
        done_bytes += reps * algo_bytes(dataclasses.replace(c, rows=rows))
        sample_desc.append(f"{c.op} {rows}x{c.width} x{reps}")
    return {"value": round(done_bytes / elapsed / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "; ".join(sample_desc) + f" ({elapsed:.1f} s, FP64, row blocks over {threads} threads)"}


def read_traffic(cfg, case):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_cfg{cfg}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_hash") != kernel_source_hash():
        return None
    v = kv.get(f"traffic_bytes[{case.op} {case.rows}x{case.width}]")
    return int(float(v)) if v else None


def bench(cfg, steps, warmup, cpu_seconds):
    cases, bufs, sets, per_case_ms, total_ms, wall = time_workload(cfg, steps, warmup)
    step_bytes = sum(algo_bytes(c) for c in cases)
    ms_per_step = total_ms / steps
    value = step_bytes * steps / (total_ms / 1e3) / 1e9
    ops = {}
    for c, ms in zip(cases, per_case_ms):
        us = ms * 1e3 / steps
        gbs = algo_bytes(c) / (us * 1e-6) / 1e9
        ops[f"{c.op} {c.rows}x{c.width}"] = {"us_per_call": round(us, 3), "GB_s": round(gbs, 1),
                                             "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4)}
    dom = int(np.argmax(per_case_ms))
    dc = cases[dom]
    dom_us = per_case_ms[dom] * 1e3 / steps
    achieved = algo_bytes(dc) / (dom_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": read_traffic(cfg, dc),
            "kernel": f"{dc.op} {dc.rows}x{dc.width}", "bytes_per_launch": algo_bytes(dc),
            "avg_launch_us": round(dom_us, 3)}
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[cfg], "config_id": cfg,
                   "cases": [f"{c.op} {c.rows}x{c.width} {c.dist}" for c in cases],
                   "rotation_sets": sets, "timing": f"one HIP graph of {steps} calls per operator on rotating "
                                                     f"buffer sets (>= 2 GiB per operator), HIP events per replay"},
        "roofline": roof,
        "ops": ops,
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "wall_s": round(wall, 4),
        "kernel_source_hash": kernel_source_hash(),
    }
    out["copy_ceiling"] = {"same_bytes_as_dominant": copy_ceiling(algo_bytes(dc)),
                           "1GiB": copy_ceiling(2 ** 30, reps=10)}
    if cfg == 2:
        out["context_m1max_us"] = M1MAX_CONTEXT_US
    if cpu_seconds > 0:
        out["cpu_baseline"] = cpu_baseline(cases, bufs, cpu_seconds)
    return out


def copy_ceiling(nbytes, reps=20):
    """GB/s of the library's streaming copy moving `nbytes` per call (half
    read, half written), on 3+ rotating buffer pairs totalling >= 2 GiB,
    timed like the reductions (one graph of `reps` calls)."""
    import torch

    import row_wise_reduction_amd as R
    n = max(1024, (nbytes // 8) // 1024 * 1024)  # floats per side
    pairs = max(3, -(-POOL_BYTES // (8 * n)))
    src = [torch.ones(n, dtype=torch.float32, device="cuda") for _ in range(pairs)]
    dst = [torch.empty_like(src[0]) for _ in range(pairs)]
    for i in range(pairs):
        R.rowred_copy(src[i], dst[i])
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for i in range(reps):
                R.rowred_copy(src[i % pairs], dst[i % pairs])
    torch.cuda.current_stream().wait_stream(stream)
    g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    return {"bytes_per_call": 8 * n, "us_per_call": round(us, 3), "GB_s": round(8 * n / (us * 1e-6) / 1e9, 1)}


def pmc_pass(cfg):
    """One dispatch of each case's kernel on buffers written just before by a
    1 GiB flush, then a 256 MiB copy (known bytes) for counter calibration."""
    import torch

    import row_wise_reduction_amd as R
    cases = WORKLOADS[cfg]
    bufs = [CaseBuffers(c, 1) for c in cases]
    flush = torch.empty(2 ** 28, dtype=torch.float32, device="cuda")
    print(f"pmc kernel_source_hash {kernel_source_hash()}", flush=True)
    torch.cuda.synchronize()
    for b in bufs:
        flush.fill_(1.0)
        b.call(0)
        torch.cuda.synchronize()
        print(f"pmc dispatch {b.case.op} {b.case.rows}x{b.case.width}", flush=True)
    n = 2 ** 26  # 256 MiB of float32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    flush.fill_(2.0)
    R.rowred_copy(src, dst)
    torch.cuda.synchronize()
    print(f"pmc copy {n * 4} bytes read, {n * 4} bytes written", flush=True)


# ---------------------------------------------------------------------------
# profile summaries (from rocprofv3 CSV output)
# ---------------------------------------------------------------------------

PMC_CMD = ("cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {ctr} --output-format csv -d <out_{ctr}> -o run -- "
           "python3 <repo>/bench.py --pmc --all > <log_{ctr}>")
TRACE_CMD = ("cd /tmp && TMPDIR=/tmp rocprofv3 --kernel-trace --stats --output-format csv -d <out> -o run -- "
             "python3 <repo>/bench.py --cpu-seconds 0")


def _csv_rows(path):
    import csv
    rows = list(csv.DictReader(open(path)))
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    return rows


def _logged_hash(log_path):
    """The kernel source hash a counter pass printed (see pmc_pass)."""
    if log_path and os.path.exists(log_path):
        for line in open(log_path, errors="replace"):
            if line.startswith("pmc kernel_source_hash "):
                return line.split()[-1]
    return "unknown"


def traffic_summary(fetch_csv, write_csv, out_dir, fetch_log=None, write_log=None):
    """Write profiles/pmc_traffic_cfg<N>.txt from the two counter passes of
    `bench.py --pmc --all`: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    scaled by what each counter reads for the 256 MiB copy that ends each
    workload's pass."""
    expected = [(cfg, c) for cfg in sorted(WORKLOAD_NAMES) for c in WORKLOADS[cfg]]
    per_cfg = {}
    for ctr, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        i = 0
        pending = []
        for row in _csv_rows(path):
            if row["Counter_Name"] != ctr:
                continue
            name = row["Kernel_Name"]
            if "rows_kernel" in name:
                cfg, case = expected[i]
                pending.append((cfg, case, float(row["Counter_Value"]), name))
                i += 1
            elif "copy_kernel" in name:
                copy_kib = float(row["Counter_Value"])
                for cfg, case, kib, kname in pending:
                    d = per_cfg.setdefault(cfg, {}).setdefault(f"{case.op} {case.rows}x{case.width}", {})
                    d[ctr] = kib
                    d[ctr + "_copy"] = copy_kib
                    d["kernel"] = kname
                pending = []
        if i != len(expected):
            raise SystemExit(f"{path}: found {i} reduction dispatches, expected {len(expected)}")
    copy_bytes = 2 ** 28  # each side of the calibration copy
    # the sources the counters were taken on (both passes must agree)
    h = _logged_hash(fetch_log)
    if _logged_hash(write_log) != h:
        h = "unknown"
    written = []
    for cfg, cases in per_cfg.items():
        lines = [f"# HBM traffic per dispatch, workload {cfg}: {WORKLOAD_NAMES[cfg]}",
                 "# Two counter passes over the same program, one dispatch per kernel on cold buffers:",
                 "#   " + PMC_CMD.format(ctr="FETCH_SIZE"),
                 "#   " + PMC_CMD.format(ctr="WRITE_SIZE"),
                 "# Counters are KiB per dispatch.  Scale: the copy kernel that ends the pass moves",
                 f"# {copy_bytes} B each way; read_scale = {copy_bytes} / (FETCH_SIZE_copy * 1024),",
                 f"# write_scale = {copy_bytes} / (WRITE_SIZE_copy * 1024).",
                 f"kernel_source_hash: {h}"]
        for key, d in cases.items():
            case = next(c for c in WORKLOADS[cfg] if f"{c.op} {c.rows}x{c.width}" == key)
            rs = copy_bytes / (d["FETCH_SIZE_copy"] * 1024)
            ws = copy_bytes / (d["WRITE_SIZE_copy"] * 1024)
            rd = d["FETCH_SIZE"] * 1024 * rs
            wr = d["WRITE_SIZE"] * 1024 * ws
            alg_r, alg_w = algo_split(case)
            lines += [f"kernel[{key}]: {d['kernel']}",
                      f"fetch_kib[{key}]: {d['FETCH_SIZE']:.2f} (copy {d['FETCH_SIZE_copy']:.2f}, "
                      f"read_scale {rs:.4f})",
                      f"write_kib[{key}]: {d['WRITE_SIZE']:.2f} (copy {d['WRITE_SIZE_copy']:.2f}, "
                      f"write_scale {ws:.4f})",
                      f"read_bytes[{key}]: {rd:.0f} (algorithmic {alg_r}, ratio {rd / alg_r:.4f})",
                      f"write_bytes[{key}]: {wr:.0f} (algorithmic {alg_w}, ratio {wr / alg_w:.4f})",
                      f"traffic_bytes[{key}]: {rd + wr:.0f}"]
        path = os.path.join(out_dir, f"pmc_traffic_cfg{cfg}.txt")
        open(path, "w").write("\n".join(lines) + "\n")
        written.append(path)
    return written


def trace_summary(stats_csv, bench_json, out_path):
    """Write the rocprofv3 kernel statistics of the default benchmark command
    next to the benchmark's own HIP-event averages."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    b = json.loads(open(bench_json).read().strip().splitlines()[-1])
    lines = [f"# rocprofv3 kernel statistics, workload {b['config']['config_id']}: {b['config']['workload']}",
             "#   " + TRACE_CMD,
             f"# kernel_source_hash: {b.get('kernel_source_hash', 'unknown')}",
             "# name | calls | total_ns | average_ns | min_ns | max_ns | percentage"]
    for r in rows:
        nm = r["Name"].replace("void rowred::(anonymous namespace)::", "")
        lines.append(" | ".join([nm, r["Calls"], r["TotalDurationNs"], f"{float(r['AverageNs']):.0f}",
                                 r["MinNs"], r["MaxNs"], f"{float(r['Percentage']):.2f}"]))
    lines.append("# benchmark (same command without the profiler): HIP-event average per call")
    for k, v in b["ops"].items():
        lines.append(f"bench[{k}]: {v['us_per_call']} us, {v['GB_s']} GB/s")
    lines.append(f"roofline: {json.dumps(b['roofline'])}")
    open(out_path, "w").write("\n".join(lines) + "\n")
    return out_path


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--all", action="store_true", help="one line per core workload 1..5 (with --pmc: 1..7)")
    ap.add_argument("--next", action="store_true", help="one line per next-step workload (6, 7, 8)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget (0: skip)")
    ap.add_argument("--pmc", action="store_true", help="counter pass (use under rocprofv3 --pmc)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "FETCH_LOG", "WRITE_LOG"),
                    help="write profiles/pmc_traffic_cfg*.txt from two counter passes and their stdout logs "
                         "(no GPU)")
    ap.add_argument("--trace-summary", nargs=3, metavar=("KERNEL_STATS_CSV", "BENCH_JSON", "OUT"),
                    help="write a kernel-trace summary (no GPU)")
    args = ap.parse_args(argv)
    if args.traffic_summary:
        fc, wc, fl, wl = args.traffic_summary
        for p in traffic_summary(fc, wc, os.path.join(ROOT, "profiles"), fl, wl):
            print(p)
        return 0
    if args.trace_summary:
        print(trace_summary(*args.trace_summary))
        return 0
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU: rows are independent, so N GPUs would each "
                                   "run the same kernel on rows/N; only --gpus 1 is measured"}))
        return 2
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        return 1
    import row_wise_reduction_amd as R
    R.lib()  # fail loudly if the HIP library is not built
    if args.pmc:
        for cfg in (sorted(WORKLOAD_NAMES) if args.all else [args.config]):
            pmc_pass(cfg)
        return 0
    cfgs = list(CORE) if args.all else list(NEXT) if args.next else [args.config]
    for cfg in cfgs:
        res = bench(cfg, args.steps, args.warmup, args.cpu_seconds if cfg == cfgs[0] else 0.0)
        print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
