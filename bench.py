#!/usr/bin/env python3
"""Benchmark of the fused FP32 row reductions on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 12] [--lean]

A step is one call of every operator of the workload on one batch of seeded
synthetic input.  The default workload is the largest single-GPU one: the
wide-row configuration (residual LayerNorm, RMSNorm and softmax on
16384x8192 FP32, inputs U[-1, 1]) plus the softmax stress configuration
(8192x32768, 8*N(0,1) + U[-80,80] row offsets, 1% -inf): four calls, 6.0 GiB
of algorithmic traffic per step.  Inputs and outputs are resident in HBM
before timing starts.  Each operator's K calls run on its own rotation of
>= 3 buffer sets totalling >= 2 GiB, so no call finds its data in the 256 MB
last-level cache; the K calls are captured in one HIP graph per operator so
the host's launch cost does not gate short kernels.  After W eager warm-up
steps the graphs are replayed, untimed, for 0.2 s; then the timed region is
ROUNDS rounds, each replaying every operator's graph once (K steps per
round), with HIP events on the launch stream around each replay.  An
operator's time per call is the median over the rounds of replay time / K,
reported with the min-max range; the step time is the median over rounds of
the round's total / K (the pages' protocol: the median of per-round
figures, with ranges rather than confidence intervals).  Each operator
also reports one cold call after a 1 GiB flush, a warm rate (K calls on one
buffer set) and its fraction of the library's copy moving the same bytes.
With --lean those extras, the A/A control and the CPU baseline are skipped,
so that a kernel trace of the run holds only the rotated graphs' calls
(plus the W eager warm-up calls).

`value` is the whole step's algorithmic bytes (one read of each input and
one write of the output, 4 B per element each) divided by its time.  The
JSON line also carries the roofline of the dominant kernel, the FP64 CPU
oracle's throughput on host cores, and per-operator figures.

    python bench.py --config 2  # one workload (1..12; see WORKLOAD_NAMES)
    python bench.py --pmc --all # counter pass: one dispatch of each kernel of
                                # workloads 1..11 on cold buffers, + a 256 MiB
                                # copy per workload for calibration
    python bench.py --all       # one JSON line per core workload (1..5)
    python bench.py --next      # plain and affine LayerNorm, row sum / min-max, any width (6-11)
    python bench.py --reload    # resident vs per-phase reload kernels, workloads 2-5
    python bench.py --pmc --reload  # its counter pass
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
WARMUP_SECONDS = 0.2  # graph replays before the timed region
ROUNDS = 5  # timed rounds of K steps; figures are their medians, with min-max

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
    9: "any width (_ws entry points): softmax 64x1048576, RMSNorm 1024x131072, residual LayerNorm 256x262144, "
       "row sum 16x4194304, softmax 7x1537",
    10: "many wide rows (plain entry points: exchange kernels with words in y's rows, row sum looped): softmax "
        "4096x65536, RMSNorm 2048x131072, residual LayerNorm 1024x65536, row sum 2048x131072",
    11: "many wide rows (_ws entry points: exchange kernels, row sum looped): softmax 4096x65536, "
        "RMSNorm 2048x131072, residual LayerNorm 1024x65536, row sum 2048x131072",
    12: "largest single-GPU configurations: residual LayerNorm + RMSNorm + softmax 16384x8192 U[-1,1], "
        "and softmax stress 8192x32768 (8*N(0,1) + U[-80,80] row offsets, 1% -inf)",
}
CORE = (1, 2, 3, 4, 5)
NEXT = (6, 7, 8, 9, 10, 11)
LARGEST = 12  # the default: workloads 4 and 5 in one step
PMC_CFGS = tuple(sorted(set(WORKLOAD_NAMES) - {LARGEST}))  # counter passes: each case once
WS_WORKLOADS = (9, 11)  # run through the _ws entry points (caller workspace)
WORKLOADS = {**synthetic.CORE_WORKLOADS, **synthetic.NEXT_WORKLOADS,
             LARGEST: synthetic.CORE_WORKLOADS[4] + synthetic.CORE_WORKLOADS[5]}


def log(*parts):
    """A progress line on stderr (the JSON result goes to stdout)."""
    print("bench:", *parts, file=sys.stderr, flush=True)


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
              "row_wise_reduction_amd/csrc/rowred_internal.h", "row_wise_reduction_amd/csrc/rowred_device.h",
              "row_wise_reduction_amd/csrc/rowred_split.hip", "row_wise_reduction_amd/csrc/rowred_looped.hip",
              "row_wise_reduction_amd/csrc/rowred_wide.hip", "row_wise_reduction_amd/csrc/rowred_flat.hip"):
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
        # the run record: each input's seed entropy and the SHA-256 of its
        # first and last MiB
        self.inputs = {t: {"seed_entropy": [int(v) for v in
                                            synthetic.seed_sequence(case.cfg, case.op, t, case.rows, case.width).entropy],
                           "sha256_first_last_MiB": synthetic.fingerprint(a)}
                       for t, a in (("x", x), ("r", r)) if a is not None}
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
        self.ws = None
        if case.cfg in WS_WORKLOADS:
            import row_wise_reduction_amd as R
            # calls are stream-ordered, so one workspace serves every set
            op = "layernorm_residual" if case.op.startswith("layernorm") else case.op
            self.ws = R.new_workspace(op, case.rows, case.width)

    def call(self, i):
        import row_wise_reduction_amd as R
        k = i % self.sets
        op = self.case.op
        if self.ws is not None:
            self.call_ws(k)
        elif op in ("layernorm", "layernorm_affine"):
            R.rowred_layernorm(self.x[k], None, self.g, self.b, self.y[k], eps=self.case.eps)
        elif op == "row_sum":
            R.rowred_row_sum(self.x[k], self.y[k])
        elif op == "row_minmax":
            R.rowred_row_minmax(self.x[k], self.y[k], self.y2[k])
        else:
            R.run_op(op, self.x[k], self.r[k], self.y[k], eps=self.case.eps)


    def plan(self):
        """The plan a call runs, as text: lanes per row x slots, threads and
        policy bits (row plans), or the exchange / split geometry and segments
        per row (row exchange plans, and _ws calls on rows wider than the
        register-resident window)."""
        import row_wise_reduction_amd as R
        op, x = self.case.op, self.x[0]
        if op in ("layernorm", "layernorm_affine"):
            p = R.rowred_layernorm_plan_query(x, None, self.g, self.b, self.y[0])
        elif op in ("row_sum", "row_minmax"):
            p = R.rowred_plan_query(op, x, self.y2[0] if op == "row_minmax" else None, self.y[0])
        else:
            p = R.rowred_plan_query(op, x, self.r[0], self.y[0])
        if self.ws is not None and p.window > 8192:
            sop = "layernorm_residual" if op.startswith("layernorm") else op
            sp = R.rowred_split_plan_query(sop, x)
            if sp.policy & R.ROWRED_POLICY_EXCHANGE:
                return f"exchange {sp.threads} x {sp.chunks}, S = {sp.segments}, {policy_names(sp.policy)}"
            if self.case.rows < 2048:
                return f"split {sp.threads} x {sp.chunks}, S = {sp.segments}, {policy_names(sp.policy)}"
        if p.policy & R.ROWRED_POLICY_EXCHANGE:
            S = p.grid // max(1, self.case.rows)
            return f"row exchange {p.threads} x {p.chunks}, S = {S}, {policy_names(p.policy)}"
        return f"{p.lanes_per_row} x {p.chunks}, {p.threads}, {policy_names(p.policy)}"

    def call_ws(self, k):
        import row_wise_reduction_amd as R
        op, ws = self.case.op, self.ws
        if op.startswith("layernorm"):
            R.rowred_layernorm_ws(self.x[k], self.r[k], self.g, self.b, self.y[k], ws, eps=self.case.eps)
        elif op == "rmsnorm":
            R.rowred_rmsnorm_ws(self.x[k], self.y[k], ws, eps=self.case.eps)
        elif op == "softmax":
            R.rowred_softmax_ws(self.x[k], self.y[k], ws)
        elif op == "row_sum":
            R.rowred_row_sum_ws(self.x[k], self.y[k], ws)
        else:
            R.rowred_row_minmax_ws(self.x[k], self.y[k], self.y2[k], ws)


POLICY_NAMES = (("ntL", 1), ("ntS", 2), ("remap", 4), ("stage", 8), ("looped", 64), ("exchange", 128),
                ("lds", 256), ("flat", 512), ("online", 1024))


def policy_names(policy):
    """Short names of a plan's policy bits (and its workgroups-per-CU cap)."""
    names = [n for n, bit in POLICY_NAMES if policy & bit and n != "exchange"]
    cap = (policy >> 12) & 15
    if cap:
        names.append(f"cap {cap}")
    return "+".join(names) or "-"


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
    bufs = []
    for c in cases:
        bufs.append(CaseBuffers(c, rotation_sets(c)))
        log(f"inputs of {c.op} {c.rows}x{c.width} resident ({bufs[-1].sets} buffer sets)")
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
    # Untimed: replay the graphs until >= WARMUP_SECONDS have passed, so the
    # first replay's setup and the GPU's clock ramp stay out of the timing.
    t = time.perf_counter()
    while True:
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()
        if time.perf_counter() - t >= WARMUP_SECONDS:
            break

    # Timed region: ROUNDS rounds of exactly `steps` steps -- each round
    # replays every case's graph once between HIP events on the stream the
    # kernels run on (torch's current stream).
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    rounds = [replay_timed(graphs) for _ in range(ROUNDS)]
    wall = time.perf_counter() - t0
    log(f"timed {ROUNDS} rounds of {steps} steps in {wall:.3f} s")
    return cases, bufs, sets, rounds, wall


def replay_timed(graphs):
    """Replay each graph once between HIP events; per-graph ms and the span."""
    import torch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in graphs]
    for g, (a, b) in zip(graphs, evs):
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs], evs[0][0].elapsed_time(evs[-1][1])


def aa_control(b, steps, rounds=5):
    """A/A control: two separately captured, identical graphs of `steps`
    calls on the same rotating buffers, replayed alternately `rounds` times.
    Their medians differ only by noise; the relative difference bounds what
    any A/B comparison on this machine can resolve."""
    import torch
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graphs = []
    with torch.cuda.stream(stream):
        for _ in range(2):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                for i in range(steps):
                    b.call(i)
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(stream)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()
    us = [[], []]
    for _ in range(rounds):
        ms, _ = replay_timed(graphs)
        for k in range(2):
            us[k].append(ms[k] * 1e3 / steps)
    a, a2 = float(np.median(us[0])), float(np.median(us[1]))
    return {"a_us": round(a, 3), "a_prime_us": round(a2, 3), "rounds": rounds,
            "rel_diff": round(abs(a - a2) / min(a, a2), 4)}


def single_and_warm(b, steps, reps=3):
    """(cold single call us, warm us per call): one eager call after a 1 GiB
    flush, median of `reps`; and a graph of `steps` calls all on buffer set
    0, so that inputs that fit the 256 MB last-level cache stay there."""
    import torch
    flush = torch.empty(2 ** 28, dtype=torch.float32, device="cuda")
    cold = []
    for _ in range(reps):
        flush.fill_(1.0)
        torch.cuda.synchronize()
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        b.call(0)
        e.record()
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(e) * 1e3)
    del flush
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for _ in range(steps):
                b.call(0)
    torch.cuda.current_stream().wait_stream(stream)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    ms, _ = replay_timed([g])
    return float(np.median(cold)), ms[0] * 1e3 / steps


def cpu_baseline(cases, bufs, seconds, threads=None):
    """The FP64 oracle on host cores, on a bounded sample of each case."""
    import oracle
    threads = threads or oracle.default_threads()
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
            "sample": "; ".join(sample_desc) + f" ({elapsed:.1f} s, FP64, row blocks over {threads} threads)",
            "cpu_model": cpu_model(), "affinity_cores": affinity_cores(),
            "thread_rule": "one thread per core of the affinity mask, at most 16 (a GPU's share of the host)"}


def affinity_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def read_traffic(case):
    """HBM bytes per launch from the committed counter summary of the case's
    workload, if it was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"pmc_traffic_cfg{case.cfg}.txt")
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


def spread(v):
    return {"n": len(v), "median": round(float(np.median(v)), 3), "min": round(min(v), 3), "max": round(max(v), 3)}


def bench(cfg, steps, warmup, cpu_seconds, lean=False):
    cases, bufs, sets, rounds, wall = time_workload(cfg, steps, warmup)
    step_bytes = sum(algo_bytes(c) for c in cases)
    # per round: each case's us per call, and the round's step time in ms
    case_us = [[r[0][i] * 1e3 / steps for r in rounds] for i in range(len(cases))]
    step_ms = [sum(r[0]) / steps for r in rounds]
    ms_per_step = float(np.median(step_ms))
    value = step_bytes / (ms_per_step / 1e3) / 1e9
    ops = {}
    for i, (c, b) in enumerate(zip(cases, bufs)):
        us = float(np.median(case_us[i]))
        gbs = algo_bytes(c) / (us * 1e-6) / 1e9
        entry = {"us_per_call": round(us, 3), "GB_s": round(gbs, 1), "frac_of_peak": round(gbs / PEAK_HBM_GBS, 4),
                 "rounds_us": spread(case_us[i]), "plan": b.plan(), "inputs": b.inputs}
        if not lean:
            cold, warm = single_and_warm(b, steps)
            copy = copy_ceiling(algo_bytes(c))
            entry.update({"frac_of_copy": round(gbs / copy["GB_s"], 4), "single_call_cold_us": round(cold, 3),
                          "warm_us_per_call": round(warm, 3)})
        ops[f"{c.op} {c.rows}x{c.width}"] = entry
    dom = int(np.argmax([np.median(u) for u in case_us]))
    dc = cases[dom]
    dom_us = float(np.median(case_us[dom]))
    achieved = algo_bytes(dc) / (dom_us * 1e-6) / 1e9
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": read_traffic(dc),
            "kernel": f"{dc.op} {dc.rows}x{dc.width}", "bytes_per_launch": algo_bytes(dc),
            "avg_launch_us": round(dom_us, 3), "avg_launch_us_rounds": spread(case_us[dom])}
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[cfg], "config_id": cfg,
                   "cases": [f"{c.op} {c.rows}x{c.width} {c.dist}" for c in cases],
                   "rotation_sets": sets,
                   "timing": f"{ROUNDS} rounds of {steps} steps; each operator's calls in one HIP graph on rotating "
                             f"buffer sets (>= 2 GiB per operator), HIP events per replay; medians over rounds"},
        "roofline": roof,
        "ops": ops,
        "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
        "ms_per_step_rounds": spread(step_ms),
        "rounds": ROUNDS,
        "wall_s": round(wall, 4),
        "kernel_source_hash": kernel_source_hash(),
    }
    if not lean:
        out["copy_ceiling"] = {"same_bytes_as_dominant": copy_ceiling(algo_bytes(dc)),
                               "1GiB": copy_ceiling(2 ** 30, reps=10)}
        out["launch_floor_us"] = launch_floor()
        out["aa_control"] = dict(kernel=f"{dc.op} {dc.rows}x{dc.width}", **aa_control(bufs[dom], steps))
    if cfg == 2:
        out["context_m1max_us"] = M1MAX_CONTEXT_US
    if cpu_seconds > 0 and not lean:
        log("oracle on host cores (cpu_baseline)")
        out["cpu_baseline"] = cpu_baseline(cases, bufs, cpu_seconds)
        out["cpu_baseline_1core"] = cpu_baseline(cases, bufs, cpu_seconds / 4, threads=1)
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
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    # the best of three timed replays: one slow replay (seen once, 10x) would
    # otherwise stand for the ceiling
    us = 1e30
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        g.replay()
        b.record()
        torch.cuda.synchronize()
        us = min(us, a.elapsed_time(b) * 1e3 / reps)
    return {"bytes_per_call": 8 * n, "us_per_call": round(us, 3), "GB_s": round(8 * n / (us * 1e-6) / 1e9, 1)}


def launch_floor(reps=50):
    """us per call of the library's copy moving one 16-byte granule, timed
    like the reductions (a graph of `reps` calls after warm-up replays): the
    fixed cost of one kernel launch, ramp and drain in this method."""
    import torch

    import row_wise_reduction_amd as R
    src = torch.ones(4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for _ in range(reps):
                R.rowred_copy(src, dst)
    torch.cuda.current_stream().wait_stream(stream)
    for _ in range(5):
        g.replay()
    torch.cuda.synchronize()
    ms, _ = replay_timed([g])
    return round(ms[0] * 1e3 / reps, 3)


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
# exchange kernels: cost of the segments per row
# ---------------------------------------------------------------------------

# softmax through explicit exchange plans at a fixed segment size, S segments
# per row, rows = 2^26 elements / width (so every S moves the same bytes and
# launches the same number of workgroups)
SEGMENT_SWEEP_S = (4, 8, 16, 32, 64, 128)
SEGMENT_GEOMETRIES = (("256 x 8", 256, 8, False), ("8 + 8 LDS", 256, 16, True))
SEGMENT_COUNTERS = ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_ANY", "GRBM_GUI_ACTIVE")


def segment_cases():
    for name, T, C, lds in SEGMENT_GEOMETRIES:
        for S in SEGMENT_SWEEP_S:
            width = S * T * C * 4
            rows = (1 << 26) // width
            if rows >= 1:
                yield name, T, C, lds, S, rows, width


def segment_sweep(calls):
    """Time softmax exchange plans across S (HIP events, median of `calls`
    calls after one untimed call); one JSON line per (geometry, S).  Under
    `rocprofv3 --pmc` the same calls give each dispatch's counters."""
    import torch

    import row_wise_reduction_amd as R
    print(f"segments kernel_source_hash {kernel_source_hash()}", flush=True)
    for name, T, C, lds, S, rows, width in segment_cases():
        case = synthetic.Case(9, "softmax", rows, width, "normal")
        x = torch.from_numpy(synthetic.case_input(case, "x")).cuda()
        y = torch.empty_like(x)
        pol = R.ROWRED_POLICY_EXCHANGE | R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | \
            (R.ROWRED_POLICY_LDS_STRIPE if lds else 0)
        plan = R.SplitPlan(threads=T, chunks=C, policy=pol)
        q = R.rowred_split_plan_query("softmax", x, plan=plan)
        assert q.segments == S, (name, S, q)
        ws = torch.empty(q.workspace_bytes, dtype=torch.uint8, device="cuda")
        R.rowred_split_run_plan("softmax", x, None, None, None, y, None, plan, ws)
        torch.cuda.synchronize()
        us = []
        for _ in range(calls):
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            R.rowred_split_run_plan("softmax", x, None, None, None, y, None, plan, ws)
            e.record()
            torch.cuda.synchronize()
            us.append(a.elapsed_time(e) * 1e3)
        status = int(ws[:8].view(torch.int64).item())
        print(json.dumps({"segments": S, "geometry": name, "rows": rows, "width": width, "calls": 1 + calls,
                          "us_per_call": round(float(np.median(us)), 2), "wait_status": status}), flush=True)
        del x, y, ws
        torch.cuda.empty_cache()


def segments_summary(counter_csv, log_path, out_path, timing_log=None):
    """profiles/pmc_exchange_segments.txt: per (geometry, S), the timed
    calls' median and the exchange kernel's counters per dispatch (mean of
    the calls): wave lifetime = SQ_WAVE_CYCLES * 4 / SQ_WAVES cycles,
    waiting share = SQ_WAIT_ANY / SQ_WAVE_CYCLES."""
    timed = [json.loads(l) for l in open(log_path) if l.startswith("{")]
    plain = {}
    if timing_log:  # the same sweep without the profiler
        for l in open(timing_log):
            if l.startswith("{"):
                t = json.loads(l)
                plain[(t["geometry"], t["segments"])] = t["us_per_call"]
    disp = {}
    for r in _csv_rows(counter_csv):
        if "seg_exchange" not in r["Kernel_Name"] and "seg_xlds" not in r["Kernel_Name"]:
            continue
        d = disp.setdefault(int(r["Dispatch_Id"]), {"name": r["Kernel_Name"]})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    ids = sorted(disp)
    lines = ["# exchange kernels (softmax) across segments per row S at a fixed segment size,",
             "# rows = 2^26 / width: same bytes and same workgroups at every S",
             "#   cd /tmp && TMPDIR=/tmp rocprofv3 --pmc " + " ".join(SEGMENT_COUNTERS) +
             " --output-format csv -d <out> -o run -- python3 <repo>/bench.py --segments > <log>",
             f"# kernel_source_hash: {_logged_hash_prefix(log_path, 'segments kernel_source_hash ')}",
             "#   python3 <repo>/bench.py --segments > <timing log>   (the same sweep without the profiler)",
             "# geometry | S | rows x width | us per call (median of 5 eager calls, without the profiler) | "
             "waves per dispatch | wave lifetime (cycles) | waiting share of wave cycles"]
    i = 0
    for t in timed:
        n = t["calls"]
        group = [disp[k] for k in ids[i:i + n]]
        i += n
        if len(group) < n:
            break
        group = group[1:]  # the untimed first call
        waves = np.mean([g.get("SQ_WAVES", 0) for g in group])
        cyc = np.mean([g.get("SQ_WAVE_CYCLES", 0) for g in group])
        wait = np.mean([g.get("SQ_WAIT_ANY", 0) for g in group])
        life = 4 * cyc / waves if waves else float("nan")
        us = plain.get((t["geometry"], t["segments"]), "-")
        lines.append(f"{t['geometry']} | {t['segments']} | {t['rows']}x{t['width']} | {us} | "
                     f"{waves:.0f} | {life:.0f} | {wait / cyc if cyc else float('nan'):.3f}")
    open(out_path, "w").write("\n".join(lines) + "\n")
    return out_path


def _logged_hash_prefix(log_path, prefix):
    for line in open(log_path, errors="replace"):
        if line.startswith(prefix):
            return line.split()[-1]
    return "unknown"


# ---------------------------------------------------------------------------
# per-phase reload A/B: the reference design's reloads as a diagnostic
# ---------------------------------------------------------------------------

RELOAD_CFGS = (2, 3, 4, 5)
# resident: the chooser's geometry on the register kernels; reload: that plan re-reading the row in
# every phase after the first; reload_cached: that without the non-temporal
# load hint, so the re-reads may hit in L2.
RELOAD_VARIANTS = ("resident", "reload", "reload_cached")


def variant_plan(case, b, variant):
    """The register-kernel plan of the chooser's geometry (exchange and
    LDS-stripe plans: one 1024-lane workgroup per row; two softmax
    collectives: the reload kernels have no one-collective form), then the
    variant's bits."""
    import row_wise_reduction_amd as R
    p = R.rowred_plan_query(case.op, b.x[0], b.r[0], b.y[0])
    L, C, T, pol = p.lanes_per_row, p.chunks, p.threads, p.policy & ~R.ROWRED_POLICY_ONLINE
    if pol & (R.ROWRED_POLICY_EXCHANGE | R.ROWRED_POLICY_LDS_STRIPE):
        L = T = 1024
        C = -(-p.window // 1024)
        pol &= R.ROWRED_POLICY_NT_LOADS | R.ROWRED_POLICY_NT_STORES | R.ROWRED_POLICY_XCD_REMAP
    if variant != "resident":
        pol |= R.ROWRED_POLICY_RELOAD
    if variant == "reload_cached":
        pol &= ~R.ROWRED_POLICY_NT_LOADS
    return R.Plan(L, 0, C, T, 0, policy=pol)


def plan_call(b, plan, i):
    import row_wise_reduction_amd as R
    k = i % b.sets
    R.rowred_run_plan(b.case.op, b.x[k], b.r[k], b.y[k], plan, eps=b.case.eps or 0.0)


def time_reload(cfg, steps, warmup, rounds=3):
    """us per call of each variant at each case of a workload: one HIP graph
    of `steps` calls per variant on rotating buffers; the rounds interleave
    the variants and the minimum over rounds is kept."""
    import torch
    ops = {}
    for case in WORKLOADS[cfg]:
        b = CaseBuffers(case, rotation_sets(case))
        plans = {v: variant_plan(case, b, v) for v in RELOAD_VARIANTS}
        for v in RELOAD_VARIANTS:
            for i in range(warmup):
                plan_call(b, plans[v], i)
        torch.cuda.synchronize()
        stream = torch.cuda.Stream()
        stream.wait_stream(torch.cuda.current_stream())
        graphs = {}
        with torch.cuda.stream(stream):
            for v in RELOAD_VARIANTS:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(steps):
                        plan_call(b, plans[v], i)
                graphs[v] = g
        torch.cuda.current_stream().wait_stream(stream)
        for g in graphs.values():
            g.replay()
        torch.cuda.synchronize()
        us = {v: [] for v in RELOAD_VARIANTS}
        for _ in range(rounds):
            for v, g in graphs.items():
                a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                g.replay()
                e.record()
                torch.cuda.synchronize()
                us[v].append(a.elapsed_time(e) * 1e3 / steps)
        entry = {}
        for v in RELOAD_VARIANTS:
            t = min(us[v])
            entry[v] = {"us_per_call": round(t, 3), "GB_s": round(algo_bytes(case) / (t * 1e-6) / 1e9, 1),
                        "policy": plans[v].policy, "rounds_us": [round(u, 3) for u in us[v]]}
        entry["reload_over_resident"] = round(entry["reload"]["us_per_call"] / entry["resident"]["us_per_call"], 3)
        entry["plan"] = f"L{plans['resident'].lanes_per_row} C{plans['resident'].chunks} T{plans['resident'].threads}"
        ops[f"{case.op} {case.rows}x{case.width}"] = entry
        del b, graphs
        torch.cuda.empty_cache()
    return {"mode": "reload_ab", "config": {"workload": WORKLOAD_NAMES[cfg], "config_id": cfg}, "steps": steps,
            "warmup": warmup, "unit": "GB/s", "ops": ops, "kernel_source_hash": kernel_source_hash(),
            "note": "GB/s counts one read of each input and one write of the output, as for the resident kernels"}


def pmc_reload_pass(cfg):
    """One dispatch of each reload variant per case, each on buffers written
    just before by a 1 GiB flush, then the 256 MiB calibration copy."""
    import torch

    import row_wise_reduction_amd as R
    flush = torch.empty(2 ** 28, dtype=torch.float32, device="cuda")
    print(f"pmc kernel_source_hash {kernel_source_hash()}", flush=True)
    for case in WORKLOADS[cfg]:
        b = CaseBuffers(case, 1)
        for v in RELOAD_VARIANTS:
            plan = variant_plan(case, b, v)
            flush.fill_(1.0)
            torch.cuda.synchronize()
            plan_call(b, plan, 0)
            torch.cuda.synchronize()
            print(f"pmc dispatch {v} {case.op} {case.rows}x{case.width}", flush=True)
        del b
    n = 2 ** 26
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
             "python3 <repo>/bench.py{args} --lean")


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


def kernel_short_name(name):
    """A library kernel's name without return type and namespaces."""
    if name.startswith("void "):
        name = name[5:]
    return name.replace("rowred::(anonymous namespace)::", "")


def is_library_reduction_kernel(name):
    """A dispatch of one of the library's reduction paths (its streaming copy
    aside): every kernel of the library lives in namespace rowred."""
    return "rowred::" in name and "copy_kernel" not in name


def traffic_summary(fetch_csv, write_csv, out_dir, fetch_log=None, write_log=None):
    """Write profiles/pmc_traffic_cfg<N>.txt from the two counter passes of
    `bench.py --pmc --all`: FETCH_SIZE and WRITE_SIZE (KiB per dispatch),
    scaled by what each counter reads for the 256 MiB copy that ends each
    workload's pass."""
    # One call per case, each after a flush fill: the library dispatches
    # between two other kernels are one call (1 to 3 dispatches).
    expected = [(cfg, c) for cfg in PMC_CFGS for c in WORKLOADS[cfg]]
    per_cfg = {}
    for ctr, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        i = 0
        pending = []   # calls since the last copy: [cfg, case, KiB, kernel names]
        in_call = False
        for row in _csv_rows(path):
            if row["Counter_Name"] != ctr:
                continue
            name = row["Kernel_Name"]
            if is_library_reduction_kernel(name):
                if not in_call:
                    if i >= len(expected):
                        raise SystemExit(f"{path}: more calls than the {len(expected)} cases")
                    pending.append([*expected[i], 0.0, []])
                    i += 1
                    in_call = True
                pending[-1][2] += float(row["Counter_Value"])
                short = kernel_short_name(name).split("(")[0]
                pending[-1][3].append(short)
            elif "copy_kernel" in name:
                copy_kib = float(row["Counter_Value"])
                for cfg, case, kib, names in pending:
                    d = per_cfg.setdefault(cfg, {}).setdefault(f"{case.op} {case.rows}x{case.width}", {})
                    d[ctr] = kib
                    d[ctr + "_copy"] = copy_kib
                    d["kernels"] = names
                pending = []
                in_call = False
            else:
                in_call = False
        if i != len(expected):
            raise SystemExit(f"{path}: found {i} calls, expected {len(expected)}")
    copy_bytes = 2 ** 28  # each side of the calibration copy
    # the sources the counters were taken on (both passes must agree)
    h = _logged_hash(fetch_log)
    if _logged_hash(write_log) != h:
        h = "unknown"
    written = []
    for cfg, cases in per_cfg.items():
        lines = [f"# HBM traffic per call (all its dispatches), workload {cfg}: {WORKLOAD_NAMES[cfg]}",
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
            lines += [f"kernel[{key}]: {' + '.join(d['kernels'])}",
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


PMC_RELOAD_CMD = ("cd /tmp && TMPDIR=/tmp rocprofv3 --pmc {ctr} --output-format csv -d <out_{ctr}> -o run -- "
                  "python3 <repo>/bench.py --pmc --reload > <log_{ctr}>")


def reload_traffic_summary(fetch_csv, write_csv, out_path, fetch_log=None, write_log=None):
    """Write the HBM traffic of the resident and reload variants from the two
    counter passes of `bench.py --pmc --reload`."""
    expected = [(cfg, c, v) for cfg in RELOAD_CFGS for c in WORKLOADS[cfg] for v in RELOAD_VARIANTS]
    got = {}
    for ctr, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        i = 0
        pending = []
        for row in _csv_rows(path):
            if row["Counter_Name"] != ctr:
                continue
            name = row["Kernel_Name"]
            if "rows_kernel" in name or "reload_kernel" in name:
                cfg, case, v = expected[i]
                want = "rows_kernel" if v == "resident" else "reload_kernel"
                if want not in name:
                    raise SystemExit(f"{path}: dispatch {i} is {name}, expected a {want} ({v})")
                pending.append((case, v, float(row["Counter_Value"])))
                i += 1
            elif "copy_kernel" in name:
                copy_kib = float(row["Counter_Value"])
                for case, v, kib in pending:
                    got.setdefault((case, v), {})[ctr] = kib * 1024 * (2 ** 28) / (copy_kib * 1024)
                pending = []
        if i != len(expected):
            raise SystemExit(f"{path}: found {i} reduction dispatches, expected {len(expected)}")
    h = _logged_hash(fetch_log)
    if _logged_hash(write_log) != h:
        h = "unknown"
    lines = ["# HBM traffic per dispatch: resident kernels vs the per-phase reload variant",
             "# (reload: every phase after the first reads x, and r, again; reload_cached: the same",
             "# without the non-temporal load hint).  One dispatch per variant on cold buffers, each",
             "# counter scaled by what it reads for the 256 MiB copy that ends each workload's pass.",
             "#   " + PMC_RELOAD_CMD.format(ctr="FETCH_SIZE"),
             "#   " + PMC_RELOAD_CMD.format(ctr="WRITE_SIZE"),
             "# reads_algorithmic: one read of each input; reads_requested: what the kernel asks",
             "# for (x and r once per phase); fetch: HBM bytes read.",
             f"kernel_source_hash: {h}"]
    for cfg in RELOAD_CFGS:
        for case in WORKLOADS[cfg]:
            alg_r, alg_w = algo_split(case)
            phases = {"layernorm_residual": 3, "rmsnorm": 2, "softmax": 3}[case.op]
            for v in RELOAD_VARIANTS:
                d = got[(case, v)]
                req = alg_r * (1 if v == "resident" else phases)
                key = f"{v} {case.op} {case.rows}x{case.width}"
                lines.append(f"fetch_bytes[{key}]: {d['FETCH_SIZE']:.0f} (reads_algorithmic {alg_r}, "
                             f"reads_requested {req}, fetch/algorithmic {d['FETCH_SIZE'] / alg_r:.4f})")
                lines.append(f"write_bytes[{key}]: {d['WRITE_SIZE']:.0f} (algorithmic {alg_w}, "
                             f"ratio {d['WRITE_SIZE'] / alg_w:.4f})")
    open(out_path, "w").write("\n".join(lines) + "\n")
    return out_path


def trace_summary(stats_csv, bench_json, out_path, trace_csv=None):
    """Write the rocprofv3 kernel statistics of a benchmark command next to
    the benchmark's own HIP-event figures (its JSON line).  With the
    per-dispatch trace, also each kernel's median duration."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    b = json.loads(open(bench_json).read().strip().splitlines()[-1])
    lines = [f"# rocprofv3 kernel statistics, workload {b['config']['config_id']}: {b['config']['workload']}",
             "#   " + TRACE_CMD.format(args=("" if b["config"]["config_id"] == LARGEST
                                         else f" --config {b['config']['config_id']}")
                                   + ("" if b["steps"] == 50 else f" --steps {b['steps']}")),
             f"# kernel_source_hash: {b.get('kernel_source_hash', 'unknown')}",
             "# name | calls | total_ns | average_ns | min_ns | max_ns | percentage"]
    for r in rows:
        nm = kernel_short_name(r["Name"])
        lines.append(" | ".join([nm, r["Calls"], r["TotalDurationNs"], f"{float(r['AverageNs']):.0f}",
                                 r["MinNs"], r["MaxNs"], f"{float(r['Percentage']):.2f}"]))
    if trace_csv:
        # one kernel may serve several shapes: keyed by kernel and grid size
        per = {}
        for r in csv.DictReader(open(trace_csv)):
            key = f"{kernel_short_name(r['Kernel_Name'])} [grid {r['Grid_Size_X']}]"
            per.setdefault(key, []).append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        lines.append("# per-dispatch durations from the kernel trace, by kernel and grid size (work-items): "
                     "name | dispatches | median_ns | p10_ns | p90_ns")
        for nm, d in sorted(per.items(), key=lambda kv: -sum(kv[1])):
            q = np.percentile(d, [50, 10, 90])
            lines.append(f"{nm} | {len(d)} | {q[0]:.0f} | {q[1]:.0f} | {q[2]:.0f}")
    lines.append("# the same run's HIP-event figures (median over rounds of replay time / calls)")
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
    ap.add_argument("--config", type=int, default=LARGEST, choices=sorted(WORKLOAD_NAMES))
    ap.add_argument("--lean", action="store_true",
                    help="time the rotated graphs only (no cold/warm calls, copy ceiling, A/A control or CPU "
                         "baseline): the command a kernel trace is taken of")
    ap.add_argument("--all", action="store_true", help="one line per core workload 1..5 (with --pmc: 1..7)")
    ap.add_argument("--next", action="store_true", help="one line per next-step workload (6-11)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget (0: skip)")
    ap.add_argument("--pmc", action="store_true", help="counter pass (use under rocprofv3 --pmc)")
    ap.add_argument("--segments", action="store_true",
                    help="softmax exchange plans at 4-128 segments per row, same bytes (timing; counters under "
                         "rocprofv3 --pmc)")
    ap.add_argument("--segments-summary", nargs="+", metavar="FILE",
                    help="COUNTER_CSV LOG [TIMING_LOG]: write profiles/pmc_exchange_segments.txt from a --segments "
                         "counter run (and the same sweep's output without the profiler)")
    ap.add_argument("--reload", action="store_true",
                    help="resident vs per-phase reload A/B at workloads 2-5 (with --pmc: its counter pass)")
    ap.add_argument("--reload-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "FETCH_LOG", "WRITE_LOG"),
                    help="write profiles/pmc_traffic_reload.txt from the two reload counter passes (no GPU)")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "FETCH_LOG", "WRITE_LOG"),
                    help="write profiles/pmc_traffic_cfg*.txt from two counter passes and their stdout logs "
                         "(no GPU)")
    ap.add_argument("--trace-summary", nargs="+", metavar="FILE",
                    help="KERNEL_STATS_CSV BENCH_JSON OUT [KERNEL_TRACE_CSV]: write a kernel-trace summary (no GPU)")
    args = ap.parse_args(argv)
    if args.traffic_summary:
        fc, wc, fl, wl = args.traffic_summary
        for p in traffic_summary(fc, wc, os.path.join(ROOT, "profiles"), fl, wl):
            print(p)
        return 0
    if args.trace_summary:
        print(trace_summary(*args.trace_summary))
        return 0
    if args.segments_summary:
        csv_path, log_path = args.segments_summary[:2]
        timing = args.segments_summary[2] if len(args.segments_summary) > 2 else None
        print(segments_summary(csv_path, log_path, os.path.join(ROOT, "profiles", "pmc_exchange_segments.txt"),
                               timing))
        return 0
    if args.reload_summary:
        fc, wc, fl, wl = args.reload_summary
        print(reload_traffic_summary(fc, wc, os.path.join(ROOT, "profiles", "pmc_traffic_reload.txt"), fl, wl))
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
    if args.pmc and args.reload:
        for cfg in RELOAD_CFGS:
            pmc_reload_pass(cfg)
        return 0
    if args.segments:
        segment_sweep(5)
        return 0
    if args.pmc:
        for cfg in (PMC_CFGS if args.all else [args.config]):
            pmc_pass(cfg)
        return 0
    if args.reload:
        for cfg in RELOAD_CFGS:
            print(json.dumps(time_reload(cfg, args.steps, args.warmup)), flush=True)
        return 0
    cfgs = list(CORE) if args.all else list(NEXT) if args.next else [args.config]
    for cfg in cfgs:
        res = bench(cfg, args.steps, args.warmup, args.cpu_seconds if cfg == cfgs[0] else 0.0, lean=args.lean)
        print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
