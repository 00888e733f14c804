"""Soft-DTW forward+backward throughput on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

Workload (the headline configuration): B=32 pairs, N=M=512, D=64, gamma=1.0,
x, y ~ N(0,1) fp32 from seed 0, unfused mode, loss = batch mean.  One step is
one pass of the whole path through the C ABI on preallocated buffers:
sdtw_forward (distances; forward and reverse sweeps of the dynamic programme
in one launch; loss) + sdtw_backward (alignment matrix from the two sweeps,
chain rule to dx and dy).  Inputs are resident in HBM when the timed region
starts.  Prints one JSON line.

Metric: DP cells per second, B*N*M / (seconds per step), plus peak memory of
the autograd path.  `roofline` describes the dominant kernel (the launch that
runs both sweeps), its duration taken from HIP events that the library
records on the launch stream (sdtw_timing); `dist` puts the distance kernel
against the HBM and fp64-MFMA roofs; `kernels` lists every launch of a step
the same way.  `cpu_baseline` is the fp64 oracle on the host, timed
on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

WORKLOAD = dict(B=32, N=512, M=512, D=64, gamma=1.0)
# Plain ALU peak of the MI355X: 256 CUs x 4 SIMDs x 16 lanes, one operation
# per lane per clock at 2.4 GHz (the datasheet's 78.6 TFLOP/s fp64 counts an
# FMA as two), i.e. 39.3 T lane-operation slots/s.
PEAK_ALU_TOPS = 256 * 4 * 16 * 2.4e9 / 1e12
# Algorithmic ALU work of one cell, forward and backward dynamic programme
# together, as the log-space formulation counts it (a logsumexp of three
# terms per sweep and the final exponential of the alignment entry): about
# 13 transcendentals (exp, log), each taking four issue slots at quarter
# rate, and about 45 other operations, i.e. 97 lane-operation slots per cell.  At the headline
# workload that is 20.7 us at PEAK_ALU_TOPS.
TRANS_PER_CELL = 13
OTHER_OPS_PER_CELL = 45
ALU_SLOTS_PER_CELL = 4 * TRANS_PER_CELL + OTHER_OPS_PER_CELL
# A narrower count, beside it: the operations of one cell in one sweep when
# the recurrence is written in base 2 -- d = Dist*log2(e)/g (1 mul), the two
# minima and two maxima that order the three predecessors (4), the two
# differences to the minimum (2), two exp2 (2), their sum with 1 (2), log2
# (1), the soft-minimum m - log2 (1) and the state t + d (1): 14 operations,
# 28 for the two sweeps, transcendentals counted once.
DP_OPS_PER_CELL = 2 * 14
# Bytes the two sweeps must move per cell: each reads Dist (4) and writes
# its fp64 state (8).
DP_BYTES_PER_CELL = 2 * (4 + 8)
DOMINANT = "dp_both"
# HBM traffic of one launch of the dominant kernel, from two rocprofv3 --pmc
# runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) on the headline workload,
# each scaled by what the same counter reads for a 256 MiB copy (FETCH_SIZE
# reads half the bytes moved, WRITE_SIZE all of them).  Valid only for the
# kernel sources it was taken on, identified by their SHA-256.
TRAFFIC_RECORD = {
    "sources": ["differentiable_series_alignment_amd/csrc/sdtw_dp.hip",
                "differentiable_series_alignment_amd/csrc/sdtw_dp_common.h",
                "differentiable_series_alignment_amd/csrc/sdtw_device.h",
                "differentiable_series_alignment_amd/csrc/sdtw_kernels.h",
                "differentiable_series_alignment_amd/csrc/sdtw_api.hip"],
    "sha256": "d97cd41000128c1cd8b38c93ca25d0d4c0a6aa5b749487fc9c628cc8deaf10e5",
    "fetch_kib": 37604, "fetch_scale": 2.0,
    "write_kib": 148110, "write_scale": 1.0,
}


# Roofs of the per-configuration bounds (MI355X datasheet): fp64 and fp32
# matrix rates, HBM bandwidth, and the dependency chain of the recurrence:
# a sweep visits the N+M-1 anti-diagonals one after another, and one step of
# the cell's chain (neighbour exchange, ordering, two exp2, a log2, the
# state) is taken as CHAIN_CYCLES clocks.
PEAK_F64_MFMA = 78.6e12
PEAK_F32_MFMA = 157.3e12
PEAK_HBM = 8.0e12
CHAIN_CYCLES = 100
CLOCK = 2.4e9


# The other configurations (tiny; feature-dimension sweep; long sequences at
# two temperatures), reported beside the headline one.
CONFIGS = ([(2, 16, 16, 1, 1.0)]
           + [(32, 256, 256, d, 1.0) for d in (1, 4, 16, 64, 128, 256)]
           + [(32, n, m, 128, g) for (n, m) in ((1024, 1024), (2048, 2048), (4096, 4096),
                                               (4096, 1000))
              for g in (1.0, 0.01)])


def step_bounds(B, N, M, D, fused):
    """Lower bounds of one fwd+bwd step (microseconds).  Stages: distances
    (2D flops per cell on fp64 MFMA; unfused also writes them, 4 B per
    cell), the sweeps (both at once unfused: the chain of N+M-1 steps,
    ALU_SLOTS_PER_CELL issue slots and 24 B per cell), the chain rule (4D flops per cell on
    fp32 MFMA; unfused reads the two fp64 states and writes E or the dy
    shares, 20 B per cell).  Fused runs the sweeps one after the other and
    recomputes the distances in each (8 B of state per cell written, then
    read).  `per_stage` puts every stage at its own roof and adds them (the
    stages run one after another); `ideal` overlaps everything (the largest
    of the summed resource times and the chain)."""
    cells = B * N * M
    io = 4 * B * (N + M) * D
    chain = (N + M - 1) * CHAIN_CYCLES / CLOCK
    alu = ALU_SLOTS_PER_CELL * cells / (PEAK_ALU_TOPS * 1e12)
    if not fused:
        t_dist = (2 * cells * D / PEAK_F64_MFMA, (4 * cells + io) / PEAK_HBM)
        t_dp = (chain, alu, 24 * cells / PEAK_HBM)
        t_rule = (4 * cells * D / PEAK_F32_MFMA, (20 * cells + 2 * io) / PEAK_HBM)
        per_stage = max(t_dist) + max(t_dp) + max(t_rule)
        mfma = t_dist[0] + t_rule[0]
        hbm = t_dist[1] + t_dp[2] + t_rule[1]
        ideal = max(mfma, hbm, alu, chain)
    else:
        t_fwd = (chain, 2 * cells * D / PEAK_F64_MFMA, (8 * cells + io) / PEAK_HBM, alu / 2)
        t_rev = (chain, 2 * cells * D / PEAK_F64_MFMA + 4 * cells * D / PEAK_F32_MFMA,
                 (8 * cells + 2 * io) / PEAK_HBM, alu / 2)
        per_stage = max(t_fwd) + max(t_rev)
        ideal = max(2 * chain, t_fwd[1] + t_rev[1], t_fwd[2] + t_rev[2])
    return {"per_stage_us": per_stage * 1e6, "ideal_us": ideal * 1e6}


def with_bounds(entry, B, N, M, D, fused):
    """Adds the bounds and the measured step's fractions of them."""
    bd = step_bounds(B, N, M, D, fused)
    t = entry["ms_per_step"] * 1e3
    entry["bound_per_stage_us"] = bd["per_stage_us"]
    entry["bound_ideal_us"] = bd["ideal_us"]
    entry["frac_per_stage"] = bd["per_stage_us"] / t
    entry["frac_ideal"] = bd["ideal_us"] / t
    return entry


def recorded_traffic():
    """Bytes per launch of the dominant kernel, or None once its sources
    differ from those the counters were taken on."""
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_RECORD["sources"]:
        with open(os.path.join(HERE, f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest() != TRAFFIC_RECORD["sha256"]:
        return None
    r = TRAFFIC_RECORD
    return 1024 * (r["fetch_kib"] * r["fetch_scale"] + r["write_kib"] * r["write_scale"])


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--headline-only", action="store_true",
                   help="skip the per-configuration table")
    p.add_argument("--counter-pass", nargs="?", const="32,512,512,64,1.0", default=None,
                   metavar="B,N,M,D,GAMMA",
                   help="for rocprofv3 --pmc runs: three unfused and three fused steps "
                        "of this workload (default: the headline one), then three "
                        "copies of 256 MiB (the counters' calibration), no output")
    p.add_argument("--summarize-counters", nargs="+", default=None, metavar="CSV",
                   help="print per-kernel averages of rocprofv3 counter_collection.csv "
                        "files (no GPU needed)")
    p.add_argument("--cells", type=float, default=None,
                   help="with --summarize-counters: DP cells per dispatch, for the "
                        "per-cell figures")
    p.add_argument("--profile-workload", default=None, metavar="B,N,M,D,GAMMA",
                   help="for rocprofv3 --kernel-trace runs: a few unfused and "
                        "fused steps of this workload, one summary line each")
    return p.parse_args()


def profile_workload(torch, L, pair_batch, spec, steps):
    """Unfused and fused fwd+bwd steps of one workload (kernel traces of
    configurations other than the headline one)."""
    b_, n_, m_, d_, g_ = spec.split(",")
    B, N, M, D, gamma = int(b_), int(n_), int(m_), int(d_), float(g_)
    xc, yc = pair_batch(B, N, M, D, seed=0)
    x, y = xc.to("cuda:0"), yc.to("cuda:0")
    for name, mode in (("unfused", L.SDTW_MODE_UNFUSED), ("fused", L.SDTW_MODE_FUSED)):
        ms = measure(L, torch, x, y, gamma, mode, steps, 2)[0]
        print(f"B={B} N={N} M={M} D={D} gamma={gamma} {name}: {ms:.3f} ms per step",
              flush=True)


def counter_pass(torch, L, pair_batch, spec):
    """Three unfused and three fused steps of one workload, then three copies
    of a 256 MiB fp32 tensor whose bytes are known, for scaling the traffic
    counters."""
    b_, n_, m_, d_, g_ = spec.split(",")
    xc, yc = pair_batch(int(b_), int(n_), int(m_), int(d_), seed=0)
    x, y = xc.to("cuda:0"), yc.to("cuda:0")
    measure(L, torch, x, y, float(g_), L.SDTW_MODE_UNFUSED, 3, 0)
    measure(L, torch, x, y, float(g_), L.SDTW_MODE_FUSED, 3, 0)
    src = torch.ones(64 * 2**20, dtype=torch.float32, device=x.device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()


def cpu_baseline(x, y, gamma, budget_s, warm=True):
    """The fp64 oracle on the host cores, on a bounded sample (whole pairs of
    the same workload) sized to about `budget_s` seconds of wall time: calls
    of min(B, threads) pairs, one pair per OpenMP thread, at least one call."""
    from oracle import oracle as O
    O.lib()
    xs, ys = x.numpy(), y.numpy()
    B, N, D = xs.shape
    M = ys.shape[1]
    threads = O.num_threads()
    if warm:
        O.value_and_grad(xs[:1, :min(N, 64)], ys[:1, :min(M, 64)], gamma, [1.0])
    npairs = min(B, threads)
    t0 = time.perf_counter()
    done = 0
    while True:
        lo = done % B
        hi = min(lo + npairs, B)
        O.value_and_grad(xs[lo:hi], ys[lo:hi], gamma, [1.0 / B] * (hi - lo))
        done += hi - lo
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done * N * M / dt, "unit": "cells/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} pairs of {N}x{M}, D={D}, gamma={gamma} (fp64 distances, "
                      f"forward, log-space backward, chain rule), {dt:.1f} s wall"}


def cpu_one_core(x, y, gamma, budget_s):
    """The oracle on one core (OpenMP limited to one thread for the call)."""
    from oracle import oracle as O
    prev = O.num_threads()
    O.set_num_threads(1)
    try:
        return cpu_baseline(x, y, gamma, budget_s, warm=False)
    finally:
        O.set_num_threads(prev)


# Counter arithmetic of the MI355X (gfx950): 8 XCDs (GRBM counters are kept
# per XCD), 256 CUs, 1024 SIMDs; one MFMA "MOP" is 512 flops; FETCH_SIZE and
# WRITE_SIZE are KiB, scaled by what they read for a copy of known size
# (FETCH_SIZE reads half the bytes a 256 MiB copy moves, WRITE_SIZE all).
N_XCD, N_CU, N_SIMD = 8, 256, 1024
FETCH_SCALE, WRITE_SCALE = 2.0, 1.0


def derived_counters(c, cells):
    """Figures per dispatch from the mean counter values `c` of one kernel:
    MFMA busy share of the SIMDs' cycles, VALU busy (rocprofv3's VALUBusy),
    MFMA flops, and per DP cell the VALU lane slots (non-MFMA VALU
    instructions x 64), transcendentals (x 64) and HBM bytes."""
    d = {}
    gui = c.get("GRBM_GUI_ACTIVE")
    if gui:
        cyc = gui / N_XCD
        d["cycles"] = cyc
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c:
            d["mfma_busy_pct"] = 100 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cyc * N_SIMD)
        if "SQ_ACTIVE_INST_VALU" in c:
            d["valu_busy_pct"] = 100 * c["SQ_ACTIVE_INST_VALU"] / N_CU / cyc
    flops = 512 * (c.get("SQ_INSTS_VALU_MFMA_MOPS_F64", 0) + c.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0))
    if "SQ_INSTS_VALU_MFMA_MOPS_F64" in c:
        d["mfma_gflop"] = flops / 1e9
    if cells:
        if "SQ_INSTS_VALU" in c and "SQ_INSTS_MFMA" in c:
            d["valu_slots_per_cell"] = 64 * (c["SQ_INSTS_VALU"] - c["SQ_INSTS_MFMA"]) / cells
        if "SQ_INSTS_VALU_TRANS_F32" in c:
            d["trans_per_cell"] = 64 * (c["SQ_INSTS_VALU_TRANS_F32"]
                                        + c.get("SQ_INSTS_VALU_TRANS_F64", 0)) / cells
        if "FETCH_SIZE" in c and "WRITE_SIZE" in c:
            d["hbm_bytes_per_cell"] = 1024 * (FETCH_SCALE * c["FETCH_SIZE"]
                                              + WRITE_SCALE * c["WRITE_SIZE"]) / cells
    if "FETCH_SIZE" in c and "WRITE_SIZE" in c:
        d["hbm_mb"] = 1024 * (FETCH_SCALE * c["FETCH_SIZE"] + WRITE_SCALE * c["WRITE_SIZE"]) / 1e6
    return d


def summarize_counters(paths, cells=None):
    """Per-kernel averages of rocprofv3 --pmc output (counter_collection.csv:
    one row per dispatch and counter, the value summed over the GPU's
    instances).  Prints one markdown row per kernel: dispatches and the mean
    value of every counter per dispatch; then the derived figures."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(list))
    for path in paths:
        with open(path) as fh:
            for r in csv.DictReader(fh):
                name = r["Kernel_Name"]
                key = (r["Dispatch_Id"], r["Counter_Name"])
                vals[name][key].append(float(r["Counter_Value"]))
    counters = sorted({c for k in vals.values() for (_, c) in k})
    means = {}
    print("| kernel | dispatches | " + " | ".join(counters) + " |")
    print("|---|---|" + "---|" * len(counters))
    for name, kv in sorted(vals.items()):
        per = defaultdict(list)
        disp = set()
        for (d, c), v in kv.items():
            per[c].append(sum(v))
            disp.add(d)
        short = name if len(name) <= 60 else name[:57] + "..."
        cols = [f"{sum(per[c]) / len(per[c]):.6g}" if per[c] else "" for c in counters]
        print(f"| `{short}` | {len(disp)} | " + " | ".join(cols) + " |")
        means[short] = {c: sum(per[c]) / len(per[c]) for c in counters if per[c]}
    rows = {k: derived_counters(v, cells) for k, v in means.items()}
    keys = [k for k in ("cycles", "mfma_busy_pct", "valu_busy_pct", "mfma_gflop",
                        "valu_slots_per_cell", "trans_per_cell", "hbm_mb",
                        "hbm_bytes_per_cell") if any(k in r for r in rows.values())]
    if keys:
        print()
        print("| kernel | " + " | ".join(keys) + " |")
        print("|---|" + "---|" * len(keys))
        for name, r in rows.items():
            print(f"| `{name}` | " + " | ".join(f"{r[k]:.4g}" if k in r else ""
                                                for k in keys) + " |")


def measure(L, torch, x, y, gamma, mode, steps, warmup):
    """Milliseconds per fwd+bwd step through the C ABI on preallocated
    buffers, timed with events on the launch stream."""
    B, N, D = x.shape
    M = y.shape[1]
    dev = x.device
    nbytes = L.sdtw_workspace_bytes(B, N, M, D, mode)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    loss = torch.empty(B, dtype=torch.float32, device=dev)
    gl = torch.full((B,), 1.0 / B, dtype=torch.float32, device=dev)
    gx = torch.empty_like(x)
    gy = torch.empty_like(y)
    stream = torch.cuda.current_stream(dev)
    s = int(stream.cuda_stream)

    def fwd():
        L.check(L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma, mode,
                               ws.data_ptr(), nbytes, loss.data_ptr(), s), "sdtw_forward")

    def bwd(grads=True):
        L.check(L.sdtw_backward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma, mode,
                                ws.data_ptr(), nbytes, gl.data_ptr(),
                                gx.data_ptr() if grads else None,
                                gy.data_ptr() if grads else None, None, s),
                "sdtw_backward")

    for _ in range(warmup):
        fwd()
        bwd()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        fwd()
        bwd()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, fwd, bwd, stream


def measure_inference(L, torch, x, y, gamma, steps, warmup):
    """Milliseconds per loss-only forward (inference mode: no state kept,
    workspace O(B*N)) through the C ABI, and the workspace size in MiB;
    None when the device cannot hold every band of a pair at once."""
    B, N, D = x.shape
    M = y.shape[1]
    mode = L.SDTW_MODE_INFERENCE
    nbytes = L.sdtw_workspace_bytes(B, N, M, D, mode)
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device)
    loss = torch.empty(B, dtype=torch.float32, device=x.device)
    s = int(torch.cuda.current_stream(x.device).cuda_stream)

    def fwd():
        return L.sdtw_forward(x.data_ptr(), y.data_ptr(), B, N, M, D, gamma, mode,
                              ws.data_ptr(), nbytes, loss.data_ptr(), s)

    if fwd() == L.SDTW_ERR_UNSUPPORTED:
        return None
    for _ in range(warmup):
        L.check(fwd(), "sdtw_forward")
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        L.check(fwd(), "sdtw_forward")
    e1.record()
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / steps
    return {"ms_per_forward": t, "cells_per_s": B * N * M / (t * 1e-3),
            "workspace_mib": nbytes / 2**20}


def peak_mib(torch, SoftDTW, x, y, gamma, fused, checkpoint=False, low_memory=False):
    """Peak device memory of one autograd fwd+bwd (SoftDTW(...)(x, y).mean()
    .backward()) above what was allocated before, and the part of it taken
    by x, y and their gradients."""
    dev = x.device
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    base = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    xg = x.clone().requires_grad_(True)
    yg = y.clone().requires_grad_(True)
    SoftDTW(gamma=gamma, fused=fused, checkpoint=checkpoint,
            low_memory=low_memory)(xg, yg).mean().backward()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated(dev) - base
    io = 2 * (xg.numel() + yg.numel()) * 4
    del xg, yg
    return peak / 2**20, (peak - io) / 2**20


def barycenter_rate(torch, softdtw_barycenter, block_waves):
    """Block-wave barycenter: 10 sequences (100, 3), Adam lr 0.1, 100
    iterations, gamma 1; each iteration is one batched fwd+bwd."""
    X = block_waves(10, 100, 3, seed=0).to("cuda:0")
    softdtw_barycenter(X, gamma=1.0, max_iter=5, lr=0.1)  # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    softdtw_barycenter(X, gamma=1.0, max_iter=100, lr=0.1)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    return {"workload": "barycenter K=10 N=M=100 D=3 gamma=1.0, 100 Adam iterations",
            "ms_per_iteration": dt * 1e3 / 100,
            "cells_per_s": 100 * 10 * 100 * 100 / dt}


def barycenter_cpu_rate(block_waves, budget_s):
    """The oracle's barycenter objective and gradient (10 pairs of 100 x 100,
    D = 3, the work of one iteration) repeated for about budget_s seconds."""
    from oracle import oracle as O
    X = block_waves(10, 100, 3, seed=0).numpy()
    z = X.mean(axis=0)
    threads = O.num_threads()
    t0 = time.perf_counter()
    it = 0
    while True:
        O.barycenter_objective_and_grad(z, X, 1.0)
        it += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"workload": "barycenter K=10 N=M=100 D=3 gamma=1.0, objective and gradient",
            "value": it * 10 * 100 * 100 / dt, "unit": "cells/s", "cores": threads,
            "kind": "oracle", "ms_per_iteration": dt * 1e3 / it,
            "sample": f"{it} iterations, {dt:.1f} s wall"}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.cells)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the workload runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch
    from differentiable_series_alignment_amd import _lib as L
    from differentiable_series_alignment_amd import SoftDTW, softdtw_barycenter
    from sdtw_inputs import block_waves, pair_batch

    L.lib()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.profile_workload:
        profile_workload(torch, L, pair_batch, args.profile_workload, 5)
        return
    dev = torch.device("cuda:0")
    W = WORKLOAD
    B, N, M, D, gamma = W["B"], W["N"], W["M"], W["D"], W["gamma"]
    xc, yc = pair_batch(B, N, M, D, seed=0)
    x, y = xc.to(dev), yc.to(dev)
    cells = B * N * M
    if args.counter_pass:
        counter_pass(torch, L, pair_batch, args.counter_pass)
        return

    ms, fwd, bwd, stream = measure(L, torch, x, y, gamma, L.SDTW_MODE_UNFUSED,
                                   args.steps, args.warmup)
    value = cells / (ms * 1e-3)

    # Per-launch durations: HIP events that the library records around each
    # of its launches, on the stream it launches on.
    L.sdtw_timing(True)
    per_kernel = {}
    for it in range(args.warmup + args.steps):
        fwd()
        bwd()
        recs = L.sdtw_timing_collect()
        if it >= args.warmup:
            for name, t in recs:
                per_kernel.setdefault(name, []).append(t)
    L.sdtw_timing(False)
    kernels = {k: {"launches_per_step": len(v) / args.steps, "avg_us": 1e3 * sum(v) / len(v)}
               for k, v in per_kernel.items()}
    dom_ms = sum(per_kernel[DOMINANT]) / len(per_kernel[DOMINANT])
    achieved = ALU_SLOTS_PER_CELL * cells / (dom_ms * 1e-3) / 1e12
    # The distance kernel against both of its roofs: HBM on its algorithmic
    # bytes (the fp32 distances written, x and y read once) and fp64 MFMA on
    # its 2*D flops per cell.
    dist_ms = sum(per_kernel["dist_skew"]) / len(per_kernel["dist_skew"])
    dist_bytes = 4 * cells + 4 * B * (N + M) * D
    dist_gbs = dist_bytes / (dist_ms * 1e-3) / 1e9
    dist_tflops = 2 * cells * D / (dist_ms * 1e-3) / 1e12
    dist = {"kernel": "distances into the band-step layout (k_dist)", "launch_us": dist_ms * 1e3,
            "algorithmic_bytes": dist_bytes, "achieved_gbs": dist_gbs,
            "frac_hbm": dist_gbs * 1e9 / PEAK_HBM, "achieved_tflops": dist_tflops,
            "frac_f64_mfma": dist_tflops * 1e12 / PEAK_F64_MFMA,
            "min_us_f64_mfma": 2 * cells * D / PEAK_F64_MFMA * 1e6,
            "min_us_hbm": dist_bytes / PEAK_HBM * 1e6}

    peak, peak_over = peak_mib(torch, SoftDTW, x, y, gamma, False)
    ms_f, _, _, _ = measure(L, torch, x, y, gamma, L.SDTW_MODE_FUSED,
                            max(5, args.steps // 5), 2)
    peak_f, peak_over_f = peak_mib(torch, SoftDTW, x, y, gamma, True)
    ms_lm, _, _, _ = measure(L, torch, x, y, gamma, L.SDTW_MODE_UNFUSED_LOWMEM,
                             max(5, args.steps // 5), 2)
    peak_lm, peak_over_lm = peak_mib(torch, SoftDTW, x, y, gamma, False, low_memory=True)
    infer = measure_inference(L, torch, x, y, gamma, max(5, args.steps // 5), 2)

    per_config = []
    if not args.headline_only:
        for (b_, n_, m_, d_, g_) in CONFIGS:
            xc2, yc2 = pair_batch(b_, n_, m_, d_, seed=0)
            x2, y2 = xc2.to(dev), yc2.to(dev)
            entry = {"workload": f"B={b_} N={n_} M={m_} D={d_} gamma={g_}"}
            for mode, name in ((L.SDTW_MODE_UNFUSED, "unfused"), (L.SDTW_MODE_FUSED, "fused"),
                               (L.SDTW_MODE_CHECKPOINT, "checkpoint"),
                               (L.SDTW_MODE_UNFUSED_LOWMEM, "unfused_low_memory")):
                t, _, _, _ = measure(L, torch, x2, y2, g_, mode, 5, 2)
                pk, pko = peak_mib(torch, SoftDTW, x2, y2, g_, mode == L.SDTW_MODE_FUSED,
                                   mode == L.SDTW_MODE_CHECKPOINT,
                                   mode == L.SDTW_MODE_UNFUSED_LOWMEM)
                entry[name] = {"ms_per_step": t, "cells_per_s": b_ * n_ * m_ / (t * 1e-3),
                               "peak_mib": pk, "peak_mib_over_io": pko}
                if mode in (L.SDTW_MODE_UNFUSED, L.SDTW_MODE_FUSED):
                    with_bounds(entry[name], b_, n_, m_, d_, mode == L.SDTW_MODE_FUSED)
            entry["inference"] = measure_inference(L, torch, x2, y2, g_, 5, 2)
            per_config.append(entry)
            del x2, y2
            torch.cuda.empty_cache()
        per_config.append(barycenter_rate(torch, softdtw_barycenter, block_waves))

    out = {
        "metric": "SoftDTW fwd+bwd DP cells/s (B*N*M/s) at B=32,N=M=512,D=64; peak MB",
        "value": value,
        "unit": "cells/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64 DP state + f32 exp/log; f64-accumulated distances; f32 chain rule",
        "data": "synthetic",
        "config": {"workload": "B=32 N=M=512 D=64 gamma=1.0 unfused fwd+bwd, batch-mean loss",
                   "B": B, "N": N, "M": M, "D": D, "gamma": gamma, "mode": "unfused"},
        "peak_mib": peak,
        "peak_mib_over_io": peak_over,
        "fused": with_bounds({"ms_per_step": ms_f, "cells_per_s": cells / (ms_f * 1e-3),
                              "peak_mib": peak_f, "peak_mib_over_io": peak_over_f},
                             B, N, M, D, True),
        "unfused_low_memory": {"ms_per_step": ms_lm, "cells_per_s": cells / (ms_lm * 1e-3),
                               "peak_mib": peak_lm, "peak_mib_over_io": peak_over_lm},
        "bounds": with_bounds({"ms_per_step": ms}, B, N, M, D, False),
        "inference": infer,
        "roofline": {"kernel": "both sweeps of the dynamic programme (k_dp_unfused)",
                     "bound": "alu", "achieved": achieved, "peak": PEAK_ALU_TOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_ALU_TOPS,
                     "ops_per_cell": ALU_SLOTS_PER_CELL,
                     "ops_note": f"{TRANS_PER_CELL} transcendentals x 4 issue slots + "
                                 f"{OTHER_OPS_PER_CELL} other lane operations per cell "
                                 "(fwd+bwd DP), against 39.3 T lane slots/s",
                     "frac_at_28_ops": DP_OPS_PER_CELL * cells / (dom_ms * 1e-3) / 1e12
                                       / PEAK_ALU_TOPS,
                     "traffic": recorded_traffic(), "traffic_unit": "bytes per launch",
                     "launch_us": dom_ms * 1e3,
                     "algorithmic_gbs": DP_BYTES_PER_CELL * cells / (dom_ms * 1e-3) / 1e9},
        "dist": dist,
        "kernels": kernels,
        "per_config": per_config,
    }
    if not args.no_cpu_baseline:
        cb = cpu_baseline(xc, yc, gamma, args.cpu_seconds)
        cb["one_core"] = cpu_one_core(xc, yc, gamma, args.cpu_seconds)
        if not args.headline_only:
            # Every other configuration, at least one call of min(B, threads)
            # pairs each (the long ones take a few seconds).
            cb["per_config"] = []
            for (b_, n_, m_, d_, g_) in CONFIGS:
                xc2, yc2 = pair_batch(b_, n_, m_, d_, seed=0)
                r = cpu_baseline(xc2, yc2, g_, 1.0, warm=False)
                r["workload"] = f"B={b_} N={n_} M={m_} D={d_} gamma={g_}"
                cb["per_config"].append(r)
            cb["per_config"].append(barycenter_cpu_rate(block_waves, 2.0))
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
