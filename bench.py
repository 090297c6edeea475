#!/usr/bin/env python3
"""Benchmark of the fp8 rowwise-scaled grouped GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one call of the grouped GEMM (group resolution, K loop, scaled
epilogue) over one batch of the workload's inputs, which are resident in HBM
before timing starts.  Prints ONE JSON line on stdout; diagnostics go to stderr.

The default workload is the dense expert (G=4, 512 rows per group, N=8192,
K=28672) through the pre-shuffled-weight entry point (weights shuffled once
before timing, as at weight load).

Timing: a clock ramp (at least 0.5 s of untimed calls, synchronised in small
batches, so that the GPU clock has settled), W counted untimed warm-up calls,
then exactly K timed calls bracketed by device synchronisation.  Each call is
also bracketed by HIP events recorded on the stream the kernel runs on, which
gives the kernel's average duration for the roofline figure.  When a workload's
bytes are small against the 256 MB Infinity Cache, calls rotate over several
copies of the inputs.  The same calls are then also timed under graph replay:
enough calls captured into one HIP graph for a replay to last about 2 ms, a clock
ramp of replays, then seven replays each bracketed by HIP events; the median per
call is reported with its minimum, interquartile range and T*/T (T* the roofline
time of the call).  The extra keys (plain weights, gate_up, padded tails, the
down-projection sweep, the quantiser) are timed that way only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fp8 rowwise grouped GEMM TFLOPS (valid rows), % fp8 MFMA peak; µs/call at M<=32"
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
MALL_BYTES = 256 * 2 ** 20    # Infinity Cache
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")

WORKLOADS = ["moe_gate_up", "moe_gate_up_preshuffle", "tiny_stacked", "dense_expert", "dense_expert_preshuffle", "padded_tails",
             "moe_gate_up_offsets", "dense_expert_batched", "moe_n_offsets", "moe_wgrad_k_offsets", "moe_gate_up_blockscale",
             "moe_gate_up_blockscale_preshuffle", "padded_blockscale"] + \
    [f"moe_down_M{m}" for m in (1, 8, 32, 256, 2048, 8192)]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make_workload(name):
    import workloads as wl
    if name == "moe_gate_up":
        return wl.moe_gate_up(), "stacked", False
    if name == "moe_gate_up_preshuffle":
        w = wl.moe_gate_up()
        w.name += "_preshuffle"
        return w, "stacked", True
    if name == "tiny_stacked":
        return wl.tiny_stacked(), "stacked", False
    if name == "dense_expert":
        return wl.dense_expert(), "stacked", False
    if name == "dense_expert_preshuffle":
        return wl.dense_expert(), "stacked", True
    if name == "padded_tails":
        return wl.padded_tails(), "padded", False
    if name == "moe_gate_up_offsets":
        # the same inputs, group boundaries given as an int32 inclusive prefix sum
        w = wl.moe_gate_up()
        w.name += "_offsets"
        return w, "offsets", False
    if name == "dense_expert_batched":
        # every group a full slab of 512 rows: the batched (3D-3D) layout
        w = wl.dense_expert()
        w.name += "_batched"
        return w, "batched", False
    if name == "moe_gate_up_blockscale":
        return wl.moe_gate_up_blockscale(), "blockscale", False
    if name == "moe_gate_up_blockscale_preshuffle":
        return wl.moe_gate_up_blockscale(), "blockscale", True
    if name == "padded_blockscale":
        return wl.padded_blockscale(), "padded_blockscale", False
    if name == "moe_n_offsets":
        return wl.moe_n_offsets(), "n_offsets", False
    if name == "moe_wgrad_k_offsets":
        return wl.moe_wgrad_k_offsets(), "k_offsets", False
    if name.startswith("moe_down_M"):
        return wl.moe_down(int(name[len("moe_down_M"):])), "stacked", False
    raise ValueError(name)


def algorithmic_work(w, layout):
    """flop = 2 N K R; bytes = R K + G_ne N K + 4 R + 4 G_ne N + 2 N R_out + 8 G.

    R = valid rows, G_ne = groups with a valid row, R_out = rows written (valid
    rows plus zeroed padding rows).  Unread weights of empty groups and unread
    padding inputs are not counted."""
    import numpy as np
    G, N, K = w.G, w.N, w.K
    if layout == "n_offsets":
        # groups own W rows: R = M rows per slab, N_valid columns, slabs of groups with columns read
        ends = np.minimum(np.maximum.accumulate(np.maximum(w.n_offsets.astype(np.int64), 0)), N)
        widths = np.diff(np.concatenate([[0], ends]))
        n_valid, g_ne, M = int(widths.sum()), int((widths > 0).sum()), w.M
        flop = 2 * M * K * n_valid
        nbytes = g_ne * M * K + n_valid * K + 4 * g_ne * M + 4 * n_valid + 2 * M * n_valid + 4 * G
        return flop, nbytes, M, g_ne
    if layout == "k_offsets":
        # groups slice K: every group writes a whole [M, N] output
        ends = np.minimum(np.maximum.accumulate(np.maximum(w.k_offsets.astype(np.int64), 0)), K)
        k_valid, M = int(ends[-1]) if G else 0, w.M
        flop = 2 * M * N * k_valid
        nbytes = M * k_valid + N * k_valid + 4 * G * M + 4 * G * N + 2 * G * M * N + 4 * G
        return flop, nbytes, G * M, G
    if layout == "blockscale":
        # stacked rows; one scale per (row, K block) and per (128 x 128) W block
        sizes = np.clip(w.M_sizes, 0, None)
        R, g_ne, nkb = int(sizes.sum()), int((sizes > 0).sum()), K // w.block_k
        flop = 2 * N * K * R
        nbytes = R * K + g_ne * N * K + 4 * R * nkb + 4 * g_ne * (N // w.block_n) * nkb + 2 * N * R + 8 * G
        return flop, nbytes, R, g_ne
    if layout == "padded_blockscale":
        # padded slabs, zeroed padding rows written; block scales per (row, K block) and W block
        em = w.expected_m
        valid = np.clip(w.zero_start_index_M, 0, em)
        R, g_ne, nkb = int(valid.sum()), int((valid > 0).sum()), K // 128
        flop = 2 * N * K * R
        nbytes = R * K + g_ne * N * K + 4 * R * nkb + 4 * g_ne * (N // 128) * nkb + 2 * N * G * em + 8 * G
        return flop, nbytes, R, g_ne
    if layout in ("stacked", "offsets", "batched"):
        sizes = np.clip(w.M_sizes, 0, None)
        R = int(min(sizes.sum(), w.total_M))
        G_ne = int(np.count_nonzero(sizes))
        R_out = R
    else:
        z = np.clip(w.zero_start_index_M, 0, w.expected_m)
        R = int(z.sum())
        G_ne = int(np.count_nonzero(z))
        R_out = G * w.expected_m
    flop = 2 * N * K * R
    nbytes = R * K + G_ne * N * K + 4 * R + 4 * G_ne * N + 2 * N * R_out + 8 * G
    return flop, nbytes, R, G_ne


def offsets_of(w):
    """int32 inclusive prefix sums of a stacked workload's group row counts."""
    import numpy as np
    return np.cumsum(np.clip(w.M_sizes, 0, None)).astype(np.int32)


# Sources that decide what the GEMM kernels do on a workload (kernels, selector,
# shared header); the activation quantiser is built from its own file.
GEMM_SOURCES = ("fp8gg_api.cpp", "fp8gg_internal.h", "fp8gg_kernels.hip")


def group_meta(w, layout):
    """The workload's group metadata as a list (row counts, valid rows or offsets)."""
    if layout in ("padded", "padded_blockscale"):
        return w.zero_start_index_M.tolist()
    if layout == "n_offsets":
        return w.n_offsets.tolist()
    if layout == "k_offsets":
        return w.k_offsets.tolist()
    return w.M_sizes.tolist()


def kernel_source_hash():
    csrc = os.path.join(ROOT, "fp8_rowwise_scaled_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f in GEMM_SOURCES:
            with open(os.path.join(csrc, f), "rb") as fh:
                h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, src_hash):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None
    when there is none for this workload or the kernels changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get("workloads", {}).get(workload)
    if not e or e.get("kernel_hash") != src_hash:
        return None
    return e.get("hbm_bytes_per_launch")


def _blas_info():
    """(vendor, threads) of numpy's BLAS as threadpoolctl reports it."""
    try:
        from threadpoolctl import threadpool_info
        for i in threadpool_info():
            if i.get("user_api") == "blas":
                return f"{i.get('internal_api')} {i.get('version')}", int(i.get("num_threads") or 1)
    except Exception:  # pragma: no cover
        pass
    return "unknown", 1


def _oracle_call(w, layout):
    import oracle
    if layout == "stacked":
        oracle.grouped_stacked(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    elif layout == "offsets":
        oracle.grouped_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, offsets_of(w))
    elif layout == "batched":
        M = w.total_M // w.G
        oracle.grouped_batched(w.XQ.reshape(w.G, M, w.K), w.WQ, w.x_scale.reshape(w.G, M), w.w_scale)
    elif layout == "blockscale":
        oracle.grouped_stacked_blockscale(w.XQ, w.WQ, w.x_scale, w.w_scale, w.M_sizes)
    elif layout == "padded_blockscale":
        oracle.grouped_dynamic_blockscale(w.XQ, w.WQ, w.x_scale, w.w_scale, w.zero_start_index_M, True)
    elif layout == "n_offsets":
        oracle.grouped_n_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, w.n_offsets)
    elif layout == "k_offsets":
        oracle.grouped_k_offsets(w.XQ, w.WQ, w.x_scale, w.w_scale, w.k_offsets)
    else:
        oracle.grouped_dynamic(w.XQ, w.WQ, w.x_scale, w.w_scale, w.zero_start_index_M, True)


def cpu_baseline(w, layout, flop, min_seconds=10.0, max_runs=50, single_thread=True):
    """The oracle as it stands on this host's cores: whole calls of the workload
    repeated until about min_seconds of CPU work (at least one call), with numpy's
    BLAS on every core of the process's affinity mask; then, single-threaded, the
    tiny workload and the down projection at total_M = 1, 8, 32."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        cores = os.cpu_count() or 1
    vendor, blas_threads = _blas_info()
    times = []
    t_all = time.perf_counter()
    while len(times) < max_runs and (time.perf_counter() - t_all) < min_seconds:
        t0 = time.perf_counter()
        _oracle_call(w, layout)
        times.append(time.perf_counter() - t0)
    med = statistics.median(times)
    out = {"value": round(flop / med / 1e12, 6), "unit": "TFLOP/s", "cores": int(blas_threads), "kind": "oracle",
           "sample": f"the full workload, {len(times)} whole call(s) over {sum(times):.1f} s, "
                     f"median {med:.3f} s per call "
                     "(e4m3fn table decode, fp64 matmul per group, fp64 scales, bf16 RNE)",
           "affinity_cores": cores, "blas": vendor, "s_per_call": round(med, 4)}
    if single_thread:
        import workloads as wl
        from threadpoolctl import threadpool_limits
        st = {}
        with threadpool_limits(limits=1):
            for name, make in [("tiny_stacked", wl.tiny_stacked)] + \
                    [(f"moe_down_M{m}", lambda m=m: wl.moe_down(m)) for m in (1, 8, 32)]:
                wx = make()
                runs = []
                t_all = time.perf_counter()
                while len(runs) < 5 and (time.perf_counter() - t_all) < 3.0:
                    t0 = time.perf_counter()
                    _oracle_call(wx, "stacked")
                    runs.append(time.perf_counter() - t0)
                st[name] = {"s_per_call": round(statistics.median(runs), 5), "calls": len(runs)}
        out["single_thread"] = st
        log("CPU oracle, one thread: " + ", ".join(f"{k} {v['s_per_call'] * 1e3:.1f} ms" for k, v in st.items()))
    log(f"CPU oracle: {out['value']:.4f} TFLOP/s, {med:.2f} s per call, BLAS {vendor} on {blas_threads} threads, "
        f"{cores} cores in the affinity mask")
    return out


def ramp(fn, seconds, batch):
    """Untimed calls, synchronised every `batch` calls, until `seconds` of wall time
    have passed: the GPU runs the workload continuously for that long, so its clock
    has settled before anything is timed."""
    import torch
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            fn(i)
            i += 1
        torch.cuda.synchronize()
    return time.perf_counter() - t0, i


def graph_stats(torch, call, ramp_s, flop, nbytes, target_us=2000.0, replays=7):
    """Per-call time under graph replay: enough calls captured into one HIP graph for
    a replay to last about `target_us`, replayed for a clock ramp, then `replays`
    replays each bracketed by HIP events.  Returns the median per-call time with its
    minimum and interquartile range, and T*/T for the roofline time
    T* = max(flop / fp8 peak, bytes / HBM peak)."""
    call(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(3):
        call(i)
    e1.record()
    torch.cuda.synchronize()
    est_us = max(e0.elapsed_time(e1) * 1e3 / 3, 1.0)
    n = max(1, min(512, math.ceil(target_us / est_us)))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            call(i)
    ramp(lambda i: g.replay(), ramp_s, 2)
    per_call = []
    for _ in range(replays):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) * 1e3 / n)
    del g
    q1, _, q3 = statistics.quantiles(per_call, n=4)
    med = statistics.median(per_call)
    t_star = max(flop / (PEAK_FP8_TFLOPS * 1e6), nbytes / (PEAK_HBM_GBS * 1e3))   # µs
    return {"us_per_call": round(med, 3), "us_min": round(min(per_call), 3), "us_iqr": round(q3 - q1, 3),
            "calls_per_graph": n, "replays": replays, "t_star_over_t": round(t_star / med, 4)}


def prepare(F, torch, w, layout, pre, rotate):
    """Device copies of the workload's inputs (`rotate` sets, resident in HBM) and
    call(i), one call of the grouped GEMM on set i % rotate."""
    dev = torch.device("cuda", 0)
    X = torch.from_numpy(w.XQ).to(dev)
    Wt = torch.from_numpy(w.WQ).to(dev)
    xs = torch.from_numpy(w.x_scale).to(dev)
    ws = torch.from_numpy(w.w_scale).to(dev)
    if layout == "n_offsets":
        meta = torch.from_numpy(w.n_offsets).to(dev)
    elif layout == "k_offsets":
        meta = torch.from_numpy(w.k_offsets).to(dev)
    elif layout == "offsets":
        meta = torch.from_numpy(offsets_of(w)).to(dev)
    elif layout == "blockscale":
        meta = torch.from_numpy(w.M_sizes).to(dev)
    elif layout == "padded_blockscale":
        meta = torch.from_numpy(w.zero_start_index_M).to(dev)
    elif layout == "batched":
        meta = torch.zeros(1, dtype=torch.int64, device=dev)   # the batched layout has no metadata
        Gb, Mb = w.G, w.total_M // w.G
        X = X.view(Gb, Mb, w.K)
        xs = xs.view(Gb, Mb)
    else:
        meta = torch.from_numpy(w.M_sizes if layout == "stacked" else w.zero_start_index_M).to(dev)
    if pre:
        Wt = F.f8f8bf16_shuffle_b(Wt)
    sets = [(X, Wt, xs, ws, meta)]
    for _ in range(rotate - 1):
        sets.append(tuple(t.clone() for t in sets[0]))
    out_shape = {"stacked": lambda: (w.total_M, w.N), "offsets": lambda: (w.total_M, w.N),
                 "blockscale": lambda: (w.total_M, w.N),
                 "padded_blockscale": lambda: (w.G, w.expected_m, w.N),
                 "batched": lambda: (w.G, w.total_M // w.G, w.N), "n_offsets": lambda: (w.M, w.N),
                 "k_offsets": lambda: (w.G, w.M, w.N),
                 "padded": lambda: (w.G, w.expected_m, w.N)}[layout]()
    outs = [torch.empty(out_shape, dtype=torch.bfloat16, device=dev) for _ in range(rotate)]
    padded = layout in ("padded", "padded_blockscale")
    fn = {("stacked", False): F.f8f8bf16_rowwise_grouped_stacked,
          ("stacked", True): F.f8f8bf16_rowwise_grouped_stacked_preshuffle,
          ("offsets", False): F.f8f8bf16_rowwise_grouped_offsets,
          ("offsets", True): F.f8f8bf16_rowwise_grouped_offsets_preshuffle,
          ("batched", False): F.f8f8bf16_rowwise_grouped_batched,
          ("batched", True): F.f8f8bf16_rowwise_grouped_batched_preshuffle,
          ("padded", False): F.f8f8bf16_rowwise_grouped_dynamic,
          ("padded", True): F.f8f8bf16_rowwise_grouped_dynamic_preshuffle,
          ("blockscale", False): F.f8f8bf16_groupwise_grouped_stacked,
          ("blockscale", True): F.f8f8bf16_groupwise_grouped_stacked_preshuffle,
          ("padded_blockscale", False): F.f8f8bf16_groupwise_grouped_dynamic,
          ("padded_blockscale", True): F.f8f8bf16_groupwise_grouped_dynamic_preshuffle,
          ("n_offsets", False): F.f8f8bf16_rowwise_grouped_n_offsets,
          ("k_offsets", False): F.f8f8bf16_rowwise_grouped_k_offsets}[(layout, pre)]

    def call(i):
        s = sets[i % rotate]
        if layout == "batched":
            fn(s[0], s[1], s[2], s[3], out=outs[i % rotate])
        elif padded:
            fn(s[0], s[1], s[2], s[3], s[4], zeroing_output_tensor=True, out=outs[i % rotate])
        else:
            fn(s[0], s[1], s[2], s[3], s[4], out=outs[i % rotate])
    return call


def time_eager(torch, call, steps, warmup, ramp_s):
    """Clock ramp, `warmup` counted untimed calls, then exactly `steps` timed calls
    between device synchronisations, each bracketed by HIP events on the stream
    the kernels are launched on (the current stream)."""
    stream = torch.cuda.current_stream()
    ramp_done, ramp_calls = ramp(call, ramp_s, 8)
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        call(i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    durs = [s.elapsed_time(e) * 1e-3 for s, e in zip(starts, ends)]
    region = starts[0].elapsed_time(ends[-1]) * 1e-3 / steps
    return {"wall": wall, "durs": durs, "avg": sum(durs) / len(durs), "median": statistics.median(durs),
            "min": min(durs), "region": region, "ramp_s": ramp_done, "ramp_calls": ramp_calls}


def roofline_of(flop, nbytes, avg, traffic):
    mfma_bound = flop / (PEAK_FP8_TFLOPS * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9)
    if mfma_bound:
        achieved = flop / avg / 1e12
        return {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_FP8_TFLOPS, 4), "traffic": traffic}
    achieved = nbytes / avg / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic}


def auto_rotate(nbytes):
    """Input copies so that the calls together touch twice the Infinity Cache."""
    return max(1, min(64, math.ceil(2 * MALL_BYTES / max(nbytes, 1))))


def rates(flop, nbytes, us):
    """TFLOP/s over valid rows and GB/s of algorithmic bytes at `us` per call, with
    their fractions of the fp8 MFMA and HBM peaks."""
    return {"TFLOP_per_s": round(flop / us / 1e6, 1), "mfma_frac": round(flop / us / 1e6 / PEAK_FP8_TFLOPS, 4),
            "GB_per_s": round(nbytes / us / 1e3, 1), "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4)}


def extra_workload(F, torch, name, ramp_s):
    """A further workload for the extra keys of the JSON line, timed under graph
    replay (median of seven replays with min and IQR, rotating over enough input
    copies to defeat the Infinity Cache)."""
    w, layout, pre = make_workload(name)
    flop, nbytes, R, _ = algorithmic_work(w, layout)
    rot = auto_rotate(nbytes)
    call = prepare(F, torch, w, layout, pre, rot)
    st = graph_stats(torch, call, ramp_s, flop, nbytes)
    r = {"workload": w.name, **st, **rates(flop, nbytes, st["us_per_call"]), "input_copies": rot}
    log(f"{name}: {st['us_per_call']:.2f} us/call (min {st['us_min']:.2f}, IQR {st['us_iqr']:.2f}), "
        f"{r['TFLOP_per_s']} TFLOP/s ({r['mfma_frac']:.1%}), {r['GB_per_s']} GB/s ({r['hbm_frac']:.1%}), "
        f"T*/T {st['t_star_over_t']:.2f}")
    del call
    torch.cuda.empty_cache()
    return r


def small_m_us_per_call(F, torch, ramp_s, totals=(1, 8, 32, 256, 2048, 8192)):
    """µs per call of the down-proj workload at each total_M, timed as the pages time
    decode-sized GEMMs: many calls captured in one HIP graph (rotating over enough
    input copies to defeat the Infinity Cache), replayed, divided by the call count."""
    import workloads as wl
    out = {}
    for m in totals:
        w = wl.moe_down(m)
        flop, nbytes, _, _ = algorithmic_work(w, "stacked")
        rot = auto_rotate(nbytes)
        call = prepare(F, torch, w, "stacked", False, rot)
        st = graph_stats(torch, call, ramp_s, flop, nbytes)
        us = st["us_per_call"]
        out[f"moe_down_M{m}"] = {**st, **rates(flop, nbytes, us), "input_copies": rot}
        log(f"down-proj M={m}: {us:.2f} us/call under graph replay (min {st['us_min']:.2f}, IQR "
            f"{st['us_iqr']:.2f}; {nbytes / us / 1e3:.0f} GB/s, {flop / us / 1e6:.0f} TFLOP/s, {rot} input copies, "
            f"T*/T {st['t_star_over_t']:.2f})")
        del call
        torch.cuda.empty_cache()
    return out


def quantize_us_per_call(F, torch, ramp_s, rows=4096, K=7168, eager_steps=0, warmup=20):
    """The rowwise activation quantiser (bf16 [rows, K] -> e4m3fn codes + fp32 row
    scales) on the gate_up activations' shape, rotating over enough input copies to
    defeat the Infinity Cache.  HBM-bound: 2 bytes read and 1 written per element,
    4 bytes written per row.  Timed under graph replay, or, with eager_steps > 0,
    as that many eager calls with HIP events around each (for profiler runs, whose
    counters are taken per dispatch)."""
    dev = torch.device("cuda", 0)
    nbytes = 3 * rows * K + 4 * rows
    rot = max(1, min(16, math.ceil(2 * MALL_BYTES / nbytes)))
    gen = torch.Generator(device=dev)
    gen.manual_seed(7001)
    xs = [torch.randn((rows, K), generator=gen, device=dev, dtype=torch.float32).to(torch.bfloat16)
          for _ in range(rot)]
    qs = [torch.empty((rows, K), dtype=torch.uint8, device=dev) for _ in range(rot)]
    ss = [torch.empty((rows,), dtype=torch.float32, device=dev) for _ in range(rot)]

    def call(i):
        F.f8f8bf16_quantize_rowwise(xs[i % rot], qs[i % rot], ss[i % rot])
    if eager_steps > 0:
        t = time_eager(torch, call, eager_steps, warmup, ramp_s)
        us = t["avg"] * 1e6
        log(f"quantize: bf16 [{rows}, {K}] -> e4m3fn: {us:.2f} us/call over {eager_steps} eager calls "
            f"({nbytes / us / 1e3:.0f} GB/s, {rot} input copies)")
        del xs, qs, ss
        return {"shape": [rows, K], "us_per_call": round(us, 3), "eager_calls": eager_steps,
                "GB_per_s": round(nbytes / us / 1e3, 1), "hbm_frac": round(nbytes / us / 1e3 / PEAK_HBM_GBS, 4),
                "input_copies": rot}
    st = graph_stats(torch, call, ramp_s, 0, nbytes)
    us = st["us_per_call"]
    gbs = nbytes / us / 1e3
    log(f"quantize: bf16 [{rows}, {K}] -> e4m3fn: {us:.2f} us/call under graph replay (min {st['us_min']:.2f}, "
        f"IQR {st['us_iqr']:.2f}; {gbs:.0f} GB/s, {rot} input copies)")
    del xs, qs, ss
    return {"shape": [rows, K], **st, "GB_per_s": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "input_copies": rot}


def copy_calibration(nbytes):
    """A plain device copy of known size, profiled beside the GEMM to scale the
    HBM byte counters."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: {nbytes} bytes read and written per copy, 5 copies")


DEFAULT_WORKLOAD = "dense_expert_preshuffle"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=WORKLOADS)
    ap.add_argument("--ramp", type=float, default=1.0,
                    help="seconds of untimed calls before the counted warm-up (default 1.0; shorter only for "
                         "profiler runs)")
    ap.add_argument("--rotate", type=int, default=0, help="input copies to rotate over (0 = automatic)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the extra workloads (plain W, gate_up, padded tails, down-proj sweep, quantiser)")
    ap.add_argument("--no-small-m", action="store_true", help="same as --no-extras")
    ap.add_argument("--quantize-only", action="store_true",
                    help="time only the rowwise activation quantiser, as --steps eager calls after --warmup "
                         "(for profiler runs); prints {\"quantize\": ...}")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain copy of this many bytes (for counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: --gpus {args.gpus} is not supported (the library has no "
              "multi-GPU path; the grouped GEMM shards by expert group, one process per GPU).", file=sys.stderr)
        sys.exit(2)
    ramp_s = max(0.0, args.ramp)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import fp8_rowwise_scaled_amd as F

    F.load()
    if args.quantize_only:
        print(json.dumps({"quantize": quantize_us_per_call(F, torch, ramp_s, eager_steps=max(1, args.steps),
                                                           warmup=args.warmup)}), flush=True)
        return
    w, layout, pre = make_workload(args.workload)
    flop, nbytes, R, G_ne = algorithmic_work(w, layout)
    log(f"workload {w.name}: layout={layout} preshuffled={pre} G={w.G} N={w.N} K={w.K} R={R} G_ne={G_ne} "
        f"flop={flop:.4g} bytes={nbytes:.4g}")
    rotate = args.rotate or auto_rotate(nbytes)
    call = prepare(F, torch, w, layout, pre, rotate)
    log(f"rotating over {rotate} input set(s); clock ramp {ramp_s:.1f} s")
    t = time_eager(torch, call, args.steps, args.warmup, ramp_s)
    avg, wall = t["avg"], t["wall"]
    ms_per_step = wall / args.steps * 1e3
    value = flop / (wall / args.steps) / 1e12
    log(f"ramp: {t['ramp_calls']} calls over {t['ramp_s']:.2f} s")
    log(f"per call: wall {ms_per_step * 1e3:.2f} us, kernel avg {avg * 1e6:.2f} us, median {t['median'] * 1e6:.2f} us, "
        f"min {t['min'] * 1e6:.2f} us, timed region / calls {t['region'] * 1e6:.2f} us")
    src_hash = kernel_source_hash()
    roof = roofline_of(flop, nbytes, avg, measured_traffic(args.workload, src_hash))
    log(f"kernel: {flop / avg / 1e12:.1f} TFLOP/s ({flop / avg / 1e12 / PEAK_FP8_TFLOPS:.1%} of fp8 peak), "
        f"{nbytes / avg / 1e9:.0f} GB/s ({nbytes / avg / 1e9 / PEAK_HBM_GBS:.1%} of HBM); source hash {src_hash}")
    # the same calls under graph replay (median of seven replays, min, IQR, T*/T)
    graph = graph_stats(torch, call, min(ramp_s, 0.5), flop, nbytes)
    log(f"graph replay: {graph['us_per_call']:.2f} us/call (min {graph['us_min']:.2f}, IQR {graph['us_iqr']:.2f}, "
        f"{graph['calls_per_graph']} calls per replay), T*/T {graph['t_star_over_t']:.2f}")
    del call
    torch.cuda.empty_cache()

    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3fn",
        "data": "synthetic",
        "config": {
            "workload": w.name + ("_preshuffle" if pre and not w.name.endswith("_preshuffle") else ""),
            "layout": layout,
            "preshuffled": pre,
            "G": w.G,
            "rows": int(w.G * w.expected_m if layout in ("padded", "padded_blockscale") else
                        (w.M if layout == "n_offsets" else (w.G * w.M if layout == "k_offsets" else w.total_M))),
            "valid_rows": R,
            "N": w.N,
            "K": w.K,
            "group_rows": group_meta(w, layout),
            "rotating_input_sets": rotate,
            "us_per_call": round(avg * 1e6, 3),
            "us_per_call_median": round(t["median"] * 1e6, 3),
            "clock_ramp_s": round(t["ramp_s"], 3),
            "clock_ramp_calls": t["ramp_calls"],
            "graph_replay": {**graph, **rates(flop, nbytes, graph["us_per_call"])},
        },
        "roofline": roof,
    }
    extras = not (args.no_extras or args.no_small_m) and args.workload == DEFAULT_WORKLOAD
    if extras:
        result["dense_expert_plain_w"] = extra_workload(F, torch, "dense_expert", ramp_s)
        result["gate_up"] = extra_workload(F, torch, "moe_gate_up_preshuffle", ramp_s)
        result["padded_tails"] = extra_workload(F, torch, "padded_tails", ramp_s)
        result["small_m"] = small_m_us_per_call(F, torch, ramp_s)
        result["quantize"] = quantize_us_per_call(F, torch, ramp_s)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        result["cpu_baseline"] = cpu_baseline(w, layout, flop, single_thread=extras)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
