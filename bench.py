"""Benchmark: exact attention forward + recompute backward on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
attn_fwd (O and the per-row statistics) followed by attn_bwd (dQ, dK, dV),
both through the C ABI, on the n = 16384 bf16 workload
(B=1, H=16, n=16384, d=64; Q, K, V, dO ~ N(0,1) from a fixed seed).

FLOP convention (algorithmic): forward 4*B*H*n^2*d (QK^T and PV), backward
10*B*H*n^2*d (score recompute, dV, dP, dQ, dK). ``value`` = 14*B*H*n^2*d per
step / step time, in TFLOP/s. Inputs are resident in HBM before timing.

Prints exactly one JSON line on stdout (everything else goes to stderr).
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""

import argparse
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s at n=16384 bf16 on 1 MI355X; % MFMA peak"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0
COPY_BYTES = 256 << 20
DOMINANT_KERNEL = "bwd_main_kernel<64, 8>"


def recorded_figures(kernel):
    """Counter figures of `kernel` from the committed rocprofv3 summaries under
    profiles/ (HBM bytes per launch, MFMA busy, ...), or {} when its source changed
    since they were taken."""
    from memory_efficient_exact_amd import rocprof
    try:
        return rocprof.current_figures(os.path.join(ROOT, "profiles"), kernel)
    except (OSError, ValueError, KeyError):
        return {}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


MIN_WARM_S = 0.2    # warm-up wall time before a timed loop (the clock leaves its idle state)
MIN_BENCH_WARM_S = 0.5  # warm-up wall time before the default mode's timed steps
MIN_TIMED_S = 0.05  # least GPU time of a timed loop


def timed_loop(fn, warmup, steps, dev):
    """Average ms per call of `fn` over back-to-back calls between two HIP events:
    at least `warmup` calls and MIN_WARM_S of warm-up first, then at least `steps`
    calls and MIN_TIMED_S of GPU time. Short calls otherwise run partly at the
    lower clock the GPU drops to while the host prepares inputs."""
    import time

    import torch
    t0, i = time.perf_counter(), 0
    while i < warmup or time.perf_counter() - t0 < MIN_WARM_S:
        fn()
        i += 1
        if i % 16 == 0:
            torch.cuda.synchronize(dev)
    count = steps
    while True:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        e0.record()
        for _ in range(count):
            fn()
        e1.record()
        torch.cuda.synchronize(dev)
        total = e0.elapsed_time(e1)
        if total >= 1e3 * MIN_TIMED_S or count >= 1 << 16:
            return total / count
        count = max(count + 1, int(count * 1e3 * MIN_TIMED_S / max(total, 1e-3)) + 1)


CPU_HEADS = 2  # heads of the workload's shape in the CPU sample (about 12 s of oracle work)


def cpu_baseline(w):
    """The fp64 oracle as it stands, on CPU_HEADS heads of the workload's shape
    (all n query rows, forward then backward), timed on this host's cores."""
    import numpy as np

    import inputgen
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = os.cpu_count() or 1
    t = inputgen.draw(1, CPU_HEADS, w.n, w.d, w.dtype, seed=w.seed, with_do=True)
    q, k, v, do = (inputgen.to_f64(t[x]) for x in ("q", "k", "v", "do"))
    t0 = time.perf_counter()
    oracle.naive_fwd(q, k, v)
    t1 = time.perf_counter()
    oracle.naive_bwd(q, k, v, do)
    t2 = time.perf_counter()
    flops = 14.0 * CPU_HEADS * w.n * w.n * w.d
    return {
        "value": flops / (t2 - t0) / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{CPU_HEADS} heads (B=1, H={CPU_HEADS}, n={w.n}, d={w.d}) of the workload's "
                   f"shape and input distribution, fp64 oracle naive_fwd + naive_bwd over all "
                   f"rows; fwd {t1 - t0:.2f} s, bwd {t2 - t1:.2f} s"),
        "host": {"cpu_count": os.cpu_count(), "affinity": len(os.sched_getaffinity(0)),
                 "machine": platform.processor() or platform.machine()},
    }


def clock_under_load(step, dev, settle_s=1.5, gap_s=1.0):
    """Graphics clocks of the XCDs, read with `amd-smi metric --clock` while `step`
    runs back to back on another thread (after the timed steps, so the timed region
    is undisturbed). The kernels run below the 2.4 GHz the published peak assumes.
    The tool reports a value that trails the load by up to about a second, so it is
    read after `settle_s` of load and again `gap_s` later, and the later reading is
    reported. Returns None when the tool is missing or its output cannot be read."""
    import shutil
    import subprocess
    import threading

    import torch
    tool = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    done = threading.Event()

    def load():
        while not done.is_set():
            step()
            torch.cuda.synchronize(dev)

    def read():
        r = subprocess.run([tool, "metric", "--clock", "--json"], capture_output=True, text=True,
                           timeout=60)
        data = json.loads(r.stdout)
        gpus = data.get("gpu_data", data) if isinstance(data, dict) else data
        clocks = gpus[0]["clock"]
        return [float(v["clk"]["value"]) for key, v in clocks.items()
                if key.startswith("gfx_") and isinstance(v, dict) and "clk" in v]

    th = threading.Thread(target=load)
    th.start()
    try:
        time.sleep(settle_s)
        first = read()
        time.sleep(gap_s)
        mhz = read()
    except (OSError, ValueError, KeyError, IndexError, TypeError, subprocess.SubprocessError):
        return None
    finally:
        done.set()
        th.join()
    if not mhz:
        return None
    mean = statistics.mean(mhz)
    return {"gfx_mhz_mean": mean, "gfx_mhz_min": min(mhz), "gfx_mhz_max": max(mhz),
            "xcds": len(mhz), "earlier_reading_mhz_mean": statistics.mean(first) if first else None,
            "peak_bf16_tflops_at_clock": PEAK_BF16_TFLOPS * mean / 2400.0,
            "source": f"amd-smi metric --clock after {settle_s + gap_s:.1f} s of the step run back "
                      "to back, after the timed steps"}


def sweep_configs(steps, warmup):
    """Per workload: forward and backward time, TFLOP/s, peak extra device
    memory beyond inputs and outputs, and the n^2 fp32 score-matrix size."""
    import torch

    import inputgen
    import memory_efficient_exact_amd as mea
    dev = torch.device("cuda:0")
    rows = []
    for name, w in inputgen.WORKLOADS.items():
        t = inputgen.make_inputs(w, with_do=True)
        q, k, v, do = (t[x].to(dev) for x in ("q", "k", "v", "do"))
        o = torch.empty_like(q)
        m = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        l = torch.empty_like(m)
        row = {"workload": name, "B": w.B, "H": w.H, "n": w.n, "d": w.d, "dtype": w.dtype,
               "n2_fp32_score_bytes": 4 * w.B * w.H * w.n * w.n}
        torch.cuda.synchronize(dev)
        before = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)

        def timed(fn):
            return timed_loop(fn, warmup, steps, dev)

        fms = timed(lambda: mea.attn_fwd(q, k, v, out=o, row_max=m, row_sum=l))
        row["fwd_ms"] = fms
        row["fwd_tflops"] = w.fwd_flops() / (fms * 1e-3) / 1e12
        row["fwd_peak_extra_bytes"] = torch.cuda.max_memory_allocated(dev) - before
        # every workload also times the backward (the training workload is the one whose
        # step includes it; for the others it is reported as extra information)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        dt = mea.DTYPE_BF16 if w.dtype == "bf16" else mea.DTYPE_F32
        ws = torch.empty(mea.attn_bwd_workspace_bytes(dt, w.B, w.H, w.n, w.d),
                         dtype=torch.uint8, device=dev)
        before = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        bms = timed(lambda: mea.attn_bwd(q, k, v, o, do, m, l, dq=dq, dk=dk, dv=dv, workspace=ws))
        row["bwd_ms"] = bms
        row["bwd_tflops"] = w.bwd_flops() / (bms * 1e-3) / 1e12
        row["workspace_bytes"] = ws.numel()
        row["bwd_peak_extra_bytes"] = torch.cuda.max_memory_allocated(dev) - before
        row["stats_bytes"] = m.numel() * 8
        rows.append(row)
        log(json.dumps(row))
        del t, q, k, v, do, o, m, l
        torch.cuda.empty_cache()
    return {"mode": "configs", "steps": steps, "warmup": warmup, "min_warm_s": MIN_WARM_S,
            "min_timed_s": MIN_TIMED_S, "rows": rows}


# Shapes for the split-key / grouped-query sweep: (name, B, H, H_kv, n_q, n_k, d, dtype, backward).
# The decoding rows are one new query per head against a long key/value cache
# with 4 query heads per key/value head, the grouped layout the pages' KV-cache
# section describes; the prefill row is the same grouping at n_q = n_k.
SPLIT_CASES = [
    ("single_head_fp32_1024", 1, 1, 1, 1024, 1024, 64, "fp32", False),
    ("multihead_bf16_4096", 4, 8, 8, 4096, 4096, 64, "bf16", False),
    ("decode_gqa_bf16_d128_16k", 1, 32, 8, 1, 16384, 128, "bf16", False),
    ("decode_gqa_bf16_d128_128k_b4", 4, 32, 8, 1, 131072, 128, "bf16", False),
    ("decode_gqa_bf16_d64_32k_b8", 8, 32, 8, 1, 32768, 64, "bf16", False),
    ("decode_gqa_fp32_d128_16k", 1, 32, 8, 1, 16384, 128, "fp32", False),
    ("prefill_gqa_bf16_d128_8k", 1, 32, 8, 8192, 8192, 128, "bf16", True),
]


def sweep_split(steps, warmup):
    """Unsplit (attn_fwd_ex) against split-key (attn_fwd_splitkv, automatic
    split count) forward time on small-grid and decoding shapes, plus the
    grouped-query backward where the row trains. Decoding is HBM-bound: its
    compulsory traffic is K and V once per key/value head, Q and O once."""
    import torch

    import inputgen
    import memory_efficient_exact_amd as mea
    dev = torch.device("cuda:0")
    rows = []
    for name, B, H, H_kv, n_q, n_k, d, dtype, backward in SPLIT_CASES:
        t = inputgen.draw_gqa(B, H, H_kv, n_q, n_k, d, dtype, seed=2000 + len(rows), with_do=backward)
        q, k, v = (t[x].to(dev) for x in ("q", "k", "v"))
        o = torch.empty_like(q)
        m = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        l = torch.empty_like(m)
        dt = mea.DTYPE_BF16 if dtype == "bf16" else mea.DTYPE_F32
        splits = mea.attn_fwd_splitkv_num_splits(dt, B, H, H_kv, n_q, n_k, d, 0)
        ws = torch.empty(max(16, mea.attn_fwd_splitkv_workspace_bytes(dt, B, H, H_kv, n_q, n_k, d, 0)),
                         dtype=torch.uint8, device=dev)

        def timed(fn):
            return timed_loop(fn, warmup, steps, dev)

        flops = 4.0 * B * H * n_q * n_k * d
        esz = q.element_size()
        hbm = (2 * B * H_kv * n_k * d + 2 * B * H * n_q * d) * esz + 8 * B * H * n_q
        ms_ex = timed(lambda: mea.attn_fwd_ex(q, k, v, out=o, row_max=m, row_sum=l))
        ms_sp = timed(lambda: mea.attn_fwd_splitkv(q, k, v, num_splits=0, out=o, row_max=m,
                                                   row_sum=l, workspace=ws))
        row = {"case": name, "B": B, "H": H, "H_kv": H_kv, "n_q": n_q, "n_k": n_k, "d": d,
               "dtype": dtype, "splits": splits,
               "fwd_ex_ms": ms_ex, "fwd_splitkv_ms": ms_sp,
               "fwd_ex_tflops": flops / (ms_ex * 1e-3) / 1e12,
               "fwd_splitkv_tflops": flops / (ms_sp * 1e-3) / 1e12,
               "compulsory_hbm_bytes": hbm,
               "fwd_splitkv_hbm_gbs": hbm / (ms_sp * 1e-3) / 1e9,
               "split_workspace_bytes": ws.numel() if splits > 1 else 0}
        if backward:
            do = t["do"].to(dev)
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            bws = torch.empty(mea.attn_bwd_ex_workspace_bytes(dt, B, H, H_kv, n_q, n_k, d),
                              dtype=torch.uint8, device=dev)
            bms = timed(lambda: mea.attn_bwd_ex(q, k, v, o, do, m, l, dq=dq, dk=dk, dv=dv,
                                                workspace=bws))
            row["bwd_ex_ms"] = bms
            row["bwd_ex_tflops"] = 2.5 * flops / (bms * 1e-3) / 1e12
        rows.append(row)
        log(json.dumps(row))
        del t, q, k, v, o, m, l, ws
        torch.cuda.empty_cache()
    return {"mode": "splitkv", "steps": steps, "warmup": warmup, "min_warm_s": MIN_WARM_S,
            "min_timed_s": MIN_TIMED_S, "rows": rows}


def sweep_memory():
    """Device memory of a forward and of a forward + backward at n = 1024 .. 16384
    (B=1, H=16, d=64, bf16), outputs allocated by the binding: the peak beyond the
    inputs and outputs (the method's overhead) must be the 8 bytes of row
    statistics per query row, plus 8 more of backward workspace (the minimum, the
    row terms), at every n, against 4*B*H*n^2 bytes for an fp32 score matrix. The
    workspace size the query reports (larger on small grids, where the backward
    splits its sweeps) is listed beside it."""
    import torch

    import inputgen
    import memory_efficient_exact_amd as mea
    dev = torch.device("cuda:0")
    rows = []
    for n in (1024, 2048, 4096, 8192, 16384):
        B, H, d = 1, 16, 64
        t = inputgen.draw(B, H, n, d, "bf16", seed=3000 + n, with_do=True)
        q, k, v, do = (t[x].to(dev) for x in ("q", "k", "v", "do"))
        io = q.numel() * q.element_size()
        torch.cuda.synchronize(dev)
        torch.cuda.empty_cache()
        base = torch.cuda.memory_allocated(dev)
        torch.cuda.reset_peak_memory_stats(dev)
        o, m, l = mea.attn_fwd(q, k, v)
        torch.cuda.synchronize(dev)
        fwd_over = torch.cuda.max_memory_allocated(dev) - base - io  # beyond the output O
        ws = torch.empty(8 * B * H * n, dtype=torch.uint8, device=dev)  # the row terms
        dq, dk, dv = mea.attn_bwd(q, k, v, o, do, m, l, workspace=ws)
        torch.cuda.synchronize(dev)
        step_over = torch.cuda.max_memory_allocated(dev) - base - 4 * io  # beyond O, dQ, dK, dV
        row = {"n": n, "B": B, "H": H, "d": d, "fwd_overhead_bytes": fwd_over,
               "fwd_overhead_per_row": fwd_over / (B * H * n),
               "step_overhead_bytes": step_over,
               "step_overhead_per_row": step_over / (B * H * n),
               "bwd_workspace_query_bytes": mea.attn_bwd_workspace_bytes(mea.DTYPE_BF16, B, H, n, d),
               "n2_fp32_score_bytes": 4 * B * H * n * n}
        rows.append(row)
        log(json.dumps(row))
        del t, q, k, v, do, o, m, l, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return {"mode": "memory", "rows": rows}


def _traffic_program(shape, mode="traffic"):
    return "python3 " + os.path.join(ROOT, "bench.py") + f" --mode {mode}" + (
        f" --shape {shape}" if shape else "")


SYNC_FWD_LAYOUTS = ("fwd row-tiled", "fwd decoding")
SYNC_BWD_ROLES = ("bwd d=64 dK/dV", "bwd d=64 dQ", "bwd d=128 dK/dV", "bwd d=128 dQ")


SYNC_COUNTERS = 7


def derive_sync(fwd_counts, bwd_counts):
    """Per tiled loop: {copy wait, barrier, loop cycles, tiles, waves, pair idle,
    pair loop} (sums over waves, core cycles; the last two over the first wave of
    each SIMD pair of 8-wave workgroups) -> cycles per tile and shares of the
    loop; pair_idle_share is the share of a SIMD's loop time in which both of its
    waves sat at the barrier."""
    out = {}
    c = SYNC_COUNTERS
    for names, counts in ((SYNC_FWD_LAYOUTS, fwd_counts), (SYNC_BWD_ROLES, bwd_counts)):
        for i, name in enumerate(names):
            wait, bar, loop, tiles, waves, pair_idle, pair_loop = counts[c * i:c * i + c]
            if tiles == 0 or loop == 0:
                continue
            out[name] = {
                "waves": waves, "tiles_per_wave": tiles / waves,
                "loop_cycles_per_tile": loop / tiles,
                "copy_wait_cycles_per_tile": wait / tiles,
                "barrier_cycles_per_tile": bar / tiles,
                "copy_wait_share": wait / loop, "barrier_share": bar / loop,
                "pair_idle_share": pair_idle / pair_loop if pair_loop else None,
            }
    return out


def run_sync(step, outputs, calls, dev):
    """Run `calls` steps through the timing library and return its end-of-tile
    counters, derived, and whether its outputs equal libmea.so's bit for bit."""
    import ctypes

    import torch

    import memory_efficient_exact_amd as mea
    step()  # libmea.so
    torch.cuda.synchronize(dev)
    ref = [x.clone() for x in outputs]
    T = mea.load(mea.timing_library_path())
    u64 = ctypes.c_ulonglong
    for fn in ("mea_sync_timers_fwd", "mea_sync_timers_bwd"):
        getattr(T, fn).argtypes = [ctypes.POINTER(u64), ctypes.c_int]
        getattr(T, fn).restype = ctypes.c_int
    fwd = (u64 * (len(SYNC_FWD_LAYOUTS) * SYNC_COUNTERS))()
    bwd = (u64 * (len(SYNC_BWD_ROLES) * SYNC_COUNTERS))()
    with mea.using(T):
        t_warm = time.perf_counter()
        while time.perf_counter() - t_warm < MIN_BENCH_WARM_S:
            step()
            torch.cuda.synchronize(dev)
        if T.mea_sync_timers_fwd(fwd, 1) or T.mea_sync_timers_bwd(bwd, 1):
            raise RuntimeError("reading the synchronisation counters failed")
        t0 = time.perf_counter()
        for _ in range(calls):
            step()
        torch.cuda.synchronize(dev)
        wall_ms = (time.perf_counter() - t0) * 1e3 / calls
        if T.mea_sync_timers_fwd(fwd, 1) or T.mea_sync_timers_bwd(bwd, 1):
            raise RuntimeError("reading the synchronisation counters failed")
    same = all(torch.equal(a, b) for a, b in zip(outputs, ref))
    return {"mode": "sync", "steps": calls, "ms_per_step_wall": wall_ms,
            "bitwise_equal_to_libmea": same, "loops": derive_sync(list(fwd), list(bwd))}


def run_probes():
    """Runs the probe program as a child process and derives, per probe, the issue
    cost of one instruction: cycles per instruction per wave and, with w waves on
    each SIMD, SIMD cycles per instruction = cycles per iteration / (w x instructions
    per iteration). VALU costs are also given relative to v_add_f32 at the same
    wave count. The mixed probes put an MFMA body and an FMA body on one SIMD (two
    waves, or interleaved in one wave): valu_hidden is the share of the VALU body's
    own time that ran under the MFMAs. The exponential mixes alternate v_exp_f32 with
    v_add_f32 or v_fma_f32: time_vs_serial_sum is 1 when they do not overlap. The
    HBM streams (2 GiB read, written, copied) give the bandwidth a plain kernel
    reaches, against which the decoding kernels are read."""
    import subprocess
    exe = os.path.join(ROOT, "memory_efficient_exact_amd", "probes", "mea_probe")
    if not os.path.exists(exe):
        sys.exit(f"{exe} is missing: build with `python -m memory_efficient_exact_amd.build`")
    log("running the issue-cost probes ...")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    if r.returncode != 0:
        sys.exit(f"probe program failed ({r.returncode}): {r.stderr[-2000:]}")
    return derive_probes(json.loads(r.stdout.strip().splitlines()[-1]))


def derive_probes(raw):
    """The derived figures of run_probes from the probe program's JSON."""
    out = {"mode": "probe", "raw": raw, "derived": {}}
    alone = {}
    for p in raw["probes"]:
        name, w = p["probe"], p["waves_per_simd"]
        if p["mfma_per_iter"] and not p["valu_per_iter"]:
            cyc = p["mfma_wave_cycles_per_iter"]
            if name == "mfma_32x32x16_bf16":  # register operands only (not the LDS-fed probes)
                alone[("mfma", w)] = cyc
            out["derived"][f"{name} w{w}"] = {
                "simd_cycles_per_mfma": cyc / (w * p["mfma_per_iter"]),
                "flop_per_cycle_per_simd": 32 * 32 * 16 * 2 * w * p["mfma_per_iter"] / cyc,
                "clock_mhz": p["clock_mhz"]}
        elif p["valu_per_iter"] and not p["mfma_per_iter"]:
            cyc = p["valu_wave_cycles_per_iter"]
            alone[(name, w)] = cyc
            out["derived"][f"{name} w{w}"] = {
                "wave_cycles_per_instr": cyc / p["valu_per_iter"],
                "simd_cycles_per_instr": cyc / (w * p["valu_per_iter"]), "clock_mhz": p["clock_mhz"]}
    for key, d in out["derived"].items():
        name, w = key.rsplit(" w", 1)
        base = alone.get(("v_add_f32", int(w)))
        if base and (name, int(w)) in alone:
            d["cost_vs_v_add_f32"] = alone[(name, int(w))] / base
        if "+" in name and (name, int(w)) in alone:
            # two kinds alternating, four of each per iteration: the time against the
            # sum of four of each alone (1: they serialise; 0.5: full overlap)
            parts = [alone.get((k, int(w))) for k in name.split("+")]
            if all(parts):
                d["time_vs_serial_sum"] = alone[(name, int(w))] / sum(c / 2 for c in parts)
    for p in raw["probes"]:
        if not (p["mfma_per_iter"] and p["valu_per_iter"]):
            continue
        w = p["waves_per_simd"]
        # the MFMA wave's time (in the two-wave probe the FMA wave runs alongside)
        cyc = p["mfma_wave_cycles_per_iter"]
        kind = "v_exp_f32" if "exp" in p["probe"] else "v_fma_f32"
        valu_alone = alone.get((kind, 1), 0.0) * p["valu_per_iter"] / 8  # one wave, alone
        mfma_alone = alone.get(("mfma", 1), 0.0)
        two_waves = p["probe"] in ("mfma_wave+fma_wave", "mfma_wave+exp_wave")
        per_simd_waves = 1 if two_waves else w
        d = {"cycles_per_iter": cyc, "mfma_per_iter_per_wave": p["mfma_per_iter"],
             "valu_per_iter_per_wave": p["valu_per_iter"], "waves_per_simd": w,
             # share of cycles the SIMD's matrix pipe is busy (32 cycles per MFMA)
             "mfma_pipe_busy": 32.0 * p["mfma_per_iter"] * per_simd_waves / cyc,
             "mfma_alone_cycles_per_iter": mfma_alone, "valu_alone_cycles_per_iter": valu_alone,
             "clock_mhz": p["clock_mhz"]}
        if two_waves:
            # the VALU wave's own time beside the MFMA wave, against its time alone
            d["valu_wave_cycles_per_iter"] = p["valu_wave_cycles_per_iter"]
            if valu_alone:
                d["valu_wave_slowdown"] = p["valu_wave_cycles_per_iter"] / valu_alone
            if mfma_alone:
                d["mfma_wave_slowdown"] = cyc / mfma_alone
        if valu_alone and mfma_alone and per_simd_waves == 1:
            # how much of the VALU work ran under the MFMAs (1: all of it)
            d["valu_hidden"] = (mfma_alone + valu_alone - cyc) / valu_alone
        out["derived"][p["probe"]] = d
    out["derived"]["atomic_dq"] = {a["mode"]: {"tb_per_s": a["tb_per_s"], "ms": a["ms"]}
                                   for a in raw["atomic_dq"]}
    out["derived"]["hbm_stream"] = {a["mode"]: {"tb_per_s": a["tb_per_s"], "ms": a["ms"]}
                                    for a in raw.get("hbm_stream", [])}
    return out


def profile_tools(args):
    """profile-plan: the rocprofv3 commands (one per pass); summarize: their reduction."""
    from memory_efficient_exact_amd import rocprof
    if not args.prof_dir:
        sys.exit("--prof-dir is required")
    program = _traffic_program(args.shape, args.pmc_mode)
    kt = "python3 " + os.path.join(ROOT, "bench.py") + (
        f" --mode {args.kt_mode}" if args.kt_mode else "") + (
        f" --shape {args.shape}" if args.kt_mode and args.shape else "") + (
        " --no-cpu-baseline" if args.no_cpu_baseline else "")
    cmds = rocprof.plan(os.path.abspath(args.prof_dir), program,
                        kt_program=kt if (args.kt_mode or not args.shape) else None)
    if args.mode == "profile-plan":
        print("\n".join(cmds))
        return
    # list only the passes this directory holds
    cmds = [c for c in cmds if " -d " not in c or os.path.isdir(c.split(" -d ")[1].split()[0])]
    timed = None
    b = {}
    if args.bench_json:
        line = [ln for ln in open(args.bench_json) if ln.strip().startswith("{")][-1]
        b = json.loads(line)
        if "warmup_steps_run" in b:
            timed = (int(b["warmup_steps_run"]), int(b["steps"]))
    summary = rocprof.collect(args.prof_dir, COPY_BYTES, timed=timed)
    agree = ""
    if timed and "fwd" in b and "bwd" in b:
        # the bench's HIP-event time per call against the trace's kernels of that call
        ks = summary.get("kernels", {})
        f_tr = sum(v.get("timed_avg_us") or 0.0 for k, v in ks.items() if k.startswith("fwd_")) / 1e3
        b_tr = sum(v.get("timed_avg_us") or 0.0 for k, v in ks.items() if k.startswith("bwd_")) / 1e3
        agree = (f" The profiled bench printed {b['fwd']['ms']:.4f} ms per forward and "
                 f"{b['bwd']['ms']:.4f} ms per backward call (HIP events on the launch stream); "
                 f"the trace's timed steps give {f_tr:.4f} ms and {b_tr:.4f} ms (each call's "
                 f"kernels summed).")
    rel = [c.replace(ROOT, "$R") for c in cmds]
    note = ("`R` is the repository root. "
            f"Summary command: `python3 bench.py --mode summarize --prof-dir {args.prof_dir}"
            + (f" --shape {args.shape}" if args.shape else "")
            + (" --bench-json <the profiled bench's stdout>" if args.bench_json else "")
            + (f" --kt-mode {args.kt_mode}" if args.kt_mode else "")
            + (f" --pmc-mode {args.pmc_mode}" if args.pmc_mode != "traffic" else "")
            + (" --probe-json <the probe run's stdout>" if args.probe_json else "")
            + "`. "
            + ("The traffic program runs one 256 MiB device copy (the counter calibration) "
               "and one step (attn_fwd, attn_bwd) of the workload. "
               if any("--pmc" in c for c in cmds) and args.pmc_mode == "traffic" else "")
            + (f"The kernel trace profiles the default bench; its timed steps are dispatches "
               f"{timed[0]}..{timed[0] + timed[1] - 1} of each per-step kernel." if timed else "")
            + agree)
    text = rocprof.render(summary, args.title, rel, note)
    if args.probe_json:
        probe = json.loads([ln for ln in open(args.probe_json) if ln.strip().startswith("{")][-1])
        head, sep, tail = text.partition("Machine-readable")
        text = head + rocprof.render_probes(probe) + "\n" + sep + tail
    print(text)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--shape", default=None,
                    help="traffic and sync modes: run the step on B,H,n,d (bf16, seed 1003) "
                         "instead of the default workload, e.g. 1,16,8192,128 for the d = 128 "
                         "kernels")
    ap.add_argument("--prof-dir", default=None,
                    help="profile-plan / summarize: directory of the rocprofv3 passes")
    ap.add_argument("--bench-json", default=None,
                    help="summarize: the JSON line the profiled default bench printed (selects "
                         "the timed steps' dispatches in the kernel trace)")
    ap.add_argument("--title", default="rocprofv3 summary", help="summarize: heading")
    ap.add_argument("--probe-json", default=None,
                    help="summarize: the JSON line `--mode probe` printed, rendered as tables")
    ap.add_argument("--pmc-mode", default="traffic",
                    help="profile-plan / summarize: bench mode the counter passes run")
    ap.add_argument("--kt-mode", default=None,
                    help="profile-plan / summarize: bench mode the kernel-trace pass runs "
                         "(default: the default bench; with --shape: the traffic program)")
    ap.add_argument("--mode", choices=("bench", "traffic", "configs", "splitkv", "memory",
                                       "profile-plan", "summarize", "probe", "sync"),
                    default="bench",
                    help="traffic: one 256 MiB copy (counter calibration) and one step, "
                         "for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE runs; configs: time "
                         "the forward on all five workloads (and the backward where the "
                         "workload trains), one JSON line with a row per workload; splitkv: "
                         "unsplit vs split-key forward on small-grid and decoding shapes; memory: "
                         "device-memory overhead per query row at n = 1024 .. 16384; "
                         "profile-plan: print the rocprofv3 commands of every pass (kernel trace "
                         "of the default bench, counter runs of --mode traffic) into --prof-dir; "
                         "summarize: reduce those passes to the markdown kept under profiles/; "
                         "probe: run the issue-cost probes (probes/mea_probe) and derive per-"
                         "instruction costs, MFMA/VALU overlap and fp32 atomic throughput; sync: "
                         "--steps steps through the timing library (libmea_synctimers.so): core "
                         "cycles per staged tile spent waiting for the tile copies and at the "
                         "barrier, per tiled loop, and a bitwise check against libmea.so")
    args = ap.parse_args()
    if args.mode in ("profile-plan", "summarize"):
        profile_tools(args)
        return
    if args.mode == "probe":
        print(json.dumps(run_probes()), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the attention "
              "kernels shard by (batch, head) with no communication, so per-GPU throughput "
              "is the single-GPU number", file=sys.stderr)
        sys.exit(2)

    import torch

    import inputgen
    import memory_efficient_exact_amd as mea

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mode == "configs":
        print(json.dumps(sweep_configs(args.steps, args.warmup)), flush=True)
        return
    if args.mode == "splitkv":
        print(json.dumps(sweep_split(args.steps, args.warmup)), flush=True)
        return
    if args.mode == "memory":
        print(json.dumps(sweep_memory()), flush=True)
        return
    w = inputgen.WORKLOADS["c3_long_bf16"]
    if args.shape is not None:
        if args.mode not in ("traffic", "sync"):
            ap.error("--shape applies to --mode traffic and --mode sync only")
        B_, H_, n_, d_ = (int(x) for x in args.shape.split(","))
        w = inputgen.Workload(f"shape_{B_}x{H_}x{n_}x{d_}", B_, H_, n_, d_, "bf16", seed=w.seed)
    t = inputgen.draw(w.B, w.H, w.n, w.d, w.dtype, seed=w.seed, with_do=True)
    q, k, v, do = (t[x].to(dev) for x in ("q", "k", "v", "do"))
    o = torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    m = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    l = torch.empty_like(m)
    ws = torch.empty(mea.attn_bwd_workspace_bytes(mea.DTYPE_BF16, w.B, w.H, w.n, w.d),
                     dtype=torch.uint8, device=dev)
    io_bytes = sum(x.numel() * x.element_size() for x in (q, k, v, do, o, dq, dk, dv, m, l))
    stream = torch.cuda.current_stream(dev)

    if args.mode == "traffic":
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE readings give
        # the factor that turns the counters into bytes.
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize(dev)
        dst.copy_(src)
        mea.attn_fwd(q, k, v, out=o, row_max=m, row_sum=l, stream=stream)
        mea.attn_bwd(q, k, v, o, do, m, l, dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream)
        torch.cuda.synchronize(dev)
        print(json.dumps({"mode": "traffic", "copy_bytes": COPY_BYTES}), flush=True)
        return

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        mea.attn_fwd(q, k, v, out=o, row_max=m, row_sum=l, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        mea.attn_bwd(q, k, v, o, do, m, l, dq=dq, dk=dk, dv=dv, workspace=ws, stream=stream)
        if ev is not None:
            ev[2].record(stream)

    if args.mode == "sync":
        r = run_sync(step, (o, m, l, dq, dk, dv), args.steps, dev)
        r["config"] = {"workload": w.name, "B": w.B, "H": w.H, "n": w.n, "d": w.d, "dtype": w.dtype}
        for name, x in r["loops"].items():
            pair = x["pair_idle_share"]
            log(f"{name}: {x['loop_cycles_per_tile']:.0f} cycles per tile per wave; copy wait "
                f"{x['copy_wait_cycles_per_tile']:.0f} ({100 * x['copy_wait_share']:.1f}%), "
                f"barrier {x['barrier_cycles_per_tile']:.0f} ({100 * x['barrier_share']:.1f}%)"
                + (f"; both waves of a SIMD at the barrier {100 * pair:.1f}%" if pair is not None
                   else ""))
        print(json.dumps(r), flush=True)
        return

    # Warm-up: at least --warmup steps and at least MIN_BENCH_WARM_S of wall time, so
    # the timed steps start on a chip that has left its idle clock (the timed step
    # count stays exactly --steps).
    t_warm, warm_steps = time.perf_counter(), 0
    while warm_steps < args.warmup or time.perf_counter() - t_warm < MIN_BENCH_WARM_S:
        step()
        warm_steps += 1
        if warm_steps % 8 == 0:
            torch.cuda.synchronize(dev)
    torch.cuda.synchronize(dev)
    warm_s = time.perf_counter() - t_warm
    before = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    stop.record(stream)
    torch.cuda.synchronize(dev)
    peak_extra = torch.cuda.max_memory_allocated(dev) - before
    total_ms = start.elapsed_time(stop)
    ms = total_ms / args.steps
    fwd_ms = [e[0].elapsed_time(e[1]) for e in evs]
    bwd_ms = [e[1].elapsed_time(e[2]) for e in evs]
    fwd_flops, bwd_flops = w.fwd_flops(), w.bwd_flops()
    value = (fwd_flops + bwd_flops) / (ms * 1e-3) / 1e12
    f_avg = statistics.mean(fwd_ms)
    b_avg = statistics.mean(bwd_ms)
    fwd_tf = fwd_flops / (f_avg * 1e-3) / 1e12
    bwd_tf = bwd_flops / (b_avg * 1e-3) / 1e12
    log(f"step {ms:.3f} ms | fwd {f_avg:.3f} ms ({fwd_tf:.1f} TFLOP/s, "
        f"{100 * fwd_tf / PEAK_BF16_TFLOPS:.1f}% of peak) | bwd {b_avg:.3f} ms ({bwd_tf:.1f} TFLOP/s)")

    # Roofline of the dominant kernel, bwd_main_kernel<64, 8> (the backward's
    # MFMA work: algorithmically 10*B*H*n^2*d flops per launch). Its average
    # launch duration is taken from HIP events around each attn_bwd call on the
    # launch stream; that call also runs the O(n*d) row pass (a few
    # microseconds), so the figure is a slight underestimate.
    fig = recorded_figures(DOMINANT_KERNEL)
    traffic = fig.get("hbm_bytes")
    roofline = {
        "kernel": DOMINANT_KERNEL,
        "bound": "mfma",
        "achieved": bwd_tf,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": bwd_tf / PEAK_BF16_TFLOPS,
        "traffic": traffic,
        "avg_launch_ms": b_avg,
        "flops_per_launch": bwd_flops,
        # from the committed counter summary of this kernel's current source (else null):
        # MFMA pipe busy share of cycles (executed MFMA work, 14/10 of the algorithmic
        # work in this design) and HBM GB/s = traffic / this run's launch time
        "mfma_busy": fig.get("mfma_busy"),
        "hbm_gbs": traffic / (b_avg * 1e-3) / 1e9 if traffic else None,
        "counters_from": fig.get("profiles"),
    }
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "warmup_s": warm_s,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "self-attention n=16384 bf16, forward + recompute backward",
                   "B": w.B, "H": w.H, "n": w.n, "d": w.d, "seed": w.seed,
                   "parallelism": "single GPU"},
        "fwd": {"ms": f_avg, "ms_median": statistics.median(fwd_ms), "ms_min": min(fwd_ms),
                "tflops": fwd_tf, "pct_peak": 100 * fwd_tf / PEAK_BF16_TFLOPS},
        "bwd": {"ms": b_avg, "ms_median": statistics.median(bwd_ms), "ms_min": min(bwd_ms),
                "tflops": bwd_tf, "pct_peak": 100 * bwd_tf / PEAK_BF16_TFLOPS},
        "pct_peak": 100 * value / PEAK_BF16_TFLOPS,
        "memory": {"io_bytes": io_bytes, "peak_extra_bytes_during_steps": peak_extra,
                   "library_overhead_bytes": 8 * w.B * w.H * w.n + ws.numel(),
                   "n2_fp32_score_matrix_bytes": 4 * w.B * w.H * w.n * w.n},
        "roofline": roofline,
    }
    out["clock"] = clock_under_load(step, dev)
    if out["clock"] is not None:
        out["roofline"]["frac_at_clock"] = bwd_tf / out["clock"]["peak_bf16_tflops_at_clock"]
        log(f"gfx clock under load: {out['clock']['gfx_mhz_mean']:.0f} MHz (mean of "
            f"{out['clock']['xcds']} XCDs)")
    if not args.no_cpu_baseline:
        log(f"timing the CPU oracle on {CPU_HEADS} heads ...")
        out["cpu_baseline"] = cpu_baseline(w)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
