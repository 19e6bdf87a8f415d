#!/usr/bin/env python3
"""Benchmark of the block-sparse attention forward on one MI355X.

Headline workload: the high-resolution video stand-in -- B=1, 24 heads,
L = 302,400 tokens (21 frames x 90x160), d = 128, bf16 Q/K/V ~ N(0,1) from
fixed seeds, a logical 128x128 block mask rasterised from the Sparse VideoGen
head patterns (heads 0-11 spatial: same frame + frame 0, frame-major; heads
12-23 temporal: |dy|,|dx| <= 2 in every frame, temporal-major). It is the
largest configuration, and it fits one GPU (7.4 GB of Q/K/V/O).

One step = one BSA call for a fresh mask: bsa_plan (host ingest, regime
lookup, physical mapping, task organisation, upload) + bsa_forward (the GPU
kernel), with Q/K/V/O resident in HBM. Kernel time is measured with HIP
events on the launch stream; effective TFLOP/s counts 4*d flops per kept
(query, key) pair, with the kept pairs counted by the CPU oracle's own mask
expansion after the timed work.

Beside the headline, the line carries one record per throughput class:
the Sparse VideoGen head-routing workload split into its 12 spatial heads
(bound by the matrix cores) and its 12 temporal heads in either layout, and
the FG-Attn M x 1 slices (both bound by the memory system), the latter with
the mask-defined gather bytes G (every 64-row query block loads each distinct
key it keeps once, as a K and a V row, plus Q read and O written once).

Prints one JSON line.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

MI355X_BF16_PEAK_TFLOPS = 2500.0  # dense bf16 MFMA
MI355X_HBM_PEAK_GBS = 8000.0
METRIC = "ms per BSA call; effective TFLOP/s on kept pairs and % of MI355X bf16 MFMA peak"
KERNEL_SRC = os.path.join(ROOT, "block_sparse_attention_fwd_amd", "csrc", "attn_fwd.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_highres.json")


def kernel_hash():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    if n and n.isdigit():
        return int(n)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# ---------------------------------------------------------------------------
# GPU timing (no oracle code is loaded until every timed region has run)
# ---------------------------------------------------------------------------

def settle_clocks(bsa, p, q, k, v, o, stream, seconds=0.3):
    """Forward launches for a while so that the GPU leaves its idle clocks
    before anything is timed (not a step, not timed)."""
    import torch
    t_end = time.perf_counter() + seconds
    n = 0
    while time.perf_counter() < t_end or n < 4:
        bsa.forward(p, q, k, v, o, stream)
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


def time_forwards(bsa, p, q, k, v, o, stream, reps):
    """`reps` forwards back to back on one plan, each bracketed by HIP events
    recorded on the launch stream; returns the per-launch times in ms."""
    import torch
    ev = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        bsa.forward(p, q, k, v, o, stream)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


MFMA_TFLOPS_PER_GHZ = 256 * 4 * 1024 / 1e3  # dense bf16: 256 CUs x 4 SIMDs x 1,024 flop per clock


def shader_clock(bsa, w, q, k, v, o, warm=4):
    """The shader clock the headline kernel runs at: `warm` forwards back to
    back, then one bsa_forward_stamped in the same stream; every task's
    shader-clock ticks over its 100 MHz ticks (their totals, and the 10th and
    90th percentiles of the per-task clocks). Not a step, not timed."""
    import numpy as np
    import torch
    from bsa_helpers import plan_workload
    p = plan_workload(w)
    stamps = torch.zeros(4 * p.info()["workgroups"], dtype=torch.int64, device="cuda:0")
    stream = torch.cuda.current_stream()
    for _ in range(warm):
        bsa.forward(p, q, k, v, o, stream)
    bsa.forward_stamped(p, q, k, v, o, stamps, stream)
    torch.cuda.synchronize()
    p.close()
    s = stamps.cpu().numpy().reshape(-1, 4).astype(np.float64)
    s = s[(s[:, 2] > s[:, 0]) & (s[:, 3] > s[:, 1])]
    clk, real = s[:, 2] - s[:, 0], s[:, 3] - s[:, 1]
    per = clk / real * 0.1
    return {"ghz": round(float(clk.sum() / real.sum() * 0.1), 4), "p10": round(float(np.percentile(per, 10)), 4),
            "p90": round(float(np.percentile(per, 90)), 4), "tasks": int(s.shape[0])}


def time_steps(w, q, k, v, o, steps, warmup):
    """Whole-path steps for the headline: plan + forward for a fresh mask each
    step. A plan is retired (its memory back to the library's pools) once an
    event shows that its forward has finished; a ring of three plans keeps the
    host planning ahead of the GPU, as a serving loop would."""
    import torch

    import block_sparse_attention_fwd_amd as bsa
    from bsa_helpers import plan_workload

    stream = torch.cuda.current_stream()
    p0 = plan_workload(w)
    settle_clocks(bsa, p0, q, k, v, o, stream, 0.5)
    p0.close()

    RING = 3
    ring = []

    def step(ev_list=None):
        if len(ring) >= RING:
            old_p, old_done = ring.pop(0)
            old_done.synchronize()
            old_p.close()
        tp = time.perf_counter()
        p = plan_workload(w)
        dt = time.perf_counter() - tp
        if ev_list is not None:
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
        bsa.forward(p, q, k, v, o, stream)
        done = torch.cuda.Event()
        done.record(stream)
        if ev_list is not None:
            e1.record(stream)
            ev_list.append((e0, e1))
        ring.append((p, done))
        return dt, p

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.synchronize()
    plan_s = 0.0
    t0 = time.perf_counter()
    for _ in range(steps):
        dt, p = step()
        plan_s += dt
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = (t1 - t0) * 1e3 / steps
    info = p.info()
    # the forwards' own time inside steps, in a separate pass (every event
    # recorded on the stream adds a little time between kernels)
    ev = []
    for _ in range(steps):
        step(ev)
    torch.cuda.synchronize()
    fwd_in_steps = sum(a.elapsed_time(b) for a, b in ev) / steps
    for pp, _ in ring:
        pp.close()
    ring.clear()

    # forward-only launches back to back on one plan (the kernel's own rate)
    p = plan_workload(w)
    for _ in range(2):
        bsa.forward(p, q, k, v, o, stream)
    torch.cuda.synchronize()
    t = time_forwards(bsa, p, q, k, v, o, stream, max(steps, 10))
    p.close()
    ts = sorted(t)
    return {"step_ms": step_ms, "plan_ms": plan_s * 1e3 / steps, "fwd_ms": sum(t) / len(t),
            "fwd_ms_median": ts[len(ts) // 2], "fwd_ms_p10": ts[len(ts) // 10], "fwd_ms_p90": ts[(9 * len(ts)) // 10],
            "fwd_ms_in_steps": fwd_in_steps, "plan_info": info}


def time_class(torch, w, reps=30, plans=3):
    """Forward time of one workload (a throughput class) on device-random
    bf16 N(0,1) inputs: one plan, warmup, then `reps` forwards timed one by one
    with events on the launch stream. The timing does not depend on values.
    The plan time is the median of `plans` plans made after one untimed plan
    (which fills the library's memory pools, as the first call of a serving
    loop would)."""
    import block_sparse_attention_fwd_amd as bsa
    from bsa_helpers import plan_workload
    g = torch.Generator(device="cuda:0")
    g.manual_seed(1000 + w.cfg)
    q, k, v = (torch.randn((w.B, w.H, w.L, w.d), generator=g, device="cuda:0").to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    plan_workload(w).close()
    plan_times = []
    for i in range(plans):
        t0 = time.perf_counter()
        p = plan_workload(w)
        plan_times.append((time.perf_counter() - t0) * 1e3)
        if i + 1 < plans:
            p.close()
    plan_ms = sorted(plan_times)[len(plan_times) // 2]
    settle_clocks(bsa, p, q, k, v, o, stream, 0.05)
    t = sorted(time_forwards(bsa, p, q, k, v, o, stream, reps))
    info = p.info()
    p.close()
    del q, k, v, o
    return {"fwd_ms_median": t[len(t) // 2], "fwd_ms_p10": t[len(t) // 10], "fwd_ms_p90": t[(9 * len(t)) // 10],
            "plan_ms": plan_ms, "regime": info["regime"], "executed_pairs": int(info["executed_pairs"])}


def class_workloads():
    """The per-class sub-calls: (name, workload, bound, description)."""
    import workloads as wl
    sp = wl.svg("A", H=12, n_spatial=12)
    sp.name = "svg_spatial_12"
    ta = wl.svg("A", H=12, n_spatial=0)
    ta.name = "svg_temporal_12_frame_major"
    tb = wl.svg("B", H=12, n_spatial=0)
    tb.name = "svg_temporal_12_temporal_major"
    fb = wl.svg("B")
    fb.name = "svg_runB_24"
    return [
        (sp, "mfma", "Sparse VideoGen: the 12 spatial heads (same frame + frame 0), frame-major, L = 20,280"),
        (ta, "hbm", "Sparse VideoGen: the 12 temporal heads (|dy|,|dx| <= 2, all frames), frame-major"),
        (tb, "hbm", "Sparse VideoGen: the 12 temporal heads, temporal-major"),
        (fb, "mfma", "Sparse VideoGen run B: all 24 heads in one call (12 spatial frame-major, 12 temporal "
                     "temporal-major)"),
        (None, "hbm", "FG-Attn M x 1 slices, M = 64: 24 heads, L = 32,760, per 64-query block a seeded key list "
                      "of density U[0.1, 0.3], 70% in runs of 4-32"),
    ]


def kept_pairs(w, oracle) -> int:
    """Kept (query, key) pairs of a workload's mask, counted by the oracle per
    head (heads with identical video masks counted once)."""
    import workloads as wl
    total = 0
    per = {}
    for b in range(w.B):
        for h in range(w.H):
            key = None
            if w.kind == wl.VIDEO:
                key = (int(w.head_pattern[h]), int(w.layout()[h]))
            if key is not None and key in per:
                total += per[key]
                continue
            c = oracle.count_pairs(w, b, h)
            if key is not None:
                per[key] = c
            total += c
    return total


# ---------------------------------------------------------------------------
# oracle legs (after the timing): parity sample, CPU baseline
# ---------------------------------------------------------------------------

def parity_sample(w, Q, K, V, o, per_head=48):
    import contextlib

    import numpy as np

    from gpu_util import compare, sample_rows
    O = o.float().cpu().numpy().astype(np.float64)
    rows = sample_rows(w, per_head=per_head)
    with contextlib.redirect_stdout(sys.stderr):  # stdout carries only the JSON line
        mx, mean = compare(w, Q, K, V, O, rows=rows, label="bench sample")
    return {"rows": int(rows.size), "max_abs": mx, "mean_abs": mean, "bar": {"max_abs": 1e-2, "mean_abs": 1e-3}}


def cpu_baseline(w, Q, K, V, P_total, rows_per_head):
    import numpy as np

    import oracle
    g = np.random.default_rng(123)
    rows = np.concatenate([h * w.L + g.choice(w.L, rows_per_head, replace=False) for h in range(w.H)]).astype(np.int64)
    oracle.lib()
    t0 = time.perf_counter()
    _, cnt = oracle.attend(w, Q, K, V, rows=rows, return_counts=True)
    dt = time.perf_counter() - t0
    P_sample = int(cnt.sum())
    ms_per_call = dt * 1e3 * P_total / P_sample
    return {"value": ms_per_call, "unit": "ms", "cores": host_threads(), "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": f"{rows.size} random query rows ({rows_per_head} per head, all {w.H} heads) of the same "
                      f"workload, {P_sample} kept pairs in {dt:.2f} s, scaled by total/sampled kept pairs "
                      f"({P_total}/{P_sample}); extrapolated",
            "effective_gflops": 4 * w.d * P_sample / dt / 1e9}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-rows-per-head", type=int, default=2000,
                    help="oracle rows per head for the CPU baseline (about 10-15 s on 16 host threads by default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--no-classes", action="store_true", help="skip the per-class records")
    ap.add_argument("--forward-only", type=int, default=0, metavar="N",
                    help="only launch N headline forwards on one plan (for counter runs) and exit")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the headline, time every configuration: one JSON line each")
    ap.add_argument("--configs", default=None,
                    help="with --all-configs: comma list of configuration names to run (tiny, svgA, svgB, "
                         "fgattn_M64, fgattn_M128, tessera0..tessera47, highres)")
    ap.add_argument("--units", action="store_true",
                    help="instead of the headline, run the unit microbenchmarks (MFMA, vector, LDS, HBM rates)")
    ap.add_argument("--occupancy", default=None, metavar="NAMES",
                    help="instead of the headline, stamped forwards of the named configurations (comma list, as "
                         "--configs): busy share of the workgroup slots, tail, shader clock per XCD class")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes 5 times (HBM counter calibration)")
    args = ap.parse_args()
    if args.configs is not None:
        unknown = set(args.configs.split(",")) - KNOWN_CONFIGS
        if unknown or not args.all_configs:
            ap.error(f"--configs needs --all-configs and names among tiny, svgA, svgB, fgattn_M64, fgattn_M128, "
                     f"tessera0..tessera47, highres (unknown: {sorted(unknown)})")
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}); heads would be sharded across GPUs with no exchange.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": 5}), flush=True)
        return
    if args.all_configs:
        all_configs(torch, wl, None if args.configs is None else set(args.configs.split(",")))
        return
    if args.units:
        for rec in unit_benchmarks():
            print(json.dumps(rec), flush=True)
        return
    if args.occupancy:
        unknown = set(args.occupancy.split(",")) - KNOWN_CONFIGS
        if unknown:
            ap.error(f"--occupancy takes configuration names (unknown: {sorted(unknown)})")
        occupancy(torch, wl, args.occupancy.split(","))
        return

    from bsa_helpers import to_device_bf16

    w = wl.highres()
    log("[bench] generating the high-res inputs (seeded, host)")
    Q, K, V = wl.make_qkv(w)
    q, k, v = to_device_bf16(Q), to_device_bf16(K), to_device_bf16(V)
    o = torch.empty_like(q)
    if args.forward_only:
        import block_sparse_attention_fwd_amd as bsa
        from bsa_helpers import plan_workload
        p = plan_workload(w)
        stream = torch.cuda.current_stream()
        t = time_forwards(bsa, p, q, k, v, o, stream, args.forward_only)
        p.close()
        print(json.dumps({"forward_only": args.forward_only, "fwd_ms": t}), flush=True)
        return

    log(f"[bench] high-res: warmup {args.warmup}, steps {args.steps}")
    r = time_steps(w, q, k, v, o, args.steps, args.warmup)
    log(f"[bench] high-res: {json.dumps({a: b for a, b in r.items() if a != 'plan_info'})}")

    import block_sparse_attention_fwd_amd as bsa
    clock = shader_clock(bsa, w, q, k, v, o)
    log(f"[bench] shader clock over a stamped forward: {json.dumps(clock)}")

    classes = {}
    if not args.no_classes:
        for cw, bound, desc in class_workloads():
            if cw is None:
                cw = wl.fgattn(M=64)
                cw.name = "fgattn_M64"
            log(f"[bench] class {cw.name}")
            c = time_class(torch, cw)
            c.update({"bound": bound, "description": desc, "workload": cw})
            classes[cw.name] = c
            torch.cuda.empty_cache()

    # ---- everything below runs after the timed work: oracle counts and checks
    import oracle
    log("[bench] counting kept pairs with the oracle")
    P = kept_pairs(w, oracle)
    flops = 4 * w.d * P
    achieved = flops / (r["fwd_ms"] * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        t = json.load(open(TRAFFIC_FILE))
        if t.get("kernel_sha") == kernel_hash():
            traffic = t["bytes_per_launch"]
    class_out = {}
    for name, c in classes.items():
        cw = c.pop("workload")
        Pc = kept_pairs(cw, oracle)
        sec = c["fwd_ms_median"] * 1e-3
        rec = {"description": c["description"], "bound": c["bound"], "heads": cw.H, "L": cw.L,
               "kept_pairs": Pc, "executed_pairs": c["executed_pairs"], "regime": c["regime"],
               "fwd_ms_median": round(c["fwd_ms_median"], 4), "fwd_ms_p10": round(c["fwd_ms_p10"], 4),
               "fwd_ms_p90": round(c["fwd_ms_p90"], 4), "plan_ms": round(c["plan_ms"], 3),
               "effective_tflops": round(4 * cw.d * Pc / sec / 1e12, 1),
               "frac_bf16_peak": round(4 * cw.d * Pc / sec / 1e12 / MI355X_BF16_PEAK_TFLOPS, 4)}
        if c["bound"] == "hbm":
            G = oracle.gather_bytes(cw, M=64)
            rec.update({"G_bytes": G, "G_GBs": round(G / sec / 1e9, 1),
                        "frac_hbm_peak": round(G / sec / 1e9 / MI355X_HBM_PEAK_GBS, 4), "target_frac": 0.6})
        else:
            rec["target_frac"] = 0.5
        class_out[name] = rec
        log(f"[bench] class {name}: {json.dumps(rec)}")

    out = {
        "metric": METRIC,
        "value": round(r["step_ms"], 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["step_ms"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V rounded to bf16; mask rasterised from the video head patterns",
        "config": {"workload": "high-res video stand-in (1440p-like): 24 heads, 21 frames x 90x160 tokens, "
                               "128x128 logical blocks rasterised from 12 spatial heads (frame-major) and 12 temporal "
                               "heads (temporal-major)",
                   "B": w.B, "H": w.H, "L": w.L, "frames": w.T, "grid": [w.Hg, w.Wg], "d": w.d,
                   "block": [w.bq, w.bk], "kept_pairs": P, "step": "bsa_plan + bsa_forward"},
        "fwd_ms": round(r["fwd_ms"], 4),
        "fwd_ms_median": round(r["fwd_ms_median"], 4),
        "fwd_ms_p10": round(r["fwd_ms_p10"], 4),
        "fwd_ms_p90": round(r["fwd_ms_p90"], 4),
        "fwd_ms_in_steps": round(r["fwd_ms_in_steps"], 4),
        "plan_ms": round(r["plan_ms"], 4),
        "effective_tflops_step": round(flops / (r["step_ms"] * 1e-3) / 1e12, 2),
        "effective_tflops_fwd": round(achieved, 2),
        "pct_bf16_peak_fwd": round(100.0 * achieved / MI355X_BF16_PEAK_TFLOPS, 2),
        "plan": r["plan_info"],
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MI355X_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MI355X_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": "bsa_fwd_bf16<4,1,128,2,kModeBlock>", "flops_per_launch": flops},
        "clock": dict(clock, mfma_peak_at_clock_tflops=round(MFMA_TFLOPS_PER_GHZ * clock["ghz"], 1),
                      frac_of_mfma_peak_at_clock=round(achieved / (MFMA_TFLOPS_PER_GHZ * clock["ghz"]), 4)),
        "classes": class_out,
    }
    if not args.no_parity:
        log("[bench] parity sample against the oracle")
        out["parity"] = parity_sample(w, Q, K, V, o)
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a row sample")
        out["cpu_baseline"] = cpu_baseline(w, Q, K, V, P, args.cpu_rows_per_head)
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------
# unit microbenchmarks (--units)
# ---------------------------------------------------------------------------

UNITS_LIB = os.path.join(ROOT, "block_sparse_attention_fwd_amd", "libbsa_units.so")
MFMA_FLOP = 2 * 32 * 32 * 16  # one v_mfma_f32_32x32x16_bf16


def unit_benchmarks():
    """The device rates the forward kernel's roofline fractions rest on,
    measured with the kernels of csrc/units.hip: MFMA throughput (alone and
    with exponentials or FMAs issued beside it, in the same wave or by a
    second wave of the SIMD), vector-unit and LDS read rates, HBM streaming
    rates. Yields one record per measurement."""
    import ctypes
    if not os.path.exists(UNITS_LIB):
        raise SystemExit(f"{UNITS_LIB} is missing: build it first (__graft_entry__.build())")
    L = ctypes.CDLL(UNITS_LIB)
    L.bsa_units_run.restype = ctypes.c_int
    L.bsa_units_run.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_double)]
    ncu = 256

    def run(which, param, iters, blocks):
        out = (ctypes.c_double * 3)()
        rc = L.bsa_units_run(which, param, iters, blocks, out)
        if rc != 0:
            raise RuntimeError(f"bsa_units_run({which}, {param}) failed: hipError {rc}")
        ms, ticks, rt = out[0], out[1], out[2]
        ghz = ticks / (rt / 100e6) / 1e9 if rt > 0 else float("nan")
        return ms, ticks, ghz

    iters = 20000
    base = None
    for which, name in ((0, "mfma"), (1, "mfma+exp same wave"), (2, "mfma+fma same wave"),
                        (3, "mfma wave + exp wave per SIMD")):
        for ne in ((0,) if which == 0 else (1, 2, 3, 4)):
            ms, ticks, ghz = run(which, ne, iters, ncu)
            mfma_waves = 4 if which == 3 else 8
            flops = ncu * mfma_waves * iters * 4 * MFMA_FLOP
            # one block per CU: two MFMA-issuing waves per SIMD (one for mode 3)
            per_simd = 2 if which != 3 else 1
            clk_per_mfma = ticks / (iters * 4 * per_simd)
            rec = {"unit": name, "per_mfma": ne, "ms": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                   "clock_ghz": round(ghz, 3), "clk_per_mfma_per_simd": round(clk_per_mfma, 2)}
            if which == 0:
                base = clk_per_mfma
            else:
                rec["vs_mfma_alone"] = round(clk_per_mfma / base, 3)
            yield rec
    for which, name in ((10, "v_exp_f32"), (11, "v_fma_f32")):
        ms, ticks, ghz = run(which, 0, iters, ncu)
        yield {"unit": name, "ms": round(ms, 4), "clock_ghz": round(ghz, 3),
               "clk_per_wave_instruction": round(ticks / (iters * 16), 2), "note": "one wave per SIMD"}
    for which, name, nbytes in ((20, "ds_read_b128", 1024), (21, "ds_read_b64_tr_b16", 512)):
        it = 4000
        ms, ticks, ghz = run(which, 0, it, ncu)
        per_cu = 8 * it * 8 * nbytes  # 8 waves x iters x 8 reads x bytes per wave read
        yield {"unit": name, "ms": round(ms, 4), "clock_ghz": round(ghz, 3),
               "bytes_per_clk_per_cu": round(per_cu / ticks, 1), "tb_per_s_chip": round(ncu * per_cu / (ms * 1e-3) / 1e12, 2)}
    for which, name in ((30, "hbm read"), (31, "hbm copy")):
        mib = 2048
        ms, ticks, ghz = run(which, mib, 0, ncu * 8)
        moved = mib * (1 << 20) * (2 if which == 31 else 1)
        yield {"unit": name, "bytes": moved, "ms": round(ms, 4), "gb_per_s": round(moved / (ms * 1e-3) / 1e9, 1),
               "frac_of_8tbs": round(moved / (ms * 1e-3) / 1e9 / MI355X_HBM_PEAK_GBS, 3)}


# ---------------------------------------------------------------------------
# every configuration (--all-configs)
# ---------------------------------------------------------------------------

KNOWN_CONFIGS = {"tiny", "svgA", "svgB", "fgattn_M64", "fgattn_M128", "highres"} | {f"tessera{i}" for i in range(48)}


def all_configs(torch, wl, only=None):
    """Every configuration at full size, one JSON line each: tiny, SVG runs A
    and B, FG-Attn slices (M = 64 and 128), the 48 Tessera-style masks (and
    the request's sum), high-res. ``only``: a set of configuration names to
    run instead of all (the request's sum then needs all 48 masks). Kept pairs
    and gather bytes are counted by the oracle after each configuration's
    timing."""
    def wanted(name):
        return only is None or name in only

    def report(w, r):
        import oracle
        P = kept_pairs(w, oracle)
        sec = r["fwd_ms_median"] * 1e-3
        G = oracle.gather_bytes(w, M=64)
        rec = {"config": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "kind": w.kind, "block": [w.bq, w.bk],
               "regime": r["regime"], "kept_pairs": P, "computed_pairs": r["executed_pairs"],
               "plan_ms": round(r["plan_ms"], 3), "fwd_ms_median": round(r["fwd_ms_median"], 4),
               "fwd_ms_p10": round(r["fwd_ms_p10"], 4), "fwd_ms_p90": round(r["fwd_ms_p90"], 4),
               "effective_tflops": round(4 * w.d * P / sec / 1e12, 1),
               "pct_bf16_peak": round(100.0 * 4 * w.d * P / sec / 1e12 / MI355X_BF16_PEAK_TFLOPS, 2),
               "G_bytes": G, "G_GBs": round(G / sec / 1e9, 1),
               "pct_hbm_peak_on_G": round(100.0 * G / sec / 1e9 / MI355X_HBM_PEAK_GBS, 2)}
        print(json.dumps(rec), flush=True)
        return rec

    timed = []
    works = [wl.tiny(), wl.svg("A"), wl.svg("B"), wl.fgattn(M=64), wl.fgattn(M=128)]
    works[3].name, works[4].name = "fgattn_M64", "fgattn_M128"
    for w in works:
        if wanted(w.name):
            log(f"[bench] {w.name}")
            timed.append((w, time_class(torch, w)))
    for i in range(48):
        if wanted(f"tessera{i}"):
            w = wl.tessera(i)
            log(f"[bench] {w.name}")
            timed.append((w, time_class(torch, w, reps=10)))
            torch.cuda.empty_cache()
    if wanted("highres"):
        w = wl.highres()
        log("[bench] highres")
        timed.append((w, time_class(torch, w, reps=10)))
    # the oracle's counts, after every timed region
    total = 0.0
    for w, r in timed:
        rec = report(w, r)
        if w.name.startswith("tessera"):
            total += rec["fwd_ms_median"]
    if only is None:
        print(json.dumps({"config": "tessera_request", "masks": 48, "sum_fwd_ms_median": round(total, 2)}), flush=True)


# ---------------------------------------------------------------------------
# launch occupancy from per-task clock stamps (--occupancy)
# ---------------------------------------------------------------------------

def config_workload(wl, name):
    """The workload of a configuration name (the names --configs takes)."""
    if name.startswith("tessera"):
        return wl.tessera(int(name[7:]))
    if name.startswith("fgattn_M"):
        w = wl.fgattn(M=int(name[8:]))
        w.name = name
        return w
    return {"tiny": wl.tiny, "svgA": lambda: wl.svg("A"), "svgB": lambda: wl.svg("B"), "highres": wl.highres}[name]()


def occupancy(torch, wl, names, launches=3):
    """Per configuration, `launches` stamped forwards (after four plain ones)
    on device-random N(0,1) inputs: the launch span, the share of the
    workgroup slots' time spent in tasks (slots = the most tasks ever running
    at once), the share of the span at its end during which fewer than 90% of
    the slots run, and per class of workgroup index mod 8 (the XCD the
    hardware deals the workgroup to) the shader clock and the time its last
    task ends. One JSON line per launch."""
    import numpy as np
    import block_sparse_attention_fwd_amd as bsa
    from bsa_helpers import plan_workload
    for name in names:
        w = config_workload(wl, name)
        g = torch.Generator(device="cuda:0")
        g.manual_seed(5)
        q, k, v = (torch.randn((w.B, w.H, w.L, w.d), generator=g, device="cuda:0").to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        p = plan_workload(w)
        info = p.info()
        n = info["workgroups"]
        for _ in range(4):
            bsa.forward(p, q, k, v, o)
        for rep in range(launches):
            stamps = torch.zeros(4 * n, dtype=torch.int64, device="cuda:0")
            bsa.forward_stamped(p, q, k, v, o, stamps)
            torch.cuda.synchronize()
            s = stamps.cpu().numpy().reshape(-1, 4).astype(np.float64)
            idx = np.arange(n)
            ok = (s[:, 3] > s[:, 1]) & (s[:, 2] > s[:, 0])
            s, idx = s[ok], idx[ok]
            st, en = s[:, 1] / 100.0, s[:, 3] / 100.0  # microseconds
            t0 = st.min()
            st, en = st - t0, en - t0
            span = float(en.max())
            ev = np.concatenate([np.stack([st, np.ones_like(st)], 1), np.stack([en, -np.ones_like(en)], 1)])
            ev = ev[np.lexsort((ev[:, 1], ev[:, 0]))]  # at equal times, ends before starts
            running = np.cumsum(ev[:, 1])
            slots = int(running.max())
            busy = float((en - st).sum() / (slots * span))
            full = np.where(running >= 0.9 * slots)[0]
            tail = span - float(ev[full[-1], 0]) if full.size else span
            cls = idx % 8
            clk = [float((s[cls == c, 2] - s[cls == c, 0]).sum() / (s[cls == c, 3] - s[cls == c, 1]).sum() * 0.1)
                   for c in range(8)]
            rec = {"config": name, "launch": rep, "regime": info["regime"], "tasks": int(s.shape[0]),
                   "span_ms": round(span / 1000, 4), "slots": slots, "busy_share": round(busy, 4),
                   "tail_share_below_90pct": round(tail / span, 4),
                   "clock_ghz_by_index_mod_8": [round(c, 3) for c in clk],
                   "last_end_ms_by_index_mod_8": [round(float(en[cls == c].max()) / 1000, 3) for c in range(8)]}
            print(json.dumps(rec), flush=True)
        p.close()
        del q, k, v, o
        torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
