#!/usr/bin/env python3
"""Benchmark of the block-sparse attention forward on one MI355X.

Workload: Sparse VideoGen head routing -- B=1, 24 heads (12 spatial: same
frame + frame 0; 12 temporal: same pixel +/-2 in y and x, every frame),
L = 20,280 tokens (13 frames x 30x52), d = 128, bf16 Q/K/V ~ N(0,1) from
fixed seeds. Run "B" (the headline) keeps the spatial heads frame-major and
permutes the temporal heads to temporal-major order; run "A" is all
frame-major and is reported beside it.

One step = one BSA call for a fresh mask: bsa_plan (host mapping, regime
lookup, task organisation, upload) + bsa_forward (the GPU kernel), with
Q/K/V/O resident in HBM. Kernel time is measured with HIP events on the
launch stream; effective TFLOP/s counts 4*d flops per kept (query, key) pair,
with the kept pairs counted by the CPU oracle's own mask expansion.

Prints one JSON line.
"""
import argparse
import contextlib
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_svg_runB.json")


def kernel_hash():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_run(w, Q, K, V, steps, warmup):
    import torch

    import block_sparse_attention_fwd_amd as bsa
    from bsa_helpers import plan_workload
    from gpu_util import to_device_bf16

    q, k, v = to_device_bf16(Q), to_device_bf16(K), to_device_bf16(V)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    # Clock settle (not a step): forward launches for about 0.3 s, so that the
    # GPU leaves its idle clocks before the warmup steps; otherwise the first
    # timed steps run while the clocks are still ramping.
    p0 = plan_workload(w)
    t_end = time.perf_counter() + 0.3
    n = 0
    while time.perf_counter() < t_end or n < 20:
        bsa.forward(p0, q, k, v, o, stream)
        n += 1
        if n % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    p0.close()

    # whole-path steps: plan + forward for a fresh mask each step. A plan is
    # retired (its memory returns to the library's pools) once an event shows
    # that its forward has finished; a ring of RING plans keeps the host
    # planning ahead of the GPU.
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
    plan_s = 0.0
    t0 = time.perf_counter()
    for _ in range(steps):
        dt, p = step()
        plan_s += dt
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms = (t1 - t0) * 1e3 / steps
    info = p.info()
    # the forwards' own time inside steps, from timing events around each
    # forward: a separate pass, since every event recorded on the stream adds
    # a few microseconds between kernels and the timed steps carry none
    ev = []
    for _ in range(steps):
        step(ev)
    torch.cuda.synchronize()
    kern_ms_inline = sum(a.elapsed_time(b) for a, b in ev) / steps
    for pp, _ in ring:
        pp.close()
    ring.clear()

    # forward-only launches back to back on a reused plan (kernel throughput)
    p = plan_workload(w)
    for _ in range(3):
        bsa.forward(p, q, k, v, o, stream)
    torch.cuda.synchronize()
    ev = []
    for _ in range(max(steps, 10)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        bsa.forward(p, q, k, v, o, stream)
        e1.record(stream)
        ev.append((e0, e1))
    torch.cuda.synchronize()
    fwd = sorted(a.elapsed_time(b) for a, b in ev)
    fwd_ms = sum(fwd) / len(fwd)
    return {"step_ms": step_ms, "plan_ms": plan_s * 1e3 / steps, "fwd_ms": fwd_ms, "fwd_ms_median": fwd[len(fwd) // 2],
            "fwd_ms_inline": kern_ms_inline, "plan_info": info}, o


def parity_sample(w, Q, K, V, o):
    import numpy as np

    from gpu_util import compare, sample_rows
    O = o.float().cpu().numpy().astype(np.float64)
    rows = sample_rows(w, per_head=8)
    with contextlib.redirect_stdout(sys.stderr):  # stdout carries only the JSON line
        mx, mean = compare(w, Q, K, V, O, rows=rows, label="bench sample")
    return {"rows": int(rows.size), "max_abs": mx, "mean_abs": mean}


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
    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    return {"value": ms_per_call, "unit": "ms", "cores": cores, "kind": "oracle",
            "sample": f"{rows.size} random query rows ({rows_per_head} per head, all {w.H} heads), {P_sample} kept pairs "
                      f"in {dt:.2f} s, scaled by total/sampled kept pairs ({P_total}/{P_sample})",
            "effective_gflops": 4 * w.d * P_sample / dt / 1e9}


def kept_pairs(w, oracle) -> int:
    """Kept (query, key) pairs of a workload's mask: block and slice masks
    counted from their descriptors, video masks by the oracle per pattern."""
    import numpy as np
    import workloads as wl
    if w.kind == wl.BLOCK:
        rows = np.minimum(np.arange(1, w.nqb + 1) * w.bq, w.L) - np.arange(w.nqb) * w.bq
        cols = np.minimum(np.arange(1, w.nkb + 1) * w.bk, w.L) - np.arange(w.nkb) * w.bk
        m = w.block.reshape(-1, w.nqb, w.nkb).astype(np.int64)
        return int(np.einsum("bij,i,j->", m, rows.astype(np.int64), cols.astype(np.int64)))
    if w.kind == wl.SLICE:
        nqb = -(-w.L // w.bq)
        rows = np.minimum(np.arange(1, nqb + 1) * w.bq, w.L) - np.arange(nqb) * w.bq
        lens = np.diff(np.asarray(w.row_ptr, dtype=np.int64)).reshape(-1, nqb)
        return int((lens * rows[None, :]).sum())
    per = {}
    total = 0
    for b in range(w.B):
        for h in range(w.H):
            key = (int(w.head_pattern[h]), int(w.head_layout[h]) if w.head_layout is not None else 0)
            if key not in per:
                per[key] = oracle.count_pairs(w, b, h)
            total += per[key]
    return total


def time_config(torch, w, P, plan_reps=5, warmup=5, reps=30):
    """Plan time (median of plan_reps host plans) and forward time (warmup
    calls, then reps calls timed one by one with events) of one workload on
    device-random bf16 inputs."""
    import block_sparse_attention_fwd_amd as bsa
    from bsa_helpers import plan_workload
    g = torch.Generator(device="cuda:0")
    g.manual_seed(w.cfg)
    q, k, v = (torch.randn((w.B, w.H, w.L, w.d), generator=g, device="cuda:0").to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    plan_ms = []
    p = None
    for _ in range(plan_reps):
        if p is not None:
            p.close()
        t0 = time.perf_counter()
        p = plan_workload(w)
        plan_ms.append((time.perf_counter() - t0) * 1e3)
    # warmup: at least `warmup` calls and 50 ms of them (clocks settle)
    n, t_end = 0, time.perf_counter() + 0.05
    while n < warmup or time.perf_counter() < t_end:
        bsa.forward(p, q, k, v, o)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ev = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        bsa.forward(p, q, k, v, o)
        e1.record()
        ev.append((e0, e1))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    info = p.info()
    p.close()
    med = t[len(t) // 2]
    flops = 4 * w.d * P
    return {"config": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "kind": w.kind, "block": [w.bq, w.bk],
            "regime": info["regime"], "task_order": info["task_order"], "kept_pairs": P,
            "computed_pairs": int(info["executed_pairs"]),
            "plan_ms_median": round(sorted(plan_ms)[len(plan_ms) // 2], 3),
            "fwd_ms_median": round(med, 4), "fwd_ms_p10": round(t[len(t) // 10], 4),
            "fwd_ms_p90": round(t[(9 * len(t)) // 10], 4),
            "effective_tflops": round(flops / (med * 1e-3) / 1e12, 1),
            "pct_bf16_peak": round(100.0 * flops / (med * 1e-3) / 1e12 / MI355X_BF16_PEAK_TFLOPS, 2)}


KNOWN_CONFIGS = {"tiny", "svgA", "svgB", "fgattn_M64", "fgattn_M128", "highres"} | {f"tessera{i}" for i in range(48)}


def all_configs(torch, oracle, wl, only=None):
    """Every configuration at full size, one JSON line each: tiny, SVG runs A
    and B, FG-Attn slices (M = 64 and 128), the 48 Tessera-style masks (and
    the request's sum), high-res. ``only``: a set of configuration names to
    run instead of all (the request's sum then needs all 48 masks)."""
    def wanted(name):
        return only is None or name in only
    works = [wl.tiny(), wl.svg("A"), wl.svg("B"), wl.fgattn(M=64), wl.fgattn(M=128)]
    works[3].name, works[4].name = "fgattn_M64", "fgattn_M128"
    # settle the clocks first (as the headline does): svg run B for 0.3 s
    time_config(torch, works[2], 1, plan_reps=1, warmup=10, reps=1)
    import block_sparse_attention_fwd_amd as bsa
    from bsa_helpers import plan_workload
    w0 = works[2]
    q0 = torch.zeros((w0.B, w0.H, w0.L, w0.d), dtype=torch.bfloat16, device="cuda:0")
    o0 = torch.empty_like(q0)
    p0 = plan_workload(w0)
    t_end = time.perf_counter() + 0.3
    n = 0
    while time.perf_counter() < t_end or n < 20:
        bsa.forward(p0, q0, q0, q0, o0)
        n += 1
        if n % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    p0.close()
    for w in works:
        if not wanted(w.name):
            continue
        log(f"[bench] {w.name}")
        print(json.dumps(time_config(torch, w, kept_pairs(w, oracle))), flush=True)
    total = 0.0
    for i in range(48):
        if not wanted(f"tessera{i}"):
            continue
        w = wl.tessera(i)
        r = time_config(torch, w, kept_pairs(w, oracle), plan_reps=3, warmup=3, reps=10)
        total += r["fwd_ms_median"]
        print(json.dumps(r), flush=True)
    if only is None:
        print(json.dumps({"config": "tessera_request", "masks": 48, "sum_fwd_ms_median": round(total, 2)}), flush=True)
    if not wanted("highres"):
        return
    w = wl.highres()
    log("[bench] highres")
    print(json.dumps(time_config(torch, w, kept_pairs(w, oracle), plan_reps=3, warmup=2, reps=10)), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-rows-per-head", type=int, default=12000,
                    help="oracle rows per head for the CPU baseline (about 10 s of CPU work by default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-parity", action="store_true")
    ap.add_argument("--runs", default="A,B", help="comma list of runs to time (the headline needs B)")
    ap.add_argument("--all-configs", action="store_true",
                    help="instead of the headline, time every configuration: one JSON line each")
    ap.add_argument("--configs", default=None,
                    help="with --all-configs: comma list of configuration names to run (tiny, svgA, svgB, "
                         "fgattn_M64, fgattn_M128, tessera0..tessera47, highres)")
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

    import oracle
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
        all_configs(torch, oracle, wl, None if args.configs is None else set(args.configs.split(",")))
        return
    wA, wB = wl.svg("A"), wl.svg("B")
    log("[bench] generating inputs")
    Q, K, V = wl.make_qkv(wB)
    log("[bench] counting kept pairs with the oracle")
    per_pattern = {}
    P = 0
    for h in range(wB.H):
        pat = int(wB.head_pattern[h])
        if pat not in per_pattern:
            per_pattern[pat] = oracle.count_pairs(wB, 0, h)
        P += per_pattern[pat]
    flops = 4 * wB.d * P

    res = {}
    runs = [r.strip() for r in args.runs.split(",") if r.strip()]
    for name, w in (("A", wA), ("B", wB)):
        if name not in runs:
            continue
        log(f"[bench] run {name}: warmup {args.warmup}, steps {args.steps}")
        r, o = time_run(w, Q, K, V, args.steps, args.warmup)
        if not args.no_parity:
            r["parity"] = parity_sample(w, Q, K, V, o)
        r["effective_tflops_step"] = flops / (r["step_ms"] * 1e-3) / 1e12
        r["effective_tflops_fwd"] = flops / (r["fwd_ms"] * 1e-3) / 1e12
        r["pct_bf16_peak_fwd"] = 100.0 * r["effective_tflops_fwd"] / MI355X_BF16_PEAK_TFLOPS
        res[name] = r
        log(f"[bench] run {name}: {json.dumps(r)}")

    B = res["B"]
    achieved = flops / (B["fwd_ms"] * 1e-3) / 1e12
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        t = json.load(open(TRAFFIC_FILE))
        if t.get("kernel_sha") == kernel_hash():
            traffic = t["bytes_per_launch"]
    out = {
        "metric": METRIC,
        "value": round(B["step_ms"], 4),
        "unit": "ms",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(B["step_ms"], 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "svg-head-routing run B (spatial heads frame-major, temporal heads temporal-major)",
                   "B": 1, "H": 24, "L": wB.L, "frames": wB.T, "grid": [wB.Hg, wB.Wg], "d": wB.d,
                   "heads": "12 spatial (same frame + frame 0), 12 temporal (|dy|,|dx| <= 2, all frames)",
                   "kept_pairs": P, "step": "bsa_plan + bsa_forward"},
        "fwd_ms": round(B["fwd_ms"], 4),
        "fwd_ms_in_steps": round(B["fwd_ms_inline"], 4),
        "plan_ms": round(B["plan_ms"], 4),
        "effective_tflops_step": round(B["effective_tflops_step"], 2),
        "effective_tflops_fwd": round(B["effective_tflops_fwd"], 2),
        "pct_bf16_peak_fwd": round(B["pct_bf16_peak_fwd"], 2),
        "run_A": ({k: (round(v, 4) if isinstance(v, float) else v) for k, v in res["A"].items() if k != "plan_info"}
                  if "A" in res else None),
        "run_B_plan": B["plan_info"],
        "parity": B.get("parity"),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": MI355X_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / MI355X_BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                     "kernel": "bsa_fwd_bf16<4,1,128,2>", "flops_per_launch": flops},
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on a row sample")
        out["cpu_baseline"] = cpu_baseline(wB, Q, K, V, P, args.cpu_rows_per_head)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
