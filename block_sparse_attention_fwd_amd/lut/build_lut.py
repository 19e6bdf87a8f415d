#!/usr/bin/env python3
"""Offline profiling that builds the regime lookup table for this GPU.

Tessera (arXiv 2609.25869), abstract: the execution regime of a request is
chosen through a lookup table built by offline profiling, which keeps
preparation cheap at run time. This script is that offline step: for every
bin of the table's features -- mask kind, logical block shape, kept-block
density, sequence length -- it plans and runs synthetic requests of that bin
with every regime that can run them, times the forward passes on the GPU and
writes the fastest regime of each bin as one rule of the table (the default
unless another wins by more than 2%).

Besides the kept-block density, block-mask bins are split by the mask's fill
(kept pairs over the pairs of its non-empty 128 x 64 tiles) and its fill2
(the same over 256 x 64 tiles), the features the planner computes: a random
layout of blocks smaller than a tile leaves most of each non-empty tile
masked, where banded, windowed and frame-aligned layouts fill them, and the
two want different tile heights. Each synthetic request's fill and fill2 are
read back from the planner, the requests of a bin are grouped by (fill bin,
fill2 bin), and each group's timings (summed over its layouts) give that
group's rule.

Inputs are seeded and synthetic (workloads module): BLOCK masks in banded,
local-window and random layouts at three densities, plus the Sparse VideoGen
head patterns rasterised at the block shape (half the heads spatial in
frame-major order, half temporal in temporal-major order, as the high-res
workload; it joins the density bin its own density falls in); video head
routing (VIDEO masks, the same head split); slice lists; Q/K/V ~ N(0,1) in
bf16, drawn on the device. The largest length bin runs 24 heads where the
mask stays under MASK_CAP bytes (4 heads for 32 x 32 blocks). Each bin's rule
names the fastest (regime, task order) pair.

Usage (on the target GPU, from the repository root):
    python3 block_sparse_attention_fwd_amd/lut/build_lut.py [--out lut/gfx950.lut] [--orders all] [--quick]
Prints one progress line per measurement and writes the table (rules plus the
measurements as comments). Rebuild the library afterwards: the default table
is compiled into it.
"""
import argparse
import os
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

TILE_REGIMES = (0, 1, 4)        # contiguous-tile regimes (block and video masks)
SLICE_RULES = ((64, 2), (128, 3))  # slice masks: the gather regime of the slice height
ORDER_NAMES = ((0, "xcd"), (1, "lpt"))  # task orders (BSA_ORDER_*: XCD-grouped, plain longest first)
ORDERS = ORDER_NAMES[:1]          # timed orders (--orders all adds lpt)
# sequence-length bins: (representative token grid T x Hg x Wg, L range of the rule, heads of the requests)
LENGTH_BINS = (
    ((4, 32, 32), (0, 8192), 24),
    ((13, 30, 52), (8193, 40000), 24),
    ((21, 45, 80), (40001, 150000), 24),
    ((21, 90, 160), (150001, 9999999999), 24),
)
MASK_CAP = 600_000_000  # bytes of a request's uint8 block mask; past it the request runs 4 heads
BLOCK_SHAPES = ((32, 32), (64, 64), (128, 128), (64, 256))
DENSITY_BINS = ((0.05, (0.0, 0.1)), (0.15, (0.1, 0.275)), (0.4, (0.275, 1.0)))
FILL_BINS = ((0.0, 0.75), (0.75, 1.0))  # low fill: random layouts of small blocks; high: banded / windowed
FILL2_BINS = ((0.0, 0.75), (0.75, 1.0))  # the same over 256-row tiles: low also for random 128-row blocks
LAYOUTS = ("banded", "local", "random")
VIDEO_LAYOUT = "video"  # the video head patterns rasterised at the block shape


def log(*a):
    print(*a, flush=True)


def oname(order):
    return dict(ORDER_NAMES)[order]


# a choice other than the default (the first timed: regime 0, or the slice
# height's gather regime, with the XCD-grouped order) must win by more than
# this fraction; within it the timings do not tell the choices apart (three
# interleaved rounds spread by about 1%)
MARGIN = 0.02


def pick(times):
    default = next(iter(times))
    best = min(times, key=times.get)
    return best if times[best] < (1.0 - MARGIN) * times[default] else default


def vname(x):
    return f"r{x[0]}/{oname(x[1])}"


def time_regimes(bsa, torch, w, regimes, q, k, v, o, reps, rounds=3):
    """Median forward time (ms) of each (regime, task order) variant on
    workload w. The variants are timed in interleaved rounds, so that clock
    and thermal drift during the sweep falls on all of them alike."""
    from bsa_helpers import plan_workload
    plans = {(r, od): plan_workload(w, force_regime=r, task_order=od) for r in regimes for od, _ in ORDERS}
    for r in regimes:  # warm the code and the clocks of each variant
        bsa.forward(plans[(r, ORDERS[0][0])], q, k, v, o)
    try:
        times = {v: [] for v in plans}
        for _ in range(rounds):
            for r in plans:
                p = plans[r]
                bsa.forward(p, q, k, v, o)
                torch.cuda.synchronize()
                ev = []
                for _ in range(reps):
                    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    a.record()
                    bsa.forward(p, q, k, v, o)
                    b.record()
                    ev.append((a, b))
                torch.cuda.synchronize()
                times[r] += [a.elapsed_time(b) for a, b in ev]
        return {r: sorted(t)[len(t) // 2] for r, t in times.items()}
    finally:
        for p in plans.values():
            p.close()


def in_bin(x, bins):
    for lo, hi in bins:
        if lo <= x <= hi:
            return (lo, hi)
    return bins[-1]


def block_rules(bq, bk, dlo, dhi, llo, lhi, groups):
    """Table lines of one (block shape, density, length) bin from its groups
    {(fill bin, fill2 bin): summed timings}. A group no layout fell into takes
    the choice of the group with the same fill bin, else of one with the same
    fill2 bin, else of any, so every (fill, fill2) in [0, 1]^2 resolves."""
    picks = {g: pick(t) for g, t in groups.items()}
    out = []
    for fb in FILL_BINS:
        for f2 in FILL2_BINS:
            best = (picks.get((fb, f2)) or next((v for (a, _), v in picks.items() if a == fb), None)
                    or next((v for (_, b), v in picks.items() if b == f2), None) or next(iter(picks.values())))
            out.append(f"block   {bq:<7d} {bk:<7d} {dlo:<10g} {dhi:<10g} {fb[0]:<7g} {fb[1]:<7g} {f2[0]:<7g} "
                       f"{f2[1]:<7g} {llo:<6d} {lhi:<10d} {best[0]} {oname(best[1])}")
    return out


def main():
    global ORDERS
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--out", default=os.path.join(HERE, "gfx950.lut"))
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--orders", choices=("xcd", "all"), default="xcd",
                    help="task orders to time: the XCD-grouped one, or also plain longest first")
    ap.add_argument("--quick", action="store_true", help="one layout per bin, two length bins")
    args = ap.parse_args()
    if args.orders == "all":
        ORDERS = ORDER_NAMES

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import torch

    import block_sparse_attention_fwd_amd as bsa
    import workloads as wl
    from bsa_helpers import plan_workload

    assert torch.cuda.is_available(), "the lookup table is built on the GPU it is for"
    d = 128
    length_bins = LENGTH_BINS[:2] if args.quick else LENGTH_BINS
    layouts = LAYOUTS[:1] if args.quick else LAYOUTS
    rules, notes, slice_rules = [], [], []
    t_start = time.time()
    for (T, Hg, Wg), (llo, lhi), H in length_bins:
        L = T * Hg * Wg
        # Q/K/V ~ N(0,1) in bf16, drawn on the device (the timings do not
        # depend on the values); requests with fewer heads use the first ones
        gen = torch.Generator(device="cuda:0")
        gen.manual_seed(9)
        q, k, v = (torch.randn((1, H, L, d), generator=gen, device="cuda:0").to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(q)
        # video head routing
        wv = wl.svg("B", H=H, T=T, Hg=Hg, Wg=Wg, d=d, cfg=9)
        tv = time_regimes(bsa, torch, wv, TILE_REGIMES, q, k, v, o, args.reps)
        best = pick(tv)
        log(f"[lut] video L={L}: " + ", ".join(f"{vname(x)} {t:.4f} ms" for x, t in tv.items()) + f" -> {vname(best)}")
        notes.append(f"video L={L} H={H}: " + " ".join(f"{vname(x)}={t:.4f}ms" for x, t in tv.items()))
        rules.append(f"video   *       *       -1         1          -1      1       {llo:<6d} {lhi:<10d} "
                     f"{best[0]} {oname(best[1])}")
        for (bq, bk) in BLOCK_SHAPES:
            Hs = H if -(-L // bq) * -(-L // bk) * H <= MASK_CAP else 4
            groups = {rb: {} for rb in DENSITY_BINS}  # density bin -> {(fill bin, fill2 bin): summed timings}
            requests = [(rho, li, lay) for rho, _ in DENSITY_BINS for li, lay in enumerate(layouts)]
            if not args.quick:
                requests.append((None, len(layouts), VIDEO_LAYOUT))
            for rho, li, lay in requests:
                if lay == VIDEO_LAYOUT:
                    w = wl.video_block_request(f"lut_{bq}x{bk}_video", 9, bq, bk, Hs, T, Hg, Wg, d)
                else:
                    w = wl.block_request(f"lut_{bq}x{bk}_{rho}_{lay}", 9, li, bq, bk, rho, lay, Hs, T, Hg, Wg, d)
                hp = plan_workload(w, device=-1)
                info = hp.info()
                hp.close()
                dens, fill, fill2 = info["mask_density"], info["mask_fill"], info["mask_fill2"]
                tt = time_regimes(bsa, torch, w, TILE_REGIMES, q, k, v, o, args.reps)
                rb = next(b for b in DENSITY_BINS if b[1][0] <= dens <= b[1][1]) if rho is None else \
                    next(b for b in DENSITY_BINS if b[0] == rho)
                g = groups[rb].setdefault((in_bin(fill, FILL_BINS), in_bin(fill2, FILL2_BINS)), {})
                for x, t in tt.items():
                    g[x] = g.get(x, 0.0) + t
                tag = f"density {dens:.3f} (bin {rb[0]})" if rho is None else f"density {rho}"
                log(f"[lut] block {bq}x{bk} {tag} {lay} L={L} H={Hs} fill {fill:.3f} fill2 {fill2:.3f}: "
                    + ", ".join(f"{vname(x)} {t:.4f} ms" for x, t in tt.items()))
                notes.append(f"block {bq}x{bk} rho={rho if rho is not None else round(dens, 3)} {lay} L={L} H={Hs} "
                             f"fill={fill:.3f} fill2={fill2:.3f}: " + " ".join(f"{vname(x)}={t:.4f}ms" for x, t in tt.items()))
            for rho, (dlo, dhi) in DENSITY_BINS:
                rules += block_rules(bq, bk, dlo, dhi, llo, lhi, groups[(rho, (dlo, dhi))])
        # slice masks: the gather regime is fixed by the slice height; the task
        # order is timed on the middle length bin (the key lists of the largest
        # one take gigabytes to generate) and applies to every length
        if (T, Hg, Wg) == LENGTH_BINS[1][0]:
            for m, r in SLICE_RULES:
                ws = wl.fgattn(H=H, T=T, Hg=Hg, Wg=Wg, d=d, M=m, cfg=9)
                ts = time_regimes(bsa, torch, ws, (r,), q, k, v, o, args.reps)
                best = pick(ts)
                log(f"[lut] slice M={m} L={L}: " + ", ".join(f"{vname(x)} {t:.4f} ms" for x, t in ts.items()) + f" -> {vname(best)}")
                notes.append(f"slice M={m} L={L}: " + " ".join(f"{vname(x)}={t:.4f}ms" for x, t in ts.items()))
                slice_rules.append(f"slice   {m:<7d} 1       0          1          -1      1       0      9999999999 "
                                   f"{r} {oname(best[1])}")
        del q, k, v, o
        torch.cuda.empty_cache()
    rules += slice_rules or [f"slice   {m:<7d} 1       0          1          -1      1       0      9999999999 {r} xcd"
                             for m, r in SLICE_RULES]
    # anything not covered (other block shapes): the default tile regime
    rules.append("block   *       *       0          1          0       1       0       1       0      9999999999 0 xcd")
    rules.append("video   *       *       -1         1          -1      1       0      9999999999 0 xcd")
    head = [
        "# Regime lookup table for gfx950 (MI355X), built by lut/build_lut.py (offline profiling).",
        "# First matching rule wins. Regimes: 0 = 128x64 tiles (4 waves), 1 = 64x64 tiles (2 waves),",
        "# 2 = 64-query gather, 3 = 128-query gather, 4 = 256x64 tiles (8 waves).",
        "# Task orders: xcd = longest first, grouped so neighbouring query tiles share an XCD; lpt = longest first.",
        "# Features: density = kept blocks / blocks; fill = kept pairs / pairs of the non-empty 128x64 tiles;",
        "# fill2 = the same over 256x64 tiles. Block lines carry the fill2 range; other lines match any fill2.",
        f"# Synthetic requests, d = {d}, bf16; median of 3 interleaved rounds of {args.reps} forwards.",
        "# kind  block_q block_k density_lo density_hi fill_lo fill_hi [fill2_lo fill2_hi] L_lo   L_hi       regime order",
    ]
    text = "\n".join(head + rules + ["#", "# measurements:"] + ["# " + n for n in notes]) + "\n"
    with open(args.out, "w") as f:
        f.write(text)
    log(f"[lut] wrote {args.out} ({len(rules)} rules) in {time.time() - t_start:.1f} s")


if __name__ == "__main__":
    np.seterr(all="ignore")
    main()
