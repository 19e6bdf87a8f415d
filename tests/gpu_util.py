"""Helpers for GPU parity tests: device tensors from seeded host data, running
the library through the C ABI, and comparing with the fp64 oracle."""
import sys

import numpy as np
import torch

import block_sparse_attention_fwd_amd as bsa
import oracle
import workloads as wl
from bsa_helpers import plan_workload, to_device_bf16, tok_of_logical

MAX_ABS = 1e-2   # bf16 inputs: max-abs error against the fp64 oracle
MEAN_ABS = 1e-3  # bf16 inputs: mean-abs error against the fp64 oracle
ROW_REL_F32 = 1e-5  # fp32 inputs: max over rows of |O - O_ref|_inf / |O_ref|_inf


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(x: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) or float32 host arrays -> cuda:0 tensor."""
    if x.dtype == np.uint16:
        return to_device_bf16(x)
    assert x.dtype == np.float32
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def run_gpu(w, Q, K, V, force_regime=-1, plan=None, fill=float("nan"), task_order=-1, rows=None):
    """Plan + forward on cuda:0 in the inputs' dtype (bf16 bits or float32);
    returns (O as float64 numpy [B][H][L][d], plan), or with ``rows`` (flat
    row ids) only those rows of O, [len(rows)][d], gathered on the device."""
    f32 = Q.dtype == np.float32
    dtype = bsa.DTYPE_F32 if f32 else bsa.DTYPE_BF16
    p = plan if plan is not None else plan_workload(w, device=0, force_regime=force_regime, dtype=dtype,
                                                    task_order=task_order)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    o = torch.full(q.shape, fill, dtype=torch.float32 if f32 else torch.bfloat16, device="cuda:0")
    bsa.forward(p, q, k, v, o)
    torch.cuda.synchronize()
    del q, k, v
    if rows is not None:
        idx = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.int64)).to("cuda:0")
        sub = o.reshape(-1, w.d).index_select(0, idx)
        return sub.float().cpu().numpy().astype(np.float64), p
    return o.float().cpu().numpy().astype(np.float64), p


def query_tile_rows(w, b, h, q0, tile):
    """Flat row ids of the logical query positions [q0, q0 + tile) of head
    (b, h): the rows one task of the kernel computes (temporal-major heads
    map logical position p*T + t to token t*HW + p)."""
    lo, hi = q0, min(q0 + tile, w.L)
    if w.layout()[h] == wl.TEMPORAL_MAJOR:
        toks = tok_of_logical(w.T, w.Hg * w.Wg)[lo:hi]
    else:
        toks = np.arange(lo, hi)
    return (b * w.H + h) * w.L + toks


def heavy_query_tile(w, b, h, tile, plan=None):
    """First logical position of a demanding query tile of head (b, h): for
    video masks, the tile with the most PARTIAL records in ``plan`` (exact
    masking on the device); for block masks, the tile whose logical block
    rows keep the most key blocks; for slice masks, the longest list."""
    if w.kind == wl.VIDEO and plan is not None:
        cnt = {}
        for r in plan.coverage(b, h):
            if r["kind"] == bsa.TILE_PARTIAL:
                key = r["q0"] // tile * tile
                cnt[key] = cnt.get(key, 0) + 1
        return max(cnt, key=cnt.get) if cnt else 0
    if w.kind == wl.BLOCK:
        per_block = w.block[b, h].astype(np.int64).sum(axis=1)
        per_tile = np.add.reduceat(per_block, np.arange(0, w.nqb, max(1, tile // w.bq))) if tile >= w.bq else per_block
        i = int(np.argmax(per_tile))
        return i * tile if tile >= w.bq else i * w.bq
    if w.kind == wl.SLICE:
        lens = np.diff(np.asarray(w.row_ptr, dtype=np.int64)).reshape(w.B, w.H, -1)[b, h]
        return int(np.argmax(lens)) * w.bq
    return 0


def thick_rows(w, tile, per_head=256, seed=0, plan=None, heads=None):
    """Per head: every row of one demanding query tile (heavy_query_tile),
    every row of the last (ragged) tile, ``per_head`` random rows and the
    first and last rows."""
    g = np.random.default_rng(seed)
    rows = []
    for b in range(w.B):
        for h in (range(w.H) if heads is None else heads):
            base = (b * w.H + h) * w.L
            rows.append(query_tile_rows(w, b, h, heavy_query_tile(w, b, h, tile, plan), tile))
            rows.append(query_tile_rows(w, b, h, (w.L - 1) // tile * tile, tile))
            rows.append(base + g.choice(w.L, per_head, replace=False))
            rows.append(base + np.array([0, w.L - 1]))
    return np.unique(np.concatenate(rows)).astype(np.int64)


def compare(w, Q, K, V, O_gpu, rows=None, label="", max_abs=MAX_ABS, mean_abs=MEAN_ABS, gathered=False):
    """Compare GPU output rows against the oracle. rows: flat row ids or None
    (all); gathered: O_gpu already holds just those rows, in that order."""
    if rows is None:
        rows = np.arange(w.B * w.H * w.L, dtype=np.int64)
    ref, cnt = oracle.attend(w, Q, K, V, rows=rows, return_counts=True)
    got = O_gpu.reshape(-1, w.d) if gathered else O_gpu.reshape(-1, w.d)[rows]
    err = np.abs(got - ref)
    mx, mean = float(err.max()), float(err.mean())
    nan = int(np.isnan(got).sum())
    zero_rows = cnt == 0
    zero_ok = bool(np.all(got[zero_rows] == 0.0))
    log(f"[parity] {label}: rows={rows.size} max_abs={mx:.3e} mean_abs={mean:.3e} nan={nan} "
        f"empty_rows={int(zero_rows.sum())} empty_exact_zero={zero_ok}")
    if not (mx <= max_abs and mean <= mean_abs and nan == 0 and zero_ok):
        row_err = np.nan_to_num(err, nan=np.inf).max(axis=1)
        for i in np.argsort(-row_err)[:8]:
            bh, q = divmod(int(rows[i]), w.L)
            log(f"    worst row: head={bh % w.H} q={q} kept={int(cnt[i])} err={row_err[i]:.3e} "
                f"got[:3]={got[i, :3]} ref[:3]={ref[i, :3]}")
        bad = row_err > max_abs
        if bad.any():
            heads = np.bincount((rows[bad] // w.L) % w.H, minlength=w.H)
            qs = rows[bad] % w.L
            log(f"    bad rows per head: {heads.tolist()}; q range {int(qs.min())}..{int(qs.max())}")
    assert nan == 0, f"{label}: {nan} NaN outputs"
    assert zero_ok, f"{label}: rows without kept keys are not exactly 0"
    assert mx <= max_abs, f"{label}: max-abs {mx}"
    assert mean <= mean_abs, f"{label}: mean-abs {mean}"
    return mx, mean


def compare_f32(w, Q, K, V, O_gpu, rows=None, label="", gathered=False):
    """fp32 build: per-row normwise relative error against the fp64 oracle
    (max over rows of |O - O_ref|_inf / |O_ref|_inf <= 1e-5); rows without a
    kept key exactly 0; elementwise relative error reported only."""
    if rows is None:
        rows = np.arange(w.B * w.H * w.L, dtype=np.int64)
    ref, cnt = oracle.attend(w, Q, K, V, rows=rows, return_counts=True)
    got = O_gpu.reshape(-1, w.d) if gathered else O_gpu.reshape(-1, w.d)[rows]
    nan = int(np.isnan(got).sum())
    zero_rows = cnt == 0
    zero_ok = bool(np.all(got[zero_rows] == 0.0))
    live = ~zero_rows
    num = np.abs(got[live] - ref[live]).max(axis=1)
    den = np.abs(ref[live]).max(axis=1)
    row_rel = num / den
    worst = float(row_rel.max()) if row_rel.size else 0.0
    elem = np.abs(got[live] - ref[live]) / np.maximum(np.abs(ref[live]), 1e-30)
    log(f"[parity f32] {label}: rows={rows.size} max_row_rel={worst:.3e} median_row_rel="
        f"{float(np.median(row_rel)) if row_rel.size else 0:.3e} max_elem_rel={float(elem.max()) if elem.size else 0:.3e} "
        f"nan={nan} empty_rows={int(zero_rows.sum())} empty_exact_zero={zero_ok}")
    if worst > ROW_REL_F32:
        idx = np.flatnonzero(live)
        for i in np.argsort(-row_rel)[:8]:
            bh, q = divmod(int(rows[idx[i]]), w.L)
            log(f"    worst row: head={bh % w.H} q={q} kept={int(cnt[idx[i]])} row_rel={row_rel[i]:.3e}")
    assert nan == 0, f"{label}: {nan} NaN outputs"
    assert zero_ok, f"{label}: rows without kept keys are not exactly 0"
    assert worst <= ROW_REL_F32, f"{label}: max row-relative error {worst}"
    return worst


def sample_rows(w, per_head=64, seed=0, tile=128):
    """Every row of each head's last (ragged) query tile plus random rows."""
    g = np.random.default_rng(seed)
    rows = []
    for b in range(w.B):
        for h in range(w.H):
            base = (b * w.H + h) * w.L
            last = (w.L - 1) // tile * tile
            rows.append(base + np.arange(last, w.L))
            rows.append(base + g.choice(w.L, per_head, replace=False))
            rows.append(base + np.array([0, w.L - 1]))
    return np.unique(np.concatenate(rows)).astype(np.int64)


def short_cases():
    """Sequences shorter than, equal to and just past one tile: BLOCK masks of
    1 to 127 tokens (32x32, 64x64 and 128x32 blocks, the diagonal kept in one
    head), video masks on 1x1x1, 2x3x5 and 3x1x7 grids (spatial, temporal in
    temporal-major order, dense), slice lists of 1 to 65 tokens with an empty
    list."""
    g = np.random.default_rng(41)
    out = []
    for L in (1, 17, 40, 64, 65, 127):
        for (bq, bk) in ((32, 32), (64, 64), (128, 32)):
            w = wl.Workload(f"short_blk{bq}x{bk}_L{L}", 140 + L, 1, 2, L, 64, 0, 0, 0, wl.BLOCK, bq, bk)
            w.block = (g.random((1, 2, w.nqb, w.nkb)) < 0.6).astype(np.uint8)
            w.block[0, 0] |= np.eye(w.nqb, w.nkb, dtype=np.uint8)
            out.append(w)
    for (T, Hg, Wg) in ((1, 1, 1), (2, 3, 5), (3, 1, 7)):
        w = wl.svg("B", H=3, T=T, Hg=Hg, Wg=Wg, d=64)
        w.name = f"short_video_{T}x{Hg}x{Wg}"
        w.head_pattern = np.array([wl.SPATIAL, wl.TEMPORAL, wl.DENSE], np.uint8)
        w.head_layout = np.array([0, 1, 1], np.uint8)
        w.radius = 1
        out.append(w)
    for L in (1, 40, 65):
        for M in (64, 128):
            w = wl.Workload(f"short_slice_M{M}_L{L}", 150 + L, 1, 2, L, 64, 0, 0, 0, wl.SLICE, M, 1)
            lists = [np.flatnonzero(g.random(L) < 0.5).astype(np.int32) for _ in range(2 * w.nqb)]
            lists[-1] = np.zeros(0, np.int32)  # a query block with an empty list
            w.row_ptr = np.concatenate([[0], np.cumsum([x.size for x in lists])]).astype(np.int64)
            w.col_idx = np.concatenate(lists).astype(np.int32)
            out.append(w)
    return out
