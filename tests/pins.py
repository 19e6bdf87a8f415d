"""Pins of the CPU oracle: checks against things other than the oracle itself.

Each ``pin_*`` takes the path of an oracle library build and returns a list of
failure messages (empty = pinned). ``test_oracle.py`` requires every pin to
hold for the real oracle; ``test_oracle_mutants.py`` plants plausible mistakes
into copies of the oracle source and requires every mutant to break a pin.
"""
import math
import os

import numpy as np
import torch

import oracle
import workloads as wl
from brute import brute_attend, element_mask, tok_of_logical

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# tiny seeded problems of every mask kind
# ---------------------------------------------------------------------------

def tiny_cases(seed=0):
    """(workload, dtype) pairs covering every kind, both layouts, ragged
    blocks, empty rows and empty lists. T*Hg*Wg = L everywhere."""
    g = np.random.default_rng(seed)
    cases = []
    # BLOCK, frame-major and temporal-major, ragged last block (L=36, blocks 8x16)
    for lay in (0, 1):
        w = wl.Workload(f"blk{lay}", 90, 1, 2, 36, 8, 3, 3, 4, wl.BLOCK, 8, 16)
        w.block = (g.random((1, 2, w.nqb, w.nkb)) < 0.45).astype(np.uint8)
        w.block[0, 1, 1, :] = 0  # a query block with no key: empty rows
        w.head_layout = np.array([lay, 1 - lay], np.uint8)
        cases.append(w)
    # BLOCK with 70 key blocks (two 64-bit words per bit row), non-power-of-2 bq
    w = wl.Workload("blkwide", 93, 1, 2, 70, 4, 2, 5, 7, wl.BLOCK, 5, 1)
    w.block = (g.random((1, 2, w.nqb, w.nkb)) < 0.3).astype(np.uint8)
    w.head_layout = np.array([0, 1], np.uint8)
    cases.append(w)
    # SLICE M=8 over L=40 (ragged last query block of 0 rows? 40 = 5*8: add ragged case too)
    for lay, (T, Hg, Wg) in ((0, (2, 4, 5)), (1, (3, 3, 5))):
        L = T * Hg * Wg
        w = wl.Workload(f"slc{lay}", 91, 1, 2, L, 6, T, Hg, Wg, wl.SLICE, 8, 1)
        nqb = w.nqb
        rp, ci = [0], []
        for e in range(2 * nqb):
            n = int(g.integers(0, 7)) if e != 3 else 0
            keys = np.sort(g.choice(L, n, replace=False)).astype(np.int32)
            ci.append(keys)
            rp.append(rp[-1] + n)
        w.row_ptr = np.array(rp, np.int64)
        w.col_idx = np.concatenate(ci).astype(np.int32)
        w.head_layout = np.array([lay, lay], np.uint8)
        cases.append(w)
    # VIDEO: spatial, temporal, dense heads; anchor frame 1 in one case
    for anchor, lay in ((0, 0), (1, 1)):
        w = wl.Workload(f"vid{anchor}", 92, 1, 3, 3 * 3 * 4, 5, 3, 3, 4, wl.VIDEO, 1, 1)
        w.head_pattern = np.array([wl.SPATIAL, wl.TEMPORAL, wl.DENSE], np.uint8)
        w.anchor, w.radius = anchor, 1
        w.head_layout = np.array([lay, lay, 0], np.uint8)
        cases.append(w)
    return cases


def rand_qkv(w, seed, dtype=np.float64, scale=1.0):
    g = np.random.default_rng(seed)
    shp = (w.B, w.H, w.L, w.d)
    Q, K, V = (g.standard_normal(shp) * scale for _ in range(3))
    if dtype == np.uint16:
        return tuple(wl.f32_to_bf16_bits(x.astype(np.float32)) for x in (Q, K, V))
    return tuple(x.astype(dtype) for x in (Q, K, V))


def as_f64(x):
    if x.dtype == np.uint16:
        return wl.bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


def _err(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_bruteforce(lib_path):
    """Oracle == pure-Python brute force (math.fsum) on tiny inputs, every kind."""
    fails = []
    for ci, w in enumerate(tiny_cases()):
        for dt in (np.float64, np.float32, np.uint16):
            Q, K, V = rand_qkv(w, 10 + ci, dt)
            O = oracle.attend(w, Q, K, V, lib_path=lib_path).reshape(w.B, w.H, w.L, w.d)
            Qf, Kf, Vf = as_f64(Q), as_f64(K), as_f64(V)
            for b in range(w.B):
                for h in range(w.H):
                    em = element_mask(w, b, h)
                    for q in range(w.L):
                        ref = brute_attend(Qf[b, h, q], Kf[b, h], Vf[b, h], em[q])
                        e = _err(O[b, h, q], ref)
                        if not e <= 1e-12:
                            fails.append(f"brute {w.name} {dt.__name__} h{h} q{q}: {e:.3g}")
                            break
    return fails


def pin_library_sdpa(lib_path):
    """Oracle == torch CPU float64 scaled_dot_product_attention with a boolean
    mask expanded independently; rows with no kept key must be exactly 0."""
    fails = []
    for ci, w in enumerate(tiny_cases(1)):
        Q, K, V = rand_qkv(w, 20 + ci)
        O = oracle.attend(w, Q, K, V, lib_path=lib_path).reshape(w.B, w.H, w.L, w.d)
        for b in range(w.B):
            for h in range(w.H):
                em = element_mask(w, b, h)
                ref = torch.nn.functional.scaled_dot_product_attention(
                    torch.from_numpy(Q[b, h])[None], torch.from_numpy(K[b, h])[None], torch.from_numpy(V[b, h])[None],
                    attn_mask=torch.from_numpy(em)[None]).numpy()[0]
                live = em.any(1)
                e = _err(O[b, h][live], ref[live])
                if not e <= 1e-12:
                    fails.append(f"sdpa {w.name} h{h}: {e:.3g}")
                if np.any(O[b, h][~live] != 0.0):
                    fails.append(f"sdpa {w.name} h{h}: empty rows not zero")
    return fails


def _dense_video(L, H=1):
    w = wl.Workload("dense", 0, 1, H, L, 1, 1, 1, L, wl.VIDEO, 1, 1)
    w.head_pattern = np.zeros(H, np.uint8)
    return w


def pin_masked_equals_deleted(lib_path):
    """Masking key k out of a row == deleting row k of K and V for that row."""
    fails = []
    for ci, w in enumerate(tiny_cases(2)):
        Q, K, V = rand_qkv(w, 30 + ci)
        O = oracle.attend(w, Q, K, V, lib_path=lib_path).reshape(w.B, w.H, w.L, w.d)
        for h in range(w.H):
            em = element_mask(w, 0, h)
            for q in range(0, w.L, 5):
                S = np.flatnonzero(em[q])
                if S.size == 0:
                    continue
                dw = _dense_video(S.size)
                dw.d = w.d
                Qd = np.repeat(Q[0, h, q][None, None, None], S.size, axis=2)
                Od = oracle.attend(dw, Qd, K[0, h, S][None, None], V[0, h, S][None, None], lib_path=lib_path)
                e = _err(O[0, h, q], Od[0])
                if not e <= 1e-13:
                    fails.append(f"deleted {w.name} h{h} q{q}: {e:.3g}")
    return fails


def _expanded(w):
    """The same problem with a 1x1-block element mask of the same pairs."""
    e = wl.Workload(w.name + "_el", w.cfg, w.B, w.H, w.L, w.d, w.T, w.Hg, w.Wg, wl.BLOCK, 1, 1)
    e.block = np.stack([np.stack([element_mask(w, b, h) for h in range(w.H)]) for b in range(w.B)]).astype(np.uint8)
    return e


def pin_block_equals_expansion(lib_path):
    """A block mask (and a slice mask) == its element-level expansion (1x1
    blocks); BLOCK_BITS == BLOCK_U8."""
    fails = []
    for ci, w in enumerate(tiny_cases(3)):
        if w.kind == wl.VIDEO:
            continue
        Q, K, V = rand_qkv(w, 40 + ci)
        O = oracle.attend(w, Q, K, V, lib_path=lib_path)
        Oe = oracle.attend(_expanded(w), Q, K, V, lib_path=lib_path)
        if not _err(O, Oe) <= 1e-13:
            fails.append(f"expansion {w.name}: {_err(O, Oe):.3g}")
        if w.kind == wl.BLOCK:
            Ob = oracle.attend(w, Q, K, V, lib_path=lib_path, bits=True)
            if not np.array_equal(O, Ob):
                fails.append(f"bits {w.name}")
    # SLICE(M) == BLOCK(M, 1) with the same bits
    for ci, w in enumerate(tiny_cases(4)):
        if w.kind != wl.SLICE:
            continue
        bw = wl.Workload(w.name + "_b", w.cfg, w.B, w.H, w.L, w.d, w.T, w.Hg, w.Wg, wl.BLOCK, w.bq, 1)
        blk = np.zeros((w.B, w.H, w.nqb, w.L), np.uint8)
        for b in range(w.B):
            for h in range(w.H):
                for i in range(w.nqb):
                    e = (b * w.H + h) * w.nqb + i
                    blk[b, h, i, w.col_idx[w.row_ptr[e]:w.row_ptr[e + 1]]] = 1
        bw.block, bw.head_layout = blk, w.head_layout
        Q, K, V = rand_qkv(w, 50 + ci)
        if not _err(oracle.attend(w, Q, K, V, lib_path=lib_path), oracle.attend(bw, Q, K, V, lib_path=lib_path)) <= 1e-13:
            fails.append(f"slice==block {w.name}")
    return fails


def pin_kv_permutation(lib_path):
    """Permuting the key/value rows together with the mask's key columns
    leaves every output unchanged."""
    fails = []
    g = np.random.default_rng(5)
    for ci, w in enumerate(tiny_cases(5)):
        e = _expanded(w)
        Q, K, V = rand_qkv(w, 60 + ci)
        O = oracle.attend(e, Q, K, V, lib_path=lib_path)
        sigma = g.permutation(w.L)
        e2 = _expanded(w)
        e2.block = e.block[..., sigma].copy()
        O2 = oracle.attend(e2, Q, K[:, :, sigma].copy(), V[:, :, sigma].copy(), lib_path=lib_path)
        if not _err(O, O2) <= 1e-12:
            fails.append(f"kvperm {w.name}: {_err(O, O2):.3g}")
    return fails


def pin_tm_equivariance(lib_path):
    """A temporal-major head == the frame-major computation on tokens
    physically stored in temporal-major order (rows permuted by reshape), with
    the output permuted back."""
    fails = []
    for ci, w in enumerate(tiny_cases(6)):
        if w.kind == wl.VIDEO:
            continue
        Q, K, V = rand_qkv(w, 70 + ci)
        O = oracle.attend(w, Q, K, V, lib_path=lib_path).reshape(w.B, w.H, w.L, w.d)
        tok = tok_of_logical(w.T, w.Hg * w.Wg)
        fm = wl.Workload(w.name + "_fm", w.cfg, w.B, w.H, w.L, w.d, w.T, w.Hg, w.Wg, w.kind, w.bq, w.bk)
        fm.block, fm.row_ptr, fm.col_idx = w.block, w.row_ptr, w.col_idx
        fm.head_layout = np.zeros(w.H, np.uint8)
        lay = w.layout()
        Qp, Kp, Vp = Q.copy(), K.copy(), V.copy()
        for h in range(w.H):
            if lay[h]:
                Qp[:, h], Kp[:, h], Vp[:, h] = Q[:, h][:, tok], K[:, h][:, tok], V[:, h][:, tok]
        Op = oracle.attend(fm, Qp, Kp, Vp, lib_path=lib_path).reshape(w.B, w.H, w.L, w.d)
        for h in range(w.H):
            ref = np.empty_like(Op[:, h])
            if lay[h]:
                ref[:, tok] = Op[:, h]
            else:
                ref = Op[:, h]
            if not _err(O[:, h], ref) <= 1e-13:
                fails.append(f"tm-equivariance {w.name} h{h}: {_err(O[:, h], ref):.3g}")
    return fails


def pin_video_layout_invariance(lib_path):
    """Video patterns are defined on token coordinates, so the head's layout
    does not change the result (run A == run B)."""
    fails = []
    for ci, w in enumerate(tiny_cases(7)):
        if w.kind != wl.VIDEO:
            continue
        Q, K, V = rand_qkv(w, 80 + ci)
        a = oracle.attend(w, Q, K, V, lib_path=lib_path)
        w2 = wl.Workload(w.name, w.cfg, w.B, w.H, w.L, w.d, w.T, w.Hg, w.Wg, w.kind, 1, 1)
        w2.head_pattern, w2.anchor, w2.radius = w.head_pattern, w.anchor, w.radius
        w2.head_layout = 1 - w.layout()
        b = oracle.attend(w2, Q, K, V, lib_path=lib_path)
        if not np.array_equal(a, b):
            fails.append(f"video layout {w.name}")
    return fails


def pin_closed_forms(lib_path):
    """Closed forms of the definition."""
    fails = []
    g = np.random.default_rng(8)
    L, d = 24, 8
    w = wl.Workload("cf", 0, 1, 1, L, d, 2, 3, 4, wl.BLOCK, 1, 1)
    Q, K, V = (g.standard_normal((1, 1, L, d)) for _ in range(3))
    # one kept key per row -> O = V[k] exactly
    sel = g.integers(0, L, L)
    w.block = np.zeros((1, 1, L, L), np.uint8)
    w.block[0, 0, np.arange(L), sel] = 1
    O = oracle.attend(w, Q, K, V, lib_path=lib_path)
    if not np.array_equal(O, V[0, 0, sel]):
        fails.append("one kept key")
    # no kept key -> exactly zero
    w.block[:] = 0
    w.block[0, 0, :, 0] = 1
    w.block[0, 0, 5, :] = 0
    O = oracle.attend(w, Q, K, V, lib_path=lib_path)
    if np.any(O[5] != 0.0) or not np.array_equal(O[3], V[0, 0, 0]):
        fails.append("empty row")
    # constant V -> O = that constant
    w.block = (g.random((1, 1, L, L)) < 0.5).astype(np.uint8)
    w.block[0, 0, np.arange(L), np.arange(L)] = 1
    Vc = np.full_like(V, 0.3)
    O = oracle.attend(w, Q, K, Vc, lib_path=lib_path)
    if not _err(O, 0.3) <= 1e-15:
        fails.append("constant V")
    # identical keys -> plain mean of the kept values
    Ki = np.repeat(K[:, :, :1], L, axis=2)
    O = oracle.attend(w, Q, Ki, V, lib_path=lib_path)
    m = w.block[0, 0].astype(bool)
    ref = np.stack([V[0, 0][m[q]].mean(0) for q in range(L)])
    if not _err(O, ref) <= 1e-14:
        fails.append("identical keys mean")
    # shifting every key by the same vector u adds q.u/sqrt(d) to every score of
    # row q: softmax unchanged
    u = g.standard_normal(d)
    O1 = oracle.attend(w, Q, K, V, lib_path=lib_path)
    O2 = oracle.attend(w, Q, K + u, V, lib_path=lib_path)
    if not _err(O1, O2) <= 1e-12:
        fails.append("key shift")
    # (2Q, K/2) gives identical scores in binary floating point
    O3 = oracle.attend(w, 2 * Q, K / 2, V, lib_path=lib_path)
    if not np.array_equal(O1, O3):
        fails.append("query/key rescale")
    # scores scaled by 1/sqrt(d): doubling Q squares the weights; check against
    # an explicit softmax of the scores written as a matrix product
    S = (Q[0, 0] @ K[0, 0].T) / math.sqrt(d)
    S = np.where(m, S, -np.inf)
    P = np.exp(S - S.max(1, keepdims=True))
    ref = (P @ V[0, 0]) / P.sum(1, keepdims=True)
    if not _err(O1, ref) <= 1e-13:
        fails.append("matrix softmax")
    return fails


def _golden_cases():
    out = []
    with open(os.path.join(GOLDEN, "worked_examples.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, d, q, keys, vals, kept, exp = [s.strip() for s in line.split(";")]
            d = int(d)
            vec = lambda s: np.array([float(x) for x in s.split(",")], np.float64)
            rows = lambda s: np.stack([vec(r) for r in s.split("|")])
            K, V = rows(keys), rows(vals)
            keep = np.ones(len(K), bool) if kept == "all" else np.zeros(len(K), bool)
            if kept not in ("all", ""):
                keep[[int(x) for x in kept.split(",")]] = True
            expv = np.zeros(d) if exp == "zero" else vec(exp)
            out.append((name, d, vec(q), K, V, keep, expv))
    return out


def pin_golden(lib_path):
    """Hand-worked examples stored under tests/golden/."""
    fails = []
    for name, d, q, K, V, keep, expv in _golden_cases():
        n = len(K)
        L = n + 1
        # row 0 is the query; rows 1..n hold the keys/values
        w = wl.Workload(name, 0, 1, 1, L, d, 1, 1, L, wl.BLOCK, 1, 1)
        Q = np.zeros((1, 1, L, d))
        Q[0, 0, 0] = q
        Kf = np.zeros((1, 1, L, d))
        Vf = np.zeros((1, 1, L, d))
        Kf[0, 0, 1:], Vf[0, 0, 1:] = K, V
        w.block = np.zeros((1, 1, L, L), np.uint8)
        w.block[0, 0, 0, 1:] = keep
        O = oracle.attend(w, Q, Kf, Vf, rows=np.array([0]), lib_path=lib_path)[0]
        if not _err(O, expv) <= 1e-14 * max(1.0, float(np.abs(expv).max())):
            fails.append(f"golden {name}: {O} vs {expv}")
    return fails


def video_pairs_closed_form(T, Hg, Wg, pattern, anchor=0, r=2):
    """Kept pairs of one video head counted from the geometry alone."""
    HW = Hg * Wg
    if pattern == wl.SPATIAL:
        # anchor-frame queries see one frame (HW keys), the others two (2 HW)
        return HW * HW + (T - 1) * HW * 2 * HW
    cy = sum(min(Hg - 1, y + r) - max(0, y - r) + 1 for y in range(Hg))
    cx = sum(min(Wg - 1, x + r) - max(0, x - r) + 1 for x in range(Wg))
    return T * T * cy * cx


def pin_counts(lib_path):
    """Pair counts: video patterns against closed forms, block and slice kinds
    against the element expansion."""
    fails = []
    for (T, Hg, Wg) in ((3, 4, 5), (2, 7, 3)):
        for pat in (wl.SPATIAL, wl.TEMPORAL):
            w = wl.Workload("cnt", 0, 1, 1, T * Hg * Wg, 1, T, Hg, Wg, wl.VIDEO, 1, 1)
            w.head_pattern = np.array([pat], np.uint8)
            got = oracle.count_pairs(w, 0, 0, lib_path=lib_path)
            want = video_pairs_closed_form(T, Hg, Wg, pat)
            if got != want:
                fails.append(f"video count {pat} {T}x{Hg}x{Wg}: {got} vs {want}")
    for w in tiny_cases(9):
        for h in range(w.H):
            got = oracle.count_pairs(w, 0, h, lib_path=lib_path)
            want = int(element_mask(w, 0, h).sum())
            if got != want:
                fails.append(f"count {w.name} h{h}: {got} vs {want}")
    return fails


def brute_union_total(w, b, h, M):
    """Sum over the M-row blocks of head (b, h)'s logical positions of the
    number of distinct keys kept by any row of the block, from the independent
    element-level mask (frame-major tokens), and the per-block key sets."""
    em = element_mask(w, b, h)
    if w.layout()[h] == wl.TEMPORAL_MAJOR:
        order = tok_of_logical(w.T, w.Hg * w.Wg)  # token at each logical position
    else:
        order = np.arange(w.L)
    sets = []
    for j0 in range(0, w.L, M):
        rows = order[j0:j0 + M]
        sets.append(em[rows].any(axis=0))
    return int(sum(int(u.sum()) for u in sets)), sets


def pin_block_union(lib_path):
    """Per-block key unions (om_block_union) and their totals (om_union_total)
    == the union of the independent element mask's rows, every kind, both
    layouts, blocks smaller than, equal to and spanning several logical query
    blocks; BLOCK_BITS == BLOCK_U8."""
    fails = []
    for w in tiny_cases(11):
        for h in range(w.H):
            for M in (3, 4, 8, 16, 64):
                want, sets = brute_union_total(w, 0, h, M)
                got = oracle.union_total(w, 0, h, M, lib_path=lib_path)
                if got != want:
                    fails.append(f"union total {w.name} h{h} M{M}: {got} vs {want}")
                for beta, u in enumerate(sets):
                    used = oracle.block_union(w, 0, h, beta, M, lib_path=lib_path).astype(bool)
                    if not np.array_equal(used, u):
                        fails.append(f"block union {w.name} h{h} M{M} block {beta}")
                        break
                if w.kind == wl.BLOCK:
                    L_ = oracle.lib(lib_path)
                    mk = oracle.Mask(w, bits=True)
                    gb = int(L_.om_union_total(oracle.ctypes.byref(mk.m), 0, h, M))
                    if gb != want:
                        fails.append(f"union total bits {w.name} h{h} M{M}: {gb} vs {want}")
    return fails


ALL_PINS = [pin_bruteforce, pin_library_sdpa, pin_masked_equals_deleted, pin_block_equals_expansion,
            pin_kv_permutation, pin_tm_equivariance, pin_video_layout_invariance, pin_closed_forms, pin_golden,
            pin_counts, pin_block_union]
