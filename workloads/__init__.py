"""Seeded synthetic workloads for block-sparse attention.

This module only *generates inputs*: query/key/value tensors and logical mask
descriptors shaped like the workloads on the source pages. It contains none of
the attention arithmetic and is the one module shared by the CPU oracle side
and the GPU path (tests and the benchmark import it; neither side imports the
other).

Token order of every tensor is frame-major: token ``i = t*Hg*Wg + y*Wg + x``.
A head may be *temporal-major*: its logical position ``j = p*T + t`` for the
token at pixel ``p = y*Wg + x`` of frame ``t`` (Sparse VideoGen / Splash
Attention summary, "Splash Attention": token layouts permuted into
temporal-major order for the temporal patterns). Block and slice masks index
logical positions of their head.

Seeds: ``numpy.random.default_rng([cfg, purpose, h, i])`` with purpose 0 = Q,
1 = K, 2 = V, 3 = mask. Values are N(0,1) drawn in float32 and rounded to
bfloat16 with round-to-nearest-even; consumers of bf16 data use those rounded
values.
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

# mask kinds / patterns / layouts (numeric values match the C ABI's enums so
# descriptors pass through unchanged; they are plain data, not arithmetic)
BLOCK, BLOCK_BITS, SLICE, VIDEO = 1, 2, 3, 4
DENSE, SPATIAL, TEMPORAL = 0, 1, 2
FRAME_MAJOR, TEMPORAL_MAJOR = 0, 1

PURPOSE_Q, PURPOSE_K, PURPOSE_V, PURPOSE_MASK = 0, 1, 2, 3


def rng(cfg: int, purpose: int, h: int = 0, i: int = 0) -> np.random.Generator:
    return np.random.default_rng([cfg, purpose, h, i])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round-to-nearest-even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass
class Workload:
    """A logical-mask problem: shapes, geometry, mask descriptor, per-head layout."""
    name: str
    cfg: int                      # seed namespace
    B: int
    H: int
    L: int
    d: int
    T: int = 0                    # video geometry (T*Hg*Wg == L when set)
    Hg: int = 0
    Wg: int = 0
    kind: int = BLOCK
    bq: int = 64                  # logical block (BLOCK); M (SLICE); 1 (VIDEO)
    bk: int = 64                  # logical block (BLOCK); 1 (SLICE, VIDEO)
    block: Optional[np.ndarray] = None      # uint8 [B][H][nqb][nkb]
    row_ptr: Optional[np.ndarray] = None    # int64 [B*H*nqb + 1]
    col_idx: Optional[np.ndarray] = None    # int32
    head_pattern: Optional[np.ndarray] = None  # uint8 [H]
    anchor: int = 0
    radius: int = 2
    head_layout: Optional[np.ndarray] = None   # uint8 [H]

    @property
    def nqb(self) -> int:
        return -(-self.L // self.bq)

    @property
    def nkb(self) -> int:
        return -(-self.L // self.bk)

    def layout(self) -> np.ndarray:
        if self.head_layout is None:
            return np.zeros(self.H, np.uint8)
        return self.head_layout

    def block_bits(self) -> np.ndarray:
        """The BLOCK mask re-encoded as uint64 bit rows [B][H][nqb][ceil(nkb/64)]."""
        assert self.block is not None
        nkb = self.block.shape[-1]
        words = -(-nkb // 64)
        padded = np.zeros(self.block.shape[:-1] + (words * 64,), np.uint8)
        padded[..., :nkb] = self.block != 0
        bits = np.packbits(padded.reshape(-1, words, 64), axis=-1, bitorder="little")
        return bits.view(np.uint64).reshape(self.block.shape[:-1] + (words,)).copy()


# ----------------------------------------------------------------------------
# Q / K / V
# ----------------------------------------------------------------------------

def _head_tensor(cfg, purpose, h, L, d, dtype):
    x = rng(cfg, purpose, h).standard_normal((L, d), dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f32":
        return x
    if dtype == "f64":
        return x.astype(np.float64)
    raise ValueError(dtype)


def make_qkv(w: Workload, dtype: str = "bf16", threads: int = 8):
    """Q, K, V as [B][H][L][d]; bf16 as uint16 bits, else float32/float64."""
    out = []
    for purpose in (PURPOSE_Q, PURPOSE_K, PURPOSE_V):
        jobs = [(b, h) for b in range(w.B) for h in range(w.H)]
        with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            parts = list(ex.map(lambda bh: _head_tensor(w.cfg * 1000 + bh[0], purpose, bh[1], w.L, w.d, dtype), jobs))
        arr = np.stack(parts).reshape(w.B, w.H, w.L, w.d)
        out.append(arr)
    return tuple(out)


# ----------------------------------------------------------------------------
# mask generators
# ----------------------------------------------------------------------------

def bernoulli_block_mask(cfg, B, H, nqb, nkb, density, force_diag=False) -> np.ndarray:
    m = np.zeros((B, H, nqb, nkb), np.uint8)
    for b in range(B):
        for h in range(H):
            m[b, h] = rng(cfg * 1000 + b, PURPOSE_MASK, h).random((nqb, nkb)) < density
            if force_diag:
                n = min(nqb, nkb)
                m[b, h, np.arange(n), np.arange(n)] = 1
    return m


def _frames_of_blocks(L, blk, HW):
    lo = np.arange(0, L, blk)
    hi = np.minimum(lo + blk, L) - 1
    return lo // HW, hi // HW


def _pixel_ranges_tm(L, blk, T):
    """Pixel index range [p0, p1] covered by each block of temporal-major positions."""
    lo = np.arange(0, L, blk)
    hi = np.minimum(lo + blk, L) - 1
    return lo // T, hi // T


def rasterize_video_block_mask(T, Hg, Wg, pattern, layout, bq, bk, anchor=0, radius=2) -> np.ndarray:
    """Block mask [nqb][nkb] that keeps a logical block iff any element pair in
    it is kept by the video pattern, in the head's own layout (FG-Attn abstract:
    block-sparse attention skips a block only when every entry in it is zero)."""
    HW = Hg * Wg
    L = T * HW
    nqb, nkb = -(-L // bq), -(-L // bk)
    if pattern == DENSE:
        return np.ones((nqb, nkb), np.uint8)
    if layout == FRAME_MAJOR:
        # element (q, k) -> frames and pixels of contiguous frame-major ranges
        if pattern == SPATIAL:
            fq0, fq1 = _frames_of_blocks(L, bq, HW)
            fk0, fk1 = _frames_of_blocks(L, bk, HW)
            overlap = (fq0[:, None] <= fk1[None, :]) & (fk0[None, :] <= fq1[:, None])
            has_anchor = (fk0 <= anchor) & (anchor <= fk1)
            return (overlap | has_anchor[None, :]).astype(np.uint8)
        # temporal, frame-major: pixel sets of each block (pixels of every frame it covers)
        return _raster_pixels(L, HW, Wg, bq, bk, radius,
                              lambda lo, hi: _fm_pixels(lo, hi, HW))
    # temporal-major layout: position j -> (pixel j // T, frame j % T)
    if pattern == SPATIAL:
        def frames(lo, hi):
            n = hi - lo + 1
            if n >= T:
                return np.ones(T, bool)
            f = np.zeros(T, bool)
            f[(lo + np.arange(n)) % T] = True
            return f
        qf = [frames(lo, min(lo + bq, L) - 1) for lo in range(0, L, bq)]
        kf = [frames(lo, min(lo + bk, L) - 1) for lo in range(0, L, bk)]
        QF = np.array(qf)
        KF = np.array(kf)
        inter = (QF.astype(np.int32) @ KF.T.astype(np.int32)) > 0
        return (inter | KF[:, anchor][None, :]).astype(np.uint8)
    return _raster_pixels(L, HW, Wg, bq, bk, radius,
                          lambda lo, hi: np.arange(lo // T, hi // T + 1))


def _fm_pixels(lo, hi, HW):
    if hi - lo + 1 >= HW:
        return np.arange(HW)
    a, b = lo % HW, hi % HW
    if a <= b:
        return np.arange(a, b + 1)
    return np.concatenate([np.arange(a, HW), np.arange(0, b + 1)])


def _raster_pixels(L, HW, Wg, bq, bk, radius, pixels_of):
    Hg = HW // Wg
    nqb, nkb = -(-L // bq), -(-L // bk)
    # which key blocks contain each pixel (a pixel may appear in several blocks)
    kblocks_of_pixel = [[] for _ in range(HW)]
    for kb in range(nkb):
        lo, hi = kb * bk, min(kb * bk + bk, L) - 1
        for p in pixels_of(lo, hi):
            kblocks_of_pixel[int(p)].append(kb)
    out = np.zeros((nqb, nkb), np.uint8)
    for qb in range(nqb):
        lo, hi = qb * bq, min(qb * bq + bq, L) - 1
        pix = pixels_of(lo, hi)
        img = np.zeros((Hg, Wg), bool)
        img.reshape(-1)[pix] = True
        # dilate by the Chebyshev radius
        dil = np.zeros_like(img)
        ys, xs = np.nonzero(img)
        for dy in range(-radius, radius + 1):
            for dx in range(-radius, radius + 1):
                yy, xx = ys + dy, xs + dx
                ok = (yy >= 0) & (yy < Hg) & (xx >= 0) & (xx < Wg)
                dil[yy[ok], xx[ok]] = True
        for p in np.flatnonzero(dil.reshape(-1)):
            for kb in kblocks_of_pixel[p]:
                out[qb, kb] = 1
    return out


def slice_lists(cfg, B, H, L, M, dens_lo=0.1, dens_hi=0.3, run_frac=0.7, run_lo=4, run_hi=32):
    """M x 1 slice key lists (FG-Attn abstract): per block of M queries a sorted
    key set. Density U[dens_lo, dens_hi]; ``run_frac`` of kept keys come from
    contiguous runs of run_lo..run_hi keys (runs placed uniformly, overlapping
    runs add only their new keys, the last run truncated), the rest uniformly
    scattered over keys not yet selected."""
    nqb = -(-L // M)
    row_ptr = np.zeros(B * H * nqb + 1, np.int64)
    lists = []
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                g = rng(cfg * 1000 + b, PURPOSE_MASK, h, i)
                rho = g.uniform(dens_lo, dens_hi)
                n = int(round(rho * L))
                n_run = int(round(run_frac * n))
                first = np.full(L, np.iinfo(np.int64).max, np.int64)
                taken = 0
                base = 0
                while True:
                    nb = max(64, 2 * (n_run - taken) // ((run_lo + run_hi) // 2) + 8)
                    ell = g.integers(run_lo, run_hi + 1, nb)
                    s = (g.random(nb) * (L - ell + 1)).astype(np.int64)
                    idx = np.repeat(np.arange(base, base + nb), ell)
                    pos = np.repeat(s, ell) + (np.arange(ell.sum()) - np.repeat(np.cumsum(ell) - ell, ell))
                    np.minimum.at(first, pos, idx)
                    base += nb
                    taken = int((first < np.iinfo(np.int64).max).sum())
                    if taken >= n_run:
                        break
                covered = np.flatnonzero(first < np.iinfo(np.int64).max)
                order = np.lexsort((covered, first[covered]))
                run_keys = covered[order[:n_run]]
                sel = np.zeros(L, bool)
                sel[run_keys] = True
                free = np.flatnonzero(~sel)
                scat = free[g.choice(free.size, n - n_run, replace=False)] if n > n_run else np.zeros(0, np.int64)
                keys = np.sort(np.concatenate([run_keys, scat])).astype(np.int32)
                lists.append(keys)
                row_ptr[(b * H + h) * nqb + i + 1] = keys.size
    row_ptr = np.cumsum(row_ptr)
    col_idx = np.concatenate(lists) if lists else np.zeros(0, np.int32)
    return row_ptr, col_idx.astype(np.int32)


# ----------------------------------------------------------------------------
# the five workloads (shapes from the source pages' workloads: 5-second clips of
# "more than 30K embeddings", M = 64 blocks, 480p/720p/1440p-like grids)
# ----------------------------------------------------------------------------

def tiny(H=2, T=4, Hg=16, Wg=16, d=64, density=0.3, blk=64, cfg=1) -> Workload:
    """H=2, L=1024 (4 x 16x16), d=64; 64x64 Bernoulli(0.3) block mask, diagonal kept."""
    L = T * Hg * Wg
    w = Workload("tiny", cfg, 1, H, L, d, T, Hg, Wg, BLOCK, blk, blk)
    w.block = bernoulli_block_mask(cfg, 1, H, w.nqb, w.nkb, density, force_diag=True)
    return w


def svg(run: str = "A", H=24, T=13, Hg=30, Wg=52, d=128, cfg=2, n_spatial=None) -> Workload:
    """Sparse VideoGen head routing: first half of the heads spatial (same frame
    plus frame 0), the rest temporal (same pixel +/-2 in y and x, every frame).
    Run "A": every head frame-major. Run "B": temporal heads temporal-major."""
    L = T * Hg * Wg
    ns = H // 2 if n_spatial is None else n_spatial
    w = Workload("svg" + run, cfg, 1, H, L, d, T, Hg, Wg, VIDEO, 1, 1)
    w.head_pattern = np.array([SPATIAL] * ns + [TEMPORAL] * (H - ns), np.uint8)
    w.anchor, w.radius = 0, 2
    lay = np.zeros(H, np.uint8)
    if run == "B":
        lay[ns:] = TEMPORAL_MAJOR
    w.head_layout = lay
    return w


def fgattn(H=24, T=21, Hg=30, Wg=52, d=128, M=64, cfg=3, **kw) -> Workload:
    """FG-Attn M x 1 slices: per 64-query block a seeded key set."""
    L = T * Hg * Wg
    w = Workload("fgattn", cfg, 1, H, L, d, T, Hg, Wg, SLICE, M, 1)
    w.row_ptr, w.col_idx = slice_lists(cfg, 1, H, L, M, **kw)
    return w


C4_SHAPES = [(32, 32), (64, 64), (128, 128), (64, 256)]
C4_DENSITIES = [0.05, 0.15, 0.4]
C4_LAYOUTS = ["banded", "local", "random"]


def c4_params(i: int):
    if i < 36:
        return C4_SHAPES[i % 4], C4_DENSITIES[(i // 4) % 3], C4_LAYOUTS[i // 12]
    g = rng(4, PURPOSE_MASK, 999, i)
    return C4_SHAPES[int(g.integers(4))], C4_DENSITIES[int(g.integers(3))], C4_LAYOUTS[int(g.integers(3))]


def _banded(L, bq, bk, rho):
    nqb, nkb = -(-L // bq), -(-L // bk)
    cq = (np.arange(nqb) * bq + np.minimum(np.arange(nqb) * bq + bq, L) - 1) / 2.0
    ck = (np.arange(nkb) * bk + np.minimum(np.arange(nkb) * bk + bk, L) - 1) / 2.0
    dist = np.abs(cq[:, None] - ck[None, :])
    vals = np.unique(dist)
    # smallest band half-width (a distance value) reaching the target density
    lo, hi = 0, vals.size - 1
    while lo < hi:
        mid = (lo + hi) // 2
        if (dist <= vals[mid]).mean() >= rho:
            hi = mid
        else:
            lo = mid + 1
    return (dist <= vals[lo]).astype(np.uint8)


def _local(T, Hg, Wg, bq, bk, rho):
    L = T * Hg * Wg
    nqb, nkb = -(-L // bq), -(-L // bk)
    rows = T * Hg
    t_of = np.arange(rows) // Hg
    y_of = np.arange(rows) % Hg
    rq0 = np.arange(nqb) * bq // Wg
    rq1 = (np.minimum(np.arange(nqb) * bq + bq, L) - 1) // Wg
    rk0 = np.arange(nkb) * bk // Wg
    rk1 = (np.minimum(np.arange(nkb) * bk + bk, L) - 1) // Wg
    best = None
    for s in range(0, max(T, Hg) + 1):
        a, b = s, 3 * s
        rk = ((np.abs(t_of[:, None] - t_of[None, :]) <= a) & (np.abs(y_of[:, None] - y_of[None, :]) <= b)).astype(np.int64)
        P = np.zeros((rows + 1, rows + 1), np.int64)
        P[1:, 1:] = rk.cumsum(0).cumsum(1)
        A0, A1 = rq0[:, None], rq1[:, None] + 1
        B0, B1 = rk0[None, :], rk1[None, :] + 1
        cnt = P[A1, B1] - P[A0, B1] - P[A1, B0] + P[A0, B0]
        m = (cnt > 0).astype(np.uint8)
        best = m
        if m.mean() >= rho:
            break
    return best


def block_request(name, cfg, i, bq, bk, rho, lay, H=24, T=21, Hg=45, Wg=80, d=128) -> Workload:
    """A BLOCK-mask request on a T x Hg x Wg token grid: layout ``lay``
    (banded / local / random) at target block density ``rho``."""
    L = T * Hg * Wg
    w = Workload(name, cfg, 1, H, L, d, T, Hg, Wg, BLOCK, bq, bk)
    if lay == "random":
        w.block = bernoulli_block_mask(cfg * 100 + i, 1, H, w.nqb, w.nkb, rho)
    else:
        one = _banded(L, bq, bk, rho) if lay == "banded" else _local(T, Hg, Wg, bq, bk, rho)
        w.block = np.broadcast_to(one, (1, H) + one.shape).copy()
    return w


def tessera(i: int, H=24, T=21, Hg=45, Wg=80, d=128, cfg=4) -> Workload:
    """Tessera-style dynamic block-sparse request, mask ``i`` of 48."""
    (bq, bk), rho, lay = c4_params(i)
    return block_request(f"tessera{i}", cfg, i, bq, bk, rho, lay, H, T, Hg, Wg, d)


def video_block_request(name, cfg, bq, bk, H, T, Hg, Wg, d) -> Workload:
    """A BLOCK-mask request whose blocks are the video head patterns
    rasterised at bq x bk: heads 0..H/2-1 spatial in frame-major order, the
    rest temporal in temporal-major order."""
    L = T * Hg * Wg
    w = Workload(name, cfg, 1, H, L, d, T, Hg, Wg, BLOCK, bq, bk)
    ns = H // 2
    sp = rasterize_video_block_mask(T, Hg, Wg, SPATIAL, FRAME_MAJOR, bq, bk)
    tp = rasterize_video_block_mask(T, Hg, Wg, TEMPORAL, TEMPORAL_MAJOR, bq, bk)
    w.block = np.stack([sp] * ns + [tp] * (H - ns))[None]
    w.head_layout = np.array([FRAME_MAJOR] * ns + [TEMPORAL_MAJOR] * (H - ns), np.uint8)
    return w


def highres(H=24, T=21, Hg=90, Wg=160, d=128, blk=128, cfg=5) -> Workload:
    """High-res: half the heads spatial (frame-major), half temporal
    (temporal-major); 128x128 logical blocks rasterised from the patterns."""
    return video_block_request("highres", cfg, blk, blk, H, T, Hg, Wg, d)


# ----------------------------------------------------------------------------
# inputs with a known head routing
# ----------------------------------------------------------------------------

PURPOSE_BOOST = 4


def routed_qkv(w: Workload, kinds, alpha: float, base: float = 0.5, dtype: str = "bf16"):
    """Q, K, V [B][H][L][d] for head routing: Q and K are base * N(0,1) plus,
    per head, alpha times a seeded unit vector shared by all tokens of one
    frame (kinds[h] == SPATIAL) or of one pixel (kinds[h] == TEMPORAL), so that
    that head's attention concentrates within frames or along pixel tracks;
    V is N(0,1). bf16 as uint16 bits (rounded once, after the sum)."""
    HW = w.Hg * w.Wg
    tok = np.arange(w.L)
    frame, pixel = tok // HW, tok % HW
    Q = np.zeros((w.B, w.H, w.L, w.d), np.float32)
    K = np.zeros_like(Q)
    V = np.zeros_like(Q)
    for b in range(w.B):
        for h in range(w.H):
            g = rng(w.cfg * 1000 + b, PURPOSE_BOOST, h)
            Q[b, h] = base * g.standard_normal((w.L, w.d), dtype=np.float32)
            K[b, h] = base * g.standard_normal((w.L, w.d), dtype=np.float32)
            V[b, h] = g.standard_normal((w.L, w.d), dtype=np.float32)
            if kinds[h] == DENSE:
                continue
            groups = w.T if kinds[h] == SPATIAL else HW
            u = g.standard_normal((groups, w.d)).astype(np.float32)
            u /= np.linalg.norm(u, axis=1, keepdims=True)
            sel = u[frame if kinds[h] == SPATIAL else pixel]
            Q[b, h] += alpha * sel
            K[b, h] += alpha * sel
    if dtype == "bf16":
        return f32_to_bf16_bits(Q), f32_to_bf16_bits(K), f32_to_bf16_bits(V)
    return Q, K, V


def sample_tokens(L: int, n: int, seed: int) -> np.ndarray:
    """n distinct query tokens drawn uniformly from [0, L), sorted."""
    return np.sort(np.random.default_rng([seed, 77]).choice(L, size=min(n, L), replace=False)).astype(np.int32)
