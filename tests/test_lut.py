"""The regime lookup table (Tessera, abstract: an execution regime chosen by a
lookup table from offline profiling): the builder's choice rule, and the
shipped table as the library compiles it in. Host planning only (device=-1),
so these run on the CPU."""
import os
import sys

import numpy as np
import pytest

import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LUT_DIR = os.path.join(ROOT, "block_sparse_attention_fwd_amd", "lut")
sys.path.insert(0, LUT_DIR)
import build_lut  # noqa: E402

bsa = pytest.importorskip("block_sparse_attention_fwd_amd")


def test_pick_keeps_the_default_within_the_margin():
    d, other, lpt = (0, 0), (1, 0), (0, 1)
    # the first entry is the default
    assert build_lut.pick({d: 1.0, other: 0.99, lpt: 0.985}) == d
    assert build_lut.pick({d: 1.0, other: 0.97, lpt: 0.99}) == other
    assert build_lut.pick({d: 1.0, other: 1.2}) == d
    # a win exactly at the margin is not enough
    assert build_lut.pick({d: 1.0, other: 1.0 - build_lut.MARGIN}) == d
    assert build_lut.pick({d: 1.0}) == d


def _lib():
    try:
        bsa.lib()
    except Exception as e:  # noqa: BLE001
        pytest.skip(f"library not built: {e}")


def _block_plan(bq, bk, L, rho, seed, lut_path=None):
    g = np.random.default_rng(seed)
    nqb, nkb = -(-L // bq), -(-L // bk)
    m = (g.random((1, 2, nqb, nkb)) < rho).astype(np.uint8)
    m[..., 0, 0] = 1
    return bsa.plan(bsa.MASK_BLOCK_U8, 1, 2, L, 64, bq, bk, data=m, lut_path=lut_path, device=-1).info()


@pytest.mark.parametrize("bq,bk", [(32, 32), (64, 64), (128, 128), (64, 256)])
@pytest.mark.parametrize("rho", [0.05, 0.2, 0.6])
def test_shipped_table_file_equals_the_compiled_table(bq, bk, rho):
    """Rules read from lut/gfx950.lut choose what the compiled-in copy does."""
    _lib()
    L = 2048
    a = _block_plan(bq, bk, L, rho, 1)
    b = _block_plan(bq, bk, L, rho, 1, lut_path=os.path.join(LUT_DIR, "gfx950.lut"))
    assert (a["regime"], a["task_order"]) == (b["regime"], b["task_order"])
    assert a["regime"] in (0, 1, 4)


def test_every_dense_bin_resolves_to_a_tile_regime():
    """Video masks and each profiled block shape get a contiguous-tile regime
    at every length bin's representative length."""
    _lib()
    for L in (1024, 20280):
        for bq, bk in [(32, 32), (64, 64), (128, 128), (64, 256)]:
            assert _block_plan(bq, bk, L, 0.15, 2)["regime"] in (0, 1, 4)
        w = wl.svg("B", H=2, T=2, Hg=16, Wg=32) if L == 1024 else wl.svg("B", H=2, T=13, Hg=30, Wg=52)
        assert w.L == L
        info = bsa.plan(bsa.MASK_VIDEO, w.B, w.H, w.L, 64, 1, 1, head_pattern=w.head_pattern, anchor_frame=0,
                        radius=2, head_layout=w.head_layout, T=w.T, Hg=w.Hg, Wg=w.Wg, device=-1).info()
        assert info["regime"] in (0, 1, 4)


def _features_by_definition(block, L, bq, bk, stride):
    """Density and fills written out from their definitions with numpy:
    density = kept blocks / blocks of the sampled logical rows; fill = kept
    pairs / pairs of the non-empty 128 x 64 tiles, over every stride-th
    128-row query tile of every head; fill2 = the same over the 256 x 64
    tiles that start at those rows (every 256-row tile when stride is 1)."""
    B, H, nqb, nkb = block.shape
    kept_blocks = blocks = 0
    kept_pairs = exec_pairs = kept2 = exec2 = 0.0
    qlen = np.minimum(np.arange(1, nqb + 1) * bq, L) - np.arange(nqb) * bq
    nqt, nkt = -(-L // 128), -(-L // 64)
    for bh in range(B * H):
        m = block.reshape(B * H, nqb, nkb)[bh].astype(bool)
        el = np.kron(m, np.ones((bq, bk), bool))[:L, :L]  # element mask (logical positions)
        for tq in range(0, nqt, stride):
            q0, q1 = tq * 128, min(tq * 128 + 128, L)
            rows = range(q0 // bq, (q1 - 1) // bq + 1)
            kept_blocks += int(m[list(rows)].sum())
            blocks += len(rows) * nkb
            sub = el[q0:q1]
            kept_pairs += float(sub.sum())
            tiles = np.pad(sub.any(axis=0), (0, nkt * 64 - L)).reshape(nkt, 64).any(axis=1)
            exec_pairs += float(tiles.sum()) * (q1 - q0) * 64
        for q0 in range(0, L, 256 * (1 if stride == 1 else stride // 2)):
            sub = el[q0:q0 + 256]
            kept2 += float(sub.sum())
            tiles = np.pad(sub.any(axis=0), (0, nkt * 64 - L)).reshape(nkt, 64).any(axis=1)
            exec2 += float(tiles.sum()) * sub.shape[0] * 64
    return kept_blocks / blocks, kept_pairs / exec_pairs, kept2 / exec2


@pytest.mark.parametrize("bq,bk", [(32, 32), (64, 64), (128, 128), (64, 256), (256, 32)])
@pytest.mark.parametrize("layout", ["random", "banded"])
def test_mask_features_match_definition(bq, bk, layout):
    """The planner's regime features (bsa_plan_info mask_density, mask_fill
    and mask_fill2) equal their definitions, on masks short enough that every
    query tile is sampled and on longer ones where every 4th is; random
    layouts of small blocks have low fill, banded ones high."""
    _lib()
    for L in (1000, 4100):
        nqb, nkb = -(-L // bq), -(-L // bk)
        g = np.random.default_rng(bq * 7 + bk)
        if layout == "random":
            m = (g.random((1, 2, nqb, nkb)) < 0.2).astype(np.uint8)
        else:
            cq = (np.arange(nqb) + 0.5) * bq
            ck = (np.arange(nkb) + 0.5) * bk
            m = np.broadcast_to((np.abs(cq[:, None] - ck[None, :]) <= 300)[None, None], (1, 2, nqb, nkb)).astype(np.uint8)
        info = bsa.plan(bsa.MASK_BLOCK_U8, 1, 2, L, 64, bq, bk, data=np.ascontiguousarray(m), device=-1).info()
        stride = 4 if -(-L // 128) >= 16 else 1
        dens, fill, fill2 = _features_by_definition(m, L, bq, bk, stride)
        assert abs(info["mask_density"] - dens) < 1e-12, (L, info["mask_density"], dens)
        assert abs(info["mask_fill"] - fill) < 1e-9, (L, info["mask_fill"], fill)
        assert abs(info["mask_fill2"] - fill2) < 1e-9, (L, info["mask_fill2"], fill2)
        if stride == 1:  # same rows: a 256-row tile computes at least its halves' pairs
            assert info["mask_fill2"] <= info["mask_fill"] + 1e-12
    if layout == "banded":
        assert info["mask_fill"] > 0.75
    elif bq < 128 or bk < 64:
        assert info["mask_fill"] < 0.75
