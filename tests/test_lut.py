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
