"""Seeded workload generators: closed-form pair counts, rasterisation against
the element-level expansion, slice-list properties, bf16 rounding."""
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from brute import element_mask
from pins import video_pairs_closed_form

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _facts():
    out = {}
    for line in open(os.path.join(GOLDEN, "page_facts.txt")):
        if line.strip() and not line.startswith("#"):
            k, v, _ = [s.strip() for s in line.split(";")]
            out[k] = v
    return out


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    x = np.concatenate([g.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3.0e38, 1e-40], np.float32)])
    ours = wl.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(wl.bf16_bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_qkv_seeded_and_reproducible():
    w = wl.tiny()
    a = wl.make_qkv(w)
    b = wl.make_qkv(w, threads=1)
    for x, y in zip(a, b):
        assert x.dtype == np.uint16 and x.shape == (1, 2, 1024, 64)
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], a[1])
    f = wl.bf16_bits_to_f32(a[0])
    assert abs(f.mean()) < 0.02 and abs(f.std() - 1) < 0.02


def test_tiny_mask():
    w = wl.tiny()
    assert w.L == 1024 and w.nqb == 16 and w.block.shape == (1, 2, 16, 16)
    assert np.all(w.block[0, :, np.arange(16), np.arange(16)] == 1)
    for h in range(2):
        for q in (0, 100, 1023):
            assert oracle.row_keys(w, 0, h, q).size >= 64
    dens = w.block.mean()
    assert 0.2 < dens < 0.5


def test_svg_pair_counts_full_size():
    """Kept pairs per head of the SVG workload (13 x 30x52): spatial
    HW^2 (2T-1), temporal T^2 * sum_y c_y * sum_x c_x."""
    assert video_pairs_closed_form(13, 30, 52, wl.SPATIAL) == 60_840_000
    assert video_pairs_closed_form(13, 30, 52, wl.TEMPORAL) == 6_181_344
    w = wl.svg("A")
    assert w.L == 20280
    assert oracle.count_pairs(w, 0, 0) == 60_840_000
    assert oracle.count_pairs(w, 0, 23) == 6_181_344
    wb = wl.svg("B")
    assert oracle.count_pairs(wb, 0, 23) == 6_181_344


@pytest.mark.parametrize("pattern", [wl.SPATIAL, wl.TEMPORAL])
@pytest.mark.parametrize("layout", [wl.FRAME_MAJOR, wl.TEMPORAL_MAJOR])
@pytest.mark.parametrize("blk", [(4, 4), (8, 16), (16, 8)])
def test_rasterised_block_mask_is_any_pair_rule(pattern, layout, blk):
    T, Hg, Wg = 3, 5, 7
    bq, bk = blk
    got = wl.rasterize_video_block_mask(T, Hg, Wg, pattern, layout, bq, bk, radius=1)
    w = wl.Workload("v", 0, 1, 1, T * Hg * Wg, 1, T, Hg, Wg, wl.VIDEO, 1, 1)
    w.head_pattern = np.array([pattern], np.uint8)
    w.radius = 1
    em = element_mask(w, 0, 0)  # token order
    L = w.L
    if layout == wl.TEMPORAL_MAJOR:
        tok = np.arange(L).reshape(T, Hg * Wg).T.reshape(-1)
        em = em[np.ix_(tok, tok)]  # logical order
    nqb, nkb = -(-L // bq), -(-L // bk)
    want = np.zeros((nqb, nkb), np.uint8)
    for i in range(nqb):
        for j in range(nkb):
            want[i, j] = em[i * bq:(i + 1) * bq, j * bk:(j + 1) * bk].any()
    assert np.array_equal(got, want)


def test_highres_statistics():
    """High-res 21 x 90x160 with 128x128 blocks: rasterised block densities and
    the total kept pairs."""
    w = wl.highres()
    assert w.L == 302_400 and w.block.shape == (1, 24, 2363, 2363)
    sp, tp = w.block[0, 0].mean(), w.block[0, 12].mean()
    assert abs(sp - 0.09353) < 5e-5, sp
    assert abs(tp - 0.005411) < 5e-6, tp
    total = sum(oracle.count_pairs(w, 0, h) for h in (0, 12)) * 12
    assert total == 108_589_744_128


def test_fgattn_lists():
    facts = _facts()
    w = wl.fgattn(H=2)
    assert w.bq == int(facts["typical_block_m"])
    assert w.L > int(facts["min_tokens_5s_clip"])
    nqb = w.nqb
    assert nqb == 512 and w.row_ptr.size == 2 * nqb + 1
    lens = np.diff(w.row_ptr)
    assert lens.min() >= round(0.1 * w.L) and lens.max() <= round(0.3 * w.L)
    assert abs(lens.mean() - 0.2 * w.L) < 0.02 * w.L
    for e in range(0, 2 * nqb, 37):
        keys = w.col_idx[w.row_ptr[e]:w.row_ptr[e + 1]]
        assert np.all(np.diff(keys) > 0) and keys[0] >= 0 and keys[-1] < w.L
        # most kept keys sit in runs: neighbours that are also kept
        kept = np.zeros(w.L + 2, bool)
        kept[keys + 1] = True
        in_run = kept[keys] | kept[keys + 2]
        assert in_run.mean() > 0.6
    w2 = wl.fgattn(H=2)
    assert np.array_equal(w.col_idx, w2.col_idx)


def test_tessera_masks():
    seen = set()
    for i in (0, 5, 10, 15, 21, 26, 31):
        (bq, bk), rho, lay = wl.c4_params(i)
        seen.add(lay)
    assert seen == {"banded", "local", "random"}
    for i in (1, 17, 29):
        (bq, bk), rho, lay = wl.c4_params(i)
        w = wl.tessera(i, H=2)
        dens = w.block.mean()
        assert dens >= rho * 0.8, (i, lay, dens, rho)
        if lay != "random":
            assert dens >= rho
