"""The mask-to-tile plan is bit-exact: the pairs the device computes (FULL
tiles whole, PARTIAL tiles through their predicate, gathered lists) are
exactly the pairs the oracle's own mask expansion keeps, each exactly once.
Host-only plans; no GPU needed."""
import numpy as np
import pytest

import block_sparse_attention_fwd_amd as bsa
import oracle
import workloads as wl
from brute import element_mask
from bsa_helpers import plan_workload, tok_of_logical


def coverage_counts(p, w, b, h):
    """uint8 [L][L] over (query token, key token): times each pair is computed."""
    L = w.L
    cnt = np.zeros((L, L), np.uint16)
    lay = w.layout()[h]
    tok = tok_of_logical(w.T, w.Hg * w.Wg) if lay == wl.TEMPORAL_MAJOR else np.arange(L)
    em_tok = element_mask(w, b, h) if w.kind == wl.VIDEO else None
    for r in p.coverage(b, h):
        qs = tok[r["q0"]:r["q1"]]
        if r["predicate"] == bsa.PRED_LIST:
            ks = tok[r["keys"]]
            cnt[np.ix_(qs, ks)] += 1
            continue
        ks = tok[r["k0"]:r["k1"]]
        if r["kind"] == bsa.TILE_FULL:
            cnt[np.ix_(qs, ks)] += 1
        elif r["predicate"] == bsa.PRED_SUBBLOCK:
            sq, sk = r["sub_q"], r["sub_k"]
            nsk = 64 // sk
            for i, qt in enumerate(range(r["q0"], r["q1"])):
                for j, kt in enumerate(range(r["k0"], r["k1"])):
                    bit = ((qt - r["q0"]) // sq) * nsk + (kt - r["k0"]) // sk
                    if (r["sub_bits"] >> bit) & 1:
                        cnt[tok[qt], tok[kt]] += 1
        elif r["predicate"] == bsa.PRED_VIDEO:
            sub = em_tok[np.ix_(qs, ks)]
            cnt[np.ix_(qs, ks)] += sub.astype(np.uint16)
        else:
            raise AssertionError(r)
    return cnt


def expected(w, b, h):
    """0/1 [L][L] from the oracle's own expansion (om_row_keys)."""
    L = w.L
    m = np.zeros((L, L), np.uint16)
    for q in range(L):
        m[q, oracle.row_keys(w, b, h, q)] = 1
    return m


def small_cases():
    out = []
    g = np.random.default_rng(3)
    # BLOCK: retain / combine / subdivide, ragged L, both layouts
    for (bq, bk) in [(64, 64), (32, 32), (128, 128), (64, 256), (32, 128), (256, 32)]:
        T, Hg, Wg = 3, 10, 11
        L = T * Hg * Wg  # 330: ragged for every block size
        w = wl.Workload(f"blk{bq}x{bk}", 7, 1, 2, L, 64, T, Hg, Wg, wl.BLOCK, bq, bk)
        w.block = (g.random((1, 2, w.nqb, w.nkb)) < 0.4).astype(np.uint8)
        w.block[0, 0, 0, :] = 1
        w.head_layout = np.array([0, 1], np.uint8)
        out.append(w)
    # SLICE M = 64 and 128, both layouts, empty lists
    for M in (64, 128):
        T, Hg, Wg = 3, 10, 11
        L = T * Hg * Wg
        w = wl.Workload(f"slice{M}", 8, 1, 2, L, 64, T, Hg, Wg, wl.SLICE, M, 1)
        nqb = w.nqb
        rp, ci = [0], []
        for e in range(2 * nqb):
            n = 0 if e == 1 else int(g.integers(1, 150))
            ci.append(np.sort(g.choice(L, n, replace=False)).astype(np.int32))
            rp.append(rp[-1] + n)
        w.row_ptr, w.col_idx = np.array(rp, np.int64), np.concatenate(ci)
        w.head_layout = np.array([0, 1], np.uint8)
        out.append(w)
    # VIDEO, small SVG-like geometry, both runs, anchor 0 and 2
    for run in ("A", "B"):
        w = wl.svg(run, H=4, T=5, Hg=7, Wg=13, d=64)
        w.head_pattern = np.array([wl.SPATIAL, wl.TEMPORAL, wl.SPATIAL, wl.DENSE], np.uint8)
        w.anchor = 2 if run == "B" else 0
        w.head_layout = np.array([0, 1, 1, 1], np.uint8) if run == "B" else np.zeros(4, np.uint8)
        out.append(w)
    return out


@pytest.mark.parametrize("w", small_cases(), ids=lambda w: w.name)
@pytest.mark.parametrize("regime", [-1, 0, 1, 4])
@pytest.mark.parametrize("order", [0, 1])
def test_plan_covers_each_kept_pair_once(w, regime, order):
    if w.kind == wl.SLICE:
        regime = -1  # slices run only in the gather regime matching M
    p = plan_workload(w, device=-1, force_regime=regime, task_order=order)
    for b in range(w.B):
        for h in range(w.H):
            got = coverage_counts(p, w, b, h)
            want = expected(w, b, h)
            bad = np.argwhere(got != want)
            assert bad.size == 0, f"{w.name} h{h}: {len(bad)} pairs wrong, first {bad[:5].tolist()}"


@pytest.mark.parametrize("regime", [0, 1, 4])
def test_video_records_are_tight(regime):
    """Video plans at wavefront granularity: every record the device computes
    (whole FULL tiles, and each wavefront's 32 rows of a PARTIAL tile) keeps at
    least one pair; FULL records keep all of theirs; a PARTIAL record whose
    keys lie inside the sequence keeps some but not all. So no wavefront runs a
    tile that holds nothing for its rows, and none masks rows it need not."""
    n_wave_records = 0
    for w in [c for c in small_cases() if c.kind == wl.VIDEO]:
        p = plan_workload(w, device=-1, force_regime=regime)
        tok_tm = tok_of_logical(w.T, w.Hg * w.Wg)
        for h in range(w.H):
            tok = tok_tm if w.layout()[h] == wl.TEMPORAL_MAJOR else np.arange(w.L)
            em = element_mask(w, 0, h)
            for r in p.coverage(0, h):
                kept = em[np.ix_(tok[r["q0"]:r["q1"]], tok[r["k0"]:r["k1"]])]
                assert kept.any(), (w.name, h, r)
                if r["kind"] == bsa.TILE_FULL:
                    assert kept.all(), (w.name, h, r)
                elif r["k1"] - r["k0"] == 64:
                    assert not kept.all(), (w.name, h, r)
                n_wave_records += r["q1"] - r["q0"] <= 32
    assert n_wave_records > 0


def test_block_bits_and_u8_give_the_same_plan():
    w = small_cases()[1]
    a = plan_workload(w, device=-1)
    b = plan_workload(w, device=-1, bits=True)
    for h in range(w.H):
        assert a.coverage(0, h) == b.coverage(0, h)


def test_every_query_tile_has_a_task():
    w = small_cases()[0]
    w.block[:] = 0
    p = plan_workload(w, device=-1)
    info = p.info()
    assert info["tiles_full"] + info["tiles_partial"] == 0
    assert info["tasks"] == w.H * -(-w.L // info["tile_q"])


@pytest.mark.parametrize("run,pattern,layout,want", [
    # (FULL, PARTIAL, EMPTY) per head for the 13 x 30x52 SVG workload at 128x64 tiles.
    # The last query tile has only 56 rows; rows past the sequence end are never
    # stored, so its 47 all-kept tiles are FULL (counting them PARTIAL would give
    # 6942 / 1001).
    ("A", wl.SPATIAL, 0, (6989, 954, 42460)),
    ("A", wl.TEMPORAL, 0, (0, 12835, 37568)),
    ("B", wl.TEMPORAL, 1, (0, 2998, 47405)),
])
def test_svg_tile_counts(run, pattern, layout, want):
    """Tile classification at full size matches the counts derived from the
    geometry (13 x 30x52, 128x64 tiles)."""
    w = wl.svg(run, H=1)
    w.head_pattern = np.array([pattern], np.uint8)
    w.head_layout = np.array([layout], np.uint8)
    info = plan_workload(w, device=-1, force_regime=0).info()
    assert (info["tiles_full"], info["tiles_partial"], info["tiles_empty"]) == want


def test_svg_plan_exact_on_sampled_query_tiles():
    """Full-size SVG plans (both runs): for sampled query tiles, the computed
    pairs equal the oracle's kept pairs exactly."""
    for run in ("A", "B"):
        w = wl.svg(run, H=24)
        p = plan_workload(w, device=-1)
        tq = p.info()["tile_q"]
        tok_tm = tok_of_logical(w.T, w.Hg * w.Wg)
        for h in (0, 11, 12, 23):
            recs = p.coverage(0, h)
            lay = w.layout()[h]
            tok = tok_tm if lay else np.arange(w.L)
            em = element_mask(w, 0, h)
            for q0 in (0, 1536, 10112, (w.L // tq) * tq):
                qs = tok[q0:min(q0 + tq, w.L)]
                cnt = np.zeros((qs.size, w.L), np.uint16)
                for r in recs:
                    if not (q0 <= r["q0"] < q0 + tq):
                        continue
                    rows = slice(r["q0"] - q0, r["q1"] - q0)
                    ks = tok[r["k0"]:r["k1"]]
                    if r["kind"] == bsa.TILE_FULL:
                        cnt[rows, ks] += 1
                    else:
                        cnt[rows, ks] += em[np.ix_(qs[rows], ks)]
                assert np.array_equal(cnt, em[qs].astype(np.uint16)), (run, h, q0)


# ---------------------------------------------------------------------------
# full-size plans (host-only): the configurations' own masks
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("regime", [-1, 0, 1, 4])
def test_tiny_plan_element_exact(regime):
    """Tiny configuration (2 heads, 1,024 tokens, 64x64 blocks): every pair of
    every head, element by element, against the oracle's expansion."""
    w = wl.tiny()
    p = plan_workload(w, device=-1, force_regime=regime)
    for h in range(w.H):
        got = coverage_counts(p, w, 0, h)
        want = expected(w, 0, h)
        assert np.array_equal(got, want), (regime, h, int((got != want).sum()))


def test_fgattn_plan_lists_exact():
    """FG-Attn slices at full size (24 heads, L = 32,760, M = 64): for sampled
    heads, the keys the plan gathers for each 64-query block, in record order,
    are exactly that block's list, each once; every block is present."""
    w = wl.fgattn()
    p = plan_workload(w, device=-1)
    nqb = w.nqb
    rp = np.asarray(w.row_ptr, dtype=np.int64)
    for h in (0, 7, 16, 23):
        got = {}
        for r in p.coverage(0, h):
            assert r["predicate"] == bsa.PRED_LIST and r["q1"] - r["q0"] <= w.bq
            got.setdefault(r["q0"], []).append(r["keys"])
        for i in range(nqb):
            e = h * nqb + i
            want = w.col_idx[rp[e]:rp[e + 1]]
            keys = np.concatenate(got.get(i * w.bq, [np.zeros(0, np.int32)]))
            assert np.array_equal(keys, want), (h, i, keys.size, want.size)


def _cell_coverage(p, w, b, h):
    """Times each logical cell is computed, from the plan's records. A cell is
    the intersection of a logical block and a physical tile (min(bq, tile_q)
    x min(bk, 64) positions): FULL records cover every cell of their tile,
    PARTIAL records the cells whose sub-block keep bit is set."""
    recs = p.coverage(b, h)
    tq = p.info()["tile_q"]
    cq, ck = min(w.bq, tq), min(w.bk, 64)
    nq, nk = -(-w.L // cq), -(-w.L // ck)
    cnt = np.zeros((nq, nk), np.uint8)
    q0 = np.array([r["q0"] for r in recs], np.int64)
    q1 = np.array([r["q1"] for r in recs], np.int64)
    k0 = np.array([r["k0"] for r in recs], np.int64)
    k1 = np.array([r["k1"] for r in recs], np.int64)
    full = np.array([r["kind"] == bsa.TILE_FULL for r in recs])
    bits = np.array([r["sub_bits"] for r in recs], np.int64)
    preds = {r["predicate"] for r in recs if r["kind"] != bsa.TILE_FULL}
    assert preds <= {bsa.PRED_SUBBLOCK}, preds
    nsk = 64 // ck
    for i in range(-(-tq // cq)):
        for j in range(-(-64 // ck)):
            rows, cols = q0 + i * cq, k0 + j * ck
            live = (rows < q1) & (cols < k1)
            keep = live & (full | (((bits >> (i * nsk + j)) & 1) == 1))
            np.add.at(cnt, (rows[keep] // cq, cols[keep] // ck), 1)
    want = np.kron(w.block[b, h].astype(np.uint8), np.ones((w.bq // cq, w.bk // ck), np.uint8))[:nq, :nk]
    return cnt, want


def _tile_elements(w, b, h, q0, q1, k0, k1):
    """Kept pairs of a rectangle of logical positions from the block mask's
    definition (every pair of a kept block), for exhaustive tile checks."""
    qb = np.arange(q0, q1) // w.bq
    kb = np.arange(k0, k1) // w.bk
    return w.block[b, h][np.ix_(qb, kb)] != 0


def _partial_tiles_exact(p, w, b, h, tiles):
    """Every PARTIAL record of the query tiles starting at ``tiles``: its
    computed pairs (sub-block bits; keys past L do not exist) equal the
    rectangle's kept pairs."""
    n = 0
    for r in p.coverage(b, h):
        if r["kind"] == bsa.TILE_FULL or r["q0"] // p.info()["tile_q"] * p.info()["tile_q"] not in tiles:
            continue
        nsk = 64 // r["sub_k"]
        qi = (np.arange(r["q0"], r["q1"]) - r["q0"]) // r["sub_q"]
        kj = (np.arange(r["k0"], r["k1"]) - r["k0"]) // r["sub_k"]
        got = ((r["sub_bits"] >> (qi[:, None] * nsk + kj[None, :])) & 1) == 1
        want = _tile_elements(w, b, h, r["q0"], r["q1"], r["k0"], r["k1"])
        assert np.array_equal(got, want), (h, r)
        n += 1
    return n


@pytest.mark.parametrize("i", [0, 4, 9, 13, 17, 22, 26, 28, 35, 39, 45])
def test_tessera_plan_cells_exact(i):
    """Tessera-style masks at full size (L = 75,600): on sampled heads every
    logical cell is computed exactly once if its block is kept and never
    otherwise; every PARTIAL tile of sampled query tiles (the last, ragged one
    included) is exact element by element. The block definition itself is
    checked against the oracle's expansion on sampled rows."""
    w = wl.tessera(i)
    p = plan_workload(w, device=-1)
    tq = p.info()["tile_q"]
    last = (w.L - 1) // tq * tq
    for h in ((0, 23) if w.bq == 32 else (0, 13, 23)):
        cnt, want = _cell_coverage(p, w, 0, h)
        assert np.array_equal(cnt, want), (i, h, int((cnt != want).sum()))
        _partial_tiles_exact(p, w, 0, h, {0, tq * 57, last})
        for q in (0, 4111, w.L - 1):
            keys = oracle.row_keys(w, 0, h, q)
            assert np.array_equal(np.flatnonzero(_tile_elements(w, 0, h, q, q + 1, 0, w.L)[0]), keys)


def test_highres_plan_cells_exact():
    """High-res at full size (L = 302,400, 128x128 blocks; spatial heads
    frame-major, temporal heads temporal-major): a spatial and a temporal head,
    every logical cell computed exactly once if kept and never otherwise; the
    ragged last query tile's PARTIAL tiles exact element by element; the block
    definition against the oracle's expansion on sampled rows (temporal-major
    positions mapped to tokens)."""
    w = wl.highres()
    p = plan_workload(w, device=-1)
    tq = p.info()["tile_q"]
    tok = tok_of_logical(w.T, w.Hg * w.Wg)
    for h in (0, 12):
        cnt, want = _cell_coverage(p, w, 0, h)
        assert np.array_equal(cnt, want), (h, int((cnt != want).sum()))
        _partial_tiles_exact(p, w, 0, h, {(w.L - 1) // tq * tq})
        for j in (0, 151234, w.L - 1):
            qtok = tok[j] if w.layout()[h] else j
            keys = oracle.row_keys(w, 0, h, qtok)
            lk = np.flatnonzero(_tile_elements(w, 0, h, j, j + 1, 0, w.L)[0])
            want_tok = np.sort(tok[lk]) if w.layout()[h] else lk
            assert np.array_equal(want_tok, keys), (h, j)
