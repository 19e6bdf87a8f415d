"""GPU parity of the head routing probe (bsa_route_heads) against the fp64
oracle's routing on the same seeded bf16 inputs.

Errors: the probe's outputs carry the bf16 path's rounding (P rounded to bf16,
fp32 sums), mean-abs about 1e-3 per output element against the oracle; the
squared difference of two outputs then moves by at most about
2 * sqrt(err) * eps + eps^2 with eps = 2e-3, so each error is compared within
4e-3 * sqrt(err) + 4e-6. The routing decision (an integer decided by floating
point) must agree wherever the two errors differ by more than twice that;
within it either pattern is accepted."""
import time

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_fwd_amd as bsa
    bsa.lib()


import block_sparse_attention_fwd_amd as bsa  # noqa: E402
from gpu_util import log, to_device  # noqa: E402


def _tol(err):
    return 4e-3 * np.sqrt(err) + 4e-6


def _check(w, Q, K, V, rows, anchor, radius, label):
    q, k, v = to_device(Q), to_device(K), to_device(V)
    pat, err = bsa.route_heads(q, k, v, w.B, w.H, w.L, w.d, w.T, w.Hg, w.Wg, rows, anchor_frame=anchor,
                               radius=radius)
    pat_o, err_o = oracle.route_heads(Q, K, V, w.T, w.Hg, w.Wg, rows, anchor=anchor, radius=radius)
    dev = np.abs(err - err_o)
    log(f"[route] {label}: max |err - oracle| / tol = {float((dev / _tol(err_o)).max()):.3f}")
    assert np.all(dev <= _tol(err_o)), (err, err_o)
    clear = np.abs(err_o[:, 0] - err_o[:, 1]) > 2 * _tol(err_o.max(axis=1))
    assert np.array_equal(pat[clear], pat_o[clear]), (pat, pat_o, err_o)
    assert set(pat.tolist()) <= {wl.SPATIAL, wl.TEMPORAL}
    return pat, err


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_rows", [1, 50, 330])
def test_route_small(d, n_rows):
    w = wl.Workload("route", 40 + d, 2, 4, 330, d, 3, 10, 11, wl.VIDEO, 1, 1)
    kinds = [wl.SPATIAL, wl.TEMPORAL, wl.DENSE, wl.TEMPORAL]
    Q, K, V = wl.routed_qkv(w, kinds, alpha=10.0)
    rows = wl.sample_tokens(w.L, n_rows, n_rows)
    log(f"[case] route small d={d} rows={n_rows}")
    pat, _ = _check(w, Q, K, V, rows, anchor=1, radius=2, label=f"small d{d} S{n_rows}")
    if n_rows > 1:
        assert pat[0] == wl.SPATIAL and pat[1] == wl.TEMPORAL and pat[3] == wl.TEMPORAL


@pytest.mark.parametrize("radius,anchor", [(0, 0), (1, 2), (12, 0)])
def test_route_radius_and_anchor(radius, anchor):
    w = wl.Workload("route", 9, 1, 3, 330, 64, 3, 10, 11, wl.VIDEO, 1, 1)
    Q, K, V = wl.routed_qkv(w, [wl.DENSE, wl.SPATIAL, wl.TEMPORAL], alpha=4.0)
    rows = wl.sample_tokens(w.L, 70, 5)
    log(f"[case] route radius={radius} anchor={anchor}")
    _check(w, Q, K, V, rows, anchor=anchor, radius=radius, label=f"r{radius} a{anchor}")


def test_route_full_size_svg():
    """SVG shape (24 heads, 13 x 30x52 tokens, d=128): 12 heads built to
    attend within frames, 12 along pixel tracks; 64 sampled query tokens.
    The probe routes them as built and matches the oracle's errors."""
    w = wl.svg("A")
    kinds = [wl.SPATIAL] * 12 + [wl.TEMPORAL] * 12
    Q, K, V = wl.routed_qkv(w, kinds, alpha=12.0)
    rows = wl.sample_tokens(w.L, 64, 2024)
    log("[case] route svg full size")
    pat, _ = _check(w, Q, K, V, rows, anchor=0, radius=2, label="svg")
    assert pat.tolist() == kinds
    q, k, v = to_device(Q), to_device(K), to_device(V)
    for _ in range(3):
        bsa.route_heads(q, k, v, w.B, w.H, w.L, w.d, w.T, w.Hg, w.Wg, rows)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 10
    for _ in range(n):
        bsa.route_heads(q, k, v, w.B, w.H, w.L, w.d, w.T, w.Hg, w.Wg, rows)
    log(f"[route] svg, 64 sampled rows: {(time.perf_counter() - t0) / n * 1e3:.3f} ms per call (synchronous)")


def test_route_argument_errors():
    w = wl.Workload("route", 9, 1, 2, 330, 64, 3, 10, 11, wl.VIDEO, 1, 1)
    Q, K, V = wl.routed_qkv(w, [wl.SPATIAL, wl.TEMPORAL], alpha=4.0)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    for kw, rows in [(dict(T=4), [0]), (dict(radius=300), [0]), (dict(anchor_frame=3), [0]), ({}, [330]), ({}, [])]:
        args = dict(T=w.T, Hg=w.Hg, Wg=w.Wg)
        args.update({x: y for x, y in kw.items() if x in ("T", "Hg", "Wg")})
        extra = {x: y for x, y in kw.items() if x not in ("T", "Hg", "Wg")}
        with pytest.raises(bsa.BSAError) as e:
            bsa.route_heads(q, k, v, w.B, w.H, w.L, w.d, args["T"], args["Hg"], args["Wg"], np.array(rows, np.int32),
                            **extra)
        assert e.value.status == bsa.ERR_INVALID_ARGUMENT
    # a device index past the last device is refused before anything runs,
    # by both entry points
    for fn in (bsa.route_heads, bsa.route_heads_noalloc):
        with pytest.raises(bsa.BSAError) as e:
            fn(q, k, v, w.B, w.H, w.L, w.d, w.T, w.Hg, w.Wg, np.array([0, 5], np.int32),
               device=torch.cuda.device_count())
        assert e.value.status == bsa.ERR_INVALID_ARGUMENT
