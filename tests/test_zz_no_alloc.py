"""The allocation-free routing entry point (bsa_route_heads_noalloc) through
the C ABI against bsa_route_heads on the same inputs: two calls in a row, the
second with a smaller input, each matching the allocating call's patterns
where the errors are clearly apart and its errors within the routing parity
tolerance (4e-3 * sqrt(err) + 4e-6). Also its limit checks."""
import numpy as np
import pytest

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


def _both(w, kinds, n_rows, seed, anchor=0, radius=2):
    Q, K, V = wl.routed_qkv(w, kinds, alpha=10.0)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    rows = wl.sample_tokens(w.L, n_rows, seed)
    args = (q, k, v, w.B, w.H, w.L, w.d, w.T, w.Hg, w.Wg, rows)
    pat_a, err_a = bsa.route_heads(*args, anchor_frame=anchor, radius=radius)
    pat_n, err_n = bsa.route_heads_noalloc(*args, anchor_frame=anchor, radius=radius)
    dev = np.abs(err_n - err_a)
    log(f"[no-alloc] {w.name} H={w.H} L={w.L} d={w.d} rows={n_rows}: max |err - err_alloc| / tol = "
        f"{float((dev / _tol(err_a)).max()):.3e}")
    assert np.all(dev <= _tol(err_a)), (err_n, err_a)
    clear = np.abs(err_a[:, 0] - err_a[:, 1]) > 2 * _tol(err_a.max(axis=1))
    assert np.array_equal(pat_n[clear], pat_a[clear]), (pat_n, pat_a)
    assert set(pat_n.tolist()) <= {wl.SPATIAL, wl.TEMPORAL}
    return pat_n


def test_noalloc_matches_allocating_call_twice():
    """Two calls in a row on the SVG shape (24 heads, 13 x 30x52 tokens,
    d = 128, 64 sampled rows), then a smaller one (4 heads, 330 tokens,
    d = 64, 50 rows): the second call runs on the array the first left
    behind."""
    w = wl.svg("A")
    kinds = [wl.SPATIAL] * 12 + [wl.TEMPORAL] * 12
    pat = _both(w, kinds, 64, 2024)
    assert pat.tolist() == kinds
    ws = wl.Workload("route_small", 41, 2, 4, 330, 64, 3, 10, 11, wl.VIDEO, 1, 1)
    pat = _both(ws, [wl.SPATIAL, wl.TEMPORAL, wl.DENSE, wl.TEMPORAL], 50, 50, anchor=1)
    assert pat[0] == wl.SPATIAL and pat[1] == wl.TEMPORAL and pat[3] == wl.TEMPORAL


def test_noalloc_limits():
    """Inputs beyond the fixed scratch are refused with UNSUPPORTED, before any
    device work; argument errors as for the allocating call."""
    w = wl.Workload("route", 9, 1, 2, 330, 64, 3, 10, 11, wl.VIDEO, 1, 1)
    Q, K, V = wl.routed_qkv(w, [wl.SPATIAL, wl.TEMPORAL], alpha=4.0)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    with pytest.raises(bsa.BSAError) as e:  # 1025 heads
        bsa.route_heads_noalloc(q, k, v, 1, 1025, w.L, w.d, w.T, w.Hg, w.Wg, [0])
    assert e.value.status == bsa.ERR_UNSUPPORTED
    big = wl.svg("A")
    Qb, Kb, Vb = (to_device(x) for x in wl.routed_qkv(big, [wl.SPATIAL] * 24, alpha=4.0))
    with pytest.raises(bsa.BSAError) as e:  # 4096 rows x 24 heads at d = 128: more than the scratch
        bsa.route_heads_noalloc(Qb, Kb, Vb, big.B, big.H, big.L, big.d, big.T, big.Hg, big.Wg,
                                np.arange(4096, dtype=np.int32))
    assert e.value.status == bsa.ERR_UNSUPPORTED and "scratch" in str(e.value)
    with pytest.raises(bsa.BSAError) as e:
        bsa.route_heads_noalloc(q, k, v, w.B, w.H, w.L, w.d, w.T, w.Hg, w.Wg, [w.L])
    assert e.value.status == bsa.ERR_INVALID_ARGUMENT
