"""Pins of the oracle's head routing (``oracle.route_heads``) against what the
reading fixes: heads built to attend within frames route spatial and heads
built to attend along pixel tracks route temporal; a pattern that keeps every
key has error exactly 0; the error is invariant under a shift of V and scales
with the square of a scale of V; the batch and the sampled rows enter as plain
means."""
import numpy as np
import pytest

import oracle
import workloads as wl


def _w(B=1, H=4, T=3, Hg=6, Wg=7, d=64, cfg=5):
    return wl.Workload("route", cfg, B, H, T * Hg * Wg, d, T, Hg, Wg, wl.VIDEO, 1, 1)


KINDS = [wl.SPATIAL, wl.TEMPORAL, wl.SPATIAL, wl.TEMPORAL]


@pytest.mark.parametrize("cfg", [5, 6, 7])
def test_constructed_heads_route_as_built(cfg):
    w = _w(cfg=cfg)
    Q, K, V = wl.routed_qkv(w, KINDS, alpha=8.0, dtype="f32")
    rows = wl.sample_tokens(w.L, 40, cfg)
    pat, err = oracle.route_heads(Q, K, V, w.T, w.Hg, w.Wg, rows, anchor=0, radius=1)
    assert pat.tolist() == KINDS
    # and by a wide margin
    for h, k in enumerate(KINDS):
        good, bad = (err[h, 0], err[h, 1]) if k == wl.SPATIAL else (err[h, 1], err[h, 0])
        assert good < 0.05 * bad


def test_pattern_keeping_every_key_has_zero_error():
    # one frame: the spatial pattern keeps every key
    w = _w(T=1, Hg=8, Wg=9)
    Q, K, V = wl.routed_qkv(w, KINDS, alpha=4.0, dtype="f32")
    rows = wl.sample_tokens(w.L, 30, 1)
    pat, err = oracle.route_heads(Q, K, V, w.T, w.Hg, w.Wg, rows, anchor=0, radius=1)
    assert np.all(err[:, 0] == 0.0) and np.all(err[:, 1] > 0)
    assert np.all(pat == wl.SPATIAL)
    # a radius covering the frame: the temporal pattern keeps every key
    w = _w(T=3, Hg=4, Wg=5)
    Q, K, V = wl.routed_qkv(w, KINDS, alpha=4.0, dtype="f32")
    rows = wl.sample_tokens(w.L, 30, 2)
    pat, err = oracle.route_heads(Q, K, V, w.T, w.Hg, w.Wg, rows, anchor=0, radius=5)
    assert np.all(err[:, 1] == 0.0) and np.all(err[:, 0] > 0)
    assert np.all(pat == wl.TEMPORAL)


def test_tie_goes_to_spatial():
    # one frame and a radius covering it: both patterns keep every key
    w = _w(T=1, Hg=4, Wg=5)
    Q, K, V = wl.routed_qkv(w, KINDS, alpha=4.0, dtype="f32")
    pat, err = oracle.route_heads(Q, K, V, w.T, w.Hg, w.Wg, np.arange(w.L), anchor=0, radius=5)
    assert np.all(err == 0.0) and np.all(pat == wl.SPATIAL)


def test_value_shift_and_scale():
    w = _w()
    Q, K, V = wl.routed_qkv(w, KINDS, alpha=3.0, dtype="f32")
    Q, K, V = (x.astype(np.float64) for x in (Q, K, V))
    rows = wl.sample_tokens(w.L, 25, 3)
    _, err = oracle.route_heads(Q, K, V, w.T, w.Hg, w.Wg, rows, anchor=1, radius=1)
    shift = np.random.default_rng(0).standard_normal((1, w.H, 1, w.d)) * 5.0
    _, err_shift = oracle.route_heads(Q, K, V + shift, w.T, w.Hg, w.Wg, rows, anchor=1, radius=1)
    np.testing.assert_allclose(err_shift, err, rtol=1e-9, atol=1e-15)
    _, err_scale = oracle.route_heads(Q, K, 3.0 * V, w.T, w.Hg, w.Wg, rows, anchor=1, radius=1)
    np.testing.assert_allclose(err_scale, 9.0 * err, rtol=1e-9, atol=1e-15)


def test_batch_and_rows_enter_as_means():
    w2 = _w(B=2)
    Q, K, V = wl.routed_qkv(w2, KINDS, alpha=3.0, dtype="f32")
    rows = wl.sample_tokens(w2.L, 40, 4)
    _, err = oracle.route_heads(Q, K, V, w2.T, w2.Hg, w2.Wg, rows, anchor=0, radius=1)
    per_b = [oracle.route_heads(Q[b:b + 1], K[b:b + 1], V[b:b + 1], w2.T, w2.Hg, w2.Wg, rows, anchor=0, radius=1)[1]
             for b in range(2)]
    np.testing.assert_allclose(err, (per_b[0] + per_b[1]) / 2, rtol=1e-12)
    half = [oracle.route_heads(Q, K, V, w2.T, w2.Hg, w2.Wg, r, anchor=0, radius=1)[1] for r in (rows[:20], rows[20:])]
    np.testing.assert_allclose(err, (half[0] + half[1]) / 2, rtol=1e-12)
