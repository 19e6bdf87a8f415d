"""Device-side planning (bsa_plan_device) of BLOCK masks held in device memory.

The plan the kernels build is checked against the host planner's plan of the
same mask, which the plan-exactness tests pin to the brute-force mapping and
the parity tests to the fp64 oracle: the same statistics, the same tile
records of every head in the same launch slots (so the same task order), and
bit-identical forward outputs. Plans whose regime comes from the lookup table
(chosen without the mask density) are checked against the oracle directly."""
import time

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
from bsa_helpers import plan_workload, plan_workload_device  # noqa: E402
from gpu_util import compare, compare_f32, log, run_gpu, sample_rows, to_device  # noqa: E402

ORDERS = [bsa.ORDER_XCD_GROUPED, bsa.ORDER_LONGEST_FIRST]
INFO_KEYS = ("regime", "tile_q", "tile_k", "gather", "tasks", "workgroups", "tiles_full", "tiles_partial",
             "tiles_empty", "gather_rows", "executed_pairs", "task_order")


def _same_plan(w, ph, pd, heads=None):
    ih, idv = ph.info(), pd.info()
    for k in INFO_KEYS:
        assert ih[k] == idv[k], (k, ih[k], idv[k])
    heads = heads if heads is not None else [(b, h) for b in range(w.B) for h in range(w.H)]
    for b, h in heads:
        assert ph.coverage(b, h) == pd.coverage(b, h), (b, h)


def _ragged_cases():
    g = np.random.default_rng(23)
    out = []
    for (bq, bk) in [(64, 64), (32, 32), (128, 128), (64, 256), (256, 32), (32, 128)]:
        T, Hg, Wg = 3, 10, 11
        L = T * Hg * Wg  # 330: ragged for every tile and block size
        w = wl.Workload(f"blk{bq}x{bk}", 90, 2, 2, L, 64, T, Hg, Wg, wl.BLOCK, bq, bk)
        w.block = (g.random((2, 2, w.nqb, w.nkb)) < 0.4).astype(np.uint8)
        w.block[0, 1, 0, :] = 0      # a query block with no kept key
        w.block[1, 0] = 1            # a dense head
        w.block[1, 1] = w.block[1, 0]  # a head equal to the previous one
        w.head_layout = np.array([0, 1], np.uint8)
        out.append(w)
    return out


@pytest.mark.parametrize("w", _ragged_cases(), ids=lambda w: w.name)
@pytest.mark.parametrize("regime", [0, 1, 4])
def test_device_plan_equals_host_plan(w, regime):
    for bits in (False, True):
        for order in ORDERS:
            log(f"[case] {w.name} regime={regime} order={order} bits={bits}")
            ph = plan_workload(w, force_regime=regime, bits=bits, task_order=order)
            pd = plan_workload_device(w, force_regime=regime, bits=bits, task_order=order)
            _same_plan(w, ph, pd)


@pytest.mark.parametrize("w", _ragged_cases()[:3], ids=lambda w: w.name)
def test_device_plan_forward_matches_oracle(w):
    Q, K, V = wl.make_qkv(w)
    for regime in (-1, 0, 4):
        log(f"[case] {w.name} device plan regime={regime}")
        pd = plan_workload_device(w, force_regime=regime)
        O, _ = run_gpu(w, Q, K, V, plan=pd)
        compare(w, Q, K, V, O, label=f"{w.name} device plan r{regime}")
        if regime >= 0:
            Oh, _ = run_gpu(w, Q, K, V, plan=plan_workload(w, force_regime=regime))
            assert np.array_equal(O, Oh)


def test_device_plan_f32():
    w = _ragged_cases()[0]
    Q, K, V = wl.make_qkv(w, dtype="f32")
    log("[case] device plan f32")
    pd = plan_workload_device(w, dtype=bsa.DTYPE_F32)
    O, _ = run_gpu(w, Q, K, V, plan=pd)
    compare_f32(w, Q, K, V, O, label="device plan f32")


def test_device_plan_empty_mask():
    w = wl.tiny()
    w.block = np.zeros_like(w.block)
    Q, K, V = wl.make_qkv(w)
    pd = plan_workload_device(w)
    info = pd.info()
    assert info["tiles_full"] == 0 and info["tiles_partial"] == 0
    O, _ = run_gpu(w, Q, K, V, plan=pd)
    assert np.all(O == 0)


@pytest.mark.parametrize("i", [0, 1, 2, 3, 13, 22, 27, 40])
def test_tessera_masks_full_size(i):
    """Full-size Tessera requests (24 heads, 21 x 45x80 tokens): the device
    plan equals the host plan of the regime the host chose; the forward of a
    device plan with its own regime matches the oracle on sampled rows."""
    w = wl.tessera(i)
    log(f"[case] tessera {i} {w.bq}x{w.bk}")
    ph = plan_workload(w)
    reg = ph.info()["regime"]
    for order in ORDERS:
        ph_o = plan_workload(w, force_regime=reg, task_order=order)
        pd_o = plan_workload_device(w, force_regime=reg, task_order=order)
        _same_plan(w, ph_o, pd_o, heads=[(0, 0), (0, 11), (0, w.H - 1)])
    pd = plan_workload_device(w)
    Q, K, V = wl.make_qkv(w)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    od = torch.full_like(q, float("nan"))
    bsa.forward(pd, q, k, v, od)
    if pd.info()["regime"] == reg:
        oh = torch.full_like(q, float("nan"))
        bsa.forward(ph, q, k, v, oh)
        torch.cuda.synchronize()
        assert torch.equal(od, oh)
    torch.cuda.synchronize()
    O = od.float().cpu().numpy().astype(np.float64)
    compare(w, Q, K, V, O, rows=sample_rows(w, per_head=16, seed=i), label=f"tessera{i} device plan")


@pytest.mark.parametrize("i", [1, 5, 9, 25, 29])
def test_device_plan_regime_without_features(i, tmp_path):
    """A mask in device memory has no host-side features, so the device
    planner takes the first lookup-table rule that holds for every density
    and fill, never a feature-restricted bin: with the compiled-in table the
    128x64-tile regime for 64x64 masks of every density and layout, and with
    a table whose first matching rule is restricted, the full-range rule
    after it."""
    w = wl.tessera(i)
    pd = plan_workload_device(w)
    assert pd.info()["regime"] == 0, (i, pd.info()["regime"])
    lut = tmp_path / "lut.txt"
    lut.write_text("block 64 64 0 0.1 0 0.75 0 9999999999 1 xcd\n"
                   "block 64 64 0 1 0 1 0 9999999999 4 lpt\n")
    pd = plan_workload_device(w, lut_path=str(lut))
    info = pd.info()
    assert (info["regime"], info["task_order"]) == (4, bsa.ORDER_LONGEST_FIRST), info
    # the host planner, which has the features, takes the restricted rule
    # where they fall into it
    ph = plan_workload(w, lut_path=str(lut), device=-1)
    hi = ph.info()
    inside = hi["mask_density"] <= 0.1 and hi["mask_fill"] <= 0.75
    assert hi["regime"] == (1 if inside else 4), hi


def test_mask_made_on_device_and_planned_on_a_side_stream():
    """A mask produced by device work (a threshold of device-random scores),
    planned on a second stream while the forward is enqueued on the current
    one: the forward waits for the planning, and the result equals the forward
    of the host plan of the same mask."""
    w = wl.tessera(5)
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(1234)
    side = torch.cuda.Stream()
    scores = torch.rand((w.B, w.H, w.nqb, w.nkb), generator=gen, device="cuda:0")
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        mask = (scores < 0.2).to(torch.uint8)
        pd = plan_workload_device(w, stream=side, mask=mask, force_regime=0)
    Q, K, V = wl.make_qkv(w)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    od = torch.full_like(q, float("nan"))
    bsa.forward(pd, q, k, v, od)  # current stream; ordered after the planning
    torch.cuda.synchronize()
    w.block = mask.cpu().numpy()
    ph = plan_workload(w, force_regime=0)
    oh = torch.full_like(q, float("nan"))
    bsa.forward(ph, q, k, v, oh)
    torch.cuda.synchronize()
    assert torch.equal(od, oh)
    _same_plan(w, ph, pd, heads=[(0, 0), (0, 7), (0, w.H - 1)])


def test_device_planning_rejects_other_kinds():
    w = wl.tiny()
    m = torch.zeros(16, dtype=torch.uint8, device="cuda:0")
    with pytest.raises(bsa.BSAError) as e:
        bsa.plan_device(bsa.MASK_VIDEO, w.B, w.H, w.L, w.d, 1, 1, m)
    assert e.value.status == bsa.ERR_UNSUPPORTED


def test_device_planning_time():
    """Planning cost of the Tessera requests: host planner (mask in host
    memory) against device planning (mask in device memory), both to a plan
    ready for the forward. Logged; the device path must not be slower than
    the host one by more than the launch overheads."""
    rows = []
    for i in (0, 1, 2, 3, 13, 26, 40):
        w = wl.tessera(i)
        md = torch.from_numpy(np.ascontiguousarray(w.block)).to("cuda:0")
        reg = plan_workload(w).info()["regime"]
        for _ in range(2):
            plan_workload(w, force_regime=reg)
            plan_workload_device(w, force_regime=reg, mask=md)
        torch.cuda.synchronize()
        n = 10
        t0 = time.perf_counter()
        for _ in range(n):
            p = plan_workload(w, force_regime=reg)
        torch.cuda.synchronize()
        th = (time.perf_counter() - t0) / n
        t0 = time.perf_counter()
        for _ in range(n):
            p = plan_workload_device(w, force_regime=reg, mask=md)
        torch.cuda.synchronize()
        td = (time.perf_counter() - t0) / n
        del p
        rows.append((i, w.bq, w.bk, th * 1e3, td * 1e3))
        log(f"[plan time] tessera{i} {w.bq}x{w.bk} host {th * 1e3:.3f} ms device {td * 1e3:.3f} ms")
    assert all(r[4] < r[3] + 2.0 for r in rows)


# ---- SLICE masks (FG-Attn M x 1 slices) planned on the device

def _slice_case(M, cfg=61, B=2, H=2, T=3, Hg=10, Wg=11):
    L = T * Hg * Wg
    w = wl.Workload(f"slice_M{M}", cfg, B, H, L, 64, T, Hg, Wg, wl.SLICE, M, 1)
    w.row_ptr, w.col_idx = wl.slice_lists(cfg, B, H, L, M)
    return w


def _plan_slice_device(w, **kw):
    rp = torch.from_numpy(np.ascontiguousarray(w.row_ptr, dtype=np.int64)).to("cuda:0")
    ci = torch.from_numpy(np.ascontiguousarray(w.col_idx, dtype=np.int32)).to("cuda:0")
    return bsa.plan_device(bsa.MASK_SLICE_CSR, w.B, w.H, w.L, w.d, w.bq, 1, row_ptr=rp, col_idx=ci,
                           nnz=int(w.row_ptr[-1]), T=w.T, Hg=w.Hg, Wg=w.Wg, head_layout=w.head_layout, **kw)


def _same_slice_plan(w, ph, pd, heads):
    ih, idv = ph.info(), pd.info()
    for k in INFO_KEYS:
        assert ih[k] == idv[k], (k, ih[k], idv[k])
    for b, h in heads:
        ch, cd = ph.coverage(b, h), pd.coverage(b, h)
        assert len(ch) == len(cd)
        for x, y in zip(ch, cd):
            xk, yk = x.pop("keys"), y.pop("keys")
            assert x == y and np.array_equal(xk, yk)


@pytest.mark.parametrize("M", [64, 128])
def test_device_slice_plan_equals_host_plan(M):
    w = _slice_case(M)
    w.head_layout = np.array([0, 1], np.uint8)
    Q, K, V = wl.make_qkv(w)
    for order in ORDERS:
        log(f"[case] slice M={M} order={order}")
        ph = plan_workload(w, task_order=order)
        pd = _plan_slice_device(w, task_order=order)
        _same_slice_plan(w, ph, pd, [(b, h) for b in range(w.B) for h in range(w.H)])
        Od, _ = run_gpu(w, Q, K, V, plan=pd)
        Oh, _ = run_gpu(w, Q, K, V, plan=ph)
        assert np.array_equal(Od, Oh)
        compare(w, Q, K, V, Od, label=f"slice M{M} device plan order {order}")


def test_device_slice_plan_full_size_fgattn():
    """FG-Attn slices at full size (24 heads, 21 x 30x52 tokens, M = 64): the
    device plan equals the host plan and runs to the same bits; planning time
    logged."""
    w = wl.fgattn()
    ph = plan_workload(w)
    pd = _plan_slice_device(w)
    _same_slice_plan(w, ph, pd, [(0, 0), (0, 13), (0, w.H - 1)])
    g = torch.Generator(device="cuda:0")
    g.manual_seed(3)
    q, k, v = (torch.randn((w.B, w.H, w.L, w.d), generator=g, device="cuda:0").to(torch.bfloat16) for _ in range(3))
    oh, od = torch.empty_like(q), torch.empty_like(q)
    bsa.forward(ph, q, k, v, oh)
    bsa.forward(pd, q, k, v, od)
    torch.cuda.synchronize()
    assert torch.equal(oh, od)
    rp = torch.from_numpy(np.ascontiguousarray(w.row_ptr, dtype=np.int64)).to("cuda:0")
    ci = torch.from_numpy(np.ascontiguousarray(w.col_idx, dtype=np.int32)).to("cuda:0")
    nnz = int(w.row_ptr[-1])
    for _ in range(2):
        p = bsa.plan_device(bsa.MASK_SLICE_CSR, w.B, w.H, w.L, w.d, w.bq, 1, row_ptr=rp, col_idx=ci, nnz=nnz)
    torch.cuda.synchronize()
    n = 5
    t0 = time.perf_counter()
    for _ in range(n):
        p = bsa.plan_device(bsa.MASK_SLICE_CSR, w.B, w.H, w.L, w.d, w.bq, 1, row_ptr=rp, col_idx=ci, nnz=nnz)
    torch.cuda.synchronize()
    td = (time.perf_counter() - t0) / n
    t0 = time.perf_counter()
    for _ in range(n):
        p = plan_workload(w)
    torch.cuda.synchronize()
    th = (time.perf_counter() - t0) / n
    del p
    log(f"[plan time] fgattn M=64 ({nnz} slice keys): host {th * 1e3:.3f} ms device {td * 1e3:.3f} ms")


def test_device_slice_plan_with_invalid_entries_is_reported_and_safe():
    """Keys out of range are clamped, a decreasing pair is used as given, a
    list whose bounds leave [0, nnz] is dropped; the plan reports
    INVALID_MASK and its forward runs (every gathered row inside the head)."""
    w = _slice_case(64, cfg=62, B=1)
    rp = np.ascontiguousarray(w.row_ptr, dtype=np.int64).copy()
    ci = np.ascontiguousarray(w.col_idx, dtype=np.int32).copy()
    ci[3] = w.L + 50     # out of range
    ci[7] = -4           # out of range
    ci[12], ci[13] = ci[13], ci[12]  # not increasing
    rpd = torch.from_numpy(rp).to("cuda:0")
    rpd[5] = int(rp[-1]) + 1000  # list 4 ends and list 5 starts past nnz
    cid = torch.from_numpy(ci).to("cuda:0")
    p = bsa.plan_device(bsa.MASK_SLICE_CSR, w.B, w.H, w.L, w.d, 64, 1, row_ptr=rpd, col_idx=cid, nnz=int(rp[-1]))
    with pytest.raises(bsa.BSAError) as e:
        p.info()
    assert e.value.status == bsa.ERR_INVALID_MASK
    Q, K, V = wl.make_qkv(w)
    O, _ = run_gpu(w, Q, K, V, plan=p)
    assert np.all(np.isfinite(O))


def test_device_plan_edge_shapes():
    """A sequence shorter than one key tile, and bit rows with stray bits
    past the last key block (ignored by the device planner): the device plan
    equals the host plan of the clean mask."""
    # the device planner chooses its regime without the mask density, so the
    # host plan is made with the regime and order the device plan took
    def host_like(w, pd, bits):
        i = pd.info()
        return plan_workload(w, bits=bits, force_regime=i["regime"], task_order=i["task_order"])

    w = wl.Workload("short", 71, 1, 3, 40, 64, 0, 0, 0, wl.BLOCK, 32, 32)
    w.block = (np.random.default_rng(5).random((1, 3, w.nqb, w.nkb)) < 0.6).astype(np.uint8)
    for bits in (False, True):
        pd = plan_workload_device(w, bits=bits)
        _same_plan(w, host_like(w, pd, bits), pd)
    w = wl.Workload("stray", 72, 1, 2, 330, 64, 0, 0, 0, wl.BLOCK, 32, 32)
    w.block = (np.random.default_rng(6).random((1, 2, w.nqb, w.nkb)) < 0.3).astype(np.uint8)
    bits = w.block_bits().copy()
    bits[..., -1] |= np.uint64(1) << np.uint64(63)  # nkb = 11: bit 63 lies past the last block
    md = torch.from_numpy(bits.view(np.int64)).to("cuda:0")
    pd = plan_workload_device(w, bits=True, mask=md)
    _same_plan(w, host_like(w, pd, True), pd)
    Q, K, V = wl.make_qkv(w)
    O, _ = run_gpu(w, Q, K, V, plan=pd)
    compare(w, Q, K, V, O, label="stray bits")


def test_device_plan_regime_ignores_density(tmp_path):
    """With a table whose rules split one block shape by density, the host
    planner takes the rule of the mask's density; the device planner, which
    never reads the mask on the host (no density, no fill), takes no
    feature-restricted rule and, with no rule for every density and fill in
    this table, falls back to the 128x64-tile regime and the XCD-grouped
    order."""
    lut = tmp_path / "split.lut"
    lut.write_text("block 32 32 0 0.5 0 1 0 9999 1 lpt\n"
                   "block 32 32 0.5 1 0 1 0 9999 4 xcd\n")
    w = wl.Workload("split", 73, 1, 2, 330, 64, 0, 0, 0, wl.BLOCK, 32, 32)
    w.block = (np.random.default_rng(7).random((1, 2, w.nqb, w.nkb)) < 0.8).astype(np.uint8)
    ih = plan_workload(w, lut_path=str(lut)).info()
    idv = plan_workload_device(w, lut_path=str(lut)).info()
    assert (ih["regime"], ih["task_order"]) == (4, bsa.ORDER_XCD_GROUPED)
    assert (idv["regime"], idv["task_order"]) == (0, bsa.ORDER_XCD_GROUPED)
