"""The C-ABI library loads, exports every function include/bsa.h declares,
and reports argument/mask errors with the documented status codes (CPU only:
host-only plans, no GPU call)."""
import os
import re

import numpy as np
import pytest

import block_sparse_attention_fwd_amd as bsa
import workloads as wl
from bsa_helpers import plan_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "bsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(bsa_[a-z_]+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 10, names
    L = bsa.lib()
    for n in names:
        assert hasattr(L, n), f"{n} declared in bsa.h but not exported"
    assert sorted(bsa.EXPORTED) == names


def test_version_and_status_strings():
    L = bsa.lib()
    assert L.bsa_abi_version() == bsa.ABI_VERSION == 7
    assert L.bsa_status_str(bsa.ERR_INVALID_MASK) == b"BSA_ERR_INVALID_MASK"
    assert L.bsa_status_str(99) == b"BSA_ERR_UNKNOWN"
    assert len(bsa.regimes()) == L.bsa_regime_count() >= 3


def _block(H=2, L=256, b=64, dens=0.5):
    g = np.random.default_rng(0)
    n = -(-L // b)
    return (g.random((1, H, n, n)) < dens).astype(np.uint8)


def expect(status, fn, *a, match=None, **k):
    with pytest.raises(bsa.BSAError) as e:
        fn(*a, **k)
    assert e.value.status == status, str(e.value)
    if match:
        assert re.search(match, str(e.value)), str(e.value)


def test_argument_errors():
    m = _block()
    P = bsa.plan
    expect(bsa.ERR_INVALID_ARGUMENT, P, bsa.MASK_BLOCK_U8, 0, 2, 256, 64, 64, 64, data=m, device=-1)
    expect(bsa.ERR_INVALID_ARGUMENT, P, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=None, device=-1)
    expect(bsa.ERR_UNSUPPORTED, P, bsa.MASK_BLOCK_U8, 1, 2, 256, 96, 64, 64, data=m, device=-1, match="head dim")
    expect(bsa.ERR_UNSUPPORTED, P, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 48, 64, data=m, device=-1, match="block shape")
    expect(bsa.ERR_INVALID_ARGUMENT, P, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, T=3, Hg=3, Wg=3, device=-1,
           match="geometry")
    expect(bsa.ERR_INVALID_ARGUMENT, P, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m,
           head_layout=np.array([0, 1], np.uint8), device=-1, match="temporal-major")
    expect(bsa.ERR_INVALID_ARGUMENT, P, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, force_regime=17, device=-1)
    expect(bsa.ERR_UNSUPPORTED, P, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, force_regime=2, device=-1,
           match="cannot run")
    expect(bsa.ERR_INVALID_ARGUMENT, P, 9, 1, 2, 256, 64, 64, 64, data=m, device=-1)


def test_mask_errors():
    L = 256
    P = bsa.plan
    rp = np.array([0, 3, 5, 5, 7, 9, 9, 9, 9], np.int64)
    good = np.array([1, 5, 9, 0, 200, 3, 4, 7, 8], np.int32)
    P(bsa.MASK_SLICE_CSR, 1, 2, L, 64, 64, 1, row_ptr=rp, col_idx=good, device=-1)
    dup = good.copy(); dup[1] = 1
    expect(bsa.ERR_INVALID_MASK, P, bsa.MASK_SLICE_CSR, 1, 2, L, 64, 64, 1, row_ptr=rp, col_idx=dup, device=-1)
    unsorted = good.copy(); unsorted[3], unsorted[4] = 200, 0
    expect(bsa.ERR_INVALID_MASK, P, bsa.MASK_SLICE_CSR, 1, 2, L, 64, 64, 1, row_ptr=rp, col_idx=unsorted, device=-1)
    oob = good.copy(); oob[2] = L
    expect(bsa.ERR_INVALID_MASK, P, bsa.MASK_SLICE_CSR, 1, 2, L, 64, 64, 1, row_ptr=rp, col_idx=oob, device=-1)
    neg = good.copy(); neg[0] = -1
    expect(bsa.ERR_INVALID_MASK, P, bsa.MASK_SLICE_CSR, 1, 2, L, 64, 64, 1, row_ptr=rp, col_idx=neg, device=-1)
    badrp = rp.copy(); badrp[2] = 2
    expect(bsa.ERR_INVALID_MASK, P, bsa.MASK_SLICE_CSR, 1, 2, L, 64, 64, 1, row_ptr=badrp, col_idx=good, device=-1)
    expect(bsa.ERR_INVALID_ARGUMENT, P, bsa.MASK_SLICE_CSR, 1, 2, L, 64, 64, 2, row_ptr=rp, col_idx=good, device=-1)
    # bit rows with bits beyond the last key block
    w = wl.Workload("b", 0, 1, 1, 200, 64, bq=64, bk=64)
    w.block = np.ones((1, 1, 4, 4), np.uint8)
    bits = w.block_bits()
    P(bsa.MASK_BLOCK_BITS, 1, 1, 200, 64, 64, 64, data=bits, device=-1)
    bits[0, 0, 1, 0] |= np.uint64(1 << 7)
    expect(bsa.ERR_INVALID_MASK, P, bsa.MASK_BLOCK_BITS, 1, 1, 200, 64, 64, 64, data=bits, device=-1)
    # video: pattern / anchor / radius / geometry
    hp = np.array([1, 2], np.uint8)
    P(bsa.MASK_VIDEO, 1, 2, 240, 64, 1, 1, head_pattern=hp, T=4, Hg=6, Wg=10, device=-1)
    expect(bsa.ERR_INVALID_MASK, P, bsa.MASK_VIDEO, 1, 2, 240, 64, 1, 1, head_pattern=np.array([1, 3], np.uint8),
           T=4, Hg=6, Wg=10, device=-1)
    expect(bsa.ERR_INVALID_MASK, P, bsa.MASK_VIDEO, 1, 2, 240, 64, 1, 1, head_pattern=hp, anchor_frame=4, T=4, Hg=6,
           Wg=10, device=-1)
    expect(bsa.ERR_INVALID_ARGUMENT, P, bsa.MASK_VIDEO, 1, 2, 240, 64, 1, 1, head_pattern=hp, device=-1)


def test_forward_rejects_host_only_plan_and_null_pointers():
    p = bsa.plan(bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=_block(), device=-1)
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.forward, p, 16, 16, 16, 16, stream=0, match="host-only")
    L = bsa.lib()
    assert L.bsa_forward(None, None, None, None, None, None) == bsa.ERR_INVALID_ARGUMENT
    # the stamped forward: stamps must be an aligned pointer; then bsa_forward's checks
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.forward_stamped, p, 16, 16, 16, 16, 0, stream=0, match="stamps")
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.forward_stamped, p, 16, 16, 16, 16, 12, stream=0, match="stamps")
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.forward_stamped, p, 16, 16, 16, 16, 16, stream=0, match="host-only")
    L.bsa_plan_destroy(None)  # NULL-safe


def test_device_planning_argument_errors():
    """bsa_plan_device rejects what it cannot plan before touching the device
    (the mask address is never read here)."""
    PD = bsa.plan_device
    expect(bsa.ERR_UNSUPPORTED, PD, bsa.MASK_VIDEO, 1, 2, 256, 64, 1, 1, 16, stream=0, match="BLOCK")
    expect(bsa.ERR_INVALID_ARGUMENT, PD, bsa.MASK_SLICE_CSR, 1, 2, 256, 64, 64, 1, stream=0, match="NULL")
    expect(bsa.ERR_INVALID_ARGUMENT, PD, bsa.MASK_SLICE_CSR, 1, 2, 256, 64, 64, 1, row_ptr=16, col_idx=16, nnz=-1,
           stream=0, match="nnz")
    expect(bsa.ERR_UNSUPPORTED, PD, bsa.MASK_SLICE_CSR, 1, 2, 256, 64, 32, 1, row_ptr=16, col_idx=16, nnz=4,
           stream=0, match="slice block")
    expect(bsa.ERR_INVALID_ARGUMENT, PD, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, 16, stream=0, device=-1,
           match="device")
    expect(bsa.ERR_INVALID_ARGUMENT, PD, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, 0, stream=0, match="NULL")
    expect(bsa.ERR_UNSUPPORTED, PD, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 48, 64, 16, stream=0, match="block shape")
    L = bsa.lib()
    assert L.bsa_plan_device(None, 1, 1, 64, 64, 64, 64, None, None, None) == bsa.ERR_INVALID_ARGUMENT


def test_request_argument_errors():
    """bsa_request_create rejects bad descriptions before touching the device."""
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.Request, 1, 2, 256, 64, depth=0, stream=0, match="depth")
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.Request, 1, 2, 256, 64, device=-1, stream=0, match="device")
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.Request, 1, 2, 256, 96, stream=0, match="shape")
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.Request, 0, 2, 256, 64, stream=0, match="shape")
    L = bsa.lib()
    assert L.bsa_request_create(None, None) == bsa.ERR_INVALID_ARGUMENT
    assert L.bsa_request_submit(None, None, 64, 64, 0, None, None, None, None) == bsa.ERR_INVALID_ARGUMENT
    assert L.bsa_request_finish(None) == bsa.ERR_INVALID_ARGUMENT
    L.bsa_request_destroy(None)  # NULL-safe


def test_route_argument_errors():
    """bsa_route_heads validates shapes, geometry and sampled rows before it
    touches the device (the tensor addresses are never read here)."""
    R = bsa.route_heads
    rows = np.array([0, 5, 17], np.int32)
    ok = dict(B=1, H=2, L=330, d=64, T=3, Hg=10, Wg=11)

    def call(rows=rows, **kw):
        a = dict(ok)
        a.update(kw)
        return R(16, 16, 16, a["B"], a["H"], a["L"], a["d"], a["T"], a["Hg"], a["Wg"], rows, stream=0,
                 **{k: v for k, v in kw.items() if k in ("anchor_frame", "radius", "device")})

    expect(bsa.ERR_INVALID_ARGUMENT, call, d=96, match="shape")
    expect(bsa.ERR_INVALID_ARGUMENT, call, T=4, match="geometry")
    expect(bsa.ERR_INVALID_ARGUMENT, call, anchor_frame=3, match="anchor")
    expect(bsa.ERR_INVALID_ARGUMENT, call, radius=257, match="radius")
    expect(bsa.ERR_INVALID_ARGUMENT, call, rows=np.array([330], np.int32), match="out of range")
    expect(bsa.ERR_INVALID_ARGUMENT, call, rows=np.zeros(0, np.int32), match="n_rows")
    expect(bsa.ERR_INVALID_ARGUMENT, call, device=-1, match="device")
    L = bsa.lib()
    assert L.bsa_route_heads(None, None, None, 1, 1, 64, 64, None, None, None, None) == bsa.ERR_INVALID_ARGUMENT


def test_simulated_allocation_failure(monkeypatch):
    monkeypatch.setenv("BSA_TEST_FAIL_ALLOC", "1")
    expect(bsa.ERR_OUT_OF_MEMORY, bsa.plan, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=_block(), device=-1)


def test_lookup_table_file(tmp_path):
    m = _block()
    f = tmp_path / "lut.txt"
    f.write_text("# test\nblock * * 0 1 0 1 0 99999 0\n")
    p = bsa.plan(bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f), device=-1)
    assert p.info()["regime"] == 0
    f.write_text("block 64 64 0 1 0 1 0 99999 1\n")
    assert bsa.plan(bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f), device=-1).info()["regime"] == 1
    f.write_text("block 64 64 0 1\n")
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.plan, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f),
           device=-1, match="malformed")
    # the fill range: a rule whose fill range excludes the mask's fill is skipped
    f.write_text("block 64 64 0 1 0 0.5 0 99999 1\nblock 64 64 0 1 0.5 1 0 99999 4\n")
    info = bsa.plan(bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f), device=-1).info()
    assert info["regime"] == (1 if info["mask_fill"] < 0.5 else 4)
    # a line with a fill2 range (fill over 256-row tiles) between fill and length
    f.write_text("block 64 64 0 1 0 1 0 0.5 0 99999 1\nblock 64 64 0 1 0 1 0.5 1 0 99999 4\n")
    info = bsa.plan(bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f), device=-1).info()
    assert 0 <= info["mask_fill2"] <= 1
    assert info["regime"] == (1 if info["mask_fill2"] < 0.5 else 4)
    f.write_text("block 64 64 0 1 0 1 0 1 0 99999\n")
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.plan, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f),
           device=-1, match="malformed")
    for bad in ("block 64 64 0 1 0.5x 1 0 99999 1", "block 64x 64 0 1 0 1 0 99999 1", "block 64 64 0 1 0 1 0 99999 1.5",
                "block 64 64 0 1 0 1 0 99999 7"):
        f.write_text(bad + "\n")
        expect(bsa.ERR_INVALID_ARGUMENT, bsa.plan, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f),
               device=-1, match="malformed|out of range")
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.plan, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m,
           lut_path=str(tmp_path / "nope"), device=-1)
    # the optional order column; an explicit task_order option overrides it
    f.write_text("block 64 64 0 1 0 1 0 99999 1 lpt\n")
    info = bsa.plan(bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f), device=-1).info()
    assert (info["regime"], info["task_order"]) == (1, bsa.ORDER_LONGEST_FIRST)
    info = bsa.plan(bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f), device=-1,
                    task_order=bsa.ORDER_XCD_GROUPED).info()
    assert (info["regime"], info["task_order"]) == (1, bsa.ORDER_XCD_GROUPED)
    f.write_text("block 64 64 0 1 0 1 0 99999 1 xcd\n")
    assert bsa.plan(bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f), device=-1).info()["task_order"] == 0
    f.write_text("block 64 64 0 1 0 1 0 99999 1 fifo\n")
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.plan, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, lut_path=str(f),
           device=-1, match="unknown order")
    expect(bsa.ERR_INVALID_ARGUMENT, bsa.plan, bsa.MASK_BLOCK_U8, 1, 2, 256, 64, 64, 64, data=m, device=-1,
           task_order=2, match="task_order")


def _task_slots(p, w):
    """{(head, q0 of the task): launch slot} from the coverage walk, and the
    task's tile count."""
    slot, ntiles = {}, {}
    tq = p.info()["tile_q"]
    for h in range(w.H):
        for r in p.coverage(0, h):
            key = (h, r["q0"] - r["q0"] % tq)
            assert slot.setdefault(key, r["task"]) == r["task"]
            ntiles.setdefault(key, set()).add(r["k0"])
    return slot, {k: len(v) for k, v in ntiles.items()}


@pytest.mark.parametrize("order", [0, 1])
def test_task_orders(order):
    """Workgroup i runs task i. Both orders put the tasks longest first (a
    task's cost class never rises along the launch); the XCD grouping puts,
    within a run of one cost class, query tiles of one head in slots 8 apart
    (one XCD), in query-tile order."""
    w = wl.svg("B")
    p = plan_workload(w, device=-1, task_order=order)
    info = p.info()
    assert info["task_order"] == order
    slot, ntiles = _task_slots(p, w)
    n = info["tasks"]
    assert len(set(slot.values())) == len(slot) == n == w.H * -(-w.L // info["tile_q"])
    assert sorted(slot.values()) == list(range(n))
    pos = {s: k for k, s in slot.items()}
    counts = [ntiles[pos[s]] for s in range(n)]
    if order == 1:
        assert counts == sorted(counts, reverse=True)
        return
    cls = [int(np.log(c) / np.log(1.3)) for c in counts]
    assert cls == sorted(cls, reverse=True)
    pairs = same = 0
    for s in range(n - 8):
        if cls[s] == cls[s + 8]:
            pairs += 1
            (h, q0), (h2, q2) = pos[s], pos[s + 8]
            same += h2 == h and q2 > q0
    assert pairs > 0.9 * n and same > 0.95 * pairs, (pairs, same, n)


def test_block_shape_range_ends():
    """The documented ranges, at both ends: BLOCK sides are powers of two in
    [32, 1024]; SLICE takes M = 64 or 128 (host-only plans)."""
    P = bsa.plan
    L = 2048
    for bq, bk in ((32, 32), (1024, 1024), (32, 1024), (1024, 32)):
        m = np.ones((1, 1, -(-L // bq), -(-L // bk)), np.uint8)
        p = P(bsa.MASK_BLOCK_U8, 1, 1, L, 64, bq, bk, data=m, device=-1)
        assert p.info()["executed_pairs"] == L * L
        p.close()
    for bq, bk in ((16, 64), (64, 16), (2048, 64), (64, 2048)):
        m = np.ones((1, 1, -(-L // bq), -(-L // bk)), np.uint8)
        expect(bsa.ERR_UNSUPPORTED, P, bsa.MASK_BLOCK_U8, 1, 1, L, 64, bq, bk, data=m, device=-1, match="block shape")
    for M in (64, 128):
        nq = -(-L // M)
        rp = np.arange(nq + 1, dtype=np.int64)
        ci = np.zeros(nq, np.int32)
        P(bsa.MASK_SLICE_CSR, 1, 1, L, 64, M, 1, row_ptr=rp, col_idx=ci, device=-1).close()
    nq = -(-L // 32)
    expect(bsa.ERR_UNSUPPORTED, P, bsa.MASK_SLICE_CSR, 1, 1, L, 64, 32, 1, row_ptr=np.arange(nq + 1, dtype=np.int64),
           col_idx=np.zeros(nq, np.int32), device=-1, match="slice block")
