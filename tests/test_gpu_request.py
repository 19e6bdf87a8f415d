"""Requests (bsa_request_*): a sequence of masks of one shape, each planned
while the forwards before it run. Every forward of a request writes the same
bits as a standalone plan + forward of its mask, and matches the fp64 oracle
within the bf16 bar, for host masks and for device-resident BLOCK masks, at
ring depths 1 and 3. The Tessera request (48 masks) is timed serialized against
pipelined."""
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
from bsa_helpers import plan_workload  # noqa: E402
from gpu_util import compare, log, to_device  # noqa: E402

T, HG, WG = 3, 10, 11
L_SMALL = T * HG * WG  # 330: ragged for every tile and block size


def _small_masks(n=8, seed=31):
    """n BLOCK masks of one shape (B=1, H=2, L=330) with varying block sizes
    and densities, and one video mask descriptor."""
    g = np.random.default_rng(seed)
    shapes = [(64, 64), (32, 32), (128, 128), (64, 256), (256, 32), (32, 128)]
    out = []
    for i in range(n):
        bq, bk = shapes[i % len(shapes)]
        w = wl.Workload(f"req{i}", 200 + i, 1, 2, L_SMALL, 64, T, HG, WG, wl.BLOCK, bq, bk)
        w.block = (g.random((1, 2, w.nqb, w.nkb)) < (0.15 + 0.1 * (i % 4))).astype(np.uint8)
        w.head_layout = np.array([0, 1], np.uint8)
        out.append(w)
    return out


def _standalone(w, q, k, v):
    p = plan_workload(w)
    o = torch.full_like(q, float("nan"))
    bsa.forward(p, q, k, v, o)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("depth", [1, 3])
@pytest.mark.parametrize("on_device", [False, True])
def test_request_outputs_equal_standalone(depth, on_device):
    masks = _small_masks()
    w0 = masks[0]
    Q, K, V = wl.make_qkv(w0)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    log(f"[case] request depth={depth} on_device={on_device}")
    req = bsa.Request(w0.B, w0.H, w0.L, w0.d, depth=depth, T=T, Hg=HG, Wg=WG, head_layout=w0.head_layout)
    outs = []
    for w in masks:
        o = torch.full_like(q, float("nan"))
        if on_device:
            md = torch.from_numpy(np.ascontiguousarray(w.block)).to("cuda:0")
            req.submit(bsa.MASK_BLOCK_U8, w.bq, w.bk, q, k, v, o, data=md, on_device=True)
        else:
            req.submit(bsa.MASK_BLOCK_U8, w.bq, w.bk, q, k, v, o, data=w.block)
        outs.append(o)
    # a video mask on the same request (host descriptor)
    hp = np.array([wl.SPATIAL, wl.TEMPORAL], np.uint8)
    ov = torch.full_like(q, float("nan"))
    req.submit(bsa.MASK_VIDEO, 1, 1, q, k, v, ov, head_pattern=hp, anchor_frame=1, radius=2)
    req.finish()
    st = req.stats()
    assert st["submitted"] == len(masks) + 1
    req.close()
    for w, o in zip(masks, outs):
        if on_device:
            md = torch.from_numpy(np.ascontiguousarray(w.block)).to("cuda:0")
            p = bsa.plan_device(bsa.MASK_BLOCK_U8, w.B, w.H, w.L, w.d, w.bq, w.bk, md, T=T, Hg=HG, Wg=WG,
                                head_layout=w.head_layout)
            ref = torch.full_like(q, float("nan"))
            bsa.forward(p, q, k, v, ref)
            torch.cuda.synchronize()
        else:
            ref = _standalone(w, q, k, v)
        assert torch.equal(o, ref), w.name
        # and each request output against the fp64 oracle directly
        compare(w, Q, K, V, o.float().cpu().numpy().astype(np.float64),
                label=f"request depth {depth} device {on_device} {w.name}")
    wv = wl.Workload("reqv", 0, 1, 2, L_SMALL, 64, T, HG, WG, wl.VIDEO, 1, 1)
    wv.head_pattern, wv.anchor, wv.radius, wv.head_layout = hp, 1, 2, w0.head_layout
    assert torch.equal(ov, _standalone(wv, q, k, v))
    compare(wv, Q, K, V, ov.float().cpu().numpy().astype(np.float64), label=f"request depth {depth} video")


def test_request_reuses_one_output_in_stream_order():
    """Forwards of a request run in submission order on its stream: a request
    that writes every mask's output into the same tensor leaves the last
    mask's output there."""
    masks = _small_masks(5, seed=7)
    w0 = masks[0]
    Q, K, V = wl.make_qkv(w0)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    o = torch.full_like(q, float("nan"))
    req = bsa.Request(w0.B, w0.H, w0.L, w0.d, depth=2, T=T, Hg=HG, Wg=WG, head_layout=w0.head_layout)
    for w in masks:
        req.submit(bsa.MASK_BLOCK_U8, w.bq, w.bk, q, k, v, o, data=w.block)
    req.close()  # finishes first
    torch.cuda.synchronize()
    assert torch.equal(o, _standalone(masks[-1], q, k, v))


def test_request_submit_error_leaves_request_usable():
    masks = _small_masks(2)
    w0 = masks[0]
    Q, K, V = wl.make_qkv(w0)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    req = bsa.Request(w0.B, w0.H, w0.L, w0.d, depth=2, T=T, Hg=HG, Wg=WG, head_layout=w0.head_layout)
    o = torch.full_like(q, float("nan"))
    with pytest.raises(bsa.BSAError) as e:
        req.submit(bsa.MASK_BLOCK_U8, 48, 64, q, k, v, o, data=w0.block)
    assert e.value.status == bsa.ERR_UNSUPPORTED
    req.submit(bsa.MASK_BLOCK_U8, w0.bq, w0.bk, q, k, v, o, data=w0.block)
    req.finish()
    req.close()
    assert torch.equal(o, _standalone(w0, q, k, v))


def test_tessera_request_pipelined():
    """The Tessera request: 48 masks (24 heads, 21 x 45x80 tokens) against one
    Q, K, V. Timed (wall clock, whole request) as plan-then-forward with a wait
    per mask, as a request with host masks, as a request with the masks
    already in device memory, and as the forwards alone on plans built
    beforehand. Logged; the pipelined request must not be slower than the
    serialized one."""
    ws = [wl.tessera(i) for i in range(48)]
    w0 = ws[0]
    g = torch.Generator(device="cuda:0")
    g.manual_seed(11)
    shp = (w0.B, w0.H, w0.L, w0.d)
    q, k, v = (torch.randn(shp, generator=g, device="cuda:0").to(torch.bfloat16) for _ in range(3))
    o = torch.empty_like(q)
    dmasks = [torch.from_numpy(np.ascontiguousarray(w.block)).to("cuda:0") for w in ws]
    kw = dict(T=w0.T, Hg=w0.Hg, Wg=w0.Wg)
    # warm the pools and the clocks
    for w in ws[:4]:
        p = bsa.plan(bsa.MASK_BLOCK_U8, w.B, w.H, w.L, w.d, w.bq, w.bk, data=w.block, **kw)
        bsa.forward(p, q, k, v, o)
        torch.cuda.synchronize()
        p.close()

    t0 = time.perf_counter()
    for w in ws:
        p = bsa.plan(bsa.MASK_BLOCK_U8, w.B, w.H, w.L, w.d, w.bq, w.bk, data=w.block, **kw)
        bsa.forward(p, q, k, v, o)
        torch.cuda.synchronize()
        p.close()
    t_serial = time.perf_counter() - t0

    def run_request(on_device):
        req = bsa.Request(w0.B, w0.H, w0.L, w0.d, depth=3, **kw)
        t0 = time.perf_counter()
        for w, md in zip(ws, dmasks):
            req.submit(bsa.MASK_BLOCK_U8, w.bq, w.bk, q, k, v, o, data=md if on_device else w.block,
                       on_device=on_device)
        req.finish()
        t = time.perf_counter() - t0
        st = req.stats()
        req.close()
        return t, st

    t_req_host, st_host = run_request(False)
    t_req_dev, st_dev = run_request(True)

    plans = [bsa.plan(bsa.MASK_BLOCK_U8, w.B, w.H, w.L, w.d, w.bq, w.bk, data=w.block, **kw) for w in ws]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for p in plans:
        bsa.forward(p, q, k, v, o)
    torch.cuda.synchronize()
    t_fwd = time.perf_counter() - t0
    for p in plans:
        p.close()
    log(f"[request] tessera 48 masks: serialized {t_serial * 1e3:.1f} ms, request host masks "
        f"{t_req_host * 1e3:.1f} ms (planning {st_host['plan_ns'] / 1e6:.1f} ms, waiting "
        f"{st_host['wait_ns'] / 1e6:.1f} ms), request device masks {t_req_dev * 1e3:.1f} ms (planning "
        f"{st_dev['plan_ns'] / 1e6:.1f} ms), forwards alone {t_fwd * 1e3:.1f} ms")
    assert t_req_host <= t_serial * 1.02
