"""Plan lifetime: a plan destroyed right after an asynchronous forward does not
hand its device memory to the next plan while the forward still reads it.
bsa_plan_destroy waits for the plan's last-use event (recorded by every
bsa_forward), so the first forward's output still matches the oracle after a
second plan of a different mask, planned at once, has taken the recycled
block and uploaded its own image into it."""
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
from gpu_util import compare, log, sample_rows, to_device  # noqa: E402


def _masks():
    """Two BLOCK masks of one shape whose plan images are about the same size
    (so the second reuses the first's pooled block), different contents."""
    T, Hg, Wg = 8, 32, 64
    L = T * Hg * Wg  # 16,384 tokens
    out = []
    for i in range(2):
        w = wl.Workload(f"life{i}", 60 + i, 1, 8, L, 128, T, Hg, Wg, wl.BLOCK, 64, 64)
        g = np.random.default_rng([60, i])
        w.block = (g.random((1, w.H, w.nqb, w.nkb)) < 0.3).astype(np.uint8)
        out.append(w)
    return out


def test_destroy_right_after_async_forward():
    w1, w2 = _masks()
    Q, K, V = wl.make_qkv(w1)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    o1 = torch.full_like(q, float("nan"))
    o2 = torch.full_like(q, float("nan"))
    log(f"[lifetime] H={w1.H} L={w1.L} d={w1.d} 64x64 blocks at 0.3")
    for rep in range(3):
        p1 = plan_workload(w1)
        bsa.forward(p1, q, k, v, o1)
        p1.close()  # no synchronisation before: destroy must wait for the forward
        p2 = plan_workload(w2)  # takes the recycled block, uploads into it
        bsa.forward(p2, q, k, v, o2)
        p2.close()
        torch.cuda.synchronize()
    O1 = o1.float().cpu().numpy().astype(np.float64)
    O2 = o2.float().cpu().numpy().astype(np.float64)
    rows = sample_rows(w1, per_head=64)
    compare(w1, Q, K, V, O1, rows=rows, label="lifetime: first plan's output")
    compare(w2, Q, K, V, O2, rows=rows, label="lifetime: second plan's output")


def test_forward_on_two_streams_then_destroy():
    """Forwards of one plan on two streams, then destroy at once: both
    outputs stay right (destroy waits for both)."""
    w1, _ = _masks()
    Q, K, V = wl.make_qkv(w1)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    oa = torch.full_like(q, float("nan"))
    ob = torch.full_like(q, float("nan"))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    p = plan_workload(w1)
    bsa.forward(p, q, k, v, oa, s1)
    bsa.forward(p, q, k, v, ob, s2)
    p.close()
    p2 = plan_workload(_masks()[1])
    p2.close()
    torch.cuda.synchronize()
    rows = sample_rows(w1, per_head=32)
    compare(w1, Q, K, V, oa.float().cpu().numpy().astype(np.float64), rows=rows, label="two streams: first")
    compare(w1, Q, K, V, ob.float().cpu().numpy().astype(np.float64), rows=rows, label="two streams: second")
