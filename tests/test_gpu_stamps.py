"""The clock-stamped forward (bsa_forward_stamped) through the C ABI: the same
output as bsa_forward bit for bit, one start/end stamp pair per workgroup that
runs a task (none for the padding workgroups), ends after starts, and a shader
clock inside the range a gfx950 runs at; fp32 plans are refused."""
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
from gpu_util import log, to_device  # noqa: E402


@pytest.mark.parametrize("name,regime", [("tiny", -1), ("svgB", 0), ("svgB", 4), ("fg64", -1)])
def test_stamped_forward_matches_and_stamps(name, regime):
    w = {"tiny": wl.tiny, "svgB": lambda: wl.svg("B"), "fg64": lambda: wl.fgattn(M=64)}[name]()
    Q, K, V = wl.make_qkv(w)
    q, k, v = to_device(Q), to_device(K), to_device(V)
    p = plan_workload(w, force_regime=regime)
    info = p.info()
    log(f"[stamps] {name} regime={info['regime']} tasks={info['tasks']} workgroups={info['workgroups']}")
    o_ref = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    o = torch.full(q.shape, float("nan"), dtype=torch.bfloat16, device="cuda:0")
    stamps = torch.zeros(4 * info["workgroups"], dtype=torch.int64, device="cuda:0")
    bsa.forward(p, q, k, v, o_ref)
    bsa.forward_stamped(p, q, k, v, o, stamps)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    s = stamps.cpu().numpy().reshape(-1, 4)
    written = s[:, 1] != 0
    assert int(written.sum()) == info["tasks"], (int(written.sum()), info["tasks"])
    s = s[written].astype(np.float64)
    assert np.all(s[:, 2] > s[:, 0]) and np.all(s[:, 3] > s[:, 1])
    ghz = (s[:, 2] - s[:, 0]).sum() / (s[:, 3] - s[:, 1]).sum() * 0.1
    log(f"[stamps] {name}: shader clock {ghz:.3f} GHz over {int(written.sum())} tasks")
    assert 0.3 < ghz < 3.5, ghz
    p.close()


def test_stamped_forward_refuses_fp32_plans():
    w = wl.tiny()
    p = plan_workload(w, dtype=bsa.DTYPE_F32)
    stamps = torch.zeros(4 * p.info()["workgroups"], dtype=torch.int64, device="cuda:0")
    x = torch.zeros((w.B, w.H, w.L, w.d), dtype=torch.float32, device="cuda:0")
    with pytest.raises(bsa.BSAError, match="bf16"):
        bsa.forward_stamped(p, x, x, x, x, stamps)
    p.close()
