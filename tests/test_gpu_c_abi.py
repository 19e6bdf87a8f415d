"""The C ABI from a plain C program: tests/c_abi_forward (built by
__graft_entry__.build() from tests/c_abi_forward.c with gcc, linked against
the in-tree libbsa.so) plans a BLOCK_U8 mask and runs the forward with its own
hipMalloc'd buffers; its output is compared with the fp64 oracle on the same
seeded inputs (bf16 bar: max-abs 1e-2, mean-abs 1e-3)."""
import os
import subprocess

import numpy as np
import pytest

import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi_forward")


def test_c_consumer_is_built_and_linked():
    """Runs on the CPU too: the program loads libbsa.so and the HIP runtime
    and stops at its usage check (exit 2) before any HIP call."""
    assert os.path.exists(EXE), "build() compiles tests/c_abi_forward"
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr


def _write_inputs(d, w, Q, K, V):
    with open(os.path.join(d, "shape.txt"), "w") as f:
        f.write(f"{w.B} {w.H} {w.L} {w.d} {w.bq} {w.bk}\n")
    np.ascontiguousarray(w.block, dtype=np.uint8).tofile(os.path.join(d, "mask.u8"))
    for name, x in (("q", Q), ("k", K), ("v", V)):
        np.ascontiguousarray(x, dtype=np.uint16).tofile(os.path.join(d, f"{name}.bf16"))


def _cases():
    out = [wl.tiny()]
    g = np.random.default_rng(21)
    for bq, bk in [(32, 32), (128, 64)]:
        T, Hg, Wg = 3, 10, 11  # L = 330: ragged for every block size
        w = wl.Workload(f"cabi{bq}x{bk}", 71, 1, 3, T * Hg * Wg, 128, T, Hg, Wg, wl.BLOCK, bq, bk)
        w.block = (g.random((1, 3, w.nqb, w.nkb)) < 0.35).astype(np.uint8)
        w.block[0, 2, 1, :] = 0  # an empty block row: its queries output 0
        out.append(w)
    return out


@pytest.mark.gpu
@pytest.mark.parametrize("w", _cases(), ids=lambda w: w.name)
def test_c_consumer_forward_matches_oracle(w, tmp_path):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(EXE):
        pytest.skip("tests/c_abi_forward is not built (build() compiles it)")
    from gpu_util import compare, log
    Q, K, V = wl.make_qkv(w)
    _write_inputs(str(tmp_path), w, Q, K, V)
    log(f"[case] C consumer {w.name}")
    r = subprocess.run([EXE, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    log(f"[c-abi] {w.name}: {r.stdout.strip()}")
    o = np.fromfile(os.path.join(str(tmp_path), "o.bf16"), dtype=np.uint16)
    O = wl.bf16_bits_to_f32(o.reshape(w.B, w.H, w.L, w.d)).astype(np.float64)
    compare(w, Q, K, V, O, label=f"C consumer {w.name}")
