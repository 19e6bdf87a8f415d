"""GPU parity of the fp32 validation build: fp32 Q, K, V, O through the C ABI
against the fp64 CPU oracle on the same seeded inputs. Bar: max over rows of
|O - O_ref|_inf / |O_ref|_inf <= 1e-5; rows with no kept key exactly 0;
every output row written (O is pre-filled with NaN)."""
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
    bsa.lib()  # fail loudly if the library is missing


from gpu_util import compare_f32, log, run_gpu, sample_rows, short_cases, thick_rows  # noqa: E402


@pytest.mark.parametrize("regime", [-1, 0, 1, 4])
def test_tiny_f32(regime):
    w = wl.tiny()
    Q, K, V = wl.make_qkv(w, "f32")
    log(f"[case] f32 tiny regime={regime}")
    O, p = run_gpu(w, Q, K, V, force_regime=regime)
    compare_f32(w, Q, K, V, O, label=f"f32 tiny r{p.info()['regime']}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("shape", [(64, 64), (32, 32), (128, 128), (64, 256), (256, 32)])
def test_small_block_f32(shape, d):
    g = np.random.default_rng(11 + d + shape[0])
    bq, bk = shape
    T, Hg, Wg = 3, 10, 11
    w = wl.Workload(f"f32blk{bq}x{bk}_d{d}", 70 + d, 1, 2, T * Hg * Wg, d, T, Hg, Wg, wl.BLOCK, bq, bk)
    w.block = (g.random((1, 2, w.nqb, w.nkb)) < 0.4).astype(np.uint8)
    w.block[0, 1, 0, :] = 0  # empty rows
    w.head_layout = np.array([0, 1], np.uint8)
    Q, K, V = wl.make_qkv(w, "f32")
    for regime in (0, 1):
        log(f"[case] f32 {w.name} regime={regime}")
        O, _ = run_gpu(w, Q, K, V, force_regime=regime)
        compare_f32(w, Q, K, V, O, label=f"f32 {w.name} r{regime}")


@pytest.mark.parametrize("run", ["A", "B"])
@pytest.mark.parametrize("d", [64, 128])
def test_small_video_f32(run, d):
    w = wl.svg(run, H=4, T=5, Hg=7, Wg=13, d=d)
    w.head_pattern = np.array([wl.SPATIAL, wl.TEMPORAL, wl.SPATIAL, wl.DENSE], np.uint8)
    w.anchor = 2 if run == "B" else 0
    w.head_layout = np.array([0, 1, 1, 1], np.uint8) if run == "B" else np.zeros(4, np.uint8)
    Q, K, V = wl.make_qkv(w, "f32")
    log(f"[case] f32 small video run={run} d={d}")
    O, _ = run_gpu(w, Q, K, V)
    compare_f32(w, Q, K, V, O, label=f"f32 video{run} d{d}")


@pytest.mark.parametrize("M", [64, 128])
def test_small_slices_f32(M):
    w = wl.fgattn(H=2, T=3, Hg=10, Wg=11, d=128, M=M, cfg=33)
    w.head_layout = np.array([0, 1], np.uint8)
    Q, K, V = wl.make_qkv(w, "f32")
    log(f"[case] f32 slices M={M}")
    O, _ = run_gpu(w, Q, K, V)
    compare_f32(w, Q, K, V, O, label=f"f32 slice M{M}")


@pytest.mark.parametrize("w", short_cases(), ids=lambda w: w.name)
def test_short_sequences_f32(w):
    """The short sequences of the bf16 suite in the fp32 build."""
    Q, K, V = wl.make_qkv(w, "f32")
    for regime in ((-1,) if w.kind == wl.SLICE else (0, 1)):
        log(f"[case] f32 {w.name} regime={regime}")
        O, p = run_gpu(w, Q, K, V, force_regime=regime)
        compare_f32(w, Q, K, V, O, label=f"f32 {w.name} r{p.info()['regime']}")


def test_all_empty_mask_f32():
    w = wl.tiny()
    w.block[:] = 0
    Q, K, V = wl.make_qkv(w, "f32")
    O, _ = run_gpu(w, Q, K, V)
    assert np.all(O == 0.0)


def test_svg_full_size_sampled_f32():
    """SVG head routing at full size, run B, fp32 build; sampled rows of every
    head, including every row of the ragged last query tile."""
    w = wl.svg("B")
    Q, K, V = wl.make_qkv(w, "f32")
    log("[case] f32 svg full run=B")
    O, p = run_gpu(w, Q, K, V)
    rows = sample_rows(w, per_head=32)
    compare_f32(w, Q, K, V, O, rows=rows, label=f"f32 svgB {p.info()['regime']}")


def test_fgattn_full_size_sampled_f32():
    """FG-Attn slices at full size (24 heads, L = 32,760, M = 64), fp32 build;
    per head the longest list's query block, the ragged last block and 256
    random rows."""
    w = wl.fgattn()
    Q, K, V = wl.make_qkv(w, "f32")
    rows = thick_rows(w, 64)
    log("[case] f32 fgattn full")
    O, p = run_gpu(w, Q, K, V, rows=rows)
    compare_f32(w, Q, K, V, O, rows=rows, gathered=True, label=f"f32 fgattn {p.info()['regime']}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("i", [28, 17, 7])
def test_tessera_full_size_sampled_f32(i):
    """Tessera-style masks at full size (24 heads, L = 75,600), fp32 build:
    32x32 random (mask 28), 64x64 local window (17), 64x256 banded (7), all at
    density 0.15; per head the heaviest query tile, the ragged last tile and
    256 random rows."""
    w = wl.tessera(i)
    Q, K, V = wl.make_qkv(w, "f32")
    rows = thick_rows(w, 256, seed=i)
    log(f"[case] f32 tessera mask {i}: {w.bq}x{w.bk}")
    O, p = run_gpu(w, Q, K, V, rows=rows)
    compare_f32(w, Q, K, V, O, rows=rows, gathered=True, label=f"f32 tessera{i} {p.info()['regime']}")


@pytest.mark.timeout(900)
def test_highres_full_size_sampled_f32():
    """High-res at full size (24 heads, L = 302,400), fp32 build; per head its
    heaviest query tile (in the head's token order), the ragged last tile and
    256 random rows."""
    w = wl.highres()
    log("[case] f32 generating high-res Q/K/V")
    Q, K, V = wl.make_qkv(w, "f32")
    rows = thick_rows(w, 128)
    log("[case] f32 highres full")
    O, p = run_gpu(w, Q, K, V, rows=rows)
    compare_f32(w, Q, K, V, O, rows=rows, gathered=True, label=f"f32 highres {p.info()['regime']}")
