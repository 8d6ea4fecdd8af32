"""fg_sgemm_streamk on the GPU: the last, partial round of tiles split along
K into per-(tile, slice) workspace slots and reduced in fixed order. Checked
against the oracle (full and sampled), bit-exact on integer inputs, and
bit-identical across repeated calls."""
import numpy as np
import pytest

import fp32_gemm_tile_amd as fg
from fp32_gemm_tile_amd import workloads as wl
import oracle
from gpu_util import check_full, check_full_blocked, log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def always_split():
    """Split every eligible tail (the default policy splits only where the
    cost model expects a gain, which few shapes reach)."""
    assert fg.fg_set_streamk_policy(1) == fg.FG_OK
    yield
    assert fg.fg_set_streamk_policy(0) == fg.FG_OK


def run_streamk(w, A, B, C=None, ws_bytes=None, c_fill=np.nan):
    import torch
    dA, _a = to_device(A)
    dB, _b = to_device(B)
    if C is None:
        C = np.full((w.M, w.LDC), c_fill, dtype=np.float32)
    dC, _c = to_device(C)
    need = fg.fg_sgemm_streamk_workspace_size(w.transA, w.transB, w.M, w.N, w.K, dA.data_ptr(),
                                              w.LDA, dB.data_ptr(), w.LDB)
    nbytes = need if ws_bytes is None else ws_bytes
    ws = torch.full((max(nbytes, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    log(f"  fg_sgemm_streamk {w.transA}{w.transB} M={w.M} N={w.N} K={w.K} alpha={w.alpha} "
        f"beta={w.beta} plan_ws={need} given={nbytes}")
    s = torch.cuda.current_stream()
    st = fg.fg_sgemm_streamk(w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.LDA,
                             dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC,
                             ws.data_ptr() if nbytes else 0, nbytes, s.cuda_stream)
    if st != fg.FG_OK:
        raise fg.FgError(st, fg.fg_last_bad_arg(), fg.fg_last_error())
    s.synchronize()
    return dC.cpu().numpy().reshape(C.shape)[:, :w.N].copy(), need


SHAPES = [
    # (M, N, K, opA, opB, alpha, beta, dist, lda, ldb, ldc)
    (1000, 1000, 500, "N", "N", 1.0, 0.0, "uniform", None, None, None),
    (2048, 2048, 384, "N", "N", 1.0, 0.0, "uniform", None, None, None),
    (3001, 2047, 1025, "T", "N", 1.5, 0.5, "normal", 3001, 2047, 2047),
    (1500, 700, 333, "N", "T", -0.5, 2.0, "normal", None, None, None),
    (777, 2100, 1000, "T", "T", 1.0, 1.0, "normal", None, None, 2101),
    (2500, 1800, 700, "N", "N", 0.75, -1.5, "normal", None, None, None),
    (1333, 2001, 555, "T", "T", 1.25, 0.5, "normal", None, None, 2003),
    (2047, 1500, 1001, "T", "N", -1.0, 1.0, "normal", None, None, None),
]


@pytest.mark.parametrize("shape", SHAPES, ids=[f"{s[0]}x{s[1]}x{s[2]}{s[3]}{s[4]}" for s in SHAPES])
def test_streamk_matches_oracle(shape):
    M, N, K, ta, tb, alpha, beta, dist, lda, ldb, ldc = shape
    w = wl.custom(M, N, K, ta, tb, alpha, beta, dist, seed=M + K, lda=lda, ldb=ldb, ldc=ldc)
    A, B, C = wl.make_inputs(w)
    out, need = run_streamk(w, A, B, C)
    check_full(w, A, B, C, out)


def test_streamk_integer_exact_and_repeatable():
    w = wl.custom(1000, 1000, 500, "N", "N", 2.0, 0.5, "int8", seed=77)
    A, B, C = wl.make_inputs(w)
    out1, need = run_streamk(w, A, B, C)
    out2, _ = run_streamk(w, A, B, C)
    assert need > 0
    cref, _ = oracle.gemm("N", "N", w.M, w.N, w.K, 2.0, A, w.LDA, B, w.LDB, 0.5, C, w.LDC)
    assert np.array_equal(out1.astype(np.float64), cref)
    assert np.array_equal(out1, out2)


def test_streamk_small_or_no_workspace():
    """Less workspace means fewer slices (still correct); none means the
    plain call, bit for bit."""
    import torch
    w = wl.custom(2048, 2048, 384, "N", "N", 1.0, 0.0, "uniform", seed=78)
    A, B, _ = wl.make_inputs(w)
    need = fg.fg_sgemm_streamk_workspace_size("N", "N", w.M, w.N, w.K)
    for nbytes in (need // 2, need // 3, 64):
        out, _ = run_streamk(w, A, B, ws_bytes=nbytes)
        check_full(w, A, B, None, out)
    plain_ws, _ = run_streamk(w, A, B, ws_bytes=0)
    dA, _a = to_device(A)
    dB, _b = to_device(B)
    dC = torch.empty(w.M * w.N, device="cuda")
    assert fg.fg_sgemm(w.transA, w.transB, w.M, w.N, w.K, 1.0, dA.data_ptr(), w.LDA,
                       dB.data_ptr(), w.LDB, 0.0, dC.data_ptr(), w.N,
                       torch.cuda.current_stream().cuda_stream) == fg.FG_OK
    torch.cuda.synchronize()
    assert np.array_equal(plain_ws, dC.cpu().numpy().reshape(w.M, w.N))


def test_streamk_shapes_exercise_the_split():
    """Most of the shapes above have a split tail with the current table (so
    the tail kernels and the slot reduction are what the oracle checks),
    across layouts, alpha/beta and unaligned rows."""
    split = [s for s in SHAPES
             if fg.fg_sgemm_streamk_workspace_size(s[3], s[4], s[0], s[1], s[2], lda=s[8],
                                                   ldb=s[9]) > 0]
    assert len(split) >= 5, split
    assert {(s[3], s[4]) for s in split} >= {("N", "N"), ("T", "N"), ("T", "T")}
    assert any(s[6] != 0 for s in split)


def test_streamk_no_tail_is_plain():
    """Whole rounds only (8192^3, 4096^3 with 256 x 256 tiles): no split. With
    the default policy the model decides, and it never splits where the
    always-split policy would not (nor asks for a larger workspace)."""
    assert fg.fg_sgemm_streamk_workspace_size("N", "N", 8192, 8192, 8192) == 0
    assert fg.fg_sgemm_streamk_workspace_size("N", "N", 4096, 4096, 4096) == 0
    shapes = [(1000, 1000, 500), (4096, 5120, 4096), (4608, 4608, 4096), (6144, 6144, 6144),
              (1536, 1536, 1536), (512, 8192, 8192)]
    always = [fg.fg_sgemm_streamk_workspace_size("N", "N", *sh) for sh in shapes]
    assert fg.fg_set_streamk_policy(0) == fg.FG_OK
    model = [fg.fg_sgemm_streamk_workspace_size("N", "N", *sh) for sh in shapes]
    assert all(m == 0 or m <= a for m, a in zip(model, always)), (model, always)
    assert sum(m == 0 for m in model) >= 1


def test_streamk_large_full():
    """A large shape whose plan has a split tail (the first of a few
    candidates that has one with the current table), every element against
    the oracle."""
    cands = [(4096, 5120, 4096), (4352, 4608, 4096), (4096, 6144, 4096), (4608, 4608, 4096),
             (5120, 5120, 4096), (6144, 6144, 6144)]
    shape = next((c for c in cands if fg.fg_sgemm_streamk_workspace_size("N", "N", *c) > 0), None)
    assert shape is not None, "no candidate has a split tail"
    log(f"  large stream-K shape {shape}")
    w = wl.custom(*shape, seed=79)
    A, B, _ = wl.make_inputs(w)
    out, need = run_streamk(w, A, B)
    assert need > 0
    assert np.all(np.isfinite(out))
    check_full_blocked(w, A, B, None, out, name=f"stream-K {shape}")
