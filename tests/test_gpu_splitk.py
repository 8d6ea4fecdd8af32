"""GPU parity of split-K (fg_sgemm_splitk) against the oracle.

Each slice sums a contiguous k range; the slices are added in ascending
order, so the result is deterministic; the float tolerance is the same
acceptance bound as the one-pass kernels (any summation order is allowed).
"""
import numpy as np
import pytest

import fp32_gemm_tile_amd as fg
from fp32_gemm_tile_amd import workloads as wl
import oracle

from gpu_util import check_full, check_full_blocked, log, to_device

pytestmark = pytest.mark.gpu

OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fg.load_library()
    yield
    torch.cuda.synchronize()


def run_splitk(w, A, B, C, splits, ws_floats=None, ws_fill=np.nan):
    import torch
    dA, _ba = to_device(A)
    dB, _bb = to_device(B)
    if C is None:
        C = np.full((w.M, w.LDC), np.nan, dtype=np.float32)
    dC, _bc = to_device(C)
    need = fg.fg_sgemm_splitk_workspace_size(w.M, w.N, max(splits, 1)) // 4
    n = ws_floats if ws_floats is not None else max(need, 1)
    ws = torch.full((n,), ws_fill, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()
    log(f"  fg_sgemm_splitk {w.transA}{w.transB} M={w.M} N={w.N} K={w.K} splits={splits} ws={n}")
    st = fg.fg_sgemm_splitk(w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.LDA,
                            dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC, splits,
                            ws.data_ptr(), n * 4, s.cuda_stream)
    if st != fg.FG_OK:
        raise fg.FgError(st, fg.fg_last_bad_arg(), fg.fg_last_error())
    s.synchronize()
    return dC.cpu().numpy().reshape(C.shape)[:, :w.N].copy()


def _pad4(n):
    return (n + 3) // 4 * 4


@pytest.mark.parametrize("ta,tb", OPS)
@pytest.mark.parametrize("splits", [2, 3, 7])
def test_splitk_ragged_float(ta, tb, splits):
    for i, (M, N, K, pad) in enumerate([(97, 131, 300, False), (128, 256, 1025, True),
                                        (33, 70, 2000, False), (256, 256, 48, True)]):
        w0 = wl.custom(M, N, K, ta, tb)
        kw = dict(lda=_pad4(w0.LDA), ldb=_pad4(w0.LDB), ldc=_pad4(w0.LDC)) if pad else {}
        w = wl.custom(M, N, K, ta, tb, alpha=1.5, beta=-0.5, dist="normal", seed=60 + i, **kw)
        A, B, C = wl.make_inputs(w)
        out = run_splitk(w, A, B, C, splits)
        check_full(w, A, B, C, out)


@pytest.mark.parametrize("ta,tb", OPS)
def test_splitk_integer_bit_exact(ta, tb):
    for (M, N, K, splits) in [(64, 96, 512, 4), (130, 33, 1000, 5), (256, 256, 64, 16)]:
        for alpha, beta in [(1.0, 0.0), (-2.0, 0.5)]:
            w = wl.custom(M, N, K, ta, tb, alpha, beta, dist="int8", seed=M + K)
            A, B, C = wl.make_inputs(w)
            out = run_splitk(w, A, B, C, splits)
            cref, _ = oracle.gemm(ta, tb, M, N, K, alpha, A, w.LDA, B, w.LDB, beta, C, w.LDC)
            assert np.array_equal(out.astype(np.float64), cref), (ta, tb, M, N, K, splits)


def test_splitk_deterministic_and_auto():
    w = wl.WORKLOADS["C2"]
    A, B, _ = wl.make_inputs(w)
    ws = 64 * 2048 * 2048  # room for 64 slices
    o1 = run_splitk(w, A, B, None, 0, ws_floats=ws)
    o2 = run_splitk(w, A, B, None, 0, ws_floats=ws, ws_fill=0.0)
    assert np.array_equal(o1, o2)
    check_full(w, A, B, None, o1)


@pytest.mark.parametrize("name", ["C1", "C3"])
def test_splitk_workloads(name):
    w = wl.WORKLOADS[name]
    A, B, C = wl.make_inputs(w)
    out = run_splitk(w, A, B, C, 0, ws_floats=16 * w.M * w.N)
    check_full(w, A, B, C, out)


def test_splitk_one_and_more_splits_than_ktiles():
    w = wl.custom(100, 100, 40, alpha=1.0, beta=0.0, seed=3)  # 2 to 5 k-tiles (BK 8 .. 32)
    A, B, _ = wl.make_inputs(w)
    o1 = run_splitk(w, A, B, None, 1, ws_floats=1)
    check_full(w, A, B, None, o1)
    o9 = run_splitk(w, A, B, None, 9, ws_floats=9 * 100 * 100)  # capped at the k-tiles
    check_full(w, A, B, None, o9)


def test_splitk_large_full():
    """One GPU's row block of 8192^3 (1024 x 8192 x 8192) with a library-chosen
    split, every element against the oracle."""
    w = wl.custom(1024, 8192, 8192, seed=77)
    A, B, _ = wl.make_inputs(w)
    out = run_splitk(w, A, B, None, 0, ws_floats=8 * 1024 * 8192)
    assert np.all(np.isfinite(out))
    check_full_blocked(w, A, B, None, out, name="split-K 1024x8192x8192")
