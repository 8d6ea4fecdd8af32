"""Leading dimensions at the library's limit (FG_MAX_LD elements).

Every kernel addresses a matrix through 32-bit byte offsets from a base that
it moves along K. Here the few-row kernels' offsets across one k block would
pass 2^32 bytes (so the calls must take the rebasing path), and the MFMA
tiles' row offsets come close to 2^31. Each matrix sits in a strided device
buffer of up to a few GB whose unused columns hold NaN: a read that lands in
the wrong place carries a NaN, or a wrong value, into the result. Inputs are
seeded and dense on the host; the oracle runs on the dense copies."""
import numpy as np
import pytest

import fp32_gemm_tile_amd as fg
from fp32_gemm_tile_amd import workloads as wl
import oracle
from oracle import compare
from gpu_util import log

pytestmark = pytest.mark.gpu
LD = fg.FG_MAX_LD


def _strided(x, ld):
    """Device buffer of (rows - 1) * ld + cols floats holding x (rows x cols)
    with leading dimension ld; everything else NaN."""
    import torch
    rows, cols = x.shape
    base = torch.full(((rows - 1) * ld + cols,), float("nan"), device="cuda")
    torch.as_strided(base, (rows, cols), (ld, 1)).copy_(torch.from_numpy(x))
    return base


def _config(kind=None, name=None):
    for c in fg.configs():
        if (kind is not None and c["kind"] == kind) or (name is not None and c["name"] == name):
            return c["id"]
    raise LookupError(kind or name)


def _run(ta, tb, M, N, K, lda, ldb, ldc, config, alpha=1.5, beta=0.5, seed=0):
    import torch
    w = wl.custom(M, N, K, ta, tb, alpha, beta, "normal", seed)
    A, B, C = wl.make_inputs(w)  # dense: lda, ldb, ldc are the minimum
    log(f"  large ld {ta}{tb} M={M} N={N} K={K} lda={lda} ldb={ldb} ldc={ldc} cfg={config}")
    dA, dB, dC = _strided(A, lda), _strided(B, ldb), _strided(C, ldc)
    s = torch.cuda.current_stream()
    st = fg.fg_sgemm_ex(ta, tb, M, N, K, alpha, dA.data_ptr(), lda, dB.data_ptr(), ldb, beta,
                        dC.data_ptr(), ldc, s.cuda_stream, config)
    assert st == fg.FG_OK, fg.fg_last_error()
    out = torch.as_strided(dC, (M, N), (ldc, 1)).cpu().numpy()
    del dA, dB, dC
    torch.cuda.empty_cache()
    cref, sabs = oracle.gemm(ta, tb, M, N, K, alpha, A, w.LDA, B, w.LDB, beta, C, w.LDC)
    ok, info = compare.check(out, cref, sabs, K, alpha, beta, C[:, :N])
    assert ok, info


class _few_kernel:
    """Force a few-row kernel family (1 vector ALU: for B stored K x N the
    instance that rebases per k step; 2 matrix cores) for a block of calls."""

    def __init__(self, kernel):
        self.kernel = kernel

    def __enter__(self):
        assert fg.fg_set_few_row_kernel(self.kernel) == fg.FG_OK

    def __exit__(self, *exc):
        assert fg.fg_set_few_row_kernel(0) == fg.FG_OK


@pytest.mark.parametrize("kernel", [1, 2])
@pytest.mark.parametrize("M", [1, 8])
def test_few_rows_b_kxn_at_max_ld(M, kernel):
    # B stored K x N: 700 rows of ldb = 2^21 (5.9 GB); byte offsets from the
    # block's first row pass 2^32 at row 512.
    with _few_kernel(kernel):
        _run("N", "N", M, 300, 700, 700, LD, LD, _config(kind=fg.FG_KIND_SKINNY))


@pytest.mark.parametrize("kernel", [1, 2])
@pytest.mark.parametrize("M", [3, 8])
@pytest.mark.parametrize("tb", ["N", "T"])
def test_few_rows_a_kxm_at_max_ld(tb, M, kernel):
    # A stored K x M with lda = 2^21 (5.9 GB), B in either layout.
    with _few_kernel(kernel):
        _run("T", tb, M, 300, 700, LD, 300 if tb == "N" else 700, 300,
             _config(kind=fg.FG_KIND_SKINNY))


@pytest.mark.parametrize("ta,tb", [("N", "N"), ("T", "T")])
def test_mfma_tiles_at_max_ld(ta, tb):
    # 256-row tiles: row offsets up to 255 * 2^21 * 4 bytes inside a tile.
    _run(ta, tb, 300, 200, 150, LD, LD, LD, _config(name="mfma_256x256x16_w2x2_s4"))


@pytest.mark.parametrize("ta,tb", [("N", "N"), ("T", "T")])
def test_valu_tiles_at_max_ld(ta, tb):
    # The vector-ALU comparison kernel's 128-row tiles at the same leading dimensions.
    _run(ta, tb, 300, 200, 150, LD, LD, LD, _config(name="valu_128x128x8_t8x8"))
