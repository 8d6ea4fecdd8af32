"""GPU parity of the few-row (memory-bound) kernel against the oracle."""
import numpy as np
import pytest

import fp32_gemm_tile_amd as fg
from fp32_gemm_tile_amd import workloads as wl
import oracle

from gpu_util import check_full, check_sampled, log, run_fg

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


def skinny_id():
    return [c["id"] for c in fg.configs() if c["kind"] == fg.FG_KIND_SKINNY][0]


class few_kernel:
    """Force the few-row kernel family (1 vector ALU, 2 matrix cores) for a
    block of calls; automatic again afterwards."""

    def __init__(self, kernel):
        self.kernel = kernel

    def __enter__(self):
        assert fg.fg_set_few_row_kernel(self.kernel) == fg.FG_OK
        log(f"  few-row kernel {self.kernel}")

    def __exit__(self, *exc):
        assert fg.fg_set_few_row_kernel(0) == fg.FG_OK


def _pad4(n):
    return (n + 3) // 4 * 4


RAGGED = [(1, 1, 1), (1, 33, 517), (2, 300, 1000), (3, 31, 7), (5, 130, 260), (8, 257, 2049),
          (13, 70, 129), (16, 8197, 300), (17, 300, 100), (32, 8200, 513), (40, 100, 64),
          (64, 33, 40)]


@pytest.mark.parametrize("kernel", [1, 2])
@pytest.mark.parametrize("ta,tb", OPS)
@pytest.mark.parametrize("aligned", [False, True])
def test_skinny_ragged(ta, tb, aligned, kernel):
    """Each few-row kernel family forced on ragged shapes (one to 64 rows;
    N from 1 to past 8192, where the matrix-core kernel takes two column sets
    per wave; K shorter than a block and not a multiple of one)."""
    cid = skinny_id()
    with few_kernel(kernel):
        for i, (M, N, K) in enumerate(RAGGED):
            w0 = wl.custom(M, N, K, ta, tb)
            kw = dict(lda=_pad4(w0.LDA), ldb=_pad4(w0.LDB), ldc=_pad4(w0.LDC)) if aligned else {}
            w = wl.custom(M, N, K, ta, tb, alpha=0.5, beta=1.25, dist="normal", seed=90 + i,
                          **kw)
            A, B, C = wl.make_inputs(w)
            out, full = run_fg(w, A, B, C, config=cid)
            check_full(w, A, B, C, out)


@pytest.mark.parametrize("kernel", [1, 2])
@pytest.mark.parametrize("ta,tb", OPS)
def test_skinny_integer_exact(ta, tb, kernel):
    cid = skinny_id()
    with few_kernel(kernel):
        for (M, N, K) in [(1, 512, 4096), (4, 65, 1000), (8, 8, 8), (12, 8200, 777),
                          (30, 100, 1500)]:
            w = wl.custom(M, N, K, ta, tb, -1.0, 0.5, dist="int8", seed=M + N)
            A, B, C = wl.make_inputs(w)
            out, _ = run_fg(w, A, B, C, config=cid)
            cref, _ = oracle.gemm(ta, tb, M, N, K, -1.0, A, w.LDA, B, w.LDB, 0.5, C, w.LDC)
            assert np.array_equal(out.astype(np.float64), cref)


@pytest.mark.parametrize("name", ["G1", "G1T", "G8", "G8T", "G32"])
def test_decode_workloads(name):
    """The few-row workloads as the library picks them (auto selection)."""
    w = wl.WORKLOADS[name]
    A, B, C = wl.make_inputs(w)
    out, _ = run_fg(w, A, B, C)
    check_full(w, A, B, C, out)
    if w.M <= 8:
        assert fg.fg_select_config(w.transA, w.transB, w.M, w.N, w.K)["kind"] == \
            fg.FG_KIND_SKINNY


def test_skinny_repeatable():
    w = wl.WORKLOADS["G8"]
    A, B, _ = wl.make_inputs(w)
    o1, _ = run_fg(w, A, B, config=skinny_id())
    o2, _ = run_fg(w, A, B, config=skinny_id())
    assert np.array_equal(o1, o2)


@pytest.mark.parametrize("ta", ["N", "T"])
def test_skinny_both_k_loops(ta):
    """B stored K x N takes the software-pipelined k loop on grids of at most
    768 workgroups of 256 (512 of 512) with more than one row per block, and
    the plain one otherwise: both, with a ragged last k block and K shorter
    than one block, against the oracle."""
    cid = skinny_id()
    with few_kernel(1):
        for i, (M, N, K) in enumerate([(8, 1000, 777), (200, 8192, 300), (130, 2047, 100),
                                       (1, 9000, 2000), (3, 4000, 1500)]):
            wgs = -(-N // 32) * -(-M // 8)
            log(f"  grid {wgs} workgroups "
                f"({'pipelined' if wgs <= 768 and M > 1 else 'plain'} loop)")
            w = wl.custom(M, N, K, ta, "N", alpha=1.5, beta=0.5, dist="normal", seed=120 + i)
            A, B, C = wl.make_inputs(w)
            out, _ = run_fg(w, A, B, C, config=cid)
            check_full(w, A, B, C, out)


@pytest.mark.parametrize("threads", [256, 512, 1024])
@pytest.mark.parametrize("ta", ["N", "T"])
def test_skinny_workgroup_sizes(threads, ta):
    """B stored K x N with each workgroup size the kernel is built for (the
    K split inside a workgroup grows with it): ragged M, N and K, alpha and
    beta, against the oracle; integer inputs bit for bit."""
    cid = skinny_id()
    assert fg.fg_set_few_row_threads(threads) == fg.FG_OK
    assert fg.fg_set_few_row_kernel(1) == fg.FG_OK
    try:
        for i, (M, N, K) in enumerate([(1, 1000, 3000), (8, 4100, 1025), (5, 300, 100),
                                       (2, 8192, 4096), (8, 257, 2049)]):
            w = wl.custom(M, N, K, ta, "N", alpha=1.5, beta=0.5, dist="normal", seed=140 + i)
            A, B, C = wl.make_inputs(w)
            out, _ = run_fg(w, A, B, C, config=cid)
            check_full(w, A, B, C, out)
        w = wl.custom(8, 777, 1500, ta, "N", alpha=2.0, beta=-1.0, dist="int8", seed=150)
        A, B, C = wl.make_inputs(w)
        out, _ = run_fg(w, A, B, C, config=cid)
        cref, _ = oracle.gemm(ta, "N", w.M, w.N, w.K, w.alpha, A, w.LDA, B, w.LDB, w.beta, C,
                              w.LDC)
        assert np.array_equal(out.astype(np.float64), cref)
    finally:
        assert fg.fg_set_few_row_threads(0) == fg.FG_OK
        assert fg.fg_set_few_row_kernel(0) == fg.FG_OK
