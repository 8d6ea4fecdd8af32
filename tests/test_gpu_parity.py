"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Tolerance (stated acceptance bound): per element
|C - C_ref| <= 8*max(K,1)*2^-24*(|alpha|*S + |beta|*|C_in|) + 1e-6 with
S = sum_k |a_ik b_kj|, and relative Frobenius error <= 1e-5. Integer-valued
inputs must match bit for bit (every partial sum is exact in binary32).
"""
import numpy as np
import pytest

import fp32_gemm_tile_amd as fg
from fp32_gemm_tile_amd import workloads as wl
import oracle

from gpu_util import check_full, check_full_blocked, log, run_fg

pytestmark = pytest.mark.gpu

OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fg.load_library()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _configs():
    try:
        return fg.configs()
    except OSError:  # library missing: the tests below then fail loudly
        return [{"id": i, "kind": fg.FG_KIND_MFMA} for i in range(7)]


def mfma_ids():
    return [c["id"] for c in _configs() if c["kind"] == fg.FG_KIND_MFMA]


def all_ids():
    return [c["id"] for c in _configs()]


def config_id(name):
    return next(c["id"] for c in fg.configs() if c["name"] == name)


HEADLINE = "mfma_256x256x16_w2x2_s4"  # the entry the 4096^3 and 8192^3 workloads run


# --- the workloads the metric and the parity cases are quoted on ----------

@pytest.mark.parametrize("name", ["C1", "C2", "C3"])
def test_workload_full_oracle(name):
    w = wl.WORKLOADS[name]
    A, B, C = wl.make_inputs(w)
    out, _ = run_fg(w, A, B, C)
    info = check_full(w, A, B, C, out)
    log(f"  {name}: max err/tol {info['max_err_over_tol']:.3g}, frob_rel {info.get('frob_rel')}")


@pytest.mark.parametrize("name", ["C4", "C5a", "C5b", "C6"])
def test_workload_full_oracle_large(name):
    """The large workloads in the launch configuration the bench times
    (automatic selection), every element against the oracle (in row blocks);
    C starts as NaN, so an element never written fails too."""
    w = wl.WORKLOADS[name]
    A, B, C = wl.make_inputs(w)
    out, _ = run_fg(w, A, B, C)
    assert np.all(np.isfinite(out))
    check_full_blocked(w, A, B, C, out)


@pytest.mark.parametrize("cfg", [-1, HEADLINE])
@pytest.mark.parametrize("ta,tb", OPS)
def test_layouts_4096_cubed_full(ta, tb, cfg):
    """4096^3 in all four layouts, with the automatic pick and with the
    headline entry forced (a grid of 256 tiles: the XCD renumbering is
    active), every element against the oracle."""
    w = wl.custom(4096, 4096, 4096, ta, tb, seed=50 + 2 * (ta == "T") + (tb == "T"))
    A, B, _ = wl.make_inputs(w)
    out, _ = run_fg(w, A, B, config=-1 if cfg == -1 else config_id(cfg))
    check_full_blocked(w, A, B, None, out, name=f"4096^3 {ta}{tb} cfg={cfg}")


@pytest.mark.parametrize("ta,tb", OPS)
def test_headline_entry_remapped_grid(ta, tb):
    """The headline entry on 2048 x 2048 x 512 (64 tiles, a multiple of 8:
    XCD renumbering on) with alpha/beta, every element."""
    w = wl.custom(2048, 2048, 512, ta, tb, alpha=0.75, beta=-1.25, dist="normal",
                  seed=60 + 2 * (ta == "T") + (tb == "T"))
    A, B, C = wl.make_inputs(w)
    out, _ = run_fg(w, A, B, C, config=config_id(HEADLINE))
    check_full(w, A, B, C, out)


# --- exactness on integer-valued inputs: catches layout/predication bugs ---

@pytest.mark.parametrize("cfg", all_ids())
@pytest.mark.parametrize("ta,tb", OPS)
def test_integer_bit_exact_every_config(cfg, ta, tb):
    rng_shapes = [(97, 131, 45), (256, 128, 32), (33, 257, 17), (1, 1, 1), (300, 5, 70)]
    for (M, N, K) in rng_shapes:
        for alpha, beta in [(1.0, 0.0), (-1.0, 2.0), (0.5, -1.0)]:
            w = wl.custom(M, N, K, ta, tb, alpha, beta, dist="int8", seed=M + N + K)
            A, B, C = wl.make_inputs(w)
            out, _ = run_fg(w, A, B, C, config=cfg)
            cref, _ = oracle.gemm(ta, tb, M, N, K, alpha, A, w.LDA, B, w.LDB, beta, C, w.LDC)
            bad = np.argwhere(out.astype(np.float64) != cref)
            assert bad.size == 0, (cfg, ta, tb, M, N, K, alpha, beta, bad[:5].tolist(),
                                   [(out[i, j], cref[i, j]) for i, j in bad[:3]])


@pytest.mark.parametrize("cfg", mfma_ids())
def test_identity_and_one_hot_layout(cfg):
    """A = I gives C = B exactly and B = I gives C = A exactly: any mix-up of
    rows, columns or k inside the kernel shows as a misplaced value."""
    rng = np.random.default_rng(1)
    for ta, tb in OPS:
        n = 160
        B = rng.standard_normal((n, 96)).astype(np.float32)
        w = wl.custom(n, 96, n, ta, tb)
        I = np.eye(n, dtype=np.float32)
        Bs = B.T.copy() if tb == "T" else B
        out, _ = run_fg(w, I, Bs, config=cfg)
        assert np.array_equal(out, B), (cfg, ta, tb)
        A = rng.standard_normal((96, n)).astype(np.float32)
        w2 = wl.custom(96, n, n, ta, tb)
        As = A.T.copy() if ta == "T" else A
        out, _ = run_fg(w2, As, I, config=cfg)
        assert np.array_equal(out, A), (cfg, ta, tb)


# --- ragged shapes, odd leading dimensions, misaligned bases ---------------

RAGGED = [(1, 1, 1), (7, 5, 3), (33, 65, 17), (129, 257, 31), (255, 129, 16),
          (300, 200, 100), (513, 97, 1025)]


@pytest.mark.parametrize("cfg", all_ids())
@pytest.mark.parametrize("ta,tb", OPS)
def test_ragged_float_every_config(cfg, ta, tb):
    for i, (M, N, K) in enumerate(RAGGED):
        w = wl.custom(M, N, K, ta, tb, alpha=1.25, beta=-0.5, dist="normal", seed=i)
        A, B, C = wl.make_inputs(w)
        out, _ = run_fg(w, A, B, C, config=cfg)
        check_full(w, A, B, C, out)


def _pad4(n):
    return (n + 3) // 4 * 4


@pytest.mark.parametrize("cfg", all_ids())
@pytest.mark.parametrize("ta,tb", OPS)
def test_ragged_aligned_rows_every_config(cfg, ta, tb):
    """Ragged M, N and K with 16-byte aligned rows (leading dimensions padded
    to a multiple of 4, padding filled with NaN): the direct-to-LDS kernels
    take these, including tiles that cross M or N and a partial last
    k-tile. NaN padding must not reach C."""
    for i, (M, N, K) in enumerate([(97, 131, 45), (300, 257, 100), (513, 190, 1025),
                                   (256, 256, 17), (31, 500, 3), (640, 384, 64)]):
        w0 = wl.custom(M, N, K, ta, tb)
        w = wl.custom(M, N, K, ta, tb, alpha=-0.75, beta=0.25, dist="normal", seed=40 + i,
                      lda=_pad4(w0.LDA), ldb=_pad4(w0.LDB), ldc=_pad4(w0.LDC))
        A, B, C = wl.make_inputs(w)
        A[:, w0.LDA:] = np.nan
        B[:, w0.LDB:] = np.nan
        C[:, N:] = 4321.0
        out, full = run_fg(w, A, B, C, config=cfg)
        check_full(w, A, B, C, out)
        assert np.all(full[:, N:] == 4321.0)


@pytest.mark.parametrize("ta,tb", OPS)
def test_padded_and_misaligned(ta, tb):
    """Leading dimensions larger than the rows (odd and multiple-of-4) and
    base pointers 1 float off 16-byte alignment; the padding of C is a guard
    band that must stay untouched."""
    for (M, N, K, pad, off) in [(130, 70, 50, 3, (1, 2, 3)), (128, 128, 64, 4, (0, 0, 0)),
                                (64, 256, 33, 5, (3, 0, 1))]:
        w0 = wl.custom(M, N, K, ta, tb)
        w = wl.custom(M, N, K, ta, tb, alpha=0.75, beta=1.5, dist="normal", seed=M,
                      lda=w0.LDA + pad, ldb=w0.LDB + pad, ldc=w0.LDC + pad)
        A, B, C = wl.make_inputs(w)
        C[:, N:] = 12345.0  # guard band
        out, full = run_fg(w, A, B, C, offsets=off)
        check_full(w, A, B, C, out)
        assert np.all(full[:, N:] == 12345.0), "C padding was written"


@pytest.mark.parametrize("cfg", mfma_ids())
@pytest.mark.parametrize("ta,tb", OPS)
def test_unaligned_c_rows_every_config(cfg, ta, tb):
    """Rows of C that are not 16-byte aligned (odd ldc, or the base 1-3 floats
    off alignment): the matrix-core entries then stage each chunk of the
    result through LDS so that a store covers consecutive elements of a row.
    Ragged M and N; the padding of C is a guard band that must stay
    untouched; with beta = 0 the old C (NaN) must not be read."""
    for i, (M, N, K, pad, coff) in enumerate([(97, 131, 45, 2, 0), (300, 257, 100, 4, 1),
                                              (129, 64, 33, 1, 3), (513, 190, 1025, 5, 2)]):
        for beta in (0.0, 0.5):
            w = wl.custom(M, N, K, ta, tb, alpha=1.5, beta=beta, dist="normal", seed=70 + i,
                          ldc=N + pad)
            A, B, C = wl.make_inputs(w)
            if C is None:
                C = np.full((M, w.LDC), np.nan, dtype=np.float32)
            C[:, N:] = 2468.0
            out, full = run_fg(w, A, B, C, config=cfg, offsets=(0, 0, coff))
            check_full(w, A, B, C, out)
            assert np.all(full[:, N:] == 2468.0), (cfg, ta, tb, M, N, K, beta)


@pytest.mark.parametrize("ta,tb", OPS)
def test_raster_bands_give_identical_results(ta, tb):
    """The tile order (band height, XCD renumbering) never changes a result:
    every tile is computed once with the same sums. 256 x 256 tiles on an
    11 x 7 grid (partial last bands for every band height tried) and on a
    grid that is a multiple of 8 (where the renumbering applies); C starts as
    NaN, so a tile left out shows."""
    import torch
    for (M, N, K) in [(2700, 1700, 96), (2048, 1024, 64)]:
        w = wl.custom(M, N, K, ta, tb, dist="int8", seed=M + K)
        A, B, C = wl.make_inputs(w)
        outs = {}
        try:
            for g, x in [(1, 0), (0, 1), (0, 0), (3, 1), (8, 1), (16, 0)]:
                assert fg.fg_set_raster(g, x) == fg.FG_OK
                outs[(g, x)], _ = run_fg(w, A, B, config=config_id(HEADLINE))
        finally:
            fg.fg_set_raster(0, 1)
        ref = outs[(1, 0)]
        cref, _ = oracle.gemm(ta, tb, M, N, K, 1.0, A, w.LDA, B, w.LDB, 0.0, None, w.LDC)
        assert np.array_equal(ref.astype(np.float64), cref), (ta, tb, M, N, K)
        for key, out in outs.items():
            assert np.array_equal(out, ref), (ta, tb, M, N, K, key)


def test_guard_rows_outside_c():
    """Nothing is written past the last row of C (the buffer continues)."""
    import torch
    M, N, K = 100, 96, 40
    w = wl.custom(M, N, K, dist="normal", seed=3)
    A, B, _ = wl.make_inputs(w)
    dA = torch.from_numpy(A).cuda()
    dB = torch.from_numpy(B).cuda()
    buf = torch.full((M + 8, N), 777.0, device="cuda")
    st = fg.fg_sgemm("N", "N", M, N, K, 1.0, dA.data_ptr(), K, dB.data_ptr(), N, 0.0,
                     buf.data_ptr(), N, 0)
    assert st == 0
    torch.cuda.synchronize()
    assert torch.all(buf[M:] == 777.0)


# --- semantics --------------------------------------------------------------

def test_beta_zero_ignores_nan_in_c():
    w = wl.custom(200, 300, 64, alpha=2.0, beta=0.0, seed=4)
    A, B, _ = wl.make_inputs(w)
    C = np.full((w.M, w.LDC), np.nan, dtype=np.float32)
    out, _ = run_fg(w, A, B, C)
    assert np.all(np.isfinite(out))
    check_full(w, A, B, None, out)


def test_nan_in_a_row_propagates():
    w = wl.custom(64, 64, 64, seed=5)
    A, B, _ = wl.make_inputs(w)
    A[7, 3] = np.nan
    out, _ = run_fg(w, A, B)
    assert np.all(np.isnan(out[7])) and np.all(np.isfinite(np.delete(out, 7, axis=0)))


@pytest.mark.parametrize("alpha,beta,K", [(0.0, 0.5, 32), (1.0, -2.0, 0), (0.0, 0.0, 16),
                                          (1.0, 0.0, 0), (0.0, 1.0, 8)])
def test_scale_only_paths(alpha, beta, K):
    """K == 0 or alpha == 0: C = beta*C, A and B never read (NaN there is fine)."""
    M, N = 50, 70
    w = wl.custom(M, N, K, alpha=alpha, beta=beta, dist="normal", seed=6)
    A = np.full((M, max(K, 1)), np.nan, dtype=np.float32)
    B = np.full((max(K, 1), N), np.nan, dtype=np.float32)
    C = np.random.default_rng(0).standard_normal((M, N)).astype(np.float32)
    out, _ = run_fg(w, A, B, C.copy())
    want = C if beta == 1.0 else (np.zeros_like(C) if beta == 0 else (beta * C.astype(np.float64)).astype(np.float32))
    assert np.array_equal(out, want)


def test_repeat_runs_bit_identical():
    w = wl.WORKLOADS["C2"]
    A, B, _ = wl.make_inputs(w)
    o1, _ = run_fg(w, A, B)
    o2, _ = run_fg(w, A, B)
    assert np.array_equal(o1, o2)


def test_runs_on_caller_stream():
    import torch
    s = torch.cuda.Stream()
    w = wl.custom(512, 384, 256, dist="normal", seed=8)
    A, B, _ = wl.make_inputs(w)
    with torch.cuda.stream(s):
        out, _ = run_fg(w, A, B, stream=s)
    check_full(w, A, B, None, out)


def test_torch_convenience_wrapper():
    import torch
    g = torch.Generator().manual_seed(0)
    A = torch.randn(300, 200, generator=g)
    B = torch.randn(200, 100, generator=g)
    C = torch.zeros(300, 100, device="cuda")
    fg.sgemm(A.cuda(), B.cuda(), C)
    torch.cuda.synchronize()
    cref, s = oracle.gemm("N", "N", 300, 100, 200, 1.0, A.numpy(), 200, B.numpy(), 100, 0.0)
    ok, info = oracle.compare.check(C.cpu().numpy(), cref, s, 200)
    assert ok, info
    # a transposed view goes through transA = T on the same storage
    At = A.t().contiguous().cuda()  # 200 x 300 storage of A^T
    C2 = torch.zeros(300, 100, device="cuda")
    fg.sgemm(At, B.cuda(), C2, transA="T")
    torch.cuda.synchronize()
    ok, info = oracle.compare.check(C2.cpu().numpy(), cref, s, 200)
    assert ok, info
    with pytest.raises(fg.FgError):
        fg.sgemm(A.cuda(), B.cuda(), C, config=1000)


def test_error_statistics_are_fp32_scale():
    """For uniform[-1,1) inputs the relative Frobenius error should be at
    binary32 rounding scale (~sqrt(K)*2^-24), far inside 1e-5; a precision
    downcast anywhere would show up as ~1e-3."""
    w = wl.custom(1024, 1024, 2048, seed=9)
    A, B, _ = wl.make_inputs(w)
    out, _ = run_fg(w, A, B)
    info = check_full(w, A, B, None, out)
    assert info["frob_rel"] < 2e-6, info


@pytest.mark.parametrize("cfg", all_ids())
def test_every_config_at_4096_cubed(cfg):
    """Every table entry, forced, on the 4096^3 workload, every element
    against the oracle: the comparison paths compute the whole product too."""
    w = wl.WORKLOADS["C6"]
    A, B, C = wl.make_inputs(w)
    out, _ = run_fg(w, A, B, C, config=cfg)
    assert np.all(np.isfinite(out))
    check_full_blocked(w, A, B, C, out, name=f"C6 cfg={cfg}")
