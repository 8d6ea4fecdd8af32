"""fg_sgemm_splitk_noalloc: split-K with the library's device-resident
scratch, for callers that cannot allocate. Its results must equal those of
fg_sgemm_splitk (caller workspace) with the same split count, bit for bit,
and pass the oracle's bound; two calls in a row share the one scratch array,
the second with a smaller problem."""
import numpy as np
import pytest

import fp32_gemm_tile_amd as fg
from fp32_gemm_tile_amd import workloads as wl

from gpu_util import check_full, log, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fg.load_library()
    yield
    torch.cuda.synchronize()


def _call(w, A, B, C, splits, noalloc):
    """One call on host arrays; returns the M x N result."""
    import torch
    dA, _a = to_device(A)
    dB, _b = to_device(B)
    Cbuf = C if C is not None else np.full((w.M, w.LDC), np.nan, dtype=np.float32)
    dC, _c = to_device(Cbuf)
    s = torch.cuda.current_stream()
    args = (w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.LDA, dB.data_ptr(),
            w.LDB, w.beta, dC.data_ptr(), w.LDC)
    log(f"  {'noalloc' if noalloc else 'workspace'} {w.transA}{w.transB} M={w.M} N={w.N} "
        f"K={w.K} splits={splits}")
    if noalloc:
        st = fg.fg_sgemm_splitk_noalloc(*args, splits, s.cuda_stream)
    else:
        need = max(fg.fg_sgemm_splitk_workspace_size(w.M, w.N, max(splits, 1)), 4)
        if splits == 0:
            need = fg.fg_sgemm_splitk_noalloc_max_bytes()  # the same room to choose in
        ws = torch.empty(need // 4, dtype=torch.float32, device="cuda")
        st = fg.fg_sgemm_splitk(*args, splits, ws.data_ptr(), need, s.cuda_stream)
    assert st == fg.FG_OK, (st, fg.fg_last_error())
    s.synchronize()
    return dC.cpu().numpy().reshape(Cbuf.shape)[:, :w.N].copy()


@pytest.mark.parametrize("splits", [8, 0])
def test_noalloc_equals_workspace_call_twice(splits):
    """A call that fills the whole scratch (1024 x 1024 x 8 slices = 32 MiB
    when 8 are asked for), then a smaller ragged one with alpha and beta:
    each equals the caller-workspace entry point bit for bit and passes the
    oracle bound."""
    cases = [wl.custom(1024, 1024, 4096, seed=91),
             wl.custom(300, 257, 1025, "T", "N", alpha=1.5, beta=0.5, dist="normal", seed=92)]
    for w in cases:
        A, B, C = wl.make_inputs(w)
        sp = splits if splits == 0 or w.M == 1024 else 3
        got = _call(w, A, B, C, sp, noalloc=True)
        want = _call(w, A, B, C, sp, noalloc=False)
        assert np.array_equal(got, want), (w.M, w.N, w.K, sp)
        check_full(w, A, B, C, got)


def test_noalloc_rejects_more_than_the_scratch():
    """M * N * splits floats above the scratch size: an error before any
    device work, naming the limit."""
    cap = fg.fg_sgemm_splitk_noalloc_max_bytes()
    assert cap == 32 << 20
    st = fg.fg_sgemm_splitk_noalloc("N", "N", 1024, 1024, 4096, 1.0, 16, 4096, 16, 1024, 0.0,
                                    16, 1024, 9, 0)
    assert st == fg.FG_ERR_INVALID_ARG and fg.fg_last_bad_arg() == 14
    assert str(cap) in fg.fg_last_error()
