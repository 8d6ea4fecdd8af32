"""The machine probes of fp32gemm_probe.h on the GPU: the MFMA-only loop
must produce the closed-form result of its fixed operands (which also pins
the lane layout of v_mfma_f32_32x32x2_f32 that the GEMM kernels rely on),
and the streaming read must sum exactly what it read."""
import numpy as np
import pytest

import fp32_gemm_tile_amd as fg
from gpu_util import log

pytestmark = pytest.mark.gpu


def _mfma_probe_expected(iters):
    """Per-lane value of the probe: lane l supplies A[l % 32][l // 32] = a(l)
    and B[l // 32][l % 32] = b(l) of one 32x32x2 product; accumulator
    register r of lane l holds C[8 (r // 4) + 4 (l // 32) + r % 4][l % 32].
    Four chains of `iters` products each, summed over the 16 registers."""
    lanes = np.arange(64, dtype=np.float64)
    a = 0.25 + lanes / 512.0
    b = 0.75 - lanes / 512.0
    A = np.stack([a[:32], a[32:]], axis=1)    # 32 x 2
    B = np.stack([b[:32], b[32:]], axis=0)    # 2 x 32
    C = A @ B
    out = np.empty(64)
    for l in range(64):
        i, h = l % 32, l // 32
        rows = [8 * (r // 4) + 4 * h + r % 4 for r in range(16)]
        out[l] = 4 * iters * C[rows, i].sum()
    return out


def test_mfma_probe_closed_form():
    import torch
    wgs, iters = 8, 5
    log(f"mfma probe wgs={wgs} iters={iters}")
    out = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device="cuda")
    assert fg.fg_probe_mfma(wgs, iters, out.data_ptr()) == fg.FG_OK
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64).reshape(wgs * 4, 64)
    want = _mfma_probe_expected(iters)
    np.testing.assert_allclose(got, np.broadcast_to(want, got.shape), rtol=1e-5)


def test_read_probe_sums_what_it_reads():
    import torch
    for n, wgs in ((1 << 20, 64), (4 * 12345, 7), (4, 3), (0, 5)):
        log(f"read probe n={n} wgs={wgs}")
        x = torch.ones(max(n, 4), dtype=torch.float32, device="cuda")
        out = torch.full((wgs * 4,), float("nan"), dtype=torch.float32, device="cuda")
        assert fg.fg_probe_read(x.data_ptr(), n, wgs, out.data_ptr()) == fg.FG_OK
        torch.cuda.synchronize()
        parts = out.cpu().numpy()
        assert np.all(np.isfinite(parts))
        assert parts.astype(np.float64).sum() == n  # integer partial sums are exact


@pytest.mark.parametrize("nbytes", [4, 16])
def test_lds_dma_lane_layout(nbytes):
    """A direct-to-LDS buffer load writes lane L's W = bytes / 4 floats to LDS
    floats W L .. W L + W - 1 of its base: the layout the GEMM's loader
    assigns its global addresses by. Lanes read src reversed, so
    out[W L + e] = src[(63 - L) W + e]; any other placement, or an LDS slot
    left unwritten (prefilled -1), fails."""
    import torch
    W = nbytes // 4
    log(f"lds dma probe bytes={nbytes}")
    src = torch.arange(64 * W, dtype=torch.float32, device="cuda") + 1000.0
    out = torch.full((64 * W,), float("nan"), dtype=torch.float32, device="cuda")
    assert fg.fg_probe_lds_dma(src.data_ptr(), nbytes, out.data_ptr()) == fg.FG_OK
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(64, W)
    want = (src.cpu().numpy().reshape(64, W))[::-1]
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]
