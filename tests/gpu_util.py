"""Helpers for the GPU tests: put seeded host arrays on the device, call the
library through its C ABI, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import fp32_gemm_tile_amd as fg
from fp32_gemm_tile_amd import workloads
import oracle
from oracle import compare


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(x, pad_floats=0):
    """Host float32 array -> flat device tensor (optionally offset by
    pad_floats elements inside a larger buffer, to test misaligned bases).
    Returns (tensor_view, base_tensor)."""
    import torch
    flat = np.ascontiguousarray(x, dtype=np.float32).ravel()
    base = torch.empty(flat.size + pad_floats + 1, dtype=torch.float32, device="cuda")
    base.fill_(float("nan"))
    view = base[pad_floats:pad_floats + flat.size]
    view.copy_(torch.from_numpy(flat))
    return view, base


def run_fg(w, A, B, C=None, config=-1, offsets=(0, 0, 0), c_fill=None, stream=None):
    """Run workload ``w`` (a workloads.Workload) on host arrays A, B (and C_in)
    through fg_sgemm_ex. Returns the M x N result (host float32) and the full
    C buffer as read back (for guard-band checks)."""
    import torch
    dA, _ba = to_device(A, offsets[0])
    dB, _bb = to_device(B, offsets[1])
    if C is None:
        C = np.full((w.M, w.LDC), np.nan if c_fill is None else c_fill, dtype=np.float32)
    dC, _bc = to_device(C, offsets[2])
    s = torch.cuda.current_stream() if stream is None else stream
    log(f"  fg_sgemm_ex {w.transA}{w.transB} M={w.M} N={w.N} K={w.K} lda={w.LDA} "
        f"ldb={w.LDB} ldc={w.LDC} alpha={w.alpha} beta={w.beta} cfg={config} off={offsets}")
    st = fg.fg_sgemm_ex(w.transA, w.transB, w.M, w.N, w.K, w.alpha, dA.data_ptr(), w.LDA,
                        dB.data_ptr(), w.LDB, w.beta, dC.data_ptr(), w.LDC,
                        s.cuda_stream, config)
    if st != fg.FG_OK:
        raise fg.FgError(st, fg.fg_last_bad_arg(), fg.fg_last_error())
    s.synchronize()
    full = dC.cpu().numpy().reshape(C.shape)
    return full[:, :w.N].copy(), full


def oracle_full(w, A, B, C):
    return oracle.gemm(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A, w.LDA, B, w.LDB,
                       w.beta, C, w.LDC)


def check_full(w, A, B, C, out):
    cref, s = oracle_full(w, A, B, C)
    cin = C[:, :w.N] if (C is not None and w.beta != 0) else None
    ok, info = compare.check(out, cref, s, w.K, w.alpha, w.beta, cin)
    assert ok, (w, info)
    return info


def row_blocks(M, block):
    for r0 in range(0, M, block):
        yield np.arange(r0, min(M, r0 + block), dtype=np.int64)


class FullCheck:
    """Every element of a large result against the oracle, one block of rows
    at a time (host memory stays bounded): the per-element bound on each
    block, the relative Frobenius bound on the whole result."""

    def __init__(self, name):
        self.name = name
        self.n = self.n_bad = 0
        self.worst = 0.0
        self.worst_at = None
        self.err2 = self.ref2 = 0.0

    def add(self, rows, info):
        self.n += info["n"]
        self.n_bad += info["n_bad"]
        if info["max_err_over_tol"] > self.worst:
            self.worst = info["max_err_over_tol"]
            i, j = info["worst_index"]
            self.worst_at = (int(rows[i]), int(j))
        self.err2 += info["frob_abs"] ** 2
        self.ref2 += info["frob_ref"] ** 2

    def finish(self):
        frob = (self.err2 ** 0.5) / (self.ref2 ** 0.5) if self.ref2 > 0 else self.err2 ** 0.5
        info = {"n": self.n, "n_bad": self.n_bad, "max_err_over_tol": self.worst,
                "worst_index": self.worst_at, "frob_rel": frob}
        log(f"  {self.name}: all {self.n} elements, max err/tol {self.worst:.3g} at "
            f"{self.worst_at}, frob_rel {frob:.3g}, {self.n_bad} outside the bound")
        assert self.n_bad == 0 and frob <= compare.FROB_REL, (self.name, info)
        return info


def check_full_blocked(w, A, B, C, out, block=1024, name=None):
    """check_full for results too large to hold the whole oracle at once."""
    fc = FullCheck(name or getattr(w, "name", "result"))
    for rows in row_blocks(w.M, block):
        cref, s = oracle.gemm_rows(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A, w.LDA, B,
                                   w.LDB, w.beta, C, w.LDC, rows=rows)
        cin = C[rows, :w.N] if (C is not None and w.beta != 0) else None
        _, info = compare.check(out[rows], cref, s, w.K, w.alpha, w.beta, cin, frob=True)
        fc.add(rows, info)
    return fc.finish()


def check_sampled(w, A, B, C, out, n=4000, seed=99, rows=(0, -1)):
    """Oracle at a seeded sample of elements plus a few whole rows."""
    ii, jj = workloads.sample_indices(w.M, w.N, n, seed=seed)
    cref, s = oracle.gemm_elems(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A, w.LDA, B,
                                w.LDB, w.beta, C, w.LDC, ii, jj)
    cin = C[ii, jj] if (C is not None and w.beta != 0) else None
    ok, info = compare.check(out[ii, jj], cref, s, w.K, w.alpha, w.beta, cin, frob=True)
    assert ok, (w.name, "sampled", info)
    rr = [r % w.M for r in rows]
    cref, s = oracle.gemm_rows(w.transA, w.transB, w.M, w.N, w.K, w.alpha, A, w.LDA, B,
                               w.LDB, w.beta, C, w.LDC, rows=rr)
    cin = C[rr, :w.N] if (C is not None and w.beta != 0) else None
    ok, info2 = compare.check(out[rr], cref, s, w.K, w.alpha, w.beta, cin)
    assert ok, (w.name, "rows", info2)
    return info
