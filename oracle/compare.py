"""Acceptance check of a binary32 GEMM result against the oracle.

TEST INFRASTRUCTURE (see the package docstring).

Bound per element, for a result computed in binary32 with any summation order
and with or without fused multiply-add:

    |C - C_ref| <= 8 * max(K, 1) * 2^-24 * (|alpha| * S + |beta| * |C_in|) + 1e-6

where S = sum_k |a_ik b_kj|. With alpha = 1 and beta = 0 this is exactly the
stated acceptance bound 8*K*2^-24*S + 1e-6; the |beta|*|C_in| term covers the
rounding of the beta*C_in product and of the final sum (a reading of the
bound for the alpha/beta epilogue, which the pages leave open).

Plus a global bound: ||C - C_ref||_F / ||C_ref||_F <= 1e-5.
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24
ABS_FLOOR = 1e-6
FROB_REL = 1e-5


def elementwise_tol(K, alpha, beta, sabs, cin=None):
    t = abs(float(alpha)) * np.asarray(sabs, dtype=np.float64)
    if beta != 0 and cin is not None:
        t = t + abs(float(beta)) * np.abs(np.asarray(cin, dtype=np.float64))
    return 8.0 * max(int(K), 1) * U32 * t + ABS_FLOOR


def check(c_gpu, c_ref, sabs, K, alpha=1.0, beta=0.0, cin=None, frob=True):
    """Return (ok, info) where info holds the worst element and the norms.

    c_gpu, c_ref, sabs (and cin if beta != 0) must have the same shape.
    """
    c_gpu = np.asarray(c_gpu, dtype=np.float64)
    c_ref = np.asarray(c_ref, dtype=np.float64)
    if c_gpu.shape != c_ref.shape:
        raise ValueError(f"shape mismatch {c_gpu.shape} vs {c_ref.shape}")
    info = {"n": int(c_ref.size)}
    if c_ref.size == 0:
        info.update(ok_elem=True, ok_frob=True)
        return True, info
    tol = elementwise_tol(K, alpha, beta, sabs, cin)
    err = np.abs(c_gpu - c_ref)
    finite = np.isfinite(c_gpu)
    bad = ~(finite & (err <= tol))
    ratio = np.where(finite, err / tol, np.inf)
    worst = int(np.argmax(ratio))
    info["max_err_over_tol"] = float(ratio.flat[worst])
    info["worst_index"] = tuple(int(v) for v in np.unravel_index(worst, c_ref.shape))
    info["n_bad"] = int(bad.sum())
    ok_elem = info["n_bad"] == 0
    ok_frob = True
    if frob:
        dn = float(np.linalg.norm(np.where(finite, c_gpu - c_ref, np.inf)))
        rn = float(np.linalg.norm(c_ref))
        info["frob_abs"] = dn
        info["frob_ref"] = rn
        if rn > 0:
            info["frob_rel"] = dn / rn
            ok_frob = dn / rn <= FROB_REL
        else:
            ok_frob = dn <= ABS_FLOOR * np.sqrt(c_ref.size)
    info["ok_elem"] = ok_elem
    info["ok_frob"] = ok_frob
    return ok_elem and ok_frob, info
