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


def epilogue_tol(K, alpha, beta, sabs, cin, v_ref, row_scale=None, col_scale=None,
                 row_bias=None, col_bias=None, act="none", per_element=False):
    """Per-element bound for the fused epilogue
    D = act(alpha * r_i * c_j * s_ij + beta * C_ij + u_i + w_j).

    The pre-activation value v carries the GEMM bound with every term of the
    sum in place of |alpha| * S and |beta| * |C_in| (each extra binary32
    rounding of the scale product and of the two bias additions is covered
    by the 8 * max(K, 1) factor, as the alpha/beta roundings are):

        tol_v = 8 * max(K, 1) * 2^-24 * (|alpha r_i c_j| S + |beta C_ij| + |u_i| + |w_j|) + 1e-6

    The activation stretches that by at most its largest slope (1 for relu,
    1.129 for gelu, 1.1 for silu) and its own binary32 evaluation adds at most
    2^-20 * |v|: a gelu whose erf is within 4e-7 of the true one (such as
    formula 7.1.26 of Abramowitz and Stegun, error 1.5e-7, evaluated in
    binary32) is off by at most 2e-7 |v|, and exp, reciprocal and the
    products around them add a few units in the last place. per_element: the four vectors are given already gathered
    at the checked elements (arrays of the shape of sabs) instead of as
    length-M / length-N vectors."""
    from .epilogue import LIPSCHITZ
    sabs = np.asarray(sabs, dtype=np.float64)
    if per_element:
        # vectors already gathered at the checked elements (shape of sabs)
        def row(v, fill):
            return fill if v is None else np.asarray(v, np.float64)
        col = row
    else:
        def row(v, fill):
            return fill if v is None else np.asarray(v, np.float64).ravel()[:, None]

        def col(v, fill):
            return fill if v is None else np.asarray(v, np.float64).ravel()[None, :]
    t = np.abs(float(alpha) * row(row_scale, 1.0) * col(col_scale, 1.0)) * sabs
    if beta != 0 and cin is not None:
        t = t + abs(float(beta)) * np.abs(np.asarray(cin, dtype=np.float64))
    t = t + np.abs(row(row_bias, 0.0)) + np.abs(col(col_bias, 0.0))
    tol_v = 8.0 * max(int(K), 1) * U32 * t + ABS_FLOOR
    if act == "none":
        return tol_v
    return LIPSCHITZ[act] * tol_v + 2.0 ** -20 * np.abs(np.asarray(v_ref, dtype=np.float64))


def check_epilogue(d_gpu, d_ref, v_ref, sabs, K, alpha, beta, cin=None, row_scale=None,
                   col_scale=None, row_bias=None, col_bias=None, act="none", frob=True,
                   per_element=False):
    """(ok, info) for a fused-epilogue result, as check() for the plain GEMM:
    every element within epilogue_tol and the relative Frobenius error of the
    whole result at most 1e-5."""
    d_gpu = np.asarray(d_gpu, dtype=np.float64)
    d_ref = np.asarray(d_ref, dtype=np.float64)
    if d_gpu.shape != d_ref.shape:
        raise ValueError(f"shape mismatch {d_gpu.shape} vs {d_ref.shape}")
    info = {"n": int(d_ref.size)}
    if d_ref.size == 0:
        return True, info
    tol = epilogue_tol(K, alpha, beta, sabs, cin, v_ref, row_scale, col_scale, row_bias,
                       col_bias, act, per_element)
    err = np.abs(d_gpu - d_ref)
    finite = np.isfinite(d_gpu)
    ratio = np.where(finite, err / tol, np.inf)
    worst = int(np.argmax(ratio))
    info["max_err_over_tol"] = float(ratio.flat[worst])
    info["worst_index"] = tuple(int(v) for v in np.unravel_index(worst, d_ref.shape))
    info["n_bad"] = int((~(finite & (err <= tol))).sum())
    ok = info["n_bad"] == 0
    if frob:
        dn = float(np.linalg.norm(np.where(finite, d_gpu - d_ref, np.inf)))
        rn = float(np.linalg.norm(d_ref))
        info["frob_rel"] = dn / rn if rn > 0 else dn
        ok = ok and (dn <= FROB_REL * rn if rn > 0 else dn <= ABS_FLOOR * np.sqrt(d_ref.size))
    return ok, info
