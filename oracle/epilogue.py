"""CPU oracle for the fused epilogue:

    D = act( alpha * r_i * c_j * (op(A) op(B))_ij + beta * C_ij + u_i + w_j )

TEST INFRASTRUCTURE (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and the CPU leg of ``bench.py`` use it.

Passage followed: "Optimising fp32 GEMM on A100", section "Performance
comparison", notes that in practice the operations before and after a GEMM
are fused into it as a prologue and an epilogue. The page names no
particular operations; the reading taken here is the plainest common one:
per-row and per-column scale factors r (length M) and c (length N) on the
product, the usual beta * C term, per-row and per-column biases u (length M)
and w (length N), then an elementwise activation. A missing vector means
ones (scales) or zeros (biases).

Activations, by their textbook definitions (no page defines them):
    none : x
    relu : max(x, 0)
    gelu : x * Phi(x) = x * (1 + erf(x / sqrt(2))) / 2   (the exact, erf form)
    silu : x * sigma(x) = x / (1 + exp(-x))

Everything here is binary64: the plain product s = op(A) op(B) comes from the
C oracle (``oracle.gemm`` with alpha = 1, beta = 0, ascending k), and the
epilogue is evaluated elementwise after it, in the order written above.
Pins: ``tests/test_oracle_epilogue.py``.
"""
from __future__ import annotations

import math

import numpy as np

ACTIVATIONS = ("none", "relu", "gelu", "silu")
# Largest slope of each activation (for the tolerance): relu 1,
# gelu Phi(x) + x phi(x) peaks at 1.1289 near x = 1.414, silu at 1.0998.
LIPSCHITZ = {"none": 1.0, "relu": 1.0, "gelu": 1.129, "silu": 1.1}


def _erf(x):
    try:
        from scipy.special import erf
        return erf(x)
    except ImportError:  # pragma: no cover - scipy is present in this image
        return np.vectorize(math.erf, otypes=[np.float64])(x)


def activation(x, kind):
    """Elementwise activation in binary64."""
    x = np.asarray(x, dtype=np.float64)
    if kind == "none":
        return x.copy()
    if kind == "relu":
        return np.maximum(x, 0.0)
    if kind == "gelu":
        return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))
    if kind == "silu":
        with np.errstate(over="ignore"):
            return x / (1.0 + np.exp(-x))
    raise ValueError(f"unknown activation {kind!r}")


def _vec(v, n, fill):
    if v is None:
        return np.full(n, fill, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64).ravel()
    if v.size != n:
        raise ValueError(f"vector of length {v.size}, expected {n}")
    return v


def pre_activation(s, alpha, beta, cin, row_scale=None, col_scale=None, row_bias=None,
                   col_bias=None):
    """v = alpha * r_i * c_j * s_ij + beta * C_ij + u_i + w_j (binary64).
    s is the plain product (M x N); cin is read only when beta != 0."""
    s = np.asarray(s, dtype=np.float64)
    M, N = s.shape
    r = _vec(row_scale, M, 1.0)
    c = _vec(col_scale, N, 1.0)
    u = _vec(row_bias, M, 0.0)
    w = _vec(col_bias, N, 0.0)
    v = float(alpha) * r[:, None] * c[None, :] * s
    if beta != 0:
        v = v + float(beta) * np.asarray(cin, dtype=np.float64)
    return v + u[:, None] + w[None, :]


def epilogue(s, alpha, beta, cin, row_scale=None, col_scale=None, row_bias=None,
             col_bias=None, act="none"):
    """D = act(pre_activation(...)) in binary64; returns (D, v)."""
    v = pre_activation(s, alpha, beta, cin, row_scale, col_scale, row_bias, col_bias)
    return activation(v, act), v


def epilogue_elems(s, alpha, beta, cin, ii, jj, row_scale=None, col_scale=None,
                   row_bias=None, col_bias=None, act="none"):
    """The same definition at a list of elements (ii[t], jj[t]): s and cin
    hold the plain product and the old C at those elements. Returns (D, v)
    of shape (len(ii),)."""
    s = np.asarray(s, dtype=np.float64)
    ii = np.asarray(ii)
    jj = np.asarray(jj)
    r = np.ones(s.shape) if row_scale is None else np.asarray(row_scale, np.float64)[ii]
    c = np.ones(s.shape) if col_scale is None else np.asarray(col_scale, np.float64)[jj]
    u = np.zeros(s.shape) if row_bias is None else np.asarray(row_bias, np.float64)[ii]
    w = np.zeros(s.shape) if col_bias is None else np.asarray(col_bias, np.float64)[jj]
    v = float(alpha) * r * c * s
    if beta != 0:
        v = v + float(beta) * np.asarray(cin, dtype=np.float64)
    v = v + u + w
    return activation(v, act), v
