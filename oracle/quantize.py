"""CPU oracle for the quantised second output of a fused GEMM epilogue.

TEST INFRASTRUCTURE (see the package docstring): only ``tests/``,
``__graft_entry__.smoke()`` and the CPU leg of ``bench.py`` use it.

Passage followed: "Optimising fp32 GEMM on A100", section "Performance
comparison", notes that the operations around a GEMM -- quantisation among
them -- are fused into it as a prologue or epilogue. The page names no
format. Reading taken here: besides the binary32 result C, the epilogue can
write a narrower copy Q of it, element by element, into a second buffer
owned by the caller, in one of two plain formats:

  bf16      Q_ij = the bfloat16 nearest to C_ij (8 significant bits, the
            binary32 exponent range), ties to even. Values that round past
            the largest bfloat16 become infinities; infinities stay; every
            NaN becomes the quiet NaN 0x7FC0.
  int8_row  Q_ij = clamp(round_half_even(fl32(C_ij * s_i)), -128, 127) with
            s_i the caller's binary32 factor of row i (e.g. 127 / max|row|);
            fl32 is the product rounded to binary32 (the quantised code is
            decided on that binary32 value, the precision of the kernel); a
            NaN gives 0, infinities saturate.

Q depends on C only, so the oracle takes C as given (binary32) and the
parity tests apply it to the GPU's own C (whose accuracy the GEMM oracle
checks separately): the codes must then agree bit for bit.

Everything here is exact: binary32 values and their products are exact in
binary64, and rounding to a grid of 2^e is done with numpy's rint (ties to
even) on exactly scaled binary64 values. Pins: ``tests/test_oracle_quantize.py``.
"""
from __future__ import annotations

import numpy as np

BF16_QNAN = 0x7FC0
BF16_MIN_SUBNORMAL_EXP = -133   # spacing of bfloat16 subnormals: 2^-133
BF16_OVERFLOW = 2.0 ** 128      # smallest magnitude that is no longer finite


def bf16_rne(c):
    """uint16 codes of the bfloat16 values nearest to binary32 `c` (ties to
    even), computed from the value: the quantum at |c| is 2^(e - 7) for
    |c| in [2^e, 2^(e+1)) (8 significant bits), at least 2^-133."""
    with np.errstate(invalid="ignore"):  # signalling NaNs convert quietly
        x = np.asarray(c, dtype=np.float32).astype(np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    nan = np.isnan(x)
    fin = np.isfinite(x)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.floor(np.log2(np.abs(np.where(fin & (x != 0), x, 1.0))))
    # log2 of a binary32 value is exact enough to floor correctly except
    # within rounding of a power of two; fix e so that 2^e <= |x| < 2^(e+1)
    ax = np.abs(np.where(fin, x, 0.0))
    e = np.where(ax >= 2.0 ** (e + 1), e + 1, e)
    e = np.where((ax > 0) & (ax < 2.0 ** e), e - 1, e)
    quantum = np.exp2(np.maximum(e - 7, BF16_MIN_SUBNORMAL_EXP))
    r = np.rint(np.where(fin, x, 0.0) / quantum) * quantum   # exact, ties to even
    overflow = fin & (np.abs(r) >= BF16_OVERFLOW)
    r = np.where(overflow, np.copysign(np.inf, x), r)
    r = np.where(fin, r, np.where(nan, 0.0, x))              # infinities stay
    # the rounded value is a bfloat16: its binary32 pattern ends in 16 zeros
    bits = r.astype(np.float32).view(np.uint32)
    # keep the sign of values that round to zero
    bits = np.where((r == 0) & np.signbit(x), np.uint32(0x80000000), bits)
    out[...] = (bits >> 16).astype(np.uint16)
    out[nan] = BF16_QNAN
    return out


def bf16_value(q):
    """binary32 values of uint16 bfloat16 codes (for reading results)."""
    q = np.asarray(q, dtype=np.uint16).astype(np.uint32) << 16
    return q.view(np.float32)


def int8_row(c, row_factor):
    """int8 codes clamp(rint(fl32(c_ij * s_i)), -128, 127); NaN -> 0."""
    c = np.asarray(c, dtype=np.float32)
    s = np.asarray(row_factor, dtype=np.float32).reshape(-1, *([1] * (c.ndim - 1)))
    with np.errstate(over="ignore", invalid="ignore"):
        prod = (c.astype(np.float64) * s.astype(np.float64)).astype(np.float32)  # fl32
        r = np.rint(prod.astype(np.float64))
        r = np.clip(np.where(np.isnan(r), 0.0, r), -128.0, 127.0)
    return r.astype(np.int8)


def quantize(c, kind, row_factor=None):
    """Q of binary32 C (2-D) in format `kind` ("bf16" or "int8_row")."""
    if kind == "bf16":
        return bf16_rne(c)
    if kind == "int8_row":
        if row_factor is None:
            raise ValueError("int8_row needs a factor per row")
        return int8_row(c, row_factor)
    raise ValueError(f"unknown quantised format {kind!r}")
