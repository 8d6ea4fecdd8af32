"""Pins for the CPU oracle: checks against facts fixed by mathematics, not by
the oracle itself. Each ``pin_*`` takes a ``gemm`` callable with the oracle's
``gemm_rows`` signature and raises AssertionError when it disagrees.

They are shared by ``test_oracle_pins.py`` (the real oracle must pass all of
them) and ``test_oracle_mutants.py`` (every planted mistake must fail one).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

U64 = 2.0 ** -53
OPS = [("N", "N"), ("N", "T"), ("T", "N"), ("T", "T")]


def store(opmat, trans, ld=None, pad_value=0.0):
    """Storage array for a logical op(X) given as rows x cols.

    trans == "T" stores the transpose; ld >= stored row length; padding
    columns hold pad_value (NaN in some pins, to prove they are not read).
    """
    x = np.asarray(opmat, dtype=np.float32)
    s = x.T if trans == "T" else x
    r, c = s.shape
    ld = max(1, c) if ld is None else ld
    out = np.full((max(r, 1), ld), pad_value, dtype=np.float32)
    out[:r, :c] = s
    return out, ld


def run(gemm, ta, tb, opA, opB, alpha=1.0, beta=0.0, Cin=None, pad=0,
        pad_value=0.0):
    opA = np.asarray(opA, dtype=np.float32)
    opB = np.asarray(opB, dtype=np.float32)
    M, K = opA.shape
    N = opB.shape[1]
    A, lda = store(opA, ta, (M if ta == "T" else K) + pad, pad_value)
    B, ldb = store(opB, tb, (K if tb == "T" else N) + pad, pad_value)
    C = None
    ldc = N
    if Cin is not None:
        C, ldc = store(Cin, "N", N + pad, pad_value)
    return gemm(ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc)


# p1: identity. Every sum has a single nonzero term, so the result is exact.
def pin_identity(gemm, rng):
    for ta, tb in OPS:
        for (m, n) in [(7, 5), (16, 33)]:
            B = rng.standard_normal((m, n)).astype(np.float32)
            c, s = run(gemm, ta, tb, np.eye(m, dtype=np.float32), B)
            assert np.array_equal(c, B.astype(np.float64)), ("I*B", ta, tb)
            assert np.array_equal(s, np.abs(B.astype(np.float64))), ("S of I*B", ta, tb)
            A = rng.standard_normal((n, m)).astype(np.float32)
            c, _ = run(gemm, ta, tb, A, np.eye(m, dtype=np.float32))
            assert np.array_equal(c, A.astype(np.float64)), ("A*I", ta, tb)


# p2: all-ones. C_ij = alpha*K + beta*c_ij exactly (integers far below 2^53).
def pin_all_ones(gemm, rng):
    for ta, tb in OPS:
        for (m, n, k) in [(3, 4, 1), (5, 9, 17), (8, 8, 300)]:
            c, s = run(gemm, ta, tb, np.ones((m, k)), np.ones((k, n)))
            assert np.all(c == k) and np.all(s == k), ("ones", ta, tb, m, n, k)
            cin = rng.integers(-5, 6, (m, n)).astype(np.float32)
            c, _ = run(gemm, ta, tb, np.ones((m, k)), np.ones((k, n)),
                       alpha=-2.0, beta=0.5, Cin=cin)
            assert np.array_equal(c, -2.0 * k + 0.5 * cin.astype(np.float64))


# p3: rank-1 (K = 1) and diagonal A: one product per element, exact in binary64.
def pin_rank1_diag(gemm, rng):
    for ta, tb in OPS:
        a = rng.standard_normal((6, 1)).astype(np.float32)
        b = rng.standard_normal((1, 11)).astype(np.float32)
        c, s = run(gemm, ta, tb, a, b)
        ref = a.astype(np.float64) @ b.astype(np.float64)  # one term: exact
        assert np.array_equal(c, ref), ("rank1", ta, tb)
        assert np.array_equal(s, np.abs(ref))
        d = rng.standard_normal(9).astype(np.float32)
        B = rng.standard_normal((9, 4)).astype(np.float32)
        c, _ = run(gemm, ta, tb, np.diag(d), B)
        assert np.array_equal(c, d.astype(np.float64)[:, None] * B.astype(np.float64))


# p4: small integers. Every partial sum is an integer well inside binary64's
# exact range, so the result must equal an integer matrix product.
def pin_integers(gemm, rng):
    for ta, tb in OPS:
        for (m, n, k, pad) in [(1, 1, 1, 0), (13, 7, 29, 3), (31, 17, 65, 1)]:
            A = rng.integers(-8, 9, (m, k))
            B = rng.integers(-8, 9, (k, n))
            Ci = rng.integers(-8, 9, (m, n))
            for alpha, beta in [(1.0, 0.0), (2.0, -1.0), (-0.5, 0.25)]:
                c, _ = run(gemm, ta, tb, A, B, alpha, beta,
                           Ci if beta != 0 else None, pad=pad, pad_value=np.nan)
                exact = A.astype(np.int64) @ B.astype(np.int64)
                want = alpha * exact.astype(np.float64)
                if beta != 0:
                    want = want + beta * Ci.astype(np.float64)
                assert np.array_equal(c, want), ("int", ta, tb, m, n, k, alpha, beta)


# p5: brute force against exact rational arithmetic on tiny shapes.
def pin_bruteforce(gemm, rng, sizes=(1, 2, 3, 5, 8)):
    for ta, tb in OPS:
        for m in sizes:
            for n in sizes:
                for k in sizes:
                    A = rng.standard_normal((m, k)).astype(np.float32)
                    B = rng.standard_normal((k, n)).astype(np.float32)
                    Ci = rng.standard_normal((m, n)).astype(np.float32)
                    alpha, beta = 1.25, -0.75
                    c, s = run(gemm, ta, tb, A, B, alpha, beta, Ci)
                    for i in range(m):
                        for j in range(n):
                            ex = Fraction(0)
                            for kk in range(k):
                                ex += Fraction(float(A[i, kk])) * Fraction(float(B[kk, j]))
                            ex = Fraction(alpha) * ex + Fraction(beta) * Fraction(float(Ci[i, j]))
                            bound = (k + 3) * U64 * (abs(alpha) * s[i, j]
                                                     + abs(beta) * abs(float(Ci[i, j]))) + 1e-300
                            err = abs(Fraction(float(c[i, j])) - ex)
                            assert err <= Fraction(bound), ("brute", ta, tb, m, n, k, i, j)


# p6: library cross-check in binary64 (a different summation, so a bound).
def pin_numpy_f64(gemm, rng):
    for ta, tb in OPS:
        m, n, k = 37, 23, 190
        A = rng.uniform(-1, 1, (m, k)).astype(np.float32)
        B = rng.uniform(-1, 1, (k, n)).astype(np.float32)
        c, s = run(gemm, ta, tb, A, B, pad=2)
        ref = A.astype(np.float64) @ B.astype(np.float64)
        assert np.all(np.abs(c - ref) <= 2 * k * U64 * s + 1e-300), ("np", ta, tb)


# p7: beta == 0 must not read C (NaN in C never reaches the output), and
# padding beyond each row's valid length is never read.
def pin_beta_zero_and_padding(gemm, rng):
    for ta, tb in OPS:
        A = rng.standard_normal((5, 7)).astype(np.float32)
        B = rng.standard_normal((7, 6)).astype(np.float32)
        nan_c = np.full((5, 6), np.nan, dtype=np.float32)
        c0, _ = run(gemm, ta, tb, A, B, 1.5, 0.0, nan_c, pad=3, pad_value=np.nan)
        c1, _ = run(gemm, ta, tb, A, B, 1.5, 0.0, None, pad=0)
        assert np.all(np.isfinite(c0)) and np.array_equal(c0, c1), ("beta0", ta, tb)


# p8: empty sum (K == 0) gives beta*C; alpha == 0 ignores A and B.
def pin_degenerate(gemm, rng):
    Ci = rng.standard_normal((4, 3)).astype(np.float32)
    c, s = gemm("N", "N", 4, 3, 0, 1.0, np.zeros(1, np.float32), 1,
                np.zeros(1, np.float32), 3, 2.0, Ci, 3)
    assert np.array_equal(c, 2.0 * Ci.astype(np.float64)) and np.all(s == 0)
    c, s = gemm("N", "N", 4, 3, 0, 1.0, np.zeros(1, np.float32), 1,
                np.zeros(1, np.float32), 3, 0.0, None, 3)
    assert np.all(c == 0)
    A = rng.standard_normal((4, 5)).astype(np.float32)
    B = rng.standard_normal((5, 3)).astype(np.float32)
    c, _ = run(gemm, "N", "N", A, B, 0.0, -1.0, Ci)
    assert np.array_equal(c, -Ci.astype(np.float64))


# Transposition consistency: a stored transpose read with "T" equals the
# untransposed matrix read with "N" (same terms in the same order).
def pin_transpose_consistency(gemm, rng):
    A = rng.standard_normal((9, 14)).astype(np.float32)
    B = rng.standard_normal((14, 10)).astype(np.float32)
    ref, _ = run(gemm, "N", "N", A, B)
    for ta, tb in OPS:
        c, _ = run(gemm, ta, tb, A, B, pad=1)
        assert np.array_equal(c, ref), ("transpose", ta, tb)
    # and a non-symmetric check that "T" really transposes: A^T B^T != A B
    Asq = rng.standard_normal((6, 6)).astype(np.float32)
    Bsq = rng.standard_normal((6, 6)).astype(np.float32)
    c_nn, _ = run(gemm, "N", "N", Asq, Bsq)
    c_tt = gemm("T", "T", 6, 6, 6, 1.0, Asq, 6, Bsq, 6, 0.0, None, 6)[0]
    want = (Asq.astype(np.float64).T @ Bsq.astype(np.float64).T)
    assert np.allclose(c_tt, want, rtol=0, atol=1e-12)
    assert not np.allclose(c_nn, c_tt)


ALL_PINS = [pin_identity, pin_all_ones, pin_rank1_diag, pin_integers,
            pin_numpy_f64, pin_beta_zero_and_padding, pin_degenerate,
            pin_transpose_consistency, pin_bruteforce]
