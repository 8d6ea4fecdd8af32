"""The oracle against its pins (closed forms, integer exactness, exact
rational brute force, a binary64 library cross-check, invariants)."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import compare
from fp32_gemm_tile_amd import workloads

from oracle_pins import ALL_PINS

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.gemm_rows, np.random.default_rng(2024))


def test_elems_equal_rows():
    rng = np.random.default_rng(7)
    for ta, tb in [("N", "N"), ("T", "N"), ("N", "T"), ("T", "T")]:
        M, N, K = 19, 23, 41
        A = rng.standard_normal((K, M) if ta == "T" else (M, K)).astype(np.float32)
        B = rng.standard_normal((N, K) if tb == "T" else (K, N)).astype(np.float32)
        C = rng.standard_normal((M, N)).astype(np.float32)
        lda, ldb = A.shape[1], B.shape[1]
        cr, sr = oracle.gemm(ta, tb, M, N, K, 0.75, A, lda, B, ldb, -1.5, C, N)
        ii, jj = workloads.sample_indices(M, N, 50, seed=3)
        ce, se = oracle.gemm_elems(ta, tb, M, N, K, 0.75, A, lda, B, ldb, -1.5, C, N, ii, jj)
        assert np.array_equal(ce, cr[ii, jj]) and np.array_equal(se, sr[ii, jj])
        rows = [M - 1, 0, 5]
        c3, s3 = oracle.gemm_rows(ta, tb, M, N, K, 0.75, A, lda, B, ldb, -1.5, C, N, rows=rows)
        assert np.array_equal(c3, cr[rows]) and np.array_equal(s3, sr[rows])


def test_storage_checks():
    with pytest.raises(ValueError):
        oracle.gemm("N", "N", 4, 4, 4, 1.0, np.zeros(15, np.float32), 4,
                    np.zeros(16, np.float32), 4, 0.0)
    with pytest.raises(ValueError):
        oracle.gemm("X", "N", 1, 1, 1, 1.0, np.zeros(1, np.float32), 1,
                    np.zeros(1, np.float32), 1, 0.0)


def test_compare_accepts_fp32_rounding_and_rejects_errors():
    """The acceptance bound holds for a plain binary32 loop (any order) and
    rejects a result with one term dropped."""
    rng = np.random.default_rng(11)
    M, N, K = 24, 20, 300
    A = (2 * rng.random((M, K), dtype=np.float32) - 1)
    B = (2 * rng.random((K, N), dtype=np.float32) - 1)
    cref, s = oracle.gemm("N", "N", M, N, K, 1.0, A, K, B, N, 0.0)
    # binary32 summation in descending k order, one rounding per step
    acc = np.zeros((M, N), dtype=np.float32)
    for k in range(K - 1, -1, -1):
        acc = (acc + np.outer(A[:, k], B[k, :]).astype(np.float32)).astype(np.float32)
    ok, info = compare.check(acc, cref, s, K)
    assert ok, info
    assert info["frob_rel"] < 1e-6
    dropped = acc - np.outer(A[:, K - 1], B[K - 1, :]).astype(np.float32)
    ok, info = compare.check(dropped, cref, s, K)
    assert not ok


def test_workload_accounting_against_pages():
    """FLOP and byte counts used for the roofline, against the figures the
    pages print (tests/golden/pages_arithmetic.json)."""
    with open(os.path.join(HERE, "golden", "pages_arithmetic.json")) as f:
        g = json.load(f)["cases"]
    w = workloads.custom(g[0]["M"], g[0]["N"], g[0]["K"])
    assert w.compulsory_bytes == g[0]["bytes_moved"]
    assert abs(w.flops / w.compulsory_bytes / g[0]["arithmetic_intensity"] - 1) < g[0]["ai_rel_tol"]
    c = g[1]
    w = workloads.custom(c["M"], c["N"], c["K"])
    assert abs(w.flops / c["flops"] - 1) < c["flops_rel_tol"]
    inp = 4 * (w.M * w.K + w.K * w.N)
    out = 4 * w.M * w.N
    assert abs(inp / c["input_bytes"] - 1) < c["input_rel_tol"]
    assert abs(out / c["output_bytes"] - 1) < c["output_rel_tol"]
    assert abs(w.flops / w.compulsory_bytes / c["arithmetic_intensity"] - 1) < c["ai_rel_tol"]
    r = g[2]
    assert abs(r["peak_flops"] / r["bandwidth"] / r["ridge"] - 1) < r["ridge_rel_tol"]


def test_workload_generators_are_seeded_and_exact():
    w = workloads.WORKLOADS["C1"]
    A1, B1, C1 = workloads.make_inputs(w)
    A2, B2, _ = workloads.make_inputs(w)
    assert C1 is None and np.array_equal(A1, A2) and np.array_equal(B1, B2)
    assert A1.dtype == np.float32 and A1.min() >= -1 and A1.max() < 1
    # every uniform value is a multiple of 2^-23
    assert np.all(A1 * np.float32(2 ** 23) == np.round(A1 * np.float32(2 ** 23)))
    w3 = workloads.WORKLOADS["C3"]
    assert (w3.a_rows, w3.a_cols, w3.LDA) == (1025, 3001, 3001)
    assert (w3.b_rows, w3.b_cols, w3.LDB, w3.LDC) == (1025, 2047, 2047, 2047)
