"""Planted mistakes in the oracle must fail a pin.

Each case copies the oracle's C source to a temporary directory, applies one
plausible mistake (a dropped term, a wrong sign, a transposed index, binary32
accumulation, ...), builds it with gcc and runs the pins against it. The
committed oracle is never modified. CPU only.
"""
import os
import shutil
import subprocess
import sys
import functools

import numpy as np
import pytest

import oracle
from fp32_gemm_tile_amd import workloads
from oracle_pins import ALL_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sgemm_oracle.c")

# (name, text to replace, replacement). Each text must occur in the source.
MUTANTS = [
    ("drop_last_term_rows", "alpha != 0.0 && k < K; ++k) {\n                    double a",
     "alpha != 0.0 && k < K - 1; ++k) {\n                    double a"),
    ("drop_first_term_elems", "for (int64_t k = 0; alpha != 0.0 && k < K; ++k) {\n        double p",
     "for (int64_t k = 1; alpha != 0.0 && k < K; ++k) {\n        double p"),
    ("beta_sign", "c += beta * (double)Cin[i * ldc + j];\n                    cref",
     "c -= beta * (double)Cin[i * ldc + j];\n                    cref"),
    ("alpha_ignored", "double c = alpha * s[j];", "double c = s[j];"),
    ("transA_swapped", "return transA ? (double)A[k * lda + i] : (double)A[i * lda + k];",
     "return transA ? (double)A[i * lda + k] : (double)A[k * lda + i];"),
    ("transB_copy_wrong", "bt[k * N + j] = B[j * ldb + k];", "bt[k * N + j] = B[k * ldb + j];"),
    ("lda_off_by_one", "(double)A[i * lda + k];", "(double)A[i * (lda - 1) + k];"),
    ("binary32_accumulation", "s[j] += p;", "s[j] = (float)(s[j] + p);"),
    ("abs_missing", "sa[j] += fabs(p);", "sa[j] += p;"),
    ("reads_c_when_beta_zero", "if (beta != 0.0)\n                        c += beta",
     "if (1)\n                        c += beta"),
    ("row_index_off_by_one", "int64_t i = rows ? rows[t] : t;",
     "int64_t i = rows ? rows[t] : (t + 1) % M;"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name}: pattern must occur exactly once"
    d = tmp_path / name
    d.mkdir()
    cpath = d / "m.c"
    cpath.write_text(src.replace(old, new))
    so = d / "libm.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-o", str(so), str(cpath), "-lm"], check=True)
    return str(so)


def _elems_vs_rows(lib):
    """Elements and rows of the same product must be the same numbers."""
    rng = np.random.default_rng(5)
    M, N, K = 9, 7, 13
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    cr, _ = oracle.gemm_rows("N", "N", M, N, K, 1.0, A, K, B, N, 0.0, lib=lib)
    ii, jj = workloads.sample_indices(M, N, 20, seed=1)
    ce, _ = oracle.gemm_elems("N", "N", M, N, K, 1.0, A, K, B, N, 0.0, None, N,
                              ii, jj, lib=lib)
    assert np.array_equal(ce, cr[ii, jj])


def run_pins_against(so_path):
    """Run every pin against the library at so_path; return the names of the
    pins that failed. Called in a child process (a planted mistake may also
    crash, e.g. by reading a C that is not there when beta == 0)."""
    lib = oracle.bind(so_path)
    gemm = functools.partial(oracle.gemm_rows, lib=lib)
    failed = []
    for pin in ALL_PINS + [None]:
        try:
            if pin is None:
                _elems_vs_rows(lib)
            else:
                pin(gemm, np.random.default_rng(2024))
        except (AssertionError, RuntimeError, ValueError):
            failed.append(pin.__name__ if pin else "elems_vs_rows")
    return failed


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("mut", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, mut):
    name, old, new = mut
    so = _build_mutant(tmp_path, name, old, new)
    code = ("import sys; sys.path[:0] = [%r, %r]; "
            "import test_oracle_mutants as t; "
            "f = t.run_pins_against(%r); print('FAILED_PINS', f); "
            "sys.exit(3 if f else 0)") % (ROOT, os.path.join(ROOT, "tests"), so)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True,
                       text=True, timeout=600)
    # exit 3: some pin failed; negative: the mutant crashed the process.
    # Either way the planted mistake did not pass unnoticed.
    assert r.returncode != 0, f"planted mistake {name} passed every pin: {r.stdout}"
    assert r.returncode == 3 or r.returncode < 0, (r.returncode, r.stderr[-2000:])
