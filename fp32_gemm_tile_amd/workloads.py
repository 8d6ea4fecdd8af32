"""Seeded synthetic SGEMM inputs (shared by the GPU tests, the bench and the
oracle checks).

This module only draws random numbers and describes shapes: it holds none of
the GEMM arithmetic, and imports neither the GPU binding nor the oracle.

Recipe (the pages fix no generator, so this is a stated choice):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64);
  * "uniform[-1,1)": ``2 * rng.random(shape, dtype=float32) - 1`` -- every value
    is a multiple of 2^-23 in [-1, 1) and exact in binary32;
  * "normal": ``rng.standard_normal(shape, dtype=float32)``;
  * "int8": ``rng.integers(-8, 9, shape)`` as float32 (small integers, for
    results that every summation order gets exactly);
  * arrays are drawn in the order A, B, C_in, each in its *storage* shape
    (rows x ld for row-major with leading dimension ld).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    transA: str = "N"
    transB: str = "N"
    alpha: float = 1.0
    beta: float = 0.0
    dist: str = "uniform"
    seed: int = 0
    lda: Optional[int] = None
    ldb: Optional[int] = None
    ldc: Optional[int] = None
    note: str = ""

    # storage shapes (row-major): op(A) is M x K, op(B) is K x N
    @property
    def a_rows(self):
        return self.K if self.transA == "T" else self.M

    @property
    def a_cols(self):
        return self.M if self.transA == "T" else self.K

    @property
    def b_rows(self):
        return self.N if self.transB == "T" else self.K

    @property
    def b_cols(self):
        return self.K if self.transB == "T" else self.N

    @property
    def LDA(self):
        return self.lda if self.lda is not None else max(1, self.a_cols)

    @property
    def LDB(self):
        return self.ldb if self.ldb is not None else max(1, self.b_cols)

    @property
    def LDC(self):
        return self.ldc if self.ldc is not None else max(1, self.N)

    @property
    def flops(self) -> int:
        """2*M*N*K: one multiply and one add per term of every output sum."""
        return 2 * self.M * self.N * self.K

    @property
    def compulsory_bytes(self) -> int:
        """Each matrix moved once: A and B read, C written (and read if
        beta != 0); 4 bytes per element."""
        c_moves = 2 if self.beta != 0 else 1
        return 4 * (self.M * self.K + self.K * self.N + c_moves * self.M * self.N)


# Shapes of the benchmark and parity workloads. C6 (4096^3) is the second
# size the headline metric is quoted at; its seed is this project's choice.
WORKLOADS = {
    "C1": Workload("C1", 256, 256, 256, seed=0,
                   note="256^3 NN, uniform[-1,1), C output only"),
    "C2": Workload("C2", 2048, 2048, 2048, seed=1,
                   note="2048^3 NN, uniform[-1,1)"),
    "C3": Workload("C3", 3001, 2047, 1025, transA="T", alpha=1.5, beta=0.5,
                   dist="normal", seed=2, lda=3001, ldb=2047, ldc=2047,
                   note="ragged TN, A stored 1025x3001, standard normal A/B/C"),
    "C4": Workload("C4", 16384, 16384, 256, seed=3,
                   note="skinny-K NN, 1 GiB of C written"),
    "C5a": Workload("C5a", 8192, 8192, 8192, seed=4,
                    note="8192^3 NN (headline)"),
    "C5b": Workload("C5b", 8192, 8192, 8192, transB="T", seed=4,
                    note="8192^3 NT, same buffers as C5a"),
    "C6": Workload("C6", 4096, 4096, 4096, seed=5,
                   note="4096^3 NN (headline)"),
    # One GPU's share of 8192^3 split by row blocks over eight GPUs (each
    # GPU holds 1024 rows of A and all of B); seed is this project's choice.
    "S8": Workload("S8", 1024, 8192, 8192, seed=8,
                   note="row block of 8192^3 over 8 GPUs: 1024 x 8192 x 8192 NN"),
    # Few-row (decode) shapes, memory-bound; seeds are this project's choice.
    "G1": Workload("G1", 1, 8192, 8192, seed=6, note="GEMV: 1 x 8192 times 8192 x 8192"),
    "G1T": Workload("G1T", 1, 8192, 8192, transB="T", seed=6,
                    note="GEMV with B stored N x K"),
    "G8": Workload("G8", 8, 8192, 8192, seed=7, note="8 rows times 8192 x 8192"),
    "G8T": Workload("G8T", 8, 8192, 8192, transB="T", seed=7,
                    note="8 rows, B stored N x K"),
    "G32": Workload("G32", 32, 8192, 8192, seed=9, note="32 rows times 8192 x 8192"),
}


def _draw(rng, dist, shape):
    if dist == "uniform":
        return 2 * rng.random(shape, dtype=np.float32) - 1
    if dist == "normal":
        return rng.standard_normal(shape, dtype=np.float32)
    if dist == "int8":
        return rng.integers(-8, 9, size=shape).astype(np.float32)
    if dist == "ones":
        return np.ones(shape, dtype=np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def make_inputs(w: Workload, with_c: Optional[bool] = None):
    """Host arrays (A, B, C_in) in storage shape for workload ``w``.

    C_in is drawn only when beta != 0 (or with_c is True); otherwise None.
    """
    rng = np.random.default_rng(w.seed)
    A = _draw(rng, w.dist, (w.a_rows, w.LDA))
    B = _draw(rng, w.dist, (w.b_rows, w.LDB))
    want_c = (w.beta != 0) if with_c is None else with_c
    C = _draw(rng, w.dist, (w.M, w.LDC)) if want_c else None
    return A, B, C


def custom(M, N, K, transA="N", transB="N", alpha=1.0, beta=0.0, dist="uniform",
           seed=0, lda=None, ldb=None, ldc=None, name="custom") -> Workload:
    return Workload(name, M, N, K, transA, transB, alpha, beta, dist, seed,
                    lda, ldb, ldc)


def sample_indices(M, N, n, seed=12345, include_corners=True):
    """Seeded element sample (ii, jj) over an M x N output, with the four
    corners and the last row/column included so ragged edges are covered."""
    rng = np.random.default_rng(seed)
    ii = rng.integers(0, M, size=n, dtype=np.int64)
    jj = rng.integers(0, N, size=n, dtype=np.int64)
    if include_corners and M > 0 and N > 0:
        ci = np.array([0, 0, M - 1, M - 1] + [M - 1] * 8 + list(range(min(M, 8))),
                      dtype=np.int64)
        cj = np.array([0, N - 1, 0, N - 1] + list(range(max(0, N - 8), N))
                      + [0] * (8 - min(N, 8)) + [N - 1] * min(M, 8), dtype=np.int64)
        k = min(ci.size, cj.size)
        ii = np.concatenate([ci[:k], ii])
        jj = np.concatenate([cj[:k], jj])
    return ii, jj
