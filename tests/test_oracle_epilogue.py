"""Pins for the fused-epilogue oracle (oracle/epilogue.py), and planted
mistakes in it that must each fail a pin. CPU only.

What fixes the expected values (none of it is the oracle's own formula):
  * values of the standard normal distribution function Phi at 0.5, 1, 2, 3
    (as tabulated in statistics references) for gelu(x) = x Phi(x);
  * the logistic function at +-ln 3, where it is exactly 3/4 and 1/4;
  * the identity f(x) - f(-x) = x, which relu, gelu (Phi(x) + Phi(-x) = 1)
    and silu (sigma(x) + sigma(-x) = 1) all satisfy;
  * exact rational arithmetic (fractions) of the whole epilogue on tiny
    dyadic inputs, with M != N so that a row vector used as a column vector
    (or the reverse) cannot pass;
  * with no vectors and no activation it must equal the plain alpha/beta
    oracle (a different code path: alpha and beta applied inside the C
    oracle).
"""
import importlib.util
import math
import os
import sys
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import epilogue as real_ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "epilogue.py")

PHI = {0.5: 0.6914624612740131, 1.0: 0.8413447460685429, 2.0: 0.9772498680518208,
       3.0: 0.9986501019683699}


def pin_gelu_phi_table(ep):
    for x, phi in PHI.items():
        assert abs(float(ep.activation(np.array([x]), "gelu")[0]) - x * phi) <= 1e-13, x
        assert abs(float(ep.activation(np.array([-x]), "gelu")[0]) + x * (1 - phi)) <= 1e-13, -x


def pin_silu_logistic(ep):
    ln3 = math.log(3.0)
    got = ep.activation(np.array([ln3, -ln3, 0.0]), "silu")
    assert abs(got[0] - 0.75 * ln3) <= 1e-15
    assert abs(got[1] + 0.25 * ln3) <= 1e-15
    assert got[2] == 0.0


def pin_odd_part_identity(ep):
    x = np.random.default_rng(3).standard_normal(1000) * 4
    for act in ("relu", "gelu", "silu"):
        d = ep.activation(x, act) - ep.activation(-x, act)
        assert np.allclose(d, x, rtol=1e-14, atol=1e-15), act
    assert np.array_equal(ep.activation(x, "relu"), np.where(x > 0, x, 0.0))
    assert np.array_equal(ep.activation(x, "none"), x)


def _dyadic(rng, shape, scale=8):
    return rng.integers(-4 * scale, 4 * scale + 1, size=shape) / scale


def pin_exact_rational(ep):
    rng = np.random.default_rng(11)
    M, N, K = 3, 5, 4
    A = _dyadic(rng, (M, K))
    B = _dyadic(rng, (K, N))
    Cin = _dyadic(rng, (M, N))
    r, c = _dyadic(rng, M), _dyadic(rng, N)
    u, w = _dyadic(rng, M), _dyadic(rng, N)
    alpha, beta = 1.5, -0.5
    s = A @ B  # exact: small dyadic values
    for vecs in [(r, c, u, w), (None, c, None, w), (r, None, u, None)]:
        d, v = ep.epilogue(s, alpha, beta, Cin, *vecs, act="none")
        dr, _ = ep.epilogue(s, alpha, beta, Cin, *vecs, act="relu")
        for i in range(M):
            for j in range(N):
                acc = sum(Fraction(A[i, k]) * Fraction(B[k, j]) for k in range(K))
                ri = Fraction(vecs[0][i]) if vecs[0] is not None else Fraction(1)
                cj = Fraction(vecs[1][j]) if vecs[1] is not None else Fraction(1)
                ui = Fraction(vecs[2][i]) if vecs[2] is not None else Fraction(0)
                wj = Fraction(vecs[3][j]) if vecs[3] is not None else Fraction(0)
                exact = (Fraction(alpha) * ri * cj * acc + Fraction(beta) * Fraction(Cin[i, j])
                         + ui + wj)
                assert Fraction(float(d[i, j])) == exact, (i, j)
                assert Fraction(float(v[i, j])) == exact, (i, j)
                assert Fraction(float(dr[i, j])) == max(exact, Fraction(0)), (i, j)


def pin_reduces_to_plain_gemm(ep):
    rng = np.random.default_rng(5)
    M, N, K = 9, 14, 33
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    Cin = rng.standard_normal((M, N)).astype(np.float32)
    s, _ = oracle.gemm("N", "N", M, N, K, 1.0, A, K, B, N, 0.0, None, N)
    want, S = oracle.gemm("N", "N", M, N, K, 1.25, A, K, B, N, -0.75, Cin, N)
    got, _ = ep.epilogue(s, 1.25, -0.75, Cin)
    bound = 2 * K * 2.0 ** -53 * (1.25 * S + 0.75 * np.abs(Cin))
    assert np.all(np.abs(got - want) <= bound + 1e-300)


PINS = [pin_gelu_phi_table, pin_silu_logistic, pin_odd_part_identity, pin_exact_rational,
        pin_reduces_to_plain_gemm]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_epilogue_oracle_pin(pin):
    pin(real_ep)


def _gelu_as7126_f32(x):
    """gelu with erf from formula 7.1.26 of Abramowitz and Stegun, every
    operation rounded to binary32 (a stand-in for an approximate device
    evaluation)."""
    f = np.float32
    x = np.asarray(x, dtype=np.float32)
    z = np.abs(x * f(0.70710678118654752))
    t = (f(1) / (f(1) + f(0.3275911) * z)).astype(np.float32)
    poly = t * (f(0.254829592) + t * (f(-0.284496736) + t * (f(1.421413741) + t * (
        f(-1.453152027) + t * f(1.061405429)))))
    e = np.copysign(f(1) - poly.astype(np.float32) * np.exp(-z * z).astype(np.float32), x)
    return (f(0.5) * x * (f(1) + e.astype(np.float32))).astype(np.float32)


def test_epilogue_tolerance_covers_approximate_gelu():
    """Formula 7.1.26 in binary32 stays inside the gelu part of the bound on
    a dense sweep of inputs (tol_v set to 0 here: only the activation's own
    error is being checked)."""
    x = np.concatenate([np.linspace(-12, 12, 200001), np.geomspace(1e-30, 1e3, 20001)])
    x = np.concatenate([x, -x]).astype(np.float32)
    got = _gelu_as7126_f32(x).astype(np.float64)
    want = real_ep.activation(x.astype(np.float64), "gelu")
    assert np.all(np.abs(got - want) <= 2.0 ** -20 * np.abs(x.astype(np.float64)) + 1e-37)


def test_epilogue_tolerance_covers_binary32_evaluation():
    """The bound of oracle.compare.epilogue_tol holds for the same epilogue
    evaluated step by step in binary32 (numpy float32, erf from binary64
    rounded), on values where the activations bend."""
    from oracle import compare
    rng = np.random.default_rng(9)
    M, N, K = 40, 30, 64
    A = rng.standard_normal((M, K)).astype(np.float32)
    B = rng.standard_normal((K, N)).astype(np.float32)
    Cin = rng.standard_normal((M, N)).astype(np.float32)
    r = rng.uniform(0.5, 2, M).astype(np.float32)
    c = rng.uniform(0.5, 2, N).astype(np.float32)
    u = rng.standard_normal(M).astype(np.float32)
    w = rng.standard_normal(N).astype(np.float32)
    s, S = oracle.gemm("N", "N", M, N, K, 1.0, A, K, B, N, 0.0, None, N)
    acc32 = (A @ B).astype(np.float32)  # binary32 products and sums
    for act in real_ep.ACTIVATIONS:
        d, v = real_ep.epilogue(s, 0.7, 0.3, Cin, r, c, u, w, act)
        v32 = (np.float32(0.7) * r[:, None] * c[None, :]) * acc32 + np.float32(0.3) * Cin
        v32 = (v32 + u[:, None]) + w[None, :]
        d32 = real_ep.activation(v32.astype(np.float64), act).astype(np.float32)
        ok, info = compare.check_epilogue(d32, d, v, S, K, 0.7, 0.3, Cin, r, c, u, w, act)
        assert ok, (act, info)


# Planted mistakes: (name, text to replace, replacement).
MUTANTS = [
    ("gelu_tanh_approximation", "return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))",
     "return 0.5 * x * (1.0 + np.tanh(0.7978845608028654 * (x + 0.044715 * x ** 3)))"),
    ("gelu_erf_without_sqrt2", "_erf(x / math.sqrt(2.0))", "_erf(x)"),
    ("silu_wrong_sign", "return x / (1.0 + np.exp(-x))", "return x / (1.0 + np.exp(x))"),
    ("relu_leaky", "return np.maximum(x, 0.0)", "return np.maximum(x, 0.01 * x)"),
    ("row_bias_as_column", "return v + u[:, None] + w[None, :]",
     "return v + u[:M, None] * 0 + u.sum() + w[None, :]"),
    ("col_bias_dropped", "return v + u[:, None] + w[None, :]", "return v + u[:, None]"),
    ("scale_on_beta_term_too",
     "v = v + float(beta) * np.asarray(cin, dtype=np.float64)\n    return v + u[:, None]",
     "v = v + float(beta) * r[:, None] * np.asarray(cin, dtype=np.float64)\n"
     "    return v + u[:, None]"),
    ("col_scale_ignored", "v = float(alpha) * r[:, None] * c[None, :] * s",
     "v = float(alpha) * r[:, None] * s"),
    ("beta_dropped",
     "v = v + float(beta) * np.asarray(cin, dtype=np.float64)\n    return v + u[:, None]",
     "v = v\n    return v + u[:, None]"),
]


def _load_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name}: pattern must occur exactly once"
    path = tmp_path / f"ep_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"ep_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_epilogue_mutant_fails_a_pin(tmp_path, name, old, new):
    mod = _load_mutant(tmp_path, name, old, new)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"


def test_epilogue_elems_equals_full():
    rng = np.random.default_rng(21)
    M, N = 7, 11
    s = rng.standard_normal((M, N))
    cin = rng.standard_normal((M, N))
    vecs = [rng.standard_normal(M), rng.standard_normal(N), rng.standard_normal(M),
            rng.standard_normal(N)]
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    for act in real_ep.ACTIVATIONS:
        d, v = real_ep.epilogue(s, 1.3, 0.4, cin, *vecs, act=act)
        de, ve = real_ep.epilogue_elems(s[ii, jj].ravel(), 1.3, 0.4, cin[ii, jj].ravel(),
                                        ii.ravel(), jj.ravel(), *vecs, act=act)
        assert np.array_equal(de, d.ravel()) and np.array_equal(ve, v.ravel()), act
        from oracle import compare
        t_full = compare.epilogue_tol(5, 1.3, 0.4, np.abs(s), cin, v, *vecs, act)
        t_el = compare.epilogue_tol(5, 1.3, 0.4, np.abs(s).ravel(), cin.ravel(), ve,
                                    vecs[0][ii.ravel()], vecs[1][jj.ravel()],
                                    vecs[2][ii.ravel()], vecs[3][jj.ravel()], act,
                                    per_element=True)
        assert np.allclose(t_full.ravel(), t_el, rtol=1e-15, atol=0), act
