"""Pins of the quantised-output oracle (oracle/quantize.py), CPU only.

The expected values come from the formats' definitions worked by hand
(bit patterns of exact ties, of the largest finite values, of subnormals),
from a library routine of another implementation (torch's binary32 ->
bfloat16 conversion), from an exhaustive check on a grid of bit patterns,
and from cases where rounding the product to binary32 first changes the
integer code. Planted mistakes in a copy of the oracle must each fail a pin.
"""
import importlib.util
import os

import numpy as np
import pytest

from oracle import quantize as real_q

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "quantize.py")


def f32(bits):
    return np.array(bits, dtype=np.uint32).view(np.float32)


# --- bf16 ---------------------------------------------------------------------

def pin_bf16_exact_and_ties(q=real_q):
    """Values already in bfloat16 keep their code; a binary32 exactly half way
    between two bfloat16 values goes to the one with an even last bit; just
    below / above half way goes down / up."""
    cases = {
        0x3F800000: 0x3F80,  # 1.0
        0xC0000000: 0xC000,  # -2.0
        0x00000000: 0x0000, 0x80000000: 0x8000,  # +-0
        0x3F808000: 0x3F80,  # 1 + 2^-8: tie, 0x3F80 is even
        0x3F818000: 0x3F82,  # tie between 0x3F81 (odd) and 0x3F82
        0x3F807FFF: 0x3F80,  # below half way
        0x3F808001: 0x3F81,  # above half way
        0xBF818000: 0xBF82,  # negative tie, magnitude to even
        0x4049FFFF: 0x404A,  # 3.1562498 -> 3.15625 (carry into the next code)
    }
    got = q.bf16_rne(f32(list(cases)))
    assert got.tolist() == list(cases.values()), [hex(v) for v in got]


def pin_bf16_specials(q=real_q):
    """Infinities stay; NaN becomes 0x7FC0; finite values that round past the
    largest bfloat16 become infinities; subnormals round on the 2^-133 grid."""
    cases = {
        0x7F800000: 0x7F80, 0xFF800000: 0xFF80,  # +-inf
        0x7FC00000: 0x7FC0, 0xFFC00001: 0x7FC0, 0x7F800001: 0x7FC0,  # NaNs
        0x7F7FFFFF: 0x7F80,  # largest binary32 -> inf
        0x7F7F7FFF: 0x7F7F,  # largest bfloat16 stays finite
        0x7F7F8000: 0x7F80,  # tie between 0x7F7F (odd) and infinity (even)
        0xFF7F8000: 0xFF80,
        0x00008000: 0x0000,  # subnormal tie -> even (zero)
        0x00018000: 0x0002,  # subnormal tie between 1 and 2 -> 2
        0x00010001: 0x0001,
        0x00000001: 0x0000,  # smallest binary32 subnormal
        0x80000001: 0x8000,  # ... keeps its sign
        0x007FFFFF: 0x0080,  # largest subnormal rounds up to the smallest normal
    }
    got = q.bf16_rne(f32(list(cases)))
    assert got.tolist() == list(cases.values()), [hex(v) for v in got]


def pin_bf16_against_torch(q=real_q):
    """torch's binary32 -> bfloat16 conversion (round to nearest even, another
    implementation) on random finite values of every magnitude and on the
    low-half patterns around each tie."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    hi = rng.integers(0, 1 << 16, 4000, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]  # finite
    lo = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    bits = (hi[:, None] << 16 | lo[None, :]).ravel()
    x = f32(bits)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy()
    got = q.bf16_rne(x)
    assert np.array_equal(got.view(np.int16), want), np.argwhere(got.view(np.int16) != want)[:5]


def pin_bf16_value_roundtrip(q=real_q):
    """Every bfloat16 code maps back to itself (all 65536 codes but NaNs)."""
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = q.bf16_value(codes)
    keep = ~np.isnan(v)
    assert np.array_equal(q.bf16_rne(v[keep]), codes[keep])


# --- int8 with a per-row factor ------------------------------------------------

def pin_int8_ties_and_saturation(q=real_q):
    c = np.array([[0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 127.5, -128.5, -129.0,
                   1000.0, -1e30, np.inf, -np.inf, np.nan, 0.49999997, -0.0, 3.0]],
                 dtype=np.float32)
    want = [0, 2, 2, 0, -2, -2, 126, 127, -128, -128, 127, -128, 127, -128, 0, 0, 0, 3]
    got = q.int8_row(c, [1.0])
    assert got.dtype == np.int8 and got.ravel().tolist() == want, got


def pin_int8_factor_per_row(q=real_q):
    """Row i uses factor s_i: [[10, -10], [10, -10]] with s = (0.25, 2) gives
    [[2, -2], [20, -20]] (2.5 -> 2 by ties to even)."""
    c = np.array([[10.0, -10.0], [10.0, -10.0]], dtype=np.float32)
    got = q.int8_row(c, np.array([0.25, 2.0], dtype=np.float32))
    assert got.tolist() == [[2, -2], [20, -20]], got


def pin_int8_product_rounded_to_binary32(q=real_q):
    """The code is decided on the binary32 product: pairs whose exact
    product lies just above k + 1/2 but rounds to exactly k + 1/2 in
    binary32 give the even neighbour, not the one the exact value is
    nearest to."""
    rng = np.random.default_rng(11)
    found = 0
    for _ in range(200000):
        s = np.float32(rng.uniform(0.5, 1.0))
        k = int(rng.integers(-100, 100))
        x = np.float32((k + 0.5) / np.float64(s))
        exact = np.float64(x) * np.float64(s)
        if np.float32(exact) != np.float32(k + 0.5) or exact == k + 0.5:
            continue
        got = int(q.int8_row(np.array([[x]], dtype=np.float32), [s])[0, 0])
        even = k if k % 2 == 0 else k + 1
        assert got == even, (float(x), float(s), exact, got)
        found += 1
        if found >= 20:
            break
    assert found >= 20


def pin_quantize_dispatch(q=real_q):
    c = np.array([[1.0, 3.0]], dtype=np.float32)
    assert q.quantize(c, "bf16").tolist() == [[0x3F80, 0x4040]]
    assert q.quantize(c, "int8_row", [2.0]).tolist() == [[2, 6]]
    with pytest.raises(ValueError):
        q.quantize(c, "int4")


PINS = [pin_bf16_exact_and_ties, pin_bf16_specials, pin_bf16_against_torch,
        pin_bf16_value_roundtrip, pin_int8_ties_and_saturation, pin_int8_factor_per_row,
        pin_int8_product_rounded_to_binary32, pin_quantize_dispatch]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_quantize_pin(pin):
    pin()


# Planted mistakes: (name, text to replace, replacement).
MUTANTS = [
    ("bf16_truncates", "r = np.rint(np.where(fin, x, 0.0) / quantum) * quantum",
     "r = np.trunc(np.where(fin, x, 0.0) / quantum) * quantum"),
    ("bf16_ties_away", "r = np.rint(np.where(fin, x, 0.0) / quantum) * quantum",
     "r = np.sign(x) * np.floor(np.abs(np.where(fin, x, 0.0)) / quantum + 0.5) * quantum"),
    ("bf16_seven_bits", "quantum = np.exp2(np.maximum(e - 7, BF16_MIN_SUBNORMAL_EXP))",
     "quantum = np.exp2(np.maximum(e - 6, BF16_MIN_SUBNORMAL_EXP))"),
    ("bf16_overflow_saturates", "r = np.where(overflow, np.copysign(np.inf, x), r)",
     "r = np.where(overflow, np.copysign(3.3895313892515355e38, x), r)"),
    ("bf16_flushes_subnormals", "BF16_MIN_SUBNORMAL_EXP = -133", "BF16_MIN_SUBNORMAL_EXP = -126"),
    ("bf16_nan_keeps_sign", "out[nan] = BF16_QNAN", "out[nan] = BF16_QNAN | (np.signbit(x[nan]) << 15)"),
    ("int8_half_up", "r = np.rint(prod.astype(np.float64))",
     "r = np.floor(prod.astype(np.float64) + 0.5)"),
    ("int8_exact_product",
     "prod = (c.astype(np.float64) * s.astype(np.float64)).astype(np.float32)  # fl32",
     "prod = c.astype(np.float64) * s.astype(np.float64)"),
    ("int8_no_saturation", "np.clip(np.where(np.isnan(r), 0.0, r), -128.0, 127.0)",
     "np.where(np.isnan(r), 0.0, r)"),
    ("int8_symmetric_range", "np.clip(np.where(np.isnan(r), 0.0, r), -128.0, 127.0)",
     "np.clip(np.where(np.isnan(r), 0.0, r), -127.0, 127.0)"),
    ("int8_nan_to_min", "np.clip(np.where(np.isnan(r), 0.0, r), -128.0, 127.0)",
     "np.clip(np.where(np.isnan(r), -128.0, r), -128.0, 127.0)"),
    ("int8_factor_per_column",
     "s = np.asarray(row_factor, dtype=np.float32).reshape(-1, *([1] * (c.ndim - 1)))",
     "s = np.asarray(row_factor, dtype=np.float32).reshape(1, -1)"),
]


def _load_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation {name}: pattern must occur exactly once"
    path = tmp_path / f"q_{name}.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"q_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_quantize_mutant_fails_a_pin(tmp_path, name, old, new):
    mod = _load_mutant(tmp_path, name, old, new)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, ValueError, IndexError, TypeError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
