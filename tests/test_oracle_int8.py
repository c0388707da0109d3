"""Pins for the CPU oracle's INT8 row-wise quantizer, W8A16 GEMV and W4A8 path.

Checked against hand-worked rows (tests/golden/int8_rows.txt,
tests/golden/actquant_rows.txt), exact invariants, an exact round trip on the
grid, integer closed forms and exact rational brute force.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from golden_io import read_cases
from synthetic_inputs import activation, bf16_bits, int4_weight, int8_layer


def bf16_value(bits: int) -> Fraction:
    return Fraction(float((np.array([bits], np.uint32) << 16).view(np.float32)[0]))


def fp16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], np.uint16).view(np.float16)[0]))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    f = np.asarray(a, np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert (oracle.bf16_to_float64(b) == f.astype(np.float64)).all(), "not bf16-exact"
    return b


# ---------------------------------------------------------------- INT8 quantizer


@pytest.mark.parametrize("case", read_cases("int8_rows.txt"), ids=lambda c: c["name"])
def test_hand_worked_rows(case):
    q, s, f = oracle.quantize_int8_rowwise(case["bits"].reshape(1, 32))
    assert int(s[0]) == case["scale"], f"{int(s[0]):#06x}"
    assert q[0].tolist() == case["codes"].tolist()
    assert f == case["flags"]


def test_int8_invariants():
    w = bf16_bits(int4_weight(64, 512, seed=41))
    w[3] = (w[3].astype(np.uint32) & 0x807F).astype(np.uint16) | 0x0100  # tiny values row
    w[5] = 0
    q, s, f = oracle.quantize_int8_rowwise(w)
    assert f == 0
    for row in range(64):
        vals = [bf16_value(int(b)) for b in w[row]]
        a = max(abs(v) for v in vals)
        sv = bf16_value(int(s[row]))
        assert sv > 0 and np.abs(q[row]).max() <= 127
        if a == 0:
            assert s[row] == 0x3F80 and not q[row].any()
            continue
        assert 127 * sv >= a
        assert 127 * bf16_value(int(s[row]) - 1) < a, "scale not minimal"
        for v, c in zip(vals, q[row]):
            assert abs(v - int(c) * sv) <= sv / 2


def test_int8_round_trip_on_grid():
    rng = np.random.default_rng(5)
    n, k = 12, 256
    qi = rng.integers(-127, 128, (n, k))
    qi[:, 0] = 127 * np.where(rng.random(n) < 0.5, 1, -1)     # |q| = 127 present
    s = np.exp2(rng.integers(-20, 10, n)).astype(np.float64)
    w_bits = to_bf16_bits(qi * s[:, None])
    q, sb, f = oracle.quantize_int8_rowwise(w_bits)
    assert f == 0
    np.testing.assert_array_equal(q, qi)
    np.testing.assert_array_equal(oracle.bf16_to_float64(sb), s)


# ---------------------------------------------------------------- W8A16


def test_w8a16_integer_closed_form():
    rng = np.random.default_rng(8)
    m, n, k = 3, 50, 256
    w = rng.integers(-127, 128, (n, k)).astype(np.int8)
    xi = rng.integers(-8, 9, (m, k))
    e = rng.integers(-4, 5, n)
    scales = to_bf16_bits(np.exp2(e) * np.where(rng.random(n) < 0.5, 1, -1))
    y = oracle.qgemm_w8a16(to_bf16_bits(xi), w, scales)
    want = (xi @ w.astype(np.int64).T).astype(np.float64) * oracle.bf16_to_float64(scales)[None, :]
    np.testing.assert_array_equal(y, want)


def test_w8a16_one_hot_and_scale_per_row():
    w, scales, _ = int8_layer(n=20, k=256, m=1, seed=3)
    w = w.numpy()
    sb = bf16_bits(scales)
    for j in (0, 100, 255):
        x = np.zeros((1, 256), np.uint16)
        x[0, j] = 0x3F80
        y = oracle.qgemm_w8a16(x, w, sb)
        want = w[:, j].astype(np.float64) * oracle.bf16_to_float64(sb)
        np.testing.assert_array_equal(y[0], want)


def test_w8a16_bruteforce_exact_rationals_tiny():
    w, scales, x = int8_layer(n=4, k=256, m=2, seed=11)
    w, sb, xb = w.numpy(), bf16_bits(scales), bf16_bits(x)
    y = oracle.qgemm_w8a16(xb, w, sb)
    for mi in range(2):
        for row in range(4):
            terms = [bf16_value(int(xb[mi, kk])) * int(w[row, kk]) for kk in range(256)]
            exact = sum(terms, Fraction(0)) * bf16_value(int(sb[row]))
            bound = (256 + 1) * Fraction(1, 2 ** 53) * sum(abs(t) for t in terms) * abs(bf16_value(int(sb[row])))
            assert abs(Fraction(y[mi, row]) - exact) <= bound


# ---------------------------------------------------------------- W4A8


@pytest.mark.parametrize("case", read_cases("actquant_rows.txt"), ids=lambda c: c["name"])
def test_actquant_hand_worked(case):
    xq, sx = oracle.actquant_int8(case["bits"].reshape(1, 32))
    assert xq[0].tolist() == case["codes"].tolist()
    assert int(sx.view(np.uint32)[0]) == case["sx"]


def test_actquant_invariants():
    x = bf16_bits(activation(4, 4096, seed=77))
    xq, sx = oracle.actquant_int8(x)
    xf = oracle.bf16_to_float64(x)
    for mi in range(4):
        a = np.abs(xf[mi]).max()
        assert np.abs(xq[mi]).max() == 127
        assert xq[mi][np.argmax(np.abs(xf[mi]))] == 127 * np.sign(xf[mi][np.argmax(np.abs(xf[mi]))])
        # within half a step (plus binary32 rounding of the step itself)
        err = np.abs(xf[mi] - xq[mi] * (a / 127.0))
        assert err.max() <= (a / 127.0) * (0.5 + 1e-5)
        assert sx[mi] == np.float32(np.float32(a) / np.float32(127.0))


def test_w4a8_equals_w4a16_when_activations_are_on_the_int8_grid():
    """x integers with absmax 127: sx = 1, xq = x, so both paths compute the same sum."""
    rng = np.random.default_rng(19)
    m, n, k = 3, 90, 512
    xi = rng.integers(-127, 128, (m, k))
    xi[:, 7] = 127
    x = to_bf16_bits(xi)
    codes, scales, zeros, _ = oracle.quantize_int4_g32(bf16_bits(int4_weight(n, k, 2)))
    xq, sx = oracle.actquant_int8(x)
    np.testing.assert_array_equal(xq, xi)
    assert (sx == 1.0).all()
    y8 = oracle.qgemm_w4a8(x, codes, scales, zeros)
    y16 = oracle.qgemm_w4a16(x, codes, scales, zeros)
    np.testing.assert_allclose(y8, y16, rtol=1e-12, atol=1e-9)


def test_w4a8_bruteforce_exact_rationals_tiny():
    m, n, k = 2, 3, 256
    codes, scales, zeros, _ = oracle.quantize_int4_g32(bf16_bits(int4_weight(n, k, 4)))
    x = bf16_bits(activation(m, k, 6))
    xq, sx = oracle.actquant_int8(x)
    y = oracle.qgemm_w4a8(x, codes, scales, zeros)
    for mi in range(m):
        for row in range(n):
            tot = Fraction(0)
            for g in range(k // 32):
                isum = sum(int(xq[mi, kk]) * (int(codes[row, kk]) - int(zeros[row, g]))
                           for kk in range(g * 32, g * 32 + 32))
                tot += fp16_value(int(scales[row, g])) * isum
            exact = Fraction(float(sx[mi])) * tot
            assert abs(Fraction(y[mi, row]) - exact) <= Fraction(1, 2 ** 40) * (abs(exact) + 1)


def test_w4a8_zero_row_gives_zero():
    codes, scales, zeros, _ = oracle.quantize_int4_g32(bf16_bits(int4_weight(8, 256, 1)))
    x = np.zeros((2, 256), np.uint16)
    x[1] = bf16_bits(activation(1, 256, 2))[0]
    y = oracle.qgemm_w4a8(x, codes, scales, zeros)
    assert (y[0] == 0).all() and (y[1] != 0).any()


def test_w4a8_span_with_an_overflowing_inverse_scale_is_a_zero_span():
    """Reading for a span whose 127/a overflows binary32 (hand-worked cases A5
    and A7): no finite inverse scale, read as a zero span.  Its row's outputs
    are exactly 0 while a row just above the threshold (case A6) is not; the
    other rows are untouched."""
    cases = {c["name"]: c for c in read_cases("actquant_rows.txt")}
    codes, scales, zeros, _ = oracle.quantize_int4_g32(bf16_bits(int4_weight(16, 256, 3)))
    x = bf16_bits(activation(4, 256, seed=8))
    clean = oracle.qgemm_w4a8(x, codes, scales, zeros)
    x[1] = 0
    x[1, 64:96] = cases["A5"]["bits"]
    x[1, 160:192] = cases["A7"]["bits"]
    x[2] = 0
    x[2, 32:64] = cases["A6"]["bits"]
    y = oracle.qgemm_w4a8(x, codes, scales, zeros)
    assert (y[1] == 0).all()
    assert (y[2] != 0).any() and np.isfinite(y[2]).all()
    np.testing.assert_array_equal(y[[0, 3]], clean[[0, 3]])
    # per group of 32: the flushed groups contribute nothing, the rest of the
    # row is as if those groups were zero
    xg = bf16_bits(activation(2, 256, seed=9))
    xg[0, 64:96] = cases["A5"]["bits"]
    xz = xg.copy()
    xz[0, 64:96] = 0
    np.testing.assert_array_equal(oracle.qgemm_w4a8_g32(xg, codes, scales, zeros),
                                  oracle.qgemm_w4a8_g32(xz, codes, scales, zeros))


# Reading: a span of activations holding a NaN or an infinity has no finite
# absmax scale; it gets sx = NaN and codes 0, and every output it reaches is NaN.
NON_FINITE = {"nan": 0x7FC0, "+inf": 0x7F80, "-inf": 0xFF80}


@pytest.mark.parametrize("kind", sorted(NON_FINITE))
def test_actquant_non_finite_row(kind):
    x = bf16_bits(activation(3, 512, seed=21))
    clean_q, clean_s = oracle.actquant_int8(x)
    x[1, 300] = NON_FINITE[kind]
    xq, sx = oracle.actquant_int8(x)
    assert np.isnan(sx[1]) and (xq[1] == 0).all()
    # the other rows are quantized as if the bad row were absent
    for r in (0, 2):
        assert sx[r] == clean_s[r] and (xq[r] == clean_q[r]).all()


@pytest.mark.parametrize("kind", sorted(NON_FINITE))
def test_w4a8_non_finite_activation_reaches_every_output_of_its_row(kind):
    m, n, k = 3, 70, 512
    codes, scales, zeros, _ = oracle.quantize_int4_g32(bf16_bits(int4_weight(n, k, 8)))
    x = bf16_bits(activation(m, k, 9))
    clean = oracle.qgemm_w4a8(x, codes, scales, zeros)
    x[2, 0] = NON_FINITE[kind]
    y = oracle.qgemm_w4a8(x, codes, scales, zeros)
    assert np.isnan(y[2]).all()
    np.testing.assert_array_equal(y[:2], clean[:2])
    assert np.isfinite(y[:2]).all()
