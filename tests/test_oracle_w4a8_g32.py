"""Pins for the oracle's W4A8 with one activation scale per group of 32.

The pages test W4A8 against the W4A16 reference's precision class, with
Gaussian activations and with a few outlier channels 20-50x larger
(executorch test_int4_quantized_gemm.py, Int4QuantizedGemmPrecisionTest,
`_activation(..., outliers=True)`), but do not give the activation quantizer.
This variant applies the per-row rule of tests/golden/actquant_rows.txt to
each group of 32 consecutive k, so an outlier only coarsens its own group.

Pins (none re-types the oracle's formula):
  * hand-worked groups: rows built from the 32-entry fixtures, one fixture per
    group, must quantize to the fixtures' codes and scales;
  * invariants: groups are independent, scaling a group by a power of two
    scales its sx and leaves its codes, every nonzero group reaches +-127;
  * closed forms: activations already on the int8 grid with absmax 127 in
    every group give exactly the W4A16 result; K = 32 is the per-row W4A8;
  * exact rationals on a tiny case, zero groups contribute nothing.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
import synthetic_inputs as si
from golden_io import read_cases

CASES = read_cases("actquant_rows.txt")


def _f32(v):
    return Fraction(float(np.float32(v)))


@pytest.mark.parametrize("order", [(0, 1, 2), (2, 0, 1), (1, 2, 0, 0), (3, 4, 5, 6), (4, 0, 6, 3, 5, 1)])
def test_groups_quantize_like_the_hand_worked_rows(order):
    bits = np.concatenate([CASES[i]["bits"] for i in order]).reshape(1, -1)
    xq, sx = oracle.actquant_int8_g32(bits)
    for g, i in enumerate(order):
        assert list(xq[0, 32 * g:32 * g + 32]) == list(CASES[i]["codes"]), (g, CASES[i]["name"])
        assert int(sx[0, g].view(np.uint32)) == CASES[i]["sx"], (g, CASES[i]["name"])


def test_groups_are_independent_and_power_of_two_equivariant():
    x = si.activation(2, 256, 11)
    xq, sx = oracle.actquant_int8_g32(si.bf16_bits(x))
    x2 = x.clone()
    x2[:, 96:128] = x2[:, 96:128] * 16          # group 3, exact in bf16
    x2[1, 200] = 0                                # and one value of group 6, row 1
    xq2, sx2 = oracle.actquant_int8_g32(si.bf16_bits(x2))
    keep = [g for g in range(8) if g != 3]
    for g in keep:
        if g == 6:
            assert (xq2[0, 192:224] == xq[0, 192:224]).all() and sx2[0, 6] == sx[0, 6]
            continue
        assert (xq2[:, 32 * g:32 * g + 32] == xq[:, 32 * g:32 * g + 32]).all(), g
        assert (sx2[:, g] == sx[:, g]).all(), g
    assert (xq2[:, 96:128] == xq[:, 96:128]).all()
    assert (sx2[:, 3] == sx[:, 3] * 16).all()


def test_every_nonzero_group_reaches_127_and_codes_are_bounded():
    x = si.activation(3, 512, 5)
    x[1, 64:96] = 0
    xq, sx = oracle.actquant_int8_g32(si.bf16_bits(x))
    g = xq.reshape(3, 16, 32).astype(np.int32)
    assert np.abs(g).max() <= 127
    amax = np.abs(g).max(axis=2)
    assert amax[1, 2] == 0 and sx[1, 2] == 0
    mask = np.ones_like(amax, bool)
    mask[1, 2] = False
    assert (amax[mask] == 127).all()


def _int4_layer(n, k, seed):
    w = si.int4_weight(n, k, seed)
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    return codes, scales, zeros


def test_equals_w4a16_when_every_group_is_on_the_int8_grid():
    n, k = 64, 512
    codes, scales, zeros = _int4_layer(n, k, 21)
    rng = np.random.default_rng(8)
    xi = rng.integers(-127, 128, (2, k))
    xi[:, ::32] = 127 * np.sign(rng.standard_normal((2, k // 32))).astype(np.int64)   # absmax 127 per group
    import torch
    x = si.bf16_bits(torch.tensor(xi, dtype=torch.bfloat16))
    xq, sx = oracle.actquant_int8_g32(x)
    assert (xq == xi).all() and (sx == 1.0).all()
    y8 = oracle.qgemm_w4a8_g32(x, codes, scales, zeros)
    y16 = oracle.qgemm_w4a16(x, codes, scales, zeros)
    np.testing.assert_allclose(y8, y16, rtol=1e-12, atol=1e-9)


def test_k32_is_the_per_row_w4a8():
    n, k = 48, 32
    codes, scales, zeros = _int4_layer(n, k, 4)
    x = si.bf16_bits(si.activation(3, k, 6))
    np.testing.assert_array_equal(oracle.qgemm_w4a8_g32(x, codes, scales, zeros),
                                  oracle.qgemm_w4a8(x, codes, scales, zeros))


def test_exact_rationals_tiny():
    n, k = 3, 96
    codes, scales, zeros = _int4_layer(n, k, 9)
    x = si.bf16_bits(si.activation(2, k, 10))
    xq, sx = oracle.actquant_int8_g32(x)
    y = oracle.qgemm_w4a8_g32(x, codes, scales, zeros)
    s = oracle.fp16_to_float64(scales)
    for m in range(2):
        for r in range(n):
            tot = Fraction(0)
            for g in range(k // 32):
                isum = sum(int(xq[m, 32 * g + i]) * (int(codes[r, 32 * g + i]) - int(zeros[r, g]))
                           for i in range(32))
                tot += _f32(sx[m, g]) * Fraction(float(s[r, g])) * isum
            assert abs(Fraction(float(y[m, r])) - tot) <= abs(tot) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 12)


def test_zero_groups_contribute_nothing():
    n, k = 32, 256
    codes, scales, zeros = _int4_layer(n, k, 12)
    x = si.activation(2, k, 13)
    x[0] = 0
    y = oracle.qgemm_w4a8_g32(si.bf16_bits(x), codes, scales, zeros)
    assert (y[0] == 0).all() and (y[1] != 0).any()
    x2 = x.clone()
    x2[1, 64:96] = 0
    part = oracle.qgemm_w4a8_g32(si.bf16_bits(x2), codes, scales, zeros)
    x3 = x.clone()
    x3[1, :64] = 0
    x3[1, 96:] = 0
    only = oracle.qgemm_w4a8_g32(si.bf16_bits(x3), codes, scales, zeros)
    # the groups add up: (all groups) = (all but group 2) + (group 2 alone)
    np.testing.assert_allclose(y[1], part[1] + only[1], rtol=1e-12, atol=1e-12)


def _outliers(x):
    """The pages' outlier recipe: channels 0, K/3, 2K/3, K-1 times 50, 35, 25, 20."""
    import torch
    k = x.shape[1]
    x = x.clone()
    for c, f in zip((0, k // 3, 2 * k // 3, k - 1), (50.0, 35.0, 25.0, 20.0)):
        x[:, c] = (x[:, c].float() * torch.tensor(f, dtype=torch.bfloat16).float()).to(torch.bfloat16)
    return x


@pytest.mark.parametrize("n,k", si.SMALL_SHAPES)
def test_precision_class_against_dense_small_shapes(n, k):
    """Why this reading exists: with one activation scale per group, the
    oracle meets the pages' dense-reference precision checks for Gaussian and
    outlier activations at every W4A8 bucket; one scale per row does not on
    the outlier case."""
    from tolerance import precision_class_failures

    w = si.int4_weight(n, k, 1200 + si.SMALL_SHAPES.index((n, k)))
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    dense = oracle.bf16_to_float64(si.bf16_bits(w))
    row_failed = False
    for m in si.DECODE_M:
        for outl in (False, True):
            x = si.activation(m, k, 9100 + 31 * si.SMALL_SHAPES.index((n, k)) + m)
            if outl:
                x = _outliers(x)
            xb = si.bf16_bits(x)
            ref_dense = oracle.bf16_to_float64(xb) @ dense.T
            a16 = oracle.qgemm_w4a16(xb, codes, scales, zeros)
            bad = precision_class_failures(oracle.qgemm_w4a8_g32(xb, codes, scales, zeros), a16, ref_dense)
            assert not bad, (m, outl, bad)
            if outl and precision_class_failures(oracle.qgemm_w4a8(xb, codes, scales, zeros), a16, ref_dense):
                row_failed = True
    assert row_failed, "per-row activation scales unexpectedly pass the outlier case here"


@pytest.mark.parametrize("bits", [0x7FC0, 0x7F80, 0xFF80], ids=["nan", "+inf", "-inf"])
def test_non_finite_activation_poisons_its_group_and_row_only(bits):
    """A NaN or infinite activation leaves its group of 32 without a finite
    scale (sx = NaN, codes 0); that group reaches every output of the row,
    which become NaN, and no other group or row changes."""
    m, n, k = 2, 40, 512
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(si.int4_weight(n, k, 3)))
    x = si.bf16_bits(si.activation(m, k, 4))
    clean_q, clean_s = oracle.actquant_int8_g32(x)
    clean_y = oracle.qgemm_w4a8_g32(x, codes, scales, zeros)
    x[0, 5 * 32 + 17] = bits
    xq, sx = oracle.actquant_int8_g32(x)
    assert np.isnan(sx[0, 5]) and (xq[0, 160:192] == 0).all()
    keep = np.ones(sx.shape, bool)
    keep[0, 5] = False
    np.testing.assert_array_equal(sx[keep], clean_s[keep])
    np.testing.assert_array_equal(np.delete(xq[0], np.s_[160:192]), np.delete(clean_q[0], np.s_[160:192]))
    np.testing.assert_array_equal(xq[1], clean_q[1])
    y = oracle.qgemm_w4a8_g32(x, codes, scales, zeros)
    assert np.isnan(y[0]).all()
    np.testing.assert_array_equal(y[1], clean_y[1])
