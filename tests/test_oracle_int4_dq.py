"""Pins for the oracle's INT4 group-32 quantizer with scale codes (uint8 code
times a per-row fp16 step, the storage of executorch
test_int4_quantized_gemm.py `_packed_with_dense`), its packed layout (version
2) and its W4A16 GEMM.

Checked against things other than the oracle itself: hand-worked rows
(tests/golden/int4_dq_rows.txt), exact invariants of the reading (minimal step,
minimal code, every value within half a step), a hand-computed byte map of
the layout, a one-hot closed form, the fp16-scale GEMM where both forms hold
the same scales, and exact rational brute force.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from golden_io import read_cases
from synthetic_inputs import bf16_bits


def fp16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], np.uint16).view(np.float16)[0]))


def bf16_value(bits: int) -> Fraction:
    return Fraction(float((np.array([bits], np.uint32) << 16).view(np.float32)[0]))


@pytest.mark.parametrize("case", read_cases("int4_dq_rows.txt", width=64), ids=lambda c: c["name"])
def test_hand_worked_rows(case):
    q, sc, st, z, f = oracle.quantize_int4_g32_dq(case["bits"].reshape(1, 64))
    assert int(st[0]) == case["step"], f"step {int(st[0]):#06x} != {case['step']:#06x}"
    assert sc[0].tolist() == [case["scode0"], case["scode1"]]
    assert z[0].tolist() == [case["zp0"], case["zp1"]]
    assert q[0].tolist() == case["codes"].tolist()
    assert f == case["flags"]


def _rows_for_invariants():
    g = torch.Generator().manual_seed(11)
    rows = []
    # randn rows whose groups have very different ranges (the codes spread over 1..255)
    w = torch.randn(8, 256, generator=g) * torch.logspace(-3, 1, 8)[torch.randperm(8, generator=g)].repeat_interleave(32)
    rows.append(w)
    rows.append(torch.randn(6, 256, generator=g) * 1e-3)
    rows.append(torch.randn(4, 256, generator=g).abs() + 0.5)            # one-sign groups
    sparse = torch.zeros(4, 256)
    sparse[torch.rand(4, 256, generator=g) < 0.05] = 3.0
    rows.append(sparse)
    return torch.cat(rows).to(torch.bfloat16)


def test_invariants_exact():
    wb = bf16_bits(_rows_for_invariants())
    n, k = wb.shape
    q, sc, st, z, f = oracle.quantize_int4_g32_dq(wb)
    assert f == 0
    for r in range(n):
        vals = [bf16_value(int(b)) for b in wb[r]]
        ranges = []
        for g in range(k // 32):
            grp = vals[32 * g:32 * g + 32]
            ranges.append(max([Fraction(0)] + grp) - min([Fraction(0)] + grp))
        big = max(ranges)
        step_bits = int(st[r])
        step = fp16_value(step_bits)
        if big == 0:
            assert step_bits == 0x3C00
        else:
            assert 3825 * step >= big, "row step too small"
            assert step_bits == 1 or 3825 * fp16_value(step_bits - 1) < big, "row step not minimal"
        for g in range(k // 32):
            c = int(sc[r, g])
            assert 1 <= c <= 255
            assert 15 * c * step >= ranges[g], "group scale does not cover its range"
            assert c == 1 or 15 * (c - 1) * step < ranges[g], "scale code not minimal"
            s = c * step
            zp = int(z[r, g])
            assert 0 <= zp <= 15
            for i in range(32):
                code = int(q[r, 32 * g + i])
                assert 0 <= code <= 15
                err = abs(vals[32 * g + i] - (code - zp) * s)
                assert err <= s / 2, f"row {r} group {g}: error {float(err)} > s/2"


def _known_pattern(n, k):
    codes = np.fromfunction(lambda r, c: (5 * r + c) % 16, (n, k), dtype=np.int64).astype(np.uint8)
    scode = np.fromfunction(lambda r, g: (7 * r + 3 * g + 1) % 256, (n, k // 32), dtype=np.int64).astype(np.uint8)
    sstep = (0x3C00 + np.arange(n)).astype(np.uint16)
    zeros = np.fromfunction(lambda r, g: (r + 3 * g) % 16, (n, k // 32), dtype=np.int64).astype(np.uint8)
    return codes, scode, sstep, zeros


def test_packed_layout_known_answer():
    """Bytes worked by hand: row block = 128-byte head of row steps + K/256 tiles of 8960 B."""
    n, k = 65, 512
    packed = oracle.pack_int4_dq(*_known_pattern(n, k))
    assert packed.size == 2 * (128 + 2 * 8960) == oracle.int4_dq_packed_bytes(n, k)
    expect = {
        0: 0x00, 1: 0x3C, 4: 0x02, 5: 0x3C,          # steps of rows 0 and 2
        128: 0x20, 129: 0x64, 128 + 16: 0x75,         # codes as in version 1
        128 + 8192: 0x01,                             # scale code (row 0, group 0) = 1
        128 + 8192 + 16 + 3: 0x18,                    # (row 2, group 3) = 14 + 9 + 1 = 24
        128 + 8704 + 4: 0x41, 128 + 8704 + 5: 0xA7,   # zeros of row 1: 1,4,7,10,13,0,3,6
        128 + 8704 + 6: 0x0D, 128 + 8704 + 7: 0x63,
        128 + 8960: 0x20,                             # tile 1 codes, row 0, k = 256, 258
        128 + 8960 + 8192: 0x19,                      # scale code (row 0, group 8) = 25
        18048: 0x40, 18049: 0x3C,                     # block 1 head: row 64 step 0x3C40
        18050: 0x00, 18051: 0x00,                     # padding row 65
        18176: 0x20, 18176 + 16: 0x00,                # row 64 codes; padding row 65 codes
        18176 + 8192: 0xC1,                           # scale code (row 64, group 0) = 449 % 256
    }
    for off, val in expect.items():
        assert packed[off] == val, f"byte {off}: {packed[off]:#04x} != {val:#04x}"


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(5)
    n, k = 130, 768
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    scode = rng.integers(0, 256, (n, k // 32)).astype(np.uint8)
    sstep = rng.integers(0, 0x7C00, n).astype(np.uint16)
    zeros = rng.integers(0, 16, (n, k // 32)).astype(np.uint8)
    c2, s2, t2, z2 = oracle.unpack_int4_dq(oracle.pack_int4_dq(codes, scode, sstep, zeros), n, k)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scode)
    np.testing.assert_array_equal(t2, sstep)
    np.testing.assert_array_equal(z2, zeros)


def test_gemm_one_hot_closed_form():
    rng = np.random.default_rng(7)
    n, k = 40, 256
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    scode = rng.integers(1, 256, (n, k // 32)).astype(np.uint8)
    sstep = rng.integers(0x0400, 0x5000, n).astype(np.uint16)
    zeros = rng.integers(0, 16, (n, k // 32)).astype(np.uint8)
    for k0 in (0, 37, 255):
        x = np.zeros((1, k), np.uint16)
        x[0, k0] = 0x3F80   # bf16 1.0
        y = oracle.qgemm_w4a16_dq(x, codes, scode, sstep, zeros)
        for r in range(n):
            want = (int(codes[r, k0]) - int(zeros[r, k0 // 32])) * int(scode[r, k0 // 32]) * fp16_value(int(sstep[r]))
            assert Fraction(y[0, r]) == want


def test_gemm_equals_fp16_scale_form_when_scales_are_fp16():
    """With power-of-two codes the group scales c*step are themselves fp16
    values: the scale-code GEMM must then equal the (separately pinned)
    fp16-scale GEMM bit for bit."""
    rng = np.random.default_rng(9)
    n, k, m = 24, 512, 3
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    scode = (1 << rng.integers(0, 8, (n, k // 32))).astype(np.uint8)
    sstep = rng.integers(0x1000, 0x4000, n).astype(np.uint16)     # 2^-11 .. 2, room for x128
    zeros = rng.integers(0, 16, (n, k // 32)).astype(np.uint8)
    s64 = scode.astype(np.float64) * sstep.view(np.float16).astype(np.float64)[:, None]
    scales = s64.astype(np.float16)
    assert (scales.astype(np.float64) == s64).all()
    x = bf16_bits(torch.randn(m, k, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16))
    y_dq = oracle.qgemm_w4a16_dq(x, codes, scode, sstep, zeros)
    y_fp16 = oracle.qgemm_w4a16(x, codes, scales.view(np.uint16), zeros)
    np.testing.assert_array_equal(y_dq, y_fp16)


def test_gemm_rational_brute_force():
    rng = np.random.default_rng(13)
    m, n, k = 2, 3, 64
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    scode = rng.integers(1, 256, (n, k // 32)).astype(np.uint8)
    sstep = rng.integers(0x0400, 0x5000, n).astype(np.uint16)
    zeros = rng.integers(0, 16, (n, k // 32)).astype(np.uint8)
    x = bf16_bits(torch.randn(m, k, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16))
    y = oracle.qgemm_w4a16_dq(x, codes, scode, sstep, zeros)
    for i in range(m):
        for r in range(n):
            exact = sum(bf16_value(int(x[i, kk])) * (int(codes[r, kk]) - int(zeros[r, kk // 32]))
                        * int(scode[r, kk // 32]) * fp16_value(int(sstep[r])) for kk in range(k))
            assert abs(Fraction(y[i, r]) - exact) <= abs(exact) * Fraction(1, 2 ** 45) + Fraction(1, 2 ** 80)


@pytest.mark.parametrize("per_group", [False, True])
def test_w4a8_equals_fp16_scale_form_when_scales_are_fp16(per_group):
    """Power-of-two codes make c*step an fp16 value: the scale-code W4A8 must
    then equal the (separately pinned) fp16-scale W4A8 bit for bit."""
    rng = np.random.default_rng(21)
    n, k, m = 24, 512, 3
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    scode = (1 << rng.integers(0, 8, (n, k // 32))).astype(np.uint8)
    sstep = rng.integers(0x1000, 0x4000, n).astype(np.uint16)
    zeros = rng.integers(0, 16, (n, k // 32)).astype(np.uint8)
    s64 = scode.astype(np.float64) * sstep.view(np.float16).astype(np.float64)[:, None]
    scales = s64.astype(np.float16)
    assert (scales.astype(np.float64) == s64).all()
    x = bf16_bits(torch.randn(m, k, generator=torch.Generator().manual_seed(6)).to(torch.bfloat16))
    if per_group:
        a = oracle.qgemm_w4a8_g32_dq(x, codes, scode, sstep, zeros)
        b = oracle.qgemm_w4a8_g32(x, codes, scales.view(np.uint16), zeros)
    else:
        a = oracle.qgemm_w4a8_dq(x, codes, scode, sstep, zeros)
        b = oracle.qgemm_w4a8(x, codes, scales.view(np.uint16), zeros)
    np.testing.assert_array_equal(a, b)


def test_w4a8_on_int8_grid_equals_w4a16():
    """Activations already on the int8 grid with absmax 127 quantize to
    themselves with sx = 1: W4A8 then equals W4A16 on the same weight."""
    rng = np.random.default_rng(22)
    n, k, m = 16, 256, 2
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    scode = rng.integers(1, 256, (n, k // 32)).astype(np.uint8)
    sstep = rng.integers(0x0400, 0x3000, n).astype(np.uint16)
    zeros = rng.integers(0, 16, (n, k // 32)).astype(np.uint8)
    xi = rng.integers(-127, 128, (m, k)).astype(np.float32)
    xi[:, 0] = 127.0
    x = (xi.view(np.uint32) >> 16).astype(np.uint16)
    a16 = oracle.qgemm_w4a16_dq(x, codes, scode, sstep, zeros)
    a8 = oracle.qgemm_w4a8_dq(x, codes, scode, sstep, zeros)
    np.testing.assert_allclose(a8, a16, rtol=1e-12, atol=1e-12)
