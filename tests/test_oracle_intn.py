"""Pins for the oracle's INT5 / INT6 group-32 quantizer (the pages' INT5/INT6
family with the INT4 recipe of `_packed_with_dense`) and its bit-plane packed
layout.

Checked against hand-worked groups (tests/golden/intn_g32_groups.txt), exact
invariants with L = 2^bits - 1 steps, an exact round trip on grid values, a
hand-computed byte map of the layout, and the dequant-then-dot GEMM's one-hot
closed form on codes above 15.
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


@pytest.mark.parametrize("case", read_cases("intn_g32_groups.txt"), ids=lambda c: c["name"])
def test_hand_worked_groups(case):
    s, z, q, f = oracle.quantize_group32_bits(case["bits"], case["width"])
    assert s == case["scale"], f"scale {s:#06x} != {case['scale']:#06x}"
    assert z == case["zp"]
    assert q.tolist() == case["codes"].tolist()
    assert f == case["flags"]


@pytest.mark.parametrize("bits", [5, 6])
def test_invariants_exact(bits):
    L = (1 << bits) - 1
    g = torch.Generator().manual_seed(20 + bits)
    w = torch.cat([torch.randn(6, 256, generator=g) * 10.0 ** torch.randint(-6, 4, (6, 1), generator=g),
                   torch.randn(2, 256, generator=g).abs() + 1.0,
                   -torch.randn(2, 256, generator=g).abs()]).to(torch.bfloat16)
    wb = bf16_bits(w)
    codes, scales, zeros, f = oracle.quantize_intn_g32(wb, bits)
    assert f == 0
    for r in range(wb.shape[0]):
        for gi in range(wb.shape[1] // 32):
            vals = [bf16_value(int(b)) for b in wb[r, 32 * gi:32 * gi + 32]]
            rng = max([Fraction(0)] + vals) - min([Fraction(0)] + vals)
            sb = int(scales[r, gi])
            s = fp16_value(sb)
            zp = int(zeros[r, gi])
            assert 0 <= zp <= L
            if rng == 0:
                assert sb == 0x3C00
                continue
            assert L * s >= rng and (sb == 1 or L * fp16_value(sb - 1) < rng), "scale not the minimal cover"
            for i, v in enumerate(vals):
                q = int(codes[r, 32 * gi + i])
                assert 0 <= q <= L
                assert abs(v - (q - zp) * s) <= s / 2


@pytest.mark.parametrize("bits", [5, 6])
def test_round_trip_on_grid(bits):
    """Values (q - zp) * s with s a power of two, q spanning 0..L: exact in
    bf16, and the quantizer must give back s, zp and q."""
    L = (1 << bits) - 1
    rng = np.random.default_rng(bits)
    for trial in range(20):
        e = int(rng.integers(-12, 4))
        s = 2.0 ** e
        zp = int(rng.integers(0, L + 1))
        q = rng.integers(0, L + 1, 32)
        q[rng.integers(0, 32)] = 0
        q[rng.integers(0, 32)] = L
        if (q == 0).sum() == 0 or (q == L).sum() == 0:
            continue
        v = ((q - zp) * s).astype(np.float32)
        b = (v.view(np.uint32) >> 16).astype(np.uint16)
        assert ((b.astype(np.uint32) << 16).view(np.float32) == v).all()
        sb, z, qq, f = oracle.quantize_group32_bits(b, bits)
        assert fp16_value(sb) == Fraction(s) and z == zp and qq.tolist() == q.tolist() and f == 0


def _pattern(n, k, bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(40 + bits)
    codes = rng.integers(0, L + 1, (n, k)).astype(np.uint8)
    codes[0] = np.arange(k) % (L + 1)
    codes[1] = 48 % (L + 1) if bits == 6 else 16
    codes[2] = 32 if bits == 6 else 0
    codes[3] = np.where(np.arange(k) % 2 == 0, 16, 0)
    scales = np.fromfunction(lambda r, g: 0x3C00 + 16 * r + g, (n, k // 32), dtype=np.int64).astype(np.uint16)
    zeros = np.fromfunction(lambda r, g: (r + 3 * g) % (L + 1), (n, k // 32), dtype=np.int64).astype(np.uint8)
    return codes, scales, zeros


def test_packed_layout_known_answer_int6():
    """Tile 64 x 256 = 8192 low-nibble bytes + 4096 plane bytes + 1024 scale + 512 zero bytes."""
    n, k = 65, 512
    packed = oracle.pack_intn(*_pattern(n, k, 6), bits=6)
    assert packed.size == 2 * 2 * 13824 == oracle.intn_packed_bytes(n, k, 6)
    # row 0, group 0: codes k = 0..31; high bit 0 set for k = 16..31 (lo dwords 2, 3 ->
    # plane dword 1): even k at bits 0,2,4,6 of bytes 4 (d = 2) and 5 (d = 3), odd k 16 higher
    assert packed[8192:8200].tolist() == [0, 0, 0, 0, 0x55, 0x55, 0x55, 0x55]
    # row 1: code 48 = 0b110000, both high bits of every code set
    assert packed[8192 + 8:8192 + 16].tolist() == [0xFF] * 8
    # row 2: code 32 = 0b100000, high bit 1 only: bits 1,3,5,7 of every byte
    assert packed[8192 + 16:8192 + 24].tolist() == [0xAA] * 8
    # row 3: 16 on even k only: the low (even) half of each plane dword
    assert packed[8192 + 24:8192 + 32].tolist() == [0x55, 0x55, 0, 0, 0x55, 0x55, 0, 0]
    assert packed[0] == 0x20 and packed[1] == 0x64      # low nibbles exactly as version 1
    assert packed[12288] == 0x00 and packed[12289] == 0x3C          # scale (row 0, group 0)
    assert packed[12288 + 32 + 6] == 0x23 and packed[12288 + 32 + 7] == 0x3C   # (row 2, group 3)
    assert packed[13312 + 8:13312 + 16].tolist() == [1, 4, 7, 10, 13, 16, 19, 22]   # zeros of row 1
    assert packed[13824 + 8192:13824 + 8200].tolist() == [0, 0, 0, 0, 0x55, 0x55, 0x55, 0x55]  # tile 1, k 256..287
    assert packed[2 * 13824 + 8192 + 8:2 * 13824 + 8192 + 16].tolist() == [0] * 8      # padding row 65


def test_packed_layout_known_answer_int5():
    """Tile 64 x 256 = 8192 low-nibble bytes + 2048 plane bytes + 1024 scale + 512 zero bytes."""
    n, k = 64, 256
    packed = oracle.pack_intn(*_pattern(n, k, 5), bits=5)
    assert packed.size == 11776 == oracle.intn_packed_bytes(n, k, 5)
    # row 0: codes k % 32 = k; the high bit for k = 16..31: even k at 4d + p (d = 2, 3 -> byte 1),
    # odd k at 16 + 4d + p (byte 3)
    assert packed[8192:8196].tolist() == [0, 0xFF, 0, 0xFF]
    assert packed[8196:8200].tolist() == [0xFF] * 4      # row 1: code 16 everywhere
    assert packed[8200:8204].tolist() == [0] * 4         # row 2: code 0
    assert packed[8204:8208].tolist() == [0xFF, 0xFF, 0, 0]   # row 3: 16 on even k
    assert packed[10240 + 16] == 0x10 and packed[10241 + 16] == 0x3C     # scale (row 1, group 0)
    assert packed[11264 + 16:11264 + 24].tolist() == [2, 5, 8, 11, 14, 17, 20, 23]   # zeros of row 2


@pytest.mark.parametrize("bits", [5, 6])
def test_pack_unpack_round_trip(bits):
    n, k = 130, 768
    codes, scales, zeros = _pattern(n, k, bits)
    c2, s2, z2 = oracle.unpack_intn(oracle.pack_intn(codes, scales, zeros, bits), n, k, bits)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(z2, zeros)


@pytest.mark.parametrize("bits", [5, 6])
def test_gemm_one_hot_on_wide_codes(bits):
    L = (1 << bits) - 1
    rng = np.random.default_rng(60 + bits)
    n, k = 32, 256
    codes = rng.integers(0, L + 1, (n, k)).astype(np.uint8)
    scales = rng.integers(0x2000, 0x4800, (n, k // 32)).astype(np.uint16)
    zeros = rng.integers(0, L + 1, (n, k // 32)).astype(np.uint8)
    for k0 in (0, 100, 255):
        x = np.zeros((1, k), np.uint16)
        x[0, k0] = 0x3F80
        y = oracle.qgemm_w4a16(x, codes, scales, zeros)
        for r in range(n):
            want = (int(codes[r, k0]) - int(zeros[r, k0 // 32])) * fp16_value(int(scales[r, k0 // 32]))
            assert Fraction(y[0, r]) == want
