"""Pins for the CPU oracle's INT4 group-32 quantizer, packed layout and W4A16 GEMM.

The oracle is checked against things other than itself: hand-worked groups
(tests/golden/int4_g32_groups.txt), exact invariants of min-max quantization,
an exact round trip on values already on the grid, a known-answer byte map of
the packed layout, closed forms (one-hot and integer inputs) and exact
rational brute force on tiny inputs.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import oracle
from golden_io import read_cases
from synthetic_inputs import bf16_bits, int4_weight

# ---------------------------------------------------------------- helpers


def fp16_value(bits: int) -> Fraction:
    """Exact value of an fp16 pattern via numpy's binary16 (not the oracle's decoder)."""
    return Fraction(float(np.array([bits], np.uint16).view(np.float16)[0]))


def bf16_value(bits: int) -> Fraction:
    return Fraction(float((np.array([bits], np.uint32) << 16).view(np.float32)[0]))


def prev_fp16(bits: int) -> int:
    return bits - 1  # positive finite fp16 patterns are ordered like their values


# ---------------------------------------------------------------- quantizer


@pytest.mark.parametrize("case", read_cases("int4_g32_groups.txt"), ids=lambda c: c["name"])
def test_hand_worked_groups(case):
    s, z, q, f = oracle.quantize_group32(case["bits"])
    assert s == case["scale"], f"scale {s:#06x} != {case['scale']:#06x}"
    assert z == case["zp"]
    assert q.tolist() == case["codes"].tolist()
    assert f == case["flags"]


def _check_group_invariants(bits32, s_bits, zp, q):
    vals = [bf16_value(int(b)) for b in bits32]
    lo = min([Fraction(0)] + vals)
    hi = max([Fraction(0)] + vals)
    r = hi - lo
    s = fp16_value(s_bits)
    assert s > 0
    assert 0 <= zp <= 15
    assert all(0 <= int(c) <= 15 for c in q)
    if r == 0:
        assert s_bits == 0x3C00 and zp == 0 and not q.any()
        return
    assert 15 * s >= r, "scale too small to cover the range"
    if s_bits > 1:
        assert 15 * fp16_value(prev_fp16(s_bits)) < r, "scale not minimal"
    for v, c in zip(vals, q):
        err = abs(v - (int(c) - zp) * s)
        assert err <= s / 2, f"dequant error {float(err)} > s/2 = {float(s) / 2}"


def _random_groups(rng, count):
    """bf16 groups of assorted character: gaussian, one-sign, tiny, wide, sparse."""
    out = []
    for i in range(count):
        kind = i % 6
        if kind == 0:
            v = rng.standard_normal(32)
        elif kind == 1:
            v = np.abs(rng.standard_normal(32)) + 3.0          # all positive, far from 0
        elif kind == 2:
            v = -np.abs(rng.standard_normal(32)) * 1e-3         # all negative, small
        elif kind == 3:
            v = rng.standard_normal(32) * 1e-30                 # tiny (fp16-subnormal scales)
        elif kind == 4:
            v = rng.standard_normal(32) * 3e4                   # large (near fp16 top)
        else:
            v = rng.standard_normal(32) * (rng.random(32) < 0.2)  # mostly zeros
        b = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)  # truncate to bf16
        out.append(b)
    return out


def test_invariants_on_assorted_groups():
    rng = np.random.default_rng(1234)
    for g in _random_groups(rng, 600):
        s, z, q, f = oracle.quantize_group32(g)
        assert f == 0
        _check_group_invariants(g, s, z, q)


def test_invariants_on_randn_weights():
    w = bf16_bits(int4_weight(48, 256, seed=5))
    codes, scales, zeros, f = oracle.quantize_int4_g32(w)
    assert f == 0
    for row in range(0, 48, 7):
        for g in range(8):
            _check_group_invariants(w[row, g * 32:(g + 1) * 32], int(scales[row, g]),
                                    int(zeros[row, g]), codes[row, g * 32:(g + 1) * 32])


def test_round_trip_is_exact_on_the_grid():
    """w = (q - zp) * s with s of <= 4 significant bits and codes 0 and 15 present in
    every group is exactly bf16; quantizing it must give back (q, zp, s)."""
    rng = np.random.default_rng(7)
    n, k = 16, 256
    q = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    q[:, 0::32] = 0
    q[:, 1::32] = 15
    zp = rng.integers(0, 16, size=(n, k // 32)).astype(np.uint8)
    mant = rng.integers(8, 16, size=(n, k // 32))           # 4 significant bits
    expo = rng.integers(-10, 3, size=(n, k // 32))
    s = mant.astype(np.float64) * np.exp2(expo - 3)
    s_bits = s.astype(np.float16).view(np.uint16)
    assert (s_bits.view(np.float16).astype(np.float64) == s).all()
    w = (q.astype(np.float64).reshape(n, -1, 32) - zp[:, :, None]) * s[:, :, None]
    w = w.reshape(n, k)
    w_bits = (w.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert (oracle.bf16_to_float64(w_bits) == w).all(), "test values must be bf16-exact"
    codes, scales, zeros, f = oracle.quantize_int4_g32(w_bits)
    assert f == 0
    np.testing.assert_array_equal(codes, q)
    np.testing.assert_array_equal(zeros, zp)
    np.testing.assert_array_equal(scales, s_bits)


def test_matrix_quantizer_is_the_group_quantizer_per_group():
    w = bf16_bits(int4_weight(5, 512, seed=9))
    codes, scales, zeros, _ = oracle.quantize_int4_g32(w)
    for row in range(5):
        for g in range(16):
            s, z, q, _ = oracle.quantize_group32(w[row, g * 32:(g + 1) * 32])
            assert scales[row, g] == s and zeros[row, g] == z
            np.testing.assert_array_equal(codes[row, g * 32:(g + 1) * 32], q)


def test_flags_are_ored_over_the_matrix():
    w = np.zeros((3, 64), np.uint16)
    w[1, 40] = 0x7F80  # +inf in row 1, group 1
    w[2, 3] = 0x4A00   # 2^21: range 2^21 > 15 * 65504 in row 2, group 0
    _, scales, _, f = oracle.quantize_int4_g32(w)
    assert f == 3
    assert scales[1, 1] == 0x7E00 and scales[2, 0] == 0x7BFF and scales[0, 0] == 0x3C00


# ---------------------------------------------------------------- packed layout


def _known_pattern(n, k):
    codes = np.fromfunction(lambda r, c: (5 * r + c) % 16, (n, k), dtype=np.int64).astype(np.uint8)
    scales = np.fromfunction(lambda r, g: 0x3C00 + 16 * r + g, (n, k // 32), dtype=np.int64).astype(np.uint16)
    zeros = np.fromfunction(lambda r, g: (r + 3 * g) % 16, (n, k // 32), dtype=np.int64).astype(np.uint8)
    return codes, scales, zeros


def test_packed_layout_known_answer():
    """Byte values worked by hand from the layout (tile = 64 rows x 256 k, 9472 B)."""
    n, k = 65, 512
    packed = oracle.pack_int4(*_known_pattern(n, k))
    assert packed.size == 2 * 2 * 9472 == oracle.int4_packed_bytes(n, k)
    expect = {
        # tile 0 (row block 0, k tile 0); row 0 codes are k % 16.
        # dword 0 nibbles p0..p7 hold k = 0, 2, 4, 6, 1, 3, 5, 7
        0: 0x20, 1: 0x64, 2: 0x31, 3: 0x75,
        4: 0xA8, 5: 0xEC, 6: 0xB9, 7: 0xFD,          # dword 1: k = 8..15
        16: 0x75,                                     # chunk (group 0, row 1): codes (5 + k) % 16
        1024: 0x20,                                   # chunk (group 1, row 0): k = 32, 34
        8192: 0x00, 8193: 0x3C,                       # scale (row 0, group 0) = 0x3C00
        8230: 0x23, 8231: 0x3C,                       # scale (row 2, group 3) = 0x3C23
        9220: 0x41, 9221: 0xA7, 9222: 0x0D, 9223: 0x63,  # zeros of row 1: 1,4,7,10,13,0,3,6
        # tile 1 (row block 0, k tile 1): group 8 onwards
        9472: 0x20,
        9472 + 8192: 0x08, 9472 + 8193: 0x3C,         # scale (row 0, group 8) = 0x3C08
        # tile 2 (row block 1, k tile 0): only row 64 is real
        18944: 0x20,                                  # row 64 codes (320 + k) % 16 = k % 16
        18944 + 16: 0x00,                             # padding row 65
        18944 + 8192 + 16: 0x00, 18944 + 8192 + 17: 0x00,
        18944 + 9216 + 4: 0x00,
    }
    for off, val in expect.items():
        assert packed[off] == val, f"byte {off}: {packed[off]:#04x} != {val:#04x}"


def test_pack_unpack_round_trip_and_padding():
    rng = np.random.default_rng(3)
    n, k = 130, 768
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    scales = rng.integers(0, 0x7C00, (n, k // 32)).astype(np.uint16)
    zeros = rng.integers(0, 16, (n, k // 32)).astype(np.uint8)
    packed = oracle.pack_int4(codes, scales, zeros)
    c2, s2, z2 = oracle.unpack_int4(packed, n, k)
    np.testing.assert_array_equal(c2, codes)
    np.testing.assert_array_equal(s2, scales)
    np.testing.assert_array_equal(z2, zeros)
    # Rows 130..191 of the last row block are all zero bytes.
    c3, s3, z3 = oracle.unpack_int4(packed, 192, k)
    assert not c3[n:].any() and not s3[n:].any() and not z3[n:].any()


def test_every_packed_bit_is_owned_by_exactly_one_field():
    """All-ones fields fill every byte of a full tile; each single code lands in one nibble."""
    n, k = 64, 256
    packed = oracle.pack_int4(np.full((n, k), 15, np.uint8), np.full((n, 8), 0xFFFF, np.uint16),
                              np.full((n, 8), 15, np.uint8))
    assert (packed == 0xFF).all()
    seen = np.zeros(9472 * 2, np.int64)
    for r in (0, 17, 63):
        for kk in range(k):
            codes = np.zeros((n, k), np.uint8)
            codes[r, kk] = 1
            p = oracle.pack_int4(codes, np.zeros((n, 8), np.uint16), np.zeros((n, 8), np.uint8))
            nz = np.flatnonzero(p)
            assert nz.size == 1 and nz[0] < 8192
            assert p[nz[0]] in (0x01, 0x10)
            seen[nz[0] * 2 + (p[nz[0]] == 0x10)] += 1
    assert seen.max() == 1


# ---------------------------------------------------------------- W4A16 GEMM


def _quantized(n, k, seed):
    return oracle.quantize_int4_g32(bf16_bits(int4_weight(n, k, seed)))[:3]


def test_one_hot_activation_returns_a_dequantized_column():
    n, k = 40, 256
    codes, scales, zeros = _quantized(n, k, 11)
    for j in (0, 31, 32, 200, 255):
        x = np.zeros((1, k), np.uint16)
        x[0, j] = 0x3F80  # 1.0
        y = oracle.qgemm_w4a16(x, codes, scales, zeros)
        for row in range(n):
            want = (int(codes[row, j]) - int(zeros[row, j // 32])) * fp16_value(int(scales[row, j // 32]))
            assert Fraction(y[0, row]) == want


def test_integer_inputs_give_the_exact_integer_product():
    """Power-of-two scales and integer activations: every partial sum is exact in
    binary64, so the oracle must equal numpy's integer matmul bit for bit."""
    rng = np.random.default_rng(21)
    m, n, k = 3, 70, 512
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    zeros = rng.integers(0, 16, (n, k // 32)).astype(np.uint8)
    e = rng.integers(-3, 4, (n, k // 32))
    scales = np.exp2(e).astype(np.float16).view(np.uint16)
    xi = rng.integers(-8, 9, (m, k))
    x = (xi.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = oracle.qgemm_w4a16(x, codes, scales, zeros)
    # Exact reference in integers: scale everything by 2^3 so all terms are integral.
    wq = codes.astype(np.int64).reshape(n, -1, 32) - zeros[:, :, None].astype(np.int64)
    w8 = (wq * (2 ** (e + 3))[:, :, None]).reshape(n, k)
    want = (xi @ w8.T).astype(np.float64) / 8.0
    np.testing.assert_array_equal(y, want)


def test_bruteforce_exact_rationals_tiny():
    m, n, k = 2, 5, 256
    codes, scales, zeros = _quantized(n, k, 13)
    x = bf16_bits(int4_weight(m, k, 17))
    y = oracle.qgemm_w4a16(x, codes, scales, zeros)
    for mi in range(m):
        for row in range(n):
            exact = Fraction(0)
            absum = Fraction(0)
            for kk in range(k):
                t = bf16_value(int(x[mi, kk])) * (int(codes[row, kk]) - int(zeros[row, kk // 32])) \
                    * fp16_value(int(scales[row, kk // 32]))
                exact += t
                absum += abs(t)
            # binary64 accumulation of exact products: |err| <= k * 2^-53 * sum|t|
            assert abs(Fraction(y[mi, row]) - exact) <= k * Fraction(1, 2 ** 53) * absum


def test_rows_are_independent_and_threads_do_not_change_results():
    n, k = 300, 512
    codes, scales, zeros = _quantized(n, k, 23)
    x1 = bf16_bits(int4_weight(1, k, 29))
    x = np.concatenate([x1, x1, bf16_bits(int4_weight(1, k, 31))])
    y1 = oracle.qgemm_w4a16(x, codes, scales, zeros, threads=1)
    y8 = oracle.qgemm_w4a16(x, codes, scales, zeros, threads=8)
    np.testing.assert_array_equal(y1, y8)
    np.testing.assert_array_equal(y1[0], y1[1])
    assert not np.array_equal(y1[0], y1[2])
