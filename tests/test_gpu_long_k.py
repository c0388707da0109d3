"""GPU parity at a long reduction: K = 131072 (512 tiles of 256 k, six times
the longest K of the pages' layers, 5376 x 21504), N = 64 and a one-row
N = 1, for every entry point and each kernel family; W8A16 at its largest K
(65536).  Long K exercises the split-K ranges, the 64-bit offsets into x and
the packed weight, and fp32 accumulation over hundreds of groups.
"""
from __future__ import annotations

import functools

import pytest
import torch

import oracle
import synthetic_inputs as si
from tolerance import assert_w16

pytestmark = pytest.mark.gpu

import gemm_decode_qgemm_amd as qg  # noqa: E402

K = 131072


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=2)
def _w(n):
    return si.int4_weight(n, K, 4000 + n)


@pytest.mark.parametrize("n", [64, 1])
@pytest.mark.parametrize("m", [1, 4, 16, 64])
def test_w4a16_long_k(dev, n, m):
    w = _w(n)
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(m, K, 10 + m)
    ref = oracle.qgemm_w4a16(si.bf16_bits(x), codes, scales, zeros, threads=oracle.hardware_threads())
    for split in (0, 1, 8):
        print(f"W4A16 N={n} K={K} M={m} split={split}", flush=True)
        y = qg.qgemm_w4a16(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32)
        assert_w16(y, ref, f"N={n} M={m} split={split}")


@pytest.mark.parametrize("m", [1, 4])
def test_w4a8_long_k(dev, m):
    n = 64
    w = _w(n)
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(m, K, 20 + m)
    xb = si.bf16_bits(x)
    assert_w16(qg.qgemm_w4a8(x.to(dev), packed, n, out_dtype=torch.float32),
               oracle.qgemm_w4a8(xb, codes, scales, zeros), f"W4A8 M={m}")
    assert_w16(qg.qgemm_w4a8_g32(x.to(dev), packed, n, out_dtype=torch.float32),
               oracle.qgemm_w4a8_g32(xb, codes, scales, zeros), f"W4A8 g32 M={m}")


@pytest.mark.parametrize("m", [1, 4, 64])
def test_scale_codes_and_int6_long_k(dev, m):
    n = 64
    w = _w(n)
    x = si.activation(m, K, 30 + m)
    xb = si.bf16_bits(x)
    c, sc, st, z, _ = oracle.quantize_int4_g32_dq(si.bf16_bits(w))
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    assert (packed.cpu().numpy() == oracle.pack_int4_dq(c, sc, st, z)).all()
    assert_w16(qg.qgemm_w4a16_dq(x.to(dev), packed, n, out_dtype=torch.float32),
               oracle.qgemm_w4a16_dq(xb, c, sc, st, z), f"scale codes M={m}")
    c6, s6, z6, _ = oracle.quantize_intn_g32(si.bf16_bits(w), 6)
    p6 = qg.quantize_intn_g32(w.to(dev), 6)
    assert (p6.cpu().numpy() == oracle.pack_intn(c6, s6, z6, 6)).all()
    assert_w16(qg.qgemm_wn_a16(x.to(dev), p6, n, 6, out_dtype=torch.float32),
               oracle.qgemm_w4a16(xb, c6, s6, z6), f"INT6 M={m}")


@pytest.mark.parametrize("m", [1, 4])
def test_w8a16_largest_k(dev, m):
    n, k = 64, 65536
    wi, s8, x = si.int8_layer(n, k, m, seed=7)
    y = qg.qgemm_w8a16(x.to(dev), wi.to(dev), s8.to(dev), out_dtype=torch.float32)
    assert_w16(y, oracle.qgemm_w8a16(si.bf16_bits(x), wi.numpy(), si.bf16_bits(s8)), f"W8A16 K=65536 M={m}")
