"""GPU parity across every activation row count and the edge shapes.

executorch test_int4_quantized_gemm.py runs each bucket with a dynamic M
inside it (`torch._dynamo.mark_dynamic(x, 0, ...)`, DYNAMIC_M tests), the
N = 257 tail (test_tail_shape), K = 256 (the smallest legal K) and
bit-equal CUDA-graph replay (test_cuda_graph_replay_matches_eager).  Here:
every M from 1 to 64 on a ragged N (the decode GEMV for M <= 4, the
matrix-core kernel with rows padded to 16 and masked above) for the INT4,
scale-code INT4 and INT5 / INT6 weights, K = 256 for every entry point, and
eager/graph bit-equality at the buckets 1, 2, 3, 4, 8, 16, 32 and 64.
"""
from __future__ import annotations

import functools

import pytest
import torch

import oracle
import synthetic_inputs as si
from tolerance import assert_w16

import gemm_decode_qgemm_amd as qg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=4)
def _layer(n, k, seed):
    w = si.int4_weight(n, k, seed)
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    return w, codes, scales, zeros


def test_every_m_from_1_to_64_ragged_n(dev):
    n, k = 320, 1024          # 320 = 5 row blocks; M = 1..64 covers all padding cases
    w, codes, scales, zeros = _layer(n, k, 61)
    packed = qg.quantize_int4_g32(w.to(dev))
    xall = si.activation(64, k, 62)
    ref = oracle.qgemm_w4a16(si.bf16_bits(xall), codes, scales, zeros)
    for m in range(1, 65):
        y = qg.qgemm_w4a16(xall[:m].contiguous().to(dev), packed, n, out_dtype=torch.float32)
        assert y.shape == (m, n)
        assert_w16(y, ref[:m], f"M={m}")


@pytest.mark.parametrize("fmt", ["dq", "int5", "int6"])
def test_every_m_from_1_to_64_ragged_n_other_layouts(dev, fmt):
    n, k = 320, 1024
    w = si.int4_weight(n, k, 67)
    xall = si.activation(64, k, 68)
    xb = si.bf16_bits(xall)
    if fmt == "dq":
        codes, scode, sstep, zeros, _ = oracle.quantize_int4_g32_dq(si.bf16_bits(w))
        packed = qg.quantize_int4_g32_dq(w.to(dev))
        ref = oracle.qgemm_w4a16_dq(xb, codes, scode, sstep, zeros)
        call = lambda x: qg.qgemm_w4a16_dq(x, packed, n, out_dtype=torch.float32)
    else:
        bits = int(fmt[3])
        codes, scales, zeros, _ = oracle.quantize_intn_g32(si.bf16_bits(w), bits)
        packed = qg.quantize_intn_g32(w.to(dev), bits)
        ref = oracle.qgemm_w4a16(xb, codes, scales, zeros)
        call = lambda x: qg.qgemm_wn_a16(x, packed, n, bits, out_dtype=torch.float32)
    for m in range(1, 65):
        y = call(xall[:m].contiguous().to(dev))
        assert y.shape == (m, n)
        assert_w16(y, ref[:m], f"{fmt} M={m}")


@pytest.mark.parametrize("m", [1, 3, 4, 16, 33, 64])
def test_k256_single_tile(dev, m):
    n, k = 257, 256
    w, codes, scales, zeros = _layer(n, k, 63)
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(m, k, 64 + m)
    xb = si.bf16_bits(x)
    assert_w16(qg.qgemm_w4a16(x.to(dev), packed, n, out_dtype=torch.float32),
               oracle.qgemm_w4a16(xb, codes, scales, zeros), f"W4A16 K=256 M={m}")
    cd, scd, std, zd, _ = oracle.quantize_int4_g32_dq(si.bf16_bits(w))
    assert_w16(qg.qgemm_w4a16_dq(x.to(dev), qg.quantize_int4_g32_dq(w.to(dev)), n, out_dtype=torch.float32),
               oracle.qgemm_w4a16_dq(xb, cd, scd, std, zd), f"W4A16 scale codes K=256 M={m}")
    for bits in (5, 6):
        cn, sn, zn, _ = oracle.quantize_intn_g32(si.bf16_bits(w), bits)
        assert_w16(qg.qgemm_wn_a16(x.to(dev), qg.quantize_intn_g32(w.to(dev), bits), n, bits,
                                   out_dtype=torch.float32),
                   oracle.qgemm_w4a16(xb, cn, sn, zn), f"INT{bits} K=256 M={m}")
    if m <= 4:
        assert_w16(qg.qgemm_w4a8(x.to(dev), packed, n, out_dtype=torch.float32),
                   oracle.qgemm_w4a8(xb, codes, scales, zeros), f"W4A8 K=256 M={m}")
        assert_w16(qg.qgemm_w4a8_g32(x.to(dev), packed, n, out_dtype=torch.float32),
                   oracle.qgemm_w4a8_g32(xb, codes, scales, zeros), f"W4A8 g32 K=256 M={m}")
        wi, si8, xw = si.int8_layer(n, k, m, seed=m)
        assert_w16(qg.qgemm_w8a16(xw.to(dev), wi.to(dev), si8.to(dev), out_dtype=torch.float32),
                   oracle.qgemm_w8a16(si.bf16_bits(xw), wi.numpy(), si.bf16_bits(si8)), f"W8A16 K=256 M={m}")


@pytest.mark.parametrize("m", [1, 2, 3, 4, 8, 16, 32, 64])
def test_graph_replay_matches_eager_every_bucket(dev, m):
    n, k = 1536, 2048
    w, *_ = _layer(n, k, 65)
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(m, k, 66 + m).to(dev)
    split = qg.default_split_k(m, n, k)
    eager = qg.qgemm_w4a16(x, packed, n)
    out = torch.empty_like(eager)
    ws = torch.empty(max(qg.workspace_bytes(m, n, k, split), 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.qgemm_w4a16(x, packed, n, out=out, workspace=ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"M={m} split={split}"
