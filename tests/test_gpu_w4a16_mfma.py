"""GPU parity: W4A16 for M = 5..64 (matrix-core path) against the CPU oracle.

Buckets 8..64 of executorch test_int4_quantized_gemm.py (SUPPORTED_BUCKETS)
on the model shapes with every split candidate, plus a spread of runtime M
(rows padded to 16 and masked, as a static bucket with a dynamic M is in the
pages' DYNAMIC_M tests) and an N tail.
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

LARGE_SHAPES = ((39936, 6656), (6656, 19968), (8448, 6656))


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=2)
def _weight(n, k, seed):
    w = si.int4_weight(n, k, seed)
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    return w, codes, scales, zeros


def _ref(x, codes, scales, zeros):
    return oracle.qgemm_w4a16(si.bf16_bits(x), codes, scales, zeros, threads=oracle.hardware_threads())


@pytest.mark.parametrize("n,k", LARGE_SHAPES)
@pytest.mark.parametrize("m", sorted(set(si.LARGE_M) | {32, 48}))
def test_mfma_large_buckets_every_split(dev, n, k, m):
    w, codes, scales, zeros = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(m, k, si.model_activation_seed(si.model_shape_index(n, k), m))
    ref = _ref(x, codes, scales, zeros)
    xd = x.to(dev)
    for split in si.SPLITS:
        y = qg.qgemm_w4a16(xd, packed, n, split_k=split, out_dtype=torch.float32)
        assert_w16(y, ref, f"{n}x{k} M={m} split={split}")
    yb = qg.qgemm_w4a16(xd, packed, n, out_dtype=torch.bfloat16)
    assert_w16(yb, ref, f"{n}x{k} M={m} bf16")


@pytest.mark.parametrize("m", [5, 8, 13, 16, 17, 32, 57, 64])
@pytest.mark.parametrize("n,k", [(768, 512), (257, 768), (1536, 512)])
def test_mfma_runtime_m_and_tails(dev, n, k, m):
    w, codes, scales, zeros = _weight(n, k, n + k)
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(m, k, 500 + m)
    ref = _ref(x, codes, scales, zeros)
    for dt in (torch.float32, torch.bfloat16):
        y = qg.qgemm_w4a16(x.to(dev), packed, n, out_dtype=dt)
        assert y.shape == (m, n)
        assert_w16(y, ref, f"{n}x{k} M={m} {dt}")


def test_mfma_matches_decode_path_row_by_row(dev):
    """Row m of an M = 16 call equals the M = 1 GEMV of row m up to fp32 rounding:
    both add the same exact products in different orders (about sqrt(K) * 2^-24
    * |y|, ~1e-4 here); a layout or masking slip would be O(1)."""
    n, k = 1024, 2048
    w, *_ = _weight(n, k, 17)
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(16, k, 6).to(dev)
    y16 = qg.qgemm_w4a16(x, packed, n, out_dtype=torch.float32)
    for r in (0, 7, 15):
        y1 = qg.qgemm_w4a16(x[r:r + 1].contiguous(), packed, n, out_dtype=torch.float32)
        torch.testing.assert_close(y16[r:r + 1], y1, rtol=1e-4, atol=1e-3)


def test_mfma_repeat_and_graph_replay_are_bit_identical(dev):
    n, k = 8448, 6656
    w, *_ = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32(w.to(dev))
    for m, split in ((16, 1), (64, 2)):
        x = si.activation(m, k, 99).to(dev)
        eager = qg.qgemm_w4a16(x, packed, n, split_k=split)
        assert torch.equal(eager, qg.qgemm_w4a16(x, packed, n, split_k=split))
        out = torch.empty_like(eager)
        ws = torch.empty(max(qg.workspace_bytes(m, n, k, split), 1), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            qg.qgemm_w4a16(x, packed, n, split_k=split, out=out, workspace=ws)
        for _ in range(3):
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"M={m} split={split}"


def test_m_above_64_is_rejected(dev):
    w, *_ = _weight(256, 256, 1)
    packed = qg.quantize_int4_g32(w.to(dev))
    with pytest.raises(qg.QGemmError) as e:
        qg.qgemm_w4a16(si.activation(65, 256, 1).to(dev), packed, 256)
    assert e.value.status == -4


@pytest.mark.parametrize("m", [32, 33, 64])
@pytest.mark.parametrize("k", [256, 512, 768])
def test_mfma_lds_form_short_k_every_split(dev, k, m):
    """The LDS-staged form on 1..3 tiles of 256 k at every legal split, so a
    workgroup's range can be a single tile: the two-buffer pipeline (32 rows)
    and the one-buffer one (33 and 64 rows) at their first and last tile,
    with N = 200 (an 8-row tail past the 64-row blocks)."""
    n = 200
    w, codes, scales, zeros = _weight(n, k, 31 * k + m)
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(m, k, 1300 + m + k)
    ref = _ref(x, codes, scales, zeros)
    xd = x.to(dev)
    for split in [s for s in si.SPLITS if s <= k // 256]:
        label = f"qgemm_w4a16 {n}x{k} M={m} split={split}"
        print(label, flush=True)
        y = qg.qgemm_w4a16(xd, packed, n, split_k=split, out_dtype=torch.float32)
        assert_w16(y, ref, label)


@pytest.mark.parametrize("m", [17, 24, 32, 33, 47, 48])
@pytest.mark.parametrize("n,k", [(320, 6656), (257, 6144), (1100, 6400)])
def test_mfma_lds_form_ragged(dev, n, k, m):
    """The LDS-staged form (17..64 rows; here 17..48, one x buffer from 33): runtime
    M inside a bucket, N tails (257, 1100), an odd tile count (K = 6400: 25
    tiles, uneven split ranges) and every legal split."""
    w, codes, scales, zeros = _weight(n, k, 7 * n + k)
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(m, k, 900 + m)
    ref = _ref(x, codes, scales, zeros)
    xd = x.to(dev)
    for split in [s for s in si.SPLITS if s <= k // 256]:
        y = qg.qgemm_w4a16(xd, packed, n, split_k=split, out_dtype=torch.float32)
        assert_w16(y, ref, f"{n}x{k} M={m} split={split}")
    yb = qg.qgemm_w4a16(xd, packed, n, out_dtype=torch.bfloat16)
    assert_w16(yb, ref, f"{n}x{k} M={m} bf16")
