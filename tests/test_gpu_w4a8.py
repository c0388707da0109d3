"""GPU parity: W4A8 (packed INT4 g32 weight x per-row int8 activations).

Two checks per case:
  * against the W4A8 oracle (same activation quantization, exact integer
    group dots) with the W4A16 bounds -- this is the parity gate;
  * against the W4A16 oracle with the precision class of executorch
    test_int4_quantized_gemm.py `_check_close` (rtol 0.03, atol 8.0, mean
    relative error below 0.02), as Int4QuantizedGemmPrecisionTest requires.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from tolerance import assert_w4a8_class, assert_w16

import gemm_decode_qgemm_amd as qg

pytestmark = pytest.mark.gpu

W4A8_SHAPES = ((8448, 6656), (6656, 19968))


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=3)
def _weight(n, k, seed):
    w = si.int4_weight(n, k, seed)
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    return w, codes, scales, zeros


def _refs(x, codes, scales, zeros):
    t = oracle.hardware_threads()
    xb = si.bf16_bits(x)
    return (oracle.qgemm_w4a8(xb, codes, scales, zeros, threads=t),
            oracle.qgemm_w4a16(xb, codes, scales, zeros, threads=t))


def _outliers(x: torch.Tensor) -> torch.Tensor:
    """Int4QuantizedGemmPrecisionTest's outlier recipe: channels 0, K/3, 2K/3
    and K-1 scaled by 50, 35, 25 and 20."""
    k = x.shape[1]
    x = x.clone()
    for c, f in zip((0, k // 3, 2 * k // 3, k - 1), (50.0, 35.0, 25.0, 20.0)):
        x[:, c] = (x[:, c].float() * f).to(torch.bfloat16)
    return x


@pytest.mark.parametrize("n,k", W4A8_SHAPES)
def test_w4a8_decode_config(dev, n, k):
    w, codes, scales, zeros = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32(w.to(dev))
    i = si.model_shape_index(n, k)
    for m in si.DECODE_M:
        x = si.activation(m, k, si.model_activation_seed(i, m))
        r8, r16 = _refs(x, codes, scales, zeros)
        for dt in (torch.float32, torch.bfloat16):
            y = qg.qgemm_w4a8(x.to(dev), packed, n, out_dtype=dt)
            assert_w16(y, r8, f"W4A8 vs W4A8 oracle {n}x{k} M={m} {dt}")
            assert_w4a8_class(y, r16, f"W4A8 vs W4A16 oracle {n}x{k} M={m} {dt}")


@pytest.mark.parametrize("n,k", [(768, 256), (257, 512), (1536, 512), (320, 6656), (64, 19968)])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_w4a8_small_shapes(dev, n, k, m):
    w, codes, scales, zeros = _weight(n, k, n + k)
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(m, k, 77 + m + n)
    r8, r16 = _refs(x, codes, scales, zeros)
    y = qg.qgemm_w4a8(x.to(dev), packed, n, out_dtype=torch.float32)
    assert_w16(y, r8, f"{n}x{k} M={m}")
    assert_w4a8_class(y, r16, f"{n}x{k} M={m}")


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_w4a8_both_workgroup_shapes_ragged_n(dev, m):
    """N = 8200: 64-row workgroups with one split (M = 1 the v_dot4c GEMV,
    M = 2..4 the matrix-instruction one) and 32-row ones with two, each with
    an 8-row tail, against the W4A8 oracle."""
    n, k = 8200, 512
    w, codes, scales, zeros = _weight(n, k, 45)
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(m, k, 70 + m)
    r8, r16 = _refs(x, codes, scales, zeros)
    for split in (1, 2):
        y = qg.qgemm_w4a8(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32)
        assert_w16(y, r8, f"N=8200 M={m} split={split}")
        assert_w4a8_class(y, r16, f"N=8200 M={m} split={split}")


@pytest.mark.parametrize("n", [8193, 10240, 10241])
def test_w4a8_matrix_instruction_gemv_row_form_edges(dev, n):
    """M = 2..4, one split, per-row and per-group scales, at the edges of the
    64-row form (N = 8193 and 10240 take it, 10241 does not)."""
    k = 256
    w, codes, scales, zeros = _weight(n, k, 91 + n)
    packed = qg.quantize_int4_g32(w.to(dev))
    t = oracle.hardware_threads()
    for m in (2, 3, 4):
        x = si.activation(m, k, 97 + m)
        xb = si.bf16_bits(x)
        print(f"qgemm_w4a8 row-form edge N={n} M={m}", flush=True)
        y = qg.qgemm_w4a8(x.to(dev), packed, n, split_k=1, out_dtype=torch.float32)
        assert_w16(y, oracle.qgemm_w4a8(xb, codes, scales, zeros, threads=t), f"per row N={n} M={m}")
        y = qg.qgemm_w4a8_g32(x.to(dev), packed, n, split_k=1, out_dtype=torch.float32)
        assert_w16(y, oracle.qgemm_w4a8_g32(xb, codes, scales, zeros, threads=t), f"per group N={n} M={m}")


@pytest.mark.parametrize("entry", ["qgemm_w4a8", "qgemm_w4a8_g32", "qgemm_w4a8_dq", "qgemm_w4a8_g32_dq"])
def test_w4a8_64_row_workgroups_non_finite_weight_row(dev, entry):
    """8448 rows at M = 2 and 4 with one split (64-row matrix-instruction
    workgroups on both layouts and scale kinds): a non-finite weight in row
    8400 of the last block makes only column 8400 of y NaN, in every row."""
    n, k = 8448, 256
    w = si.int4_weight(n, k, 8).clone()
    w[8400, 3] = float("-inf")
    dq = entry.endswith("_dq")
    packed = (qg.quantize_int4_g32_dq if dq else qg.quantize_int4_g32)(w.to(dev))
    fn = getattr(qg, entry)
    for m in (2, 4):
        y = fn(si.activation(m, k, 9 + m).to(dev), packed, n, split_k=1, out_dtype=torch.float32).cpu()
        assert torch.isnan(y[:, 8400]).all(), f"{entry} M={m}"
        assert torch.isfinite(torch.cat([y[:, :8400], y[:, 8401:]], dim=1)).all(), f"{entry} M={m}"


def test_w4a8_every_split(dev):
    n, k = 320, 6656
    w, codes, scales, zeros = _weight(n, k, 12)
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(3, k, 5)
    r8, _ = _refs(x, codes, scales, zeros)
    for split in si.SPLITS:
        y = qg.qgemm_w4a8(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32)
        assert_w16(y, r8, f"split={split}")


def test_w4a8_on_the_int8_grid_matches_w4a16(dev):
    """x already integer with absmax 127: xq = x and sx = 1, so W4A8 and W4A16
    compute the same sum; the GPU must agree with the W4A16 oracle to fp32
    rounding (catches any dropped product or wrong byte order)."""
    n, k = 512, 4096
    w, codes, scales, zeros = _weight(n, k, 31)
    packed = qg.quantize_int4_g32(w.to(dev))
    rng = np.random.default_rng(3)
    xi = rng.integers(-127, 128, (2, k))
    xi[:, 5] = 127
    x = torch.tensor(xi, dtype=torch.bfloat16)
    _, r16 = _refs(x, codes, scales, zeros)
    y = qg.qgemm_w4a8(x.to(dev), packed, n, out_dtype=torch.float32)
    err = np.abs(y.cpu().numpy().astype(np.float64) - r16)
    assert err.max() <= 1e-5 * np.abs(r16).max() + 1e-3


def test_w4a8_one_hot_rows(dev):
    n, k = 128, 512
    w, codes, scales, zeros = _weight(n, k, 8)
    packed = qg.quantize_int4_g32(w.to(dev))
    for j in (0, 7, 30, 31, 100, 511):
        x = torch.zeros(1, k, dtype=torch.bfloat16)
        x[0, j] = 3.0
        r8, _ = _refs(x, codes, scales, zeros)
        y = qg.qgemm_w4a8(x.to(dev), packed, n, out_dtype=torch.float32).cpu().numpy()
        np.testing.assert_allclose(y, r8, rtol=1e-6, atol=1e-6, err_msg=f"one-hot at k={j}")


def test_w4a8_zero_row_is_zero(dev):
    n, k = 256, 768
    w, codes, scales, zeros = _weight(n, k, 2)
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(2, k, 3)
    x[0] = 0
    y = qg.qgemm_w4a8(x.to(dev), packed, n, out_dtype=torch.float32).cpu()
    assert (y[0] == 0).all() and (y[1] != 0).any()


def test_w4a8_outlier_activations_parity(dev):
    """Outlier rows still match the W4A8 oracle (same quantization)."""
    n, k = 8448, 6656
    w, codes, scales, zeros = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32(w.to(dev))
    x = _outliers(si.activation(4, k, 4301))
    r8, _ = _refs(x, codes, scales, zeros)
    assert_w16(qg.qgemm_w4a8(x.to(dev), packed, n, out_dtype=torch.float32), r8, "outliers")


@pytest.mark.xfail(reason="per-row int8 activation scales lose the small channels when a few "
                          "channels are 20-50x larger; finer activation groups are the next step",
                   strict=False)
def test_w4a8_outlier_precision_class(dev):
    n, k = 8448, 6656
    w, codes, scales, zeros = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32(w.to(dev))
    x = _outliers(si.activation(4, k, 4301))
    _, r16 = _refs(x, codes, scales, zeros)
    assert_w4a8_class(qg.qgemm_w4a8(x.to(dev), packed, n, out_dtype=torch.float32), r16, "outliers")


def test_w4a8_rejects_m_above_64(dev):
    w, *_ = _weight(256, 256, 1)
    packed = qg.quantize_int4_g32(w.to(dev))
    with pytest.raises(qg.QGemmError) as e:
        qg.qgemm_w4a8(si.activation(65, 256, 1).to(dev), packed, 256)
    assert e.value.status == -4


def test_w4a8_graph_replay_is_bit_identical(dev):
    n, k = 8448, 6656
    w, *_ = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32(w.to(dev))
    x = si.activation(2, k, 9).to(dev)
    eager = qg.qgemm_w4a8(x, packed, n)
    out = torch.empty_like(eager)
    ws = torch.empty(max(qg.workspace_bytes(2, n, k), 1), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.qgemm_w4a8(x, packed, n, out=out, workspace=ws)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
