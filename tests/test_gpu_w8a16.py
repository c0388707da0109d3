"""GPU parity: INT8 row-wise quantizer (bit-exact) and W8A16 (tolerance: the
GEMV at 1..4 rows, the matrix cores at 5..64) against the CPU oracle, through
the C ABI.

The layer is gpt-fast issue #114's WeightOnlyInt8Linear: int8 [out, in]
weight, one bf16 scale per output row, y = (x . W^T) * scale; its benchmark
size is D = 8192.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from golden_io import read_cases
from tolerance import assert_w16

import gemm_decode_qgemm_amd as qg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _ref(x, w, s):
    return oracle.qgemm_w8a16(si.bf16_bits(x), w.numpy(), si.bf16_bits(s),
                              threads=oracle.hardware_threads())


# ------------------------------------------------------------------ quantizer


@pytest.mark.parametrize("n,k", [(64, 256), (257, 768), (1000, 4096), (8192, 8192)])
def test_quantize_int8_bit_exact(dev, n, k):
    w = si.int4_weight(n, k, 7 + n)            # bf16 standard normal weights
    q, s = qg.quantize_int8_rowwise(w.to(dev))
    rq, rs, flags = oracle.quantize_int8_rowwise(si.bf16_bits(w))
    assert flags == 0
    np.testing.assert_array_equal(q.cpu().numpy(), rq)
    np.testing.assert_array_equal(si.bf16_bits(s.cpu()), rs)


def test_quantize_int8_hand_worked_rows(dev):
    cases = read_cases("int8_rows.txt")
    k = 256
    rows = []
    for c in cases:
        r = np.zeros(k, np.uint16)
        r[:32] = c["bits"]
        r[100:132] = c["bits"]           # the same values again further along
        rows.append(r)
    w = np.stack(rows)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    q, s = qg.quantize_int8_rowwise(si.bits_to_bf16(w).to(dev), status=status)
    q, s = q.cpu().numpy(), si.bf16_bits(s.cpu())
    flags = 0
    for i, c in enumerate(cases):
        assert int(s[i]) == c["scale"], c["name"]
        assert q[i, :32].tolist() == c["codes"].tolist(), c["name"]
        assert q[i, 100:132].tolist() == c["codes"].tolist(), c["name"]
        flags |= c["flags"]
    assert int(status.item()) == flags


# ------------------------------------------------------------------ W8A16 GEMV


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 16, 33, 64])
def test_w8a16_gpt_fast_config(dev, m):
    """N = K = 8192, int8 uniform in [-127, 127], bf16 randn scales and x."""
    w, s, x = si.int8_layer(m=m)
    ref = _ref(x, w, s)
    for dt in (torch.float32, torch.bfloat16):
        y = qg.qgemm_w8a16(x.to(dev), w.to(dev), s.to(dev), out_dtype=dt)
        assert_w16(y, ref, f"W8A16 8192x8192 M={m} {dt}")


@pytest.mark.parametrize("n,k", [(1, 256), (17, 768), (257, 1280), (600, 4096), (333, 6656),
                                 (64, 19968), (48, 65536)])
@pytest.mark.parametrize("m", [1, 3, 4, 5, 17, 48, 64])
def test_w8a16_shapes_and_tails(dev, n, k, m):
    w, s, x = si.int8_layer(n=n, k=k, m=m, seed=n + k + m)
    ref = _ref(x, w, s)
    y = qg.qgemm_w8a16(x.to(dev), w.to(dev), s.to(dev), out_dtype=torch.float32)
    assert_w16(y, ref, f"{n}x{k} M={m}")


@pytest.mark.parametrize("m", [17, 24, 32, 33])
def test_w8a16_64_row_workgroups_on_tall_layers(dev, m):
    """From 16384 rows every M takes the LDS-staged form with workgroups of
    64 weight rows (4 n-tiles); N = 32801 leaves a 33-row tail in the last
    workgroup."""
    n, k = 32801, 256
    w, s, x = si.int8_layer(n=n, k=k, m=m, seed=700 + m)
    ref = _ref(x, w, s)
    print(f"qgemm_w8a16 {n}x{k} M={m}", flush=True)
    for dt in (torch.float32, torch.bfloat16):
        y = qg.qgemm_w8a16(x.to(dev), w.to(dev), s.to(dev), out_dtype=dt)
        assert_w16(y, ref, f"{n}x{k} M={m} {dt}")


@pytest.mark.parametrize("n,m", [(16400, 5), (16400, 64), (4097, 40), (6000, 33), (300, 64), (4096, 49)])
def test_w8a16_lds_form_tile_counts(dev, n, m):
    """The LDS-staged form (4 n-tiles per workgroup from 16384 rows, 2 above
    4096, 1 below; above 32 activation rows on smaller layers) on 1..7 tiles
    of 256 k, so its three-way unrolled tile loop leaves at every point, with
    ragged N (16400 = 256 * 64 + 16, 4097, 300) and ragged M."""
    for tiles in range(1, 8):
        k = 256 * tiles
        w, s, x = si.int8_layer(n=n, k=k, m=m, seed=900 + n + m + tiles)
        ref = _ref(x, w, s)
        label = f"qgemm_w8a16 {n}x{k} M={m}"
        print(label, flush=True)
        y = qg.qgemm_w8a16(x.to(dev), w.to(dev), s.to(dev), out_dtype=torch.float32)
        assert_w16(y, ref, label)


def test_w8a16_quantized_weight_round_trip(dev):
    """Quantize bf16 weights on the GPU, then run the GEMV on them."""
    n, k = 512, 4096
    wb = si.int4_weight(n, k, 3)
    q, s = qg.quantize_int8_rowwise(wb.to(dev))
    x = si.activation(2, k, 4)
    ref = _ref(x, q.cpu(), s.cpu())
    assert_w16(qg.qgemm_w8a16(x.to(dev), q, s, out_dtype=torch.float32), ref, "round trip")


def test_w8a16_every_bucket_ragged_n(dev):
    """Every M from 1 to 64 (GEMV to 4, the matrix cores above, rows masked
    to 16-row tiles) on N = 257 (a 1-row tail past the 32-row workgroups)."""
    n, k = 257, 1024
    w, s, _ = si.int8_layer(n=n, k=k, m=1, seed=5)
    wd, sd = w.to(dev), s.to(dev)
    for m in range(1, 65):
        x = si.activation(m, k, 300 + m)
        assert_w16(qg.qgemm_w8a16(x.to(dev), wd, sd, out_dtype=torch.float32), _ref(x, w, s), f"M={m}")


def test_w8a16_argument_errors(dev):
    w, s, x = si.int8_layer(n=64, k=512, m=65, seed=1)
    with pytest.raises(qg.QGemmError) as e:
        qg.qgemm_w8a16(x.to(dev), w.to(dev), s.to(dev))
    assert e.value.status == -4             # QG_E_M_RANGE
    w2, s2, x2 = si.int8_layer(n=64, k=300, m=1, seed=1)
    with pytest.raises(qg.QGemmError) as e:
        qg.qgemm_w8a16(x2.to(dev), w2.to(dev), s2.to(dev))
    assert e.value.status == -3             # QG_E_K_MULTIPLE


@pytest.mark.parametrize("n,k", [(4096, 8192), (6000, 4096), (16400, 2048)])
@pytest.mark.parametrize("m", [1, 16, 64])
def test_w8a16_repeat_and_graph_replay_are_bit_identical(dev, n, k, m):
    """Every form (GEMV, register form, LDS-staged form with 1, 2 and 4
    n-tiles per workgroup): repeated calls and graph replays give the same
    bits."""
    w, s, x = si.int8_layer(n=n, k=k, m=m, seed=9)
    w, s, x = w.to(dev), s.to(dev), x.to(dev)
    eager = qg.qgemm_w8a16(x, w, s)
    assert torch.equal(eager, qg.qgemm_w8a16(x, w, s))
    out = torch.empty_like(eager)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        qg.qgemm_w8a16(x, w, s, out=out)
    for _ in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager)
