"""GPU parity: INT4 g32 quantizer (bit-exact) and W4A16 decode GEMV (tolerance)
against the CPU oracle, through the C ABI.

Shapes, seeds and buckets follow executorch test_int4_quantized_gemm.py
(MODEL_SHAPES, SMALL_SHAPES, the N = 257 tail, every split candidate, an
illegal split, repeat and graph-replay determinism).
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from golden_io import read_cases
from tolerance import assert_w16

pytestmark = pytest.mark.gpu

import gemm_decode_qgemm_amd as qg  # noqa: E402  (fails loudly if the library is not built)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=4)
def _weight(n: int, k: int, seed: int):
    """(bf16 CPU weight, oracle codes/scales/zeros, oracle packed bytes)."""
    w = si.int4_weight(n, k, seed)
    codes, scales, zeros, flags = oracle.quantize_int4_g32(si.bf16_bits(w))
    assert flags == 0
    return w, codes, scales, zeros


def _gpu_packed(w, dev):
    return qg.quantize_int4_g32(w.to(dev))


def _ref(x, codes, scales, zeros):
    return oracle.qgemm_w4a16(si.bf16_bits(x), codes, scales, zeros, threads=oracle.hardware_threads())


# ------------------------------------------------------------------ quantizer

QUANT_SHAPES = [(768, 256), (256, 768), (1536, 512), (257, 256), (1, 512), (63, 1024)]


@pytest.mark.parametrize("n,k", QUANT_SHAPES)
def test_quantize_bit_exact_small(dev, n, k):
    w, codes, scales, zeros = _weight(n, k, n + k)
    packed = _gpu_packed(w, dev).cpu().numpy()
    ref = oracle.pack_int4(codes, scales, zeros)
    assert packed.size == ref.size
    if not np.array_equal(packed, ref):
        c, s, z = oracle.unpack_int4(packed, n, k)
        bad = np.argwhere(s != scales)[:5]
        raise AssertionError(f"packed bytes differ ({int((packed != ref).sum())} bytes); "
                             f"first scale mismatches at {bad.tolist()}")


@pytest.mark.parametrize("n,k", si.MODEL_SHAPES)
def test_quantize_bit_exact_model_shapes(dev, n, k):
    w, codes, scales, zeros = _weight(n, k, si.model_weight_seed(n, k))
    packed = _gpu_packed(w, dev).cpu().numpy()
    assert np.array_equal(packed, oracle.pack_int4(codes, scales, zeros))


def test_quantize_hand_worked_groups(dev):
    """Every hand-worked group, placed in different rows and group slots."""
    cases = read_cases("int4_g32_groups.txt")
    n, k = 70, 512
    w = si.bf16_bits(si.int4_weight(n, k, 99)).copy()
    where = {}
    for i, c in enumerate(cases):
        row, g = (7 * i) % n, (3 * i + 1) % (k // 32)
        w[row, g * 32:(g + 1) * 32] = c["bits"]
        where[(row, g)] = c
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    packed = qg.quantize_int4_g32(si.bits_to_bf16(w).to(dev), status=status)
    codes, scales, zeros = oracle.unpack_int4(packed.cpu().numpy(), n, k)
    for (row, g), c in where.items():
        assert scales[row, g] == c["scale"], c["name"]
        assert zeros[row, g] == c["zp"], c["name"]
        assert codes[row, g * 32:(g + 1) * 32].tolist() == c["codes"].tolist(), c["name"]
    want_flags = 0
    for c in cases:
        want_flags |= c["flags"]
    assert int(status.item()) == want_flags
    rc, rs, rz, rf = oracle.quantize_int4_g32(w)
    assert rf == want_flags
    assert np.array_equal(packed.cpu().numpy(), oracle.pack_int4(rc, rs, rz))


def test_quantize_adversarial_groups(dev):
    """Ties at half steps, one-sign, tiny (subnormal fp16 scales), huge, sparse groups."""
    rng = np.random.default_rng(5)
    n, k = 128, 1024
    v = rng.standard_normal((n, k))
    v[0::6] = np.abs(v[0::6]) + 5.0
    v[1::6] = -np.abs(v[1::6]) * 1e-3
    v[2::6] *= 1e-30
    v[3::6] *= 6e4
    v[4::6] *= rng.random((len(range(4, n, 6)), k)) < 0.1
    # rows 5::6: values on a coarse grid so that many v/s land on half steps
    v[5::6] = np.round(v[5::6] * 4) / 8
    bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    packed = qg.quantize_int4_g32(si.bits_to_bf16(bits).to(dev)).cpu().numpy()
    codes, scales, zeros, _ = oracle.quantize_int4_g32(bits)
    assert np.array_equal(packed, oracle.pack_int4(codes, scales, zeros))


# ------------------------------------------------------------------ W4A16 GEMV

SMALL_CASES = [(768, 256), (256, 768), (1536, 512), (257, 512), (257, 256), (512, 8192)]


@pytest.mark.parametrize("n,k", SMALL_CASES)
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_w4a16_small_shapes(dev, n, k, m):
    w, codes, scales, zeros = _weight(n, k, n + k)
    packed = _gpu_packed(w, dev)
    x = si.activation(m, k, 1000 + n + m)
    ref = _ref(x, codes, scales, zeros)
    for dt in (torch.float32, torch.bfloat16):
        y = qg.qgemm_w4a16(x.to(dev), packed, n, out_dtype=dt)
        assert y.shape == (m, n) and y.dtype == dt
        assert_w16(y, ref, f"{n}x{k} M={m} {dt}")


def test_w4a16_tiny_config(dev):
    w, x = si.tiny_inputs()
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    packed = _gpu_packed(w, dev)
    ref = _ref(x, codes, scales, zeros)
    for dt in (torch.float32, torch.bfloat16):
        assert_w16(qg.qgemm_w4a16(x.to(dev), packed, 768, out_dtype=dt), ref, f"tiny {dt}")


@pytest.mark.parametrize("n,k", si.MODEL_SHAPES)
def test_w4a16_model_shapes_decode_buckets(dev, n, k):
    w, codes, scales, zeros = _weight(n, k, si.model_weight_seed(n, k))
    packed = _gpu_packed(w, dev)
    i = si.model_shape_index(n, k)
    for m in si.DECODE_M:
        x = si.activation(m, k, si.model_activation_seed(i, m))
        ref = _ref(x, codes, scales, zeros)
        for dt in (torch.float32, torch.bfloat16):
            y = qg.qgemm_w4a16(x.to(dev), packed, n, out_dtype=dt)
            assert_w16(y, ref, f"{n}x{k} M={m} {dt}")


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_w4a16_every_split(dev, m):
    n, k = 256, 4096
    w, codes, scales, zeros = _weight(n, k, 91)
    packed = _gpu_packed(w, dev)
    x = si.activation(m, k, 300 + m)
    ref = _ref(x, codes, scales, zeros)
    for split in si.SPLITS:
        y = qg.qgemm_w4a16(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32)
        assert_w16(y, ref, f"split={split} M={m}")


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_w4a16_both_workgroup_shapes_ragged_n(dev, m):
    """N = 8200 (8200 % 64 = 8): 257 workgroups of 32 rows or 129 of 64.  With
    one split the library takes 64-row workgroups (M = 1 the v_dot2c GEMV,
    M = 2..4 the matrix-instruction one), with two splits 32-row ones; both
    must mask the 8-row tail and match the oracle."""
    n, k = 8200, 512
    w, codes, scales, zeros = _weight(n, k, 44)
    packed = _gpu_packed(w, dev)
    x = si.activation(m, k, 60 + m)
    ref = _ref(x, codes, scales, zeros)
    for split in (1, 2):
        for dt in (torch.float32, torch.bfloat16):
            y = qg.qgemm_w4a16(x.to(dev), packed, n, split_k=split, out_dtype=dt)
            assert_w16(y, ref, f"N=8200 M={m} split={split} {dt}")


@pytest.mark.parametrize("n", [8193, 10240, 10241])
def test_w4a16_matrix_instruction_gemv_row_form_edges(dev, n):
    """M = 2..4, one split, at the edges of the 64-row form: N = 8193 (257
    32-row blocks, the first N that takes 64-row workgroups, 129 of them, the
    last with one live row), N = 10240 (160 blocks of 64, the last N that
    does) and N = 10241 (back to 32-row workgroups)."""
    k = 256
    w, codes, scales, zeros = _weight(n, k, 90 + n)
    packed = _gpu_packed(w, dev)
    for m in (2, 3, 4):
        x = si.activation(m, k, 95 + m)
        ref = _ref(x, codes, scales, zeros)
        print(f"qgemm_w4a16 row-form edge N={n} M={m}", flush=True)
        y = qg.qgemm_w4a16(x.to(dev), packed, n, split_k=1, out_dtype=torch.float32)
        assert_w16(y, ref, f"N={n} M={m}")


@pytest.mark.parametrize("m", [2, 4])
def test_w4a16_64_row_workgroups_non_finite_row(dev, m):
    """8448 rows at M = 2..4 and one split (64-row matrix-instruction
    workgroups): a non-finite weight in row 8400 of the last block makes only
    column 8400 of y NaN, in every activation row."""
    n, k = 8448, 256
    w = si.int4_weight(n, k, 8).clone()
    w[8400, 3] = float("-inf")
    packed = _gpu_packed(w, dev)
    y = qg.qgemm_w4a16(si.activation(m, k, 9).to(dev), packed, n, split_k=1, out_dtype=torch.float32).cpu()
    assert torch.isnan(y[:, 8400]).all()
    assert torch.isfinite(torch.cat([y[:, :8400], y[:, 8401:]], dim=1)).all()


@pytest.mark.parametrize("n", [4097, 5000, 6600, 8191, 8192, 8193])
def test_w4a16_prefetch_grid(dev, n):
    """M = 1 with at most one 32-row workgroup per CU (2 x 64-row blocks x
    split <= 256) takes the two-register-set loop: 130 workgroups at N = 4097
    (one live row in the last), the padded rows of a partial last block, and
    the edge at N = 8192 (256 workgroups, prefetching) against 8193 (258, the
    plain loop); split 0 (the default) and 1, both output types."""
    k = 768
    w, codes, scales, zeros = _weight(n, k, 70 + n)
    packed = _gpu_packed(w, dev)
    x = si.activation(1, k, 80 + n)
    ref = _ref(x, codes, scales, zeros)
    print(f"qgemm_w4a16 prefetch grid N={n}", flush=True)
    for split in (0, 1):
        for dt in (torch.float32, torch.bfloat16):
            y = qg.qgemm_w4a16(x.to(dev), packed, n, split_k=split, out_dtype=dt)
            assert_w16(y, ref, f"N={n} split={split} {dt}")


def test_w4a16_uneven_split_partition(dev):
    """K = 6656 has 26 tiles: splits 4 and 8 give uneven ranges (7,7,6,6 / 4,4,3,...)."""
    n, k = 320, 6656
    w, codes, scales, zeros = _weight(n, k, 5)
    packed = _gpu_packed(w, dev)
    x = si.activation(3, k, 17)
    ref = _ref(x, codes, scales, zeros)
    for split in si.SPLITS:
        y = qg.qgemm_w4a16(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32)
        assert_w16(y, ref, f"split={split}")


def test_illegal_split_is_rejected(dev):
    w, *_ = _weight(256, 768, 3)
    packed = _gpu_packed(w, dev)
    x = si.activation(1, 768, 4).to(dev)
    with pytest.raises(qg.QGemmError) as e:
        qg.qgemm_w4a16(x, packed, 256, split_k=4)          # 768 / 256 = 3 < 4
    assert e.value.status == -5
    with pytest.raises(qg.QGemmError):
        qg.qgemm_w4a16(x, packed, 256, split_k=3)


def test_repeat_and_graph_replay_are_bit_identical(dev):
    n, k = 8448, 6656
    w, *_ = _weight(n, k, si.model_weight_seed(n, k))
    packed = _gpu_packed(w, dev)
    for m in (1, 4):
        x = si.activation(m, k, 77 + m).to(dev)
        for split in (1, 2, 8):
            eager = qg.qgemm_w4a16(x, packed, n, split_k=split)
            again = qg.qgemm_w4a16(x, packed, n, split_k=split)
            assert torch.equal(eager, again)
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
                assert torch.equal(out, eager), f"replay differs (m={m}, split={split})"
                _ = qg.qgemm_w4a16(x, packed, n, split_k=1)   # eager work between replays
