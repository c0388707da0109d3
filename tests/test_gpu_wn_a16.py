"""GPU parity of the INT5 / INT6 group-32 path (the INT5/INT6 family of
executorch pull request #23737, quantized with the INT4 recipe of
test_int4_quantized_gemm.py `_packed_with_dense` at 2^bits - 1 steps): the
quantizer bit for bit and the GEMVs (M = 1..4) and matrix-core kernels
(M = 5..64, the pull request's buckets 16 and 64 among them) within tolerance, against the CPU
oracle, through the C ABI.  Layer shapes: the INT6 ones the pull request lists
(4096x5376, 5376x21504, 6656x19968, 1024x6656); INT5 runs two INT4/INT6 shapes
(the pull request names the count of INT5 layers, not their shapes).
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

INT6_SHAPES = ((4096, 5376), (5376, 21504), (6656, 19968), (1024, 6656))
INT5_SHAPES = ((6656, 4096), (1024, 6656))
LAYERS = [(6, n, k) for n, k in INT6_SHAPES] + [(5, n, k) for n, k in INT5_SHAPES]


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=4)
def _weight(n: int, k: int, bits: int, seed: int):
    w = si.int4_weight(n, k, seed)
    codes, scales, zeros, flags = oracle.quantize_intn_g32(si.bf16_bits(w), bits)
    assert flags == 0
    return w, codes, scales, zeros


def _ref(x, codes, scales, zeros):
    # the dequant-then-dot reference takes codes of any width
    return oracle.qgemm_w4a16(si.bf16_bits(x), codes, scales, zeros, threads=oracle.hardware_threads())


@pytest.mark.parametrize("bits", [5, 6])
@pytest.mark.parametrize("n,k", [(768, 256), (257, 512), (63, 1024), (1, 256)])
def test_quantize_intn_bit_exact_small(dev, bits, n, k):
    w, codes, scales, zeros = _weight(n, k, bits, n + k + bits)
    packed = qg.quantize_intn_g32(w.to(dev), bits).cpu().numpy()
    ref = oracle.pack_intn(codes, scales, zeros, bits)
    assert packed.size == ref.size == qg.intn_packed_bytes(n, k, bits)
    assert np.array_equal(packed, ref), f"{int((packed != ref).sum())} bytes differ"


@pytest.mark.parametrize("bits,n,k", LAYERS)
def test_quantize_intn_bit_exact_layers(dev, bits, n, k):
    print(f"quantize_intn_g32 INT{bits} {n}x{k}", flush=True)
    w, codes, scales, zeros = _weight(n, k, bits, n ^ k)
    packed = qg.quantize_intn_g32(w.to(dev), bits).cpu().numpy()
    assert np.array_equal(packed, oracle.pack_intn(codes, scales, zeros, bits))


def test_quantize_intn_hand_worked_groups(dev):
    cases = read_cases("intn_g32_groups.txt")
    for bits in (5, 6):
        n, k = 40, 512
        w = si.bf16_bits(si.int4_weight(n, k, 7 + bits)).copy()
        where = {}
        for i, c in enumerate(x for x in cases if x["width"] == bits):
            row, g = (5 * i + 2) % n, (3 * i + 1) % (k // 32)
            w[row, 32 * g:32 * g + 32] = c["bits"]
            where[(row, g)] = c
        status = torch.zeros(1, dtype=torch.int32, device=dev)
        packed = qg.quantize_intn_g32(si.bits_to_bf16(w).to(dev), bits, status=status).cpu().numpy()
        codes, scales, zeros = oracle.unpack_intn(packed, n, k, bits)
        flags = 0
        for (row, g), c in where.items():
            flags |= c["flags"]
            assert scales[row, g] == c["scale"], c["name"]
            assert zeros[row, g] == c["zp"], c["name"]
            assert codes[row, 32 * g:32 * g + 32].tolist() == c["codes"].tolist(), c["name"]
        assert int(status.item()) == flags
        rc, rs, rz, rf = oracle.quantize_intn_g32(w, bits)
        assert rf == flags
        assert np.array_equal(packed, oracle.pack_intn(rc, rs, rz, bits))


@pytest.mark.parametrize("bits", [5, 6])
def test_quantize_intn_adversarial_groups(dev, bits):
    rng = np.random.default_rng(30 + bits)
    n, k = 96, 512
    v = rng.standard_normal((n, k))
    v[0::6] = np.abs(v[0::6]) + 5.0
    v[1::6] = -np.abs(v[1::6]) * 1e-3
    v[2::6] *= 1e-30
    v[3::6] *= 6e4
    v[4::6] *= rng.random((len(range(4, n, 6)), k)) < 0.1
    v[5::6] = np.round(v[5::6] * 16) / 32
    bits16 = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    packed = qg.quantize_intn_g32(si.bits_to_bf16(bits16).to(dev), bits).cpu().numpy()
    codes, scales, zeros, _ = oracle.quantize_intn_g32(bits16, bits)
    assert np.array_equal(packed, oracle.pack_intn(codes, scales, zeros, bits))


@pytest.mark.parametrize("bits", [5, 6])
@pytest.mark.parametrize("n,k", [(768, 256), (257, 512), (1536, 512), (512, 8192)])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_wn_a16_small_shapes(dev, bits, n, k, m):
    w, codes, scales, zeros = _weight(n, k, bits, n + k + bits)
    packed = qg.quantize_intn_g32(w.to(dev), bits)
    x = si.activation(m, k, 500 + n + bits + m)
    ref = _ref(x, codes, scales, zeros)
    for dt in (torch.float32, torch.bfloat16):
        y = qg.qgemm_wn_a16(x.to(dev), packed, n, bits, out_dtype=dt)
        assert y.shape == (m, n) and y.dtype == dt
        assert_w16(y, ref, f"INT{bits} {n}x{k} M={m} {dt}")


@pytest.mark.parametrize("bits,n,k", LAYERS)
def test_wn_a16_layers(dev, bits, n, k):
    w, codes, scales, zeros = _weight(n, k, bits, n ^ k)
    packed = qg.quantize_intn_g32(w.to(dev), bits)
    for m in si.DECODE_M:
        print(f"qgemm_wn_a16 INT{bits} {n}x{k} M={m}", flush=True)
        x = si.activation(m, k, 900 + bits + m)
        ref = _ref(x, codes, scales, zeros)
        for dt in (torch.float32, torch.bfloat16):
            assert_w16(qg.qgemm_wn_a16(x.to(dev), packed, n, bits, out_dtype=dt), ref,
                       f"INT{bits} {n}x{k} M={m} {dt}")


@pytest.mark.parametrize("bits", [5, 6])
@pytest.mark.parametrize("m", [1, 4])
def test_wn_a16_every_split_uneven(dev, bits, m):
    n, k = 257, 6656
    w, codes, scales, zeros = _weight(n, k, bits, 77)
    packed = qg.quantize_intn_g32(w.to(dev), bits)
    x = si.activation(m, k, 33 + m)
    ref = _ref(x, codes, scales, zeros)
    for split in si.SPLITS:
        y = qg.qgemm_wn_a16(x.to(dev), packed, n, bits, split_k=split, out_dtype=torch.float32)
        assert_w16(y, ref, f"INT{bits} M={m} split={split}")


@pytest.mark.parametrize("bits", [5, 6])
@pytest.mark.parametrize("m", [2, 3, 4])
def test_wn_a16_64_row_workgroups_ragged_n(dev, bits, m):
    """N = 8200 (8200 % 64 = 8) at M = 2..4: one split takes 64-row
    matrix-instruction workgroups (129, the last with 8 live rows), two
    splits 32-row ones."""
    n, k = 8200, 512
    w, codes, scales, zeros = _weight(n, k, bits, 48 + bits)
    packed = qg.quantize_intn_g32(w.to(dev), bits)
    x = si.activation(m, k, 62 + bits + m)
    ref = _ref(x, codes, scales, zeros)
    print(f"qgemm_wn_a16 INT{bits} 64-row workgroups N=8200 M={m}", flush=True)
    for split in (1, 2):
        for dt in (torch.float32, torch.bfloat16):
            y = qg.qgemm_wn_a16(x.to(dev), packed, n, bits, split_k=split, out_dtype=dt)
            assert_w16(y, ref, f"INT{bits} N=8200 M={m} split={split} {dt}")


@pytest.mark.parametrize("bits", [5, 6])
@pytest.mark.parametrize("m", [5, 8, 16, 17, 32, 33, 48, 64])
def test_wn_a16_matrix_core_runtime_m_and_tails(dev, bits, m):
    """Rows padded to 16 and masked; N = 257 leaves a one-row tail block."""
    for n, k in ((257, 768), (768, 512)):
        w, codes, scales, zeros = _weight(n, k, bits, n + k + bits)
        packed = qg.quantize_intn_g32(w.to(dev), bits)
        x = si.activation(m, k, 700 + m + bits)
        ref = _ref(x, codes, scales, zeros)
        for dt in (torch.float32, torch.bfloat16):
            assert_w16(qg.qgemm_wn_a16(x.to(dev), packed, n, bits, out_dtype=dt), ref,
                       f"INT{bits} {n}x{k} M={m} {dt}")


@pytest.mark.parametrize("n,k", INT6_SHAPES)
@pytest.mark.parametrize("m", [16, 64])
def test_wn_a16_int6_layers_large_buckets(dev, n, k, m):
    print(f"qgemm_wn_a16 INT6 {n}x{k} M={m}", flush=True)
    w, codes, scales, zeros = _weight(n, k, 6, n ^ k)
    packed = qg.quantize_intn_g32(w.to(dev), 6)
    x = si.activation(m, k, 1200 + m)
    ref = _ref(x, codes, scales, zeros)
    assert_w16(qg.qgemm_wn_a16(x.to(dev), packed, n, 6, out_dtype=torch.float32), ref, f"INT6 {n}x{k} M={m}")


@pytest.mark.parametrize("bits", [5, 6])
@pytest.mark.parametrize("m", [16, 64])
def test_wn_a16_matrix_core_every_split(dev, bits, m):
    n, k = 320, 6656
    w, codes, scales, zeros = _weight(n, k, bits, 91)
    packed = qg.quantize_intn_g32(w.to(dev), bits)
    x = si.activation(m, k, 61 + m)
    ref = _ref(x, codes, scales, zeros)
    for split in si.SPLITS:
        y = qg.qgemm_wn_a16(x.to(dev), packed, n, bits, split_k=split, out_dtype=torch.float32)
        assert_w16(y, ref, f"INT{bits} M={m} split={split}")


def test_wn_a16_graph_replay_bit_identical(dev):
    n, k = 6656, 19968
    w, *_ = _weight(n, k, 6, n ^ k)
    packed = qg.quantize_intn_g32(w.to(dev), 6)
    for m, split in ((1, 1), (1, 4), (4, 1), (16, 2), (64, 4)):
        x = si.activation(m, k, 5 + m).to(dev)
        eager = qg.qgemm_wn_a16(x, packed, n, 6, split_k=split)
        assert torch.equal(eager, qg.qgemm_wn_a16(x, packed, n, 6, split_k=split))
        out = torch.empty_like(eager)
        ws = torch.empty(max(qg.workspace_bytes(m, n, k, split), 1), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            qg.qgemm_wn_a16(x, packed, n, 6, split_k=split, out=out, workspace=ws)
        for _ in range(3):
            out.zero_()
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay differs (m={m}, split={split})"
            _ = qg.qgemm_wn_a16(x, packed, n, 6, split_k=1)


def test_wn_a16_rejects_bad_width_and_m(dev):
    w, *_ = _weight(256, 768, 6, 3)
    packed = qg.quantize_intn_g32(w.to(dev), 6)
    with pytest.raises(qg.QGemmError) as e:
        qg.qgemm_wn_a16(si.activation(1, 768, 1).to(dev), packed, 256, 7)
    assert e.value.status == -10
    with pytest.raises(qg.QGemmError) as e:
        qg.qgemm_wn_a16(si.activation(65, 768, 1).to(dev), packed, 256, 6)
    assert e.value.status == -4
