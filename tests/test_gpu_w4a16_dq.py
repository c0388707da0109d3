"""GPU parity of the scale-code form of the INT4 g32 weight (uint8 scale code
times a per-row fp16 step, the stored form of executorch
test_int4_quantized_gemm.py `_packed_with_dense`): the quantizer bit for bit,
the W4A16 kernels (M = 1..64) within tolerance, against the CPU oracle, through
the C ABI.  Shapes, buckets, the N = 257 tail and every split follow the same
page as the fp16-scale tests.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from golden_io import read_cases
from tolerance import assert_w16, assert_w4a8_class

pytestmark = pytest.mark.gpu

import gemm_decode_qgemm_amd as qg  # noqa: E402  (fails loudly if the library is not built)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=4)
def _weight(n: int, k: int, seed: int):
    w = si.int4_weight(n, k, seed)
    codes, scode, sstep, zeros, flags = oracle.quantize_int4_g32_dq(si.bf16_bits(w))
    assert flags == 0
    return w, codes, scode, sstep, zeros


def _ref(x, codes, scode, sstep, zeros):
    return oracle.qgemm_w4a16_dq(si.bf16_bits(x), codes, scode, sstep, zeros, threads=oracle.hardware_threads())


# ------------------------------------------------------------------ quantizer

@pytest.mark.parametrize("n,k", [(768, 256), (256, 768), (1536, 512), (257, 256), (1, 512), (63, 1024)]
                         + list(si.MODEL_SHAPES))
def test_quantize_dq_bit_exact(dev, n, k):
    seed = si.model_weight_seed(n, k) if (n, k) in si.MODEL_SHAPES else n + k
    w, codes, scode, sstep, zeros = _weight(n, k, seed)
    print(f"quantize_int4_g32_dq {n}x{k}", flush=True)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    packed = qg.quantize_int4_g32_dq(w.to(dev), status=status).cpu().numpy()
    ref = oracle.pack_int4_dq(codes, scode, sstep, zeros)
    assert packed.size == ref.size == qg.int4_dq_packed_bytes(n, k)
    if not np.array_equal(packed, ref):
        c, s, t, z = oracle.unpack_int4_dq(packed, n, k)
        raise AssertionError(f"{int((packed != ref).sum())} bytes differ; steps differ in "
                             f"{int((t != sstep).sum())} rows, scale codes in {int((s != scode).sum())} groups")
    assert int(status.item()) == 0


def test_quantize_dq_hand_worked_rows(dev):
    """Each hand-worked row in a 256-wide row whose other groups are zero (the
    row's largest range is unchanged), plus random rows around them."""
    cases = read_cases("int4_dq_rows.txt", width=64)
    n, k = 70, 256
    w = si.bf16_bits(si.int4_weight(n, k, 123)).copy()
    where = {}
    for i, c in enumerate(cases):
        row = (11 * i + 3) % n
        w[row] = 0
        w[row, :64] = c["bits"]
        where[row] = c
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    packed = qg.quantize_int4_g32_dq(si.bits_to_bf16(w).to(dev), status=status).cpu().numpy()
    codes, scode, sstep, zeros = oracle.unpack_int4_dq(packed, n, k)
    want_flags = 0
    for row, c in where.items():
        want_flags |= c["flags"]
        assert int(sstep[row]) == c["step"], c["name"]
        assert scode[row, :2].tolist() == [c["scode0"], c["scode1"]], c["name"]
        assert zeros[row, :2].tolist() == [c["zp0"], c["zp1"]], c["name"]
        assert codes[row, :64].tolist() == c["codes"].tolist(), c["name"]
        if c["flags"] & 1 == 0:
            assert scode[row, 2:].tolist() == [1] * 6 and not codes[row, 64:].any(), c["name"]
    assert int(status.item()) == want_flags
    rc, rs, rt, rz, rf = oracle.quantize_int4_g32_dq(w)
    assert rf == want_flags
    assert np.array_equal(packed, oracle.pack_int4_dq(rc, rs, rt, rz))


def test_quantize_dq_adversarial_rows(dev):
    """Groups of very different ranges in one row, one-sign, tiny (subnormal
    steps), huge, sparse and half-step rows."""
    rng = np.random.default_rng(8)
    n, k = 128, 1024
    v = rng.standard_normal((n, k)) * np.repeat(10.0 ** rng.uniform(-4, 2, (n, k // 32)), 32, axis=1)
    v[0::6] = np.abs(v[0::6]) + 5.0
    v[1::6] = -np.abs(v[1::6]) * 1e-3
    v[2::6] *= 1e-30
    v[3::6] *= 6e4
    v[4::6] *= rng.random((len(range(4, n, 6)), k)) < 0.1
    v[5::6] = np.round(v[5::6] * 4) / 8
    bits = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    packed = qg.quantize_int4_g32_dq(si.bits_to_bf16(bits).to(dev)).cpu().numpy()
    codes, scode, sstep, zeros, _ = oracle.quantize_int4_g32_dq(bits)
    assert np.array_equal(packed, oracle.pack_int4_dq(codes, scode, sstep, zeros))


# ------------------------------------------------------------------ W4A16 GEMV

@pytest.mark.parametrize("n,k", [(768, 256), (256, 768), (1536, 512), (257, 512), (512, 8192)])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_w4a16_dq_small_shapes(dev, n, k, m):
    w, codes, scode, sstep, zeros = _weight(n, k, n + k)
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    x = si.activation(m, k, 1000 + n + m)
    ref = _ref(x, codes, scode, sstep, zeros)
    print(f"qgemm_w4a16_dq {n}x{k} M={m}", flush=True)
    for dt in (torch.float32, torch.bfloat16):
        y = qg.qgemm_w4a16_dq(x.to(dev), packed, n, out_dtype=dt)
        assert y.shape == (m, n) and y.dtype == dt
        assert_w16(y, ref, f"{n}x{k} M={m} {dt}")


@pytest.mark.parametrize("n,k", si.MODEL_SHAPES)
def test_w4a16_dq_model_shapes_decode_buckets(dev, n, k):
    w, codes, scode, sstep, zeros = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    i = si.model_shape_index(n, k)
    for m in si.DECODE_M:
        print(f"qgemm_w4a16_dq {n}x{k} M={m}", flush=True)
        x = si.activation(m, k, si.model_activation_seed(i, m))
        ref = _ref(x, codes, scode, sstep, zeros)
        for dt in (torch.float32, torch.bfloat16):
            assert_w16(qg.qgemm_w4a16_dq(x.to(dev), packed, n, out_dtype=dt), ref, f"{n}x{k} M={m} {dt}")


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_w4a16_dq_every_split_uneven(dev, m):
    """K = 6656 (26 tiles: uneven ranges at splits 4 and 8) and a ragged N."""
    n, k = 257, 6656
    w, codes, scode, sstep, zeros = _weight(n, k, 31)
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    x = si.activation(m, k, 40 + m)
    ref = _ref(x, codes, scode, sstep, zeros)
    for split in si.SPLITS:
        y = qg.qgemm_w4a16_dq(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32)
        assert_w16(y, ref, f"split={split} M={m}")


def test_w4a16_dq_non_finite_row_gives_nan(dev):
    n, k = 64, 256
    w = si.int4_weight(n, k, 3).clone()
    w[5, 17] = float("inf")
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    y = qg.qgemm_w4a16_dq(si.activation(1, k, 2).to(dev), packed, n, out_dtype=torch.float32).cpu()
    assert torch.isnan(y[0, 5])
    assert torch.isfinite(torch.cat([y[0, :5], y[0, 6:]])).all()


@pytest.mark.parametrize("n", [4097, 6600, 8192, 8193])
def test_w4a16_dq_prefetch_grid(dev, n):
    """The two-register-set loop (M = 1, at most 256 workgroups of 32 rows)
    on the scale-code layout, on both sides of the 256-workgroup edge."""
    k = 512
    w, codes, scode, sstep, zeros = _weight(n, k, 90 + n)
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    x = si.activation(1, k, 95 + n)
    ref = _ref(x, codes, scode, sstep, zeros)
    print(f"qgemm_w4a16_dq prefetch grid N={n}", flush=True)
    for dt in (torch.float32, torch.bfloat16):
        assert_w16(qg.qgemm_w4a16_dq(x.to(dev), packed, n, out_dtype=dt), ref, f"N={n} {dt}")


def test_w4a16_dq_prefetch_grid_non_finite_row(dev):
    """N = 6656 (208 workgroups, prefetching): a non-finite weight in row 70
    makes that row's step NaN, and only y[70] may be NaN."""
    n, k = 6656, 256
    w = si.int4_weight(n, k, 4).clone()
    w[70, 9] = float("inf")
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    y = qg.qgemm_w4a16_dq(si.activation(1, k, 6).to(dev), packed, n, out_dtype=torch.float32).cpu()
    assert torch.isnan(y[0, 70])
    assert torch.isfinite(torch.cat([y[0, :70], y[0, 71:]])).all()


@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_w4a16_dq_64_row_workgroups_ragged_n(dev, m):
    """N = 8200 at M = 1..4: one split takes 64-row workgroups (129, the last
    with 8 live rows; M >= 2 on the matrix instruction), two splits 32-row
    ones; both read each row's step from its block's head."""
    n, k = 8200, 512
    w, codes, scode, sstep, zeros = _weight(n, k, 46)
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    x = si.activation(m, k, 61 + m)
    ref = _ref(x, codes, scode, sstep, zeros)
    print(f"qgemm_w4a16_dq 64-row workgroups N=8200 M={m}", flush=True)
    for split in (1, 2):
        for dt in (torch.float32, torch.bfloat16):
            y = qg.qgemm_w4a16_dq(x.to(dev), packed, n, split_k=split, out_dtype=dt)
            assert_w16(y, ref, f"N=8200 M={m} split={split} {dt}")


def test_w4a16_dq_64_row_workgroups_non_finite_row(dev):
    """8448 rows (64-row workgroups at M = 1): a non-finite weight in row 8400
    of the last block makes only y[8400] NaN."""
    n, k = 8448, 256
    w = si.int4_weight(n, k, 8).clone()
    w[8400, 3] = float("-inf")
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    y = qg.qgemm_w4a16_dq(si.activation(1, k, 9).to(dev), packed, n, out_dtype=torch.float32).cpu()
    assert torch.isnan(y[0, 8400])
    assert torch.isfinite(torch.cat([y[0, :8400], y[0, 8401:]])).all()


def test_w4a16_dq_repeat_and_graph_replay_are_bit_identical(dev):
    n, k = 8448, 6656
    w, *_ = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    for m in (1, 4):
        x = si.activation(m, k, 77 + m).to(dev)
        for split in (1, 4):
            eager = qg.qgemm_w4a16_dq(x, packed, n, split_k=split)
            assert torch.equal(eager, qg.qgemm_w4a16_dq(x, packed, n, split_k=split))
            out = torch.empty_like(eager)
            ws = torch.empty(max(qg.workspace_bytes(m, n, k, split), 1), dtype=torch.uint8, device=dev)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                qg.qgemm_w4a16_dq(x, packed, n, split_k=split, out=out, workspace=ws)
            for _ in range(3):
                out.zero_()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                assert torch.equal(out, eager), f"replay differs (m={m}, split={split})"
                _ = qg.qgemm_w4a16_dq(x, packed, n, split_k=1)


def test_w4a16_dq_rejects_m_above_64(dev):
    w, *_ = _weight(256, 768, 3)
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    with pytest.raises(qg.QGemmError) as e:
        qg.qgemm_w4a16_dq(si.activation(65, 768, 1).to(dev), packed, 256)
    assert e.value.status == -4


@pytest.mark.parametrize("m", [5, 8, 16, 17, 32, 33, 48, 64])
def test_w4a16_dq_matrix_core_runtime_m_and_tails(dev, m):
    """The matrix-core kernels on the scale-code layout; N = 257 leaves a one-row tail block."""
    for n, k in ((257, 768), (768, 512)):
        w, codes, scode, sstep, zeros = _weight(n, k, n + k)
        packed = qg.quantize_int4_g32_dq(w.to(dev))
        x = si.activation(m, k, 800 + m)
        ref = _ref(x, codes, scode, sstep, zeros)
        for dt in (torch.float32, torch.bfloat16):
            assert_w16(qg.qgemm_w4a16_dq(x.to(dev), packed, n, out_dtype=dt), ref, f"{n}x{k} M={m} {dt}")


@pytest.mark.parametrize("n,k", [(39936, 6656), (6656, 19968), (8448, 6656)])
@pytest.mark.parametrize("m", [16, 64])
def test_w4a16_dq_large_buckets(dev, n, k, m):
    print(f"qgemm_w4a16_dq {n}x{k} M={m}", flush=True)
    w, codes, scode, sstep, zeros = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    x = si.activation(m, k, 1300 + m)
    ref = _ref(x, codes, scode, sstep, zeros)
    for split in (0, 2):
        y = qg.qgemm_w4a16_dq(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32)
        assert_w16(y, ref, f"{n}x{k} M={m} split={split}")


# ------------------------------------------------------------------ W4A8 on scale codes

@pytest.mark.parametrize("per_group", [False, True])
@pytest.mark.parametrize("n,k", [(768, 256), (257, 512), (1536, 512)])
@pytest.mark.parametrize("m", [1, 2, 3, 4])
def test_w4a8_dq_small_shapes(dev, per_group, n, k, m):
    w, codes, scode, sstep, zeros = _weight(n, k, n + k)
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    x = si.activation(m, k, 1400 + n + m)
    xb = si.bf16_bits(x)
    fn, ref_fn = ((qg.qgemm_w4a8_g32_dq, oracle.qgemm_w4a8_g32_dq) if per_group
                  else (qg.qgemm_w4a8_dq, oracle.qgemm_w4a8_dq))
    ref = ref_fn(xb, codes, scode, sstep, zeros)
    for dt in (torch.float32, torch.bfloat16):
        assert_w16(fn(x.to(dev), packed, n, out_dtype=dt), ref, f"{n}x{k} M={m} group={per_group} {dt}")


@pytest.mark.parametrize("n,k", [(8448, 6656), (6656, 19968)])
def test_w4a8_dq_config_shapes(dev, n, k):
    """The W4A8 layer shapes and buckets 1..4: parity with the W4A8 oracle and
    the pages' precision class against the W4A16 oracle."""
    w, codes, scode, sstep, zeros = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    i = si.model_shape_index(n, k)
    for m in si.DECODE_M:
        print(f"qgemm_w4a8_dq {n}x{k} M={m}", flush=True)
        x = si.activation(m, k, si.model_activation_seed(i, m))
        xb = si.bf16_bits(x)
        ref16 = _ref(x, codes, scode, sstep, zeros)
        for fn, ref_fn in ((qg.qgemm_w4a8_dq, oracle.qgemm_w4a8_dq), (qg.qgemm_w4a8_g32_dq, oracle.qgemm_w4a8_g32_dq)):
            y = fn(x.to(dev), packed, n, out_dtype=torch.float32)
            assert_w16(y, ref_fn(xb, codes, scode, sstep, zeros, threads=oracle.hardware_threads()),
                       f"{fn.__name__} {n}x{k} M={m}")
            assert_w4a8_class(y, ref16, f"{fn.__name__} vs W4A16 {n}x{k} M={m}")


@pytest.mark.parametrize("m", [1, 4])
def test_w4a8_dq_every_split(dev, m):
    n, k = 257, 6656
    w, codes, scode, sstep, zeros = _weight(n, k, 31)
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    x = si.activation(m, k, 90 + m)
    xb = si.bf16_bits(x)
    for fn, ref_fn in ((qg.qgemm_w4a8_dq, oracle.qgemm_w4a8_dq), (qg.qgemm_w4a8_g32_dq, oracle.qgemm_w4a8_g32_dq)):
        ref = ref_fn(xb, codes, scode, sstep, zeros)
        for split in si.SPLITS:
            y = fn(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32)
            assert_w16(y, ref, f"{fn.__name__} M={m} split={split}")


def test_w4a8_dq_graph_replay_bit_identical(dev):
    n, k = 6656, 19968
    w, *_ = _weight(n, k, si.model_weight_seed(n, k))
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    for fn in (qg.qgemm_w4a8_dq, qg.qgemm_w4a8_g32_dq):
        for m, split in ((1, 1), (4, 1), (2, 4)):
            x = si.activation(m, k, 120 + m).to(dev)
            eager = fn(x, packed, n, split_k=split)
            assert torch.equal(eager, fn(x, packed, n, split_k=split))
            out = torch.empty_like(eager)
            ws = torch.empty(max(qg.workspace_bytes(m, n, k, split), 1), dtype=torch.uint8, device=dev)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(x, packed, n, split_k=split, out=out, workspace=ws)
            for _ in range(3):
                out.zero_()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                assert torch.equal(out, eager), f"{fn.__name__} replay differs (m={m}, split={split})"
                _ = fn(x, packed, n, split_k=1)
