"""Exact-arithmetic GPU pins: inputs on which every product and every partial
sum is exact in binary32, so the GPU's fp32 output must equal the oracle's
value (rounded once to binary32) bit for bit, whatever the kernel's order of
summation.  A dropped, doubled or misplaced product, a wrong zero point or
scale on a single group, or a lost DPP / matrix-instruction result changes
the output by at least one unit and fails here, where the W4A16 tolerance
(1e-2 * mean|ref| + 1e-3) might let it through.

  * grid weights: every group is (q - zp) * 2^e with e in {-2, -1, 0}, zp and
    the codes random and every group holding the codes 0 and L (L = 15, 31,
    63), so the quantizer returns exactly those codes, zero points and
    power-of-two scales; activations are small integers.  Every dequantized
    weight times x is an integer multiple of 2^-2 and every partial sum stays
    below 2^22 of those units.  Run on qgemm_w4a16, qgemm_wn_a16 (INT5, INT6)
    and, with activations on the int8 grid (the largest |x| of every row, or
    of every group of 32, is 127, so sx = 1 and xq = x), on qgemm_w4a8 and
    qgemm_w4a8_g32.
  * one-hot activations (x = e_j): y[:, n] = (q[n, j] - zp) * s exactly, on
    random weights and every layout (the scale-code layout, whose scales
    c * step have up to 19 significant bits, included).
  * W8A16 with integer x: the sum is exact, and y = fp32(sum) * scale is one
    rounding of the exact product.
All at M = 1, 2, 3, 4, 5, 16, 33, 64 (every kernel family), every legal split,
N = 8200 (64-row GEMV workgroups and an 8-row tail) and N = 768.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si

import gemm_decode_qgemm_amd as qg

pytestmark = pytest.mark.gpu

K = 2048
BUCKETS = (1, 2, 3, 4, 5, 16, 33, 64)
SPLITS = (1, 2, 4, 8)


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


def _bf16(v: np.ndarray) -> torch.Tensor:
    t = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(t.double(), torch.tensor(v, dtype=torch.float64)), "values must be bf16-exact"
    return t


@functools.lru_cache(maxsize=8)
def _grid_weight(n: int, levels: int, seed: int) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    g = K // 32
    q = rng.integers(0, levels + 1, (n, g, 32))
    a = rng.integers(0, 32, (n, g))
    b = (a + rng.integers(1, 32, (n, g))) % 32                 # a != b
    rows, grp = np.meshgrid(np.arange(n), np.arange(g), indexing="ij")
    q[rows, grp, a] = 0
    q[rows, grp, b] = levels
    zp = rng.integers(0, levels + 1, (n, g, 1))
    e = rng.integers(-2, 1, (n, g, 1))
    return _bf16(((q - zp) * np.ldexp(1.0, e)).reshape(n, K))


def _int_x(m: int, lim: int, seed: int, peak: int | None = None, per_group: bool = False) -> torch.Tensor:
    """Integers in [-lim, lim]; with `peak`, one entry of every row (or of every
    group of 32) is +-peak, so that row's (group's) absmax is exactly peak."""
    rng = np.random.default_rng(seed)
    x = rng.integers(-lim, lim + 1, (m, K))
    if peak is not None:
        spans = K // 32 if per_group else 1
        width = K // spans
        for r in range(m):
            for s in range(spans):
                x[r, s * width + rng.integers(0, width)] = peak * (1 if rng.random() < 0.5 else -1)
    return _bf16(x.astype(np.float64))


def _one_hot(m: int, cols) -> torch.Tensor:
    x = np.zeros((m, K))
    for r, c in enumerate(cols):
        x[r, c] = 1.0
    return _bf16(x)


def _hot_columns(m: int, call: int) -> list[int]:
    """Columns for one call: group edges and tile edges first, then a stride
    that walks every column over the calls."""
    edges = [0, 1, 7, 8, 31, 32, 127, 128, 255, 256, K - 256, K - 33, K - 32, K - 1]
    cols = [(edges[(call * m + r) % len(edges)] if call == 0 else (call * 97 + r * 131) % K) for r in range(m)]
    return cols


def _assert_exact(y: torch.Tensor, ref: np.ndarray, label: str) -> None:
    got = y.cpu().numpy()
    want = ref.astype(np.float32)
    bad = got != want
    assert not bad.any(), (f"{label}: {int(bad.sum())} of {bad.size} outputs differ; first at "
                           f"{np.argwhere(bad)[0].tolist()}: {got[bad][0]!r} vs {want[bad][0]!r}")


def _splits(m):
    return [s for s in SPLITS if s <= K // 256]


# ---------------------------------------------------------------- grid weights


GRID_ENTRIES = {
    # name: (levels, weight kind, GPU entry (None: qgemm_wn_a16), oracle GEMM, |x| limit,
    #        activation absmax per span (None: not on the int8 grid), one span per group of 32)
    "w4a16": (15, "int4", qg.qgemm_w4a16, oracle.qgemm_w4a16, 31, None, False),
    "w5a16": (31, "int5", None, oracle.qgemm_w4a16, 31, None, False),
    "w6a16": (63, "int6", None, oracle.qgemm_w4a16, 15, None, False),
    "w4a8": (15, "int4", qg.qgemm_w4a8, oracle.qgemm_w4a8, 15, 127, False),
    "w4a8_g32": (15, "int4", qg.qgemm_w4a8_g32, oracle.qgemm_w4a8_g32, 15, 127, True),
}


def _quantize_grid(dev, kind, w):
    wb = si.bf16_bits(w)
    if kind == "int4":
        codes, scales, zeros, flags = oracle.quantize_int4_g32(wb)
        packed = qg.quantize_int4_g32(w.to(dev))
        ref_packed = oracle.pack_int4(codes, scales, zeros)
    else:
        bits = int(kind[3])
        codes, scales, zeros, flags = oracle.quantize_intn_g32(wb, bits)
        packed = qg.quantize_intn_g32(w.to(dev), bits)
        ref_packed = oracle.pack_intn(codes, scales, zeros, bits)
    assert flags == 0
    assert np.array_equal(packed.cpu().numpy(), ref_packed), "packed grid weight differs from the oracle"
    # the grid is reproduced exactly: power-of-two scales
    s = oracle.fp16_to_float64(scales)
    assert (np.frexp(s)[0] == 0.5).all(), "grid scales must come back as powers of two"
    return packed, (codes, scales, zeros)


@pytest.mark.parametrize("n", [768, 8200])
@pytest.mark.parametrize("entry", sorted(GRID_ENTRIES))
def test_grid_weight_integer_activations_exact(dev, entry, n):
    levels, kind, fn, ref_fn, lim, peak, per_group = GRID_ENTRIES[entry]
    w = _grid_weight(n, levels, 900 + levels + n)
    packed, parts = _quantize_grid(dev, kind, w)
    if fn is None:
        bits = int(kind[3])

        def fn(x, p, nn, **kw):
            return qg.qgemm_wn_a16(x, p, nn, bits, **kw)
    for m in BUCKETS:
        x = _int_x(m, lim, 1000 + m, peak, per_group)
        ref = ref_fn(si.bf16_bits(x), *parts, threads=oracle.hardware_threads())
        xd = x.to(dev)
        for split in _splits(m):
            label = f"{entry} N={n} M={m} split={split}"
            print(label, flush=True)
            y = fn(xd, packed, n, split_k=split, out_dtype=torch.float32)
            _assert_exact(y, ref, label)


# ---------------------------------------------------------------- one-hot


@functools.lru_cache(maxsize=4)
def _random_weight(n: int):
    return si.int4_weight(n, K, 1300 + n)


ONE_HOT_ENTRIES = ["w4a16", "w4a16_dq", "w5a16", "w6a16"]


def _one_hot_setup(dev, entry, n):
    w = _random_weight(n)
    wb = si.bf16_bits(w)
    if entry == "w4a16":
        codes, scales, zeros, _ = oracle.quantize_int4_g32(wb)
        packed = qg.quantize_int4_g32(w.to(dev))

        def ref(xb):
            return oracle.qgemm_w4a16(xb, codes, scales, zeros, threads=oracle.hardware_threads())

        return packed, ref, qg.qgemm_w4a16
    if entry == "w4a16_dq":
        codes, scode, sstep, zeros, _ = oracle.quantize_int4_g32_dq(wb)
        packed = qg.quantize_int4_g32_dq(w.to(dev))

        def ref(xb):
            return oracle.qgemm_w4a16_dq(xb, codes, scode, sstep, zeros, threads=oracle.hardware_threads())

        return packed, ref, qg.qgemm_w4a16_dq
    bits = int(entry[1])
    codes, scales, zeros, _ = oracle.quantize_intn_g32(wb, bits)
    packed = qg.quantize_intn_g32(w.to(dev), bits)

    def ref(xb):
        return oracle.qgemm_w4a16(xb, codes, scales, zeros, threads=oracle.hardware_threads())

    def fn(x, p, nn, **kw):
        return qg.qgemm_wn_a16(x, p, nn, bits, **kw)

    return packed, ref, fn


@pytest.mark.parametrize("n", [768, 8200])
@pytest.mark.parametrize("entry", ONE_HOT_ENTRIES)
def test_one_hot_activations_exact(dev, entry, n):
    packed, ref_fn, fn = _one_hot_setup(dev, entry, n)
    for m in BUCKETS:
        calls = K // 64 if (m == 64 and n == 768) else 2     # every column of K once
        for call in range(calls):
            cols = list(range(call * 64, call * 64 + 64)) if calls > 2 else _hot_columns(m, call)
            x = _one_hot(m, cols)
            ref = ref_fn(si.bf16_bits(x))
            xd = x.to(dev)
            for split in _splits(m) if call == 0 else (0,):
                label = f"{entry} N={n} M={m} split={split} columns {cols[:4]}..."
                print(label, flush=True)
                y = fn(xd, packed, n, split_k=split, out_dtype=torch.float32)
                _assert_exact(y, ref, label)


# ---------------------------------------------------------------- W8A16


@pytest.mark.parametrize("n", [768, 8200, 16400])
def test_w8a16_integer_activations_one_rounding(dev, n):
    torch.manual_seed(77 + n)
    w = torch.randint(-127, 128, (n, K), dtype=torch.int8)
    scale = torch.randn(n, dtype=torch.bfloat16)
    wd, sd = w.to(dev), scale.to(dev)
    for m in BUCKETS:
        x = _int_x(m, 15, 1500 + m)     # |partial sums of x * (w + 128)| < 2^24
        ref = oracle.qgemm_w8a16(si.bf16_bits(x), w.numpy(), si.bf16_bits(scale),
                                 threads=oracle.hardware_threads())
        label = f"w8a16 N={n} M={m}"
        print(label, flush=True)
        y = qg.qgemm_w8a16(x.to(dev), wd, sd, out_dtype=torch.float32)
        _assert_exact(y, ref, label)


# ---------------------------------------------------------------- W4A8 on scale codes


@pytest.mark.parametrize("entry", ["qgemm_w4a8_dq", "qgemm_w4a8_g32_dq"])
def test_w4a8_scale_codes_tight(dev, entry):
    """Scale codes c * step carry up to 19 significant bits, so s * I rounds:
    each output must be within (groups + 2) * 2^-24 of sum_g |s_g * I_g| of
    the oracle's value (activations on the int8 grid: sx = 1, xq = x)."""
    n = 8200
    per_group = entry == "qgemm_w4a8_g32_dq"
    w = _random_weight(n)
    codes, scode, sstep, zeros, _ = oracle.quantize_int4_g32_dq(si.bf16_bits(w))
    packed = qg.quantize_int4_g32_dq(w.to(dev))
    fn = getattr(qg, entry)
    ref_fn = getattr(oracle, entry)
    g = K // 32
    step = oracle.fp16_to_float64(sstep)[:, None]
    s = scode.astype(np.float64) * step                                  # [n, g]
    wi = (codes.astype(np.int64).reshape(n, g, 32) - zeros.astype(np.int64)[:, :, None])
    for m in BUCKETS:
        x = _int_x(m, 15, 1700 + m, 127, per_group)
        xi = np.rint(oracle.bf16_to_float64(si.bf16_bits(x))).astype(np.int64).reshape(m, g, 32)
        mag = np.einsum("mgk,ngk->mng", xi, wi)                          # exact integer group dots
        bound = (g + 2) * 2.0 ** -24 * np.abs(mag * s[None]).sum(axis=2)
        ref = ref_fn(si.bf16_bits(x), codes, scode, sstep, zeros, threads=oracle.hardware_threads())
        for split in _splits(m):
            label = f"{entry} N={n} M={m} split={split}"
            print(label, flush=True)
            y = fn(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32).cpu().double().numpy()
            over = np.abs(y - ref) > bound
            assert not over.any(), f"{label}: {int(over.sum())} outputs outside (G+2) * 2^-24 * sum|s*I|"
