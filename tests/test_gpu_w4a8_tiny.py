"""GPU parity for activation spans at the bottom of the binary32 range (W4A8).

The pages do not say what int8 activation quantization does with a span
whose inverse scale 127/a overflows binary32 (executorch
test_int4_quantized_gemm.py, Int4QuantizedGemmPrecisionTest, says only "int8
activations").  The reading taken: such a span has no finite inverse scale
and is a zero span (sx = 0, codes 0); 127/a is finite exactly when
a >= 255 * 2^-129 (hand-worked cases A4-A7 of tests/golden/actquant_rows.txt).

Checked on every W4A8 entry point, both packed layouts, buckets 1..4 and the
matrix-core and slice paths above 4 rows, both workgroup shapes (N = 8200 and
N = 768), one and two splits:
  * a span just below the threshold (j * 2^-130, |j| <= 254) gives exactly
    what a zero span gives: per row, an all-zero output row; per group, the
    output of the same x with that group set to 0, bit for bit;
  * a span just above it (j * 2^-129, one j = 255) keeps its scale: its row
    (all other groups zero, for per-group scales) is nonzero and within 1e-4
    of the row's largest output of the oracle, which keeps the subnormal sx;
  * the ordinary rows are bit-identical to a call without the tiny spans and
    within the W4A16 bounds of the oracle.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from tolerance import assert_w16

import gemm_decode_qgemm_amd as qg

pytestmark = pytest.mark.gpu

K = 512


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=4)
def _weight(n, dq):
    w = si.int4_weight(n, K, 610 + n)
    if dq:
        codes, scode, sstep, zeros, _ = oracle.quantize_int4_g32_dq(si.bf16_bits(w))
        return w, (codes, scode, sstep, zeros)
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    return w, (codes, scales, zeros)


ENTRIES = {
    "qgemm_w4a8": (False, False, qg.qgemm_w4a8, oracle.qgemm_w4a8),
    "qgemm_w4a8_g32": (False, True, qg.qgemm_w4a8_g32, oracle.qgemm_w4a8_g32),
    "qgemm_w4a8_dq": (True, False, qg.qgemm_w4a8_dq, oracle.qgemm_w4a8_dq),
    "qgemm_w4a8_g32_dq": (True, True, qg.qgemm_w4a8_g32_dq, oracle.qgemm_w4a8_g32_dq),
}


def _tiny(length, seed, below):
    """bf16 j * 2^-130 with |j| <= 254 (127/a overflows), or j * 2^-129 with
    one j = 255 (the smallest absmax whose 127/a is finite); every value is
    exact in bf16 (the smallest ones are bf16 subnormals)."""
    rng = np.random.default_rng(seed)
    if below:
        j = rng.integers(-254, 255, length)
        j[length // 3] = 254
        v = j * 2.0 ** -130
    else:
        j = rng.integers(-255, 256, length)
        j[length // 2] = 255
        v = j * 2.0 ** -129
    t = torch.tensor(v, dtype=torch.float32).to(torch.bfloat16)
    assert torch.equal(t.double(), torch.tensor(v, dtype=torch.float64)), "tiny values must be bf16-exact"
    return t


def _cases(m, group):
    """(x, flush_rows, border_rows, zero_equivalent_x) for one bucket: x with a
    flushed span and a span just above the threshold; zero_equivalent_x is x
    with the flushed span set to 0."""
    x = si.activation(m, K, 720 + m)
    out = []
    if not group:
        if m == 1:
            out.append((_tiny(K, 1, True).reshape(1, K), [0], []))
            out.append((_tiny(K, 2, False).reshape(1, K), [], [0]))
        else:
            xt = x.clone()
            xt[0] = _tiny(K, 3, True)
            xt[m - 1] = _tiny(K, 4, False)
            out.append((xt, [0], [m - 1]))
        return [(xt, fr, br, None) for xt, fr, br in out]
    # per group: row 0 has a flushed group 2 and a border group 5 among
    # ordinary groups; the border row holds group 3 only
    xt = x.clone()
    xt[0, 64:96] = _tiny(32, 5, True)
    xt[0, 160:192] = _tiny(32, 6, False)
    xz = xt.clone()
    xz[0, 64:96] = 0
    res = [(xt, [], [], xz)]
    xb = x.clone() if m > 1 else torch.zeros(1, K, dtype=torch.bfloat16)
    xb[m - 1] = 0
    xb[m - 1, 96:128] = _tiny(32, 7, False)
    res.append((xb, [], [m - 1], None))
    return res


@pytest.mark.parametrize("n", [768, 8200])
@pytest.mark.parametrize("entry", sorted(ENTRIES))
def test_tiny_activation_spans(dev, entry, n):
    dq, group, fn, ref_fn = ENTRIES[entry]
    w, parts = _weight(n, dq)
    packed = (qg.quantize_int4_g32_dq if dq else qg.quantize_int4_g32)(w.to(dev))
    for m in (1, 2, 3, 4, 8, 16):
        for ci, (xt, flush_rows, border_rows, xz) in enumerate(_cases(m, group)):
            ref = ref_fn(si.bf16_bits(xt), *parts, threads=oracle.hardware_threads())
            for r in flush_rows:
                assert (ref[r] == 0).all()
            plain = [r for r in range(m) if r not in flush_rows and r not in border_rows]
            if not group:
                xc = xt.clone()
                xc[flush_rows + border_rows] = 0      # the ordinary rows alone
            for split in (1, 2):
                label = f"{entry} N={n} M={m} case={ci} split={split}"
                print(label, flush=True)
                y = fn(xt.to(dev), packed, n, split_k=split, out_dtype=torch.float32).cpu()
                assert torch.isfinite(y).all(), label
                for r in flush_rows:
                    assert (y[r] == 0).all(), f"{label}: flushed row {r} not zero"
                for r in border_rows:
                    rr = ref[r]
                    assert (rr != 0).any()
                    err = np.abs(y[r].double().numpy() - rr)
                    assert err.max() <= 1e-4 * np.abs(rr).max(), f"{label}: border row {r}"
                    assert ((y[r] != 0).numpy() | (rr == 0)).all(), f"{label}: border row {r} flushed"
                if xz is not None:
                    yz = fn(xz.to(dev), packed, n, split_k=split, out_dtype=torch.float32).cpu()
                    assert torch.equal(y, yz), f"{label}: flushed group differs from a zero group"
                if plain and not group:
                    yc = fn(xc.to(dev), packed, n, split_k=split, out_dtype=torch.float32).cpu()
                    assert torch.equal(y[plain], yc[plain]), label
                if plain:
                    assert_w16(y[plain], ref[plain], label)
