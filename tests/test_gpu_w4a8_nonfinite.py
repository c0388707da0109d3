"""GPU parity for non-finite activations under W4A8.

Neither executorch's Int4QuantizedGemmPrecisionTest nor the other pages say
what int8 activation quantization does with a NaN or an infinity.  The
reading taken: a span (a row for per-row scales, a group of 32 for per-group
scales) holding one has no finite absmax scale, so every output of that
activation row is NaN; the other rows do not change.  Checked on every W4A8
entry point, both packed layouts, buckets 1..4 and 8, both workgroup shapes
(N = 8200 with an 8-row tail, N = 768) and one and two splits: the bad row is
NaN on the GPU and in the oracle, the clean rows are bit-identical to a call
without the bad value and within the W4A16 bounds of the oracle.
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
BAD = {"nan": float("nan"), "+inf": float("inf"), "-inf": float("-inf")}


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=4)
def _weight(n, dq):
    w = si.int4_weight(n, K, 600 + n)
    if dq:
        codes, scode, sstep, zeros, _ = oracle.quantize_int4_g32_dq(si.bf16_bits(w))
        return w, (codes, scode, sstep, zeros)
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    return w, (codes, scales, zeros)


ENTRIES = {
    "qgemm_w4a8": (False, qg.qgemm_w4a8, oracle.qgemm_w4a8),
    "qgemm_w4a8_g32": (False, qg.qgemm_w4a8_g32, oracle.qgemm_w4a8_g32),
    "qgemm_w4a8_dq": (True, qg.qgemm_w4a8_dq, oracle.qgemm_w4a8_dq),
    "qgemm_w4a8_g32_dq": (True, qg.qgemm_w4a8_g32_dq, oracle.qgemm_w4a8_g32_dq),
}


@pytest.mark.parametrize("kind", sorted(BAD))
@pytest.mark.parametrize("n", [768, 8200])
@pytest.mark.parametrize("entry", sorted(ENTRIES))
def test_non_finite_activation_gives_a_nan_row(dev, entry, n, kind):
    dq, fn, ref_fn = ENTRIES[entry]
    w, parts = _weight(n, dq)
    packed = (qg.quantize_int4_g32_dq if dq else qg.quantize_int4_g32)(w.to(dev))
    for m in (1, 2, 3, 4, 8):
        bad = m // 2
        x = si.activation(m, K, 700 + m)
        xbad = x.clone()
        xbad[bad, 37] = BAD[kind]
        ref = ref_fn(si.bf16_bits(xbad), *parts, threads=oracle.hardware_threads())
        assert np.isnan(ref[bad]).all()
        keep = [r for r in range(m) if r != bad]
        for split in (1, 2):
            label = f"{entry} N={n} M={m} split={split} {kind} in row {bad}"
            print(label, flush=True)
            y_clean = fn(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32).cpu()
            y = fn(xbad.to(dev), packed, n, split_k=split, out_dtype=torch.float32).cpu()
            assert torch.isnan(y[bad]).all(), label
            assert torch.equal(y[keep], y_clean[keep]), label
            if keep:
                assert_w16(y[keep], ref[keep], label)
