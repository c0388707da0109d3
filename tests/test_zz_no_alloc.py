"""qgemm_w4a16_noalloc through the C ABI: the split-K partial sums in the
library's static device scratch instead of a caller workspace.

Checked against qgemm_w4a16 at the same split (the same kernels, so the
outputs must be bit-identical) and against the oracle (the W4A16 bound), on
consecutive calls whose sizes shrink and then grow again, so that a call
reading what an earlier, larger call left in the scratch would show; an
explicit split whose partials exceed the scratch is refused with nothing
launched.
"""
from __future__ import annotations

import numpy as np
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


def _layer(dev, n, k, m, seed):
    w = si.int4_weight(n, k, seed)
    x = si.activation(m, k, seed + 1)
    codes, scales, zeros, _ = oracle.quantize_int4_g32(si.bf16_bits(w))
    return qg.quantize_int4_g32(w.to(dev)), x, (codes, scales, zeros)


def _check(dev, packed, x, parts, n, split, out_dtype, label, rows=None):
    xd = x.to(dev)
    y = qg.qgemm_w4a16_noalloc(xd, packed, n, split_k=split, out_dtype=out_dtype)
    y_ref = qg.qgemm_w4a16(xd, packed, n, split_k=split, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), f"{label}: differs from qgemm_w4a16 at the same split"
    rows = list(range(x.shape[0])) if rows is None else rows
    ref = oracle.qgemm_w4a16(si.bf16_bits(x[rows]), *parts, threads=oracle.hardware_threads())
    assert_w16(y[rows].cpu(), ref, label)


def test_noalloc_matches_qgemm_w4a16_on_consecutive_calls(dev):
    big = _layer(dev, 8448, 6656, 64, 41)
    small = _layer(dev, 768, 512, 3, 43)
    mid = _layer(dev, 6656, 4096, 16, 45)
    steps = [
        (big, 8448, 4, torch.float32, "8448x6656 M=64 split 4 (8.6 MB of partials)"),
        (small, 768, 2, torch.bfloat16, "768x512 M=3 split 2"),
        (mid, 6656, 8, torch.float32, "6656x4096 M=16 split 8"),
        (small, 768, 0, torch.float32, "768x512 M=3 default split"),
        (big, 8448, 2, torch.bfloat16, "8448x6656 M=64 split 2"),
        (small, 768, 1, torch.float32, "768x512 M=3 split 1 (no scratch)"),
    ]
    for (packed, x, parts), n, split, dt, label in steps:
        print(label, flush=True)
        rows = [0, 31, 63] if x.shape[0] == 64 else None
        _check(dev, packed, x, parts, n, split, dt, label, rows)


def test_noalloc_refuses_a_split_beyond_the_scratch(dev):
    n, k, m = 39936, 6656, 64
    packed = torch.zeros(qg.int4_packed_bytes(n, k), dtype=torch.uint8, device=dev)
    x = torch.zeros((m, k), dtype=torch.bfloat16, device=dev)
    y = torch.full((m, n), 7.0, dtype=torch.float32, device=dev)
    with pytest.raises(qg.QGemmError) as ei:
        qg.qgemm_w4a16_noalloc(x, packed, n, split_k=8, out_dtype=torch.float32, out=y)
    assert ei.value.status == -11
    torch.cuda.synchronize()
    assert bool((y == 7.0).all()), "a refused call must launch nothing"
    # the default split of the same shape needs no scratch at all
    qg.qgemm_w4a16_noalloc(x, packed, n, out_dtype=torch.float32, out=y)
    torch.cuda.synchronize()
    assert bool((y == 0).all())
