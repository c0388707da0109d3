"""GPU parity: W4A8 at every decode bucket above 4 rows.

The pages' buckets run to 64 rows (executorch test_int4_quantized_gemm.py,
SUPPORTED_BUCKETS).  At M = 5..64 the W4A8 entry points quantize x once into
the workspace and run the bf16 matrix-core kernel on the exact int8 values,
one pass over the weight: per-row scales are applied after the sum over K,
per-group scales to each group's integer dot.  Checked on every W4A8 entry
point and both packed layouts against the matching W4A8 oracle with the
W4A16 bounds: ragged M (5, 33), M = 8, 16, 64, ragged N, one and two splits
and the default, both output dtypes, every split on both paths; the pages'
W4A8 layer shapes at M = 16 and 64 with the precision class against the W4A16
oracle (gaussian activations); rows independent of the rows padded next to
them; bit-equal graph replay.
"""
from __future__ import annotations

import functools

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from tolerance import assert_w16, assert_w4a8_class

import gemm_decode_qgemm_amd as qg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=6)
def _weight(n, k, seed, dq):
    w = si.int4_weight(n, k, seed)
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


def _packed(w, dq, dev):
    return (qg.quantize_int4_g32_dq if dq else qg.quantize_int4_g32)(w.to(dev))


@pytest.mark.parametrize("n,k", [(257, 512), (768, 256), (1536, 1024)])
@pytest.mark.parametrize("entry", sorted(ENTRIES))
def test_buckets_above_4_small_shapes(dev, entry, n, k):
    dq, fn, ref_fn = ENTRIES[entry]
    w, parts = _weight(n, k, n + k, dq)
    packed = _packed(w, dq, dev)
    for m in (5, 8, 16, 33, 64):
        x = si.activation(m, k, 3000 + m + n)
        ref = ref_fn(si.bf16_bits(x), *parts, threads=oracle.hardware_threads())
        for split in [sp for sp in (0, 1, 2) if sp <= k // 256]:
            for dt in (torch.float32, torch.bfloat16):
                label = f"{entry} {n}x{k} M={m} split={split} {dt}"
                print(label, flush=True)
                assert_w16(fn(x.to(dev), packed, n, split_k=split, out_dtype=dt), ref, label)


@pytest.mark.parametrize("n,k", [(8448, 6656), (6656, 19968)])
@pytest.mark.parametrize("entry", ["qgemm_w4a8", "qgemm_w4a8_g32"])
def test_buckets_16_and_64_layer_shapes(dev, entry, n, k):
    """The pages' W4A8 layer shapes at the MFMA buckets: parity with the W4A8
    oracle and, on gaussian activations, the precision class against W4A16."""
    dq, fn, ref_fn = ENTRIES[entry]
    w, parts = _weight(n, k, si.model_weight_seed(n, k), dq)
    packed = _packed(w, dq, dev)
    i = si.model_shape_index(n, k)
    t = oracle.hardware_threads()
    for m in (16, 64):
        x = si.activation(m, k, si.model_activation_seed(i, m))
        xb = si.bf16_bits(x)
        ref8 = ref_fn(xb, *parts, threads=t)
        ref16 = oracle.qgemm_w4a16(xb, *parts, threads=t)
        label = f"{entry} {n}x{k} M={m}"
        print(label, flush=True)
        y = fn(x.to(dev), packed, n, out_dtype=torch.float32)
        assert_w16(y, ref8, label + " vs W4A8 oracle")
        assert_w4a8_class(y, ref16, label + " vs W4A16 oracle")


def test_rows_are_independent_of_their_padding(dev):
    """An M = 13 call runs the 16-row kernel with 3 padded rows: its rows are
    bit-identical to the first 13 rows of an M = 16 call whose last 3 rows
    hold other activations (same kernel and split), on every W4A8 entry
    point."""
    n, k = 1000, 2048
    x16 = si.activation(16, k, 18)
    x16[13:] = si.activation(3, k, 19) * 40       # different scales in the extra rows
    x13 = x16[:13].contiguous()
    for dq in (False, True):
        w, _ = _weight(n, k, 17, dq)
        packed = _packed(w, dq, dev)
        fns = (qg.qgemm_w4a8_dq, qg.qgemm_w4a8_g32_dq) if dq else (qg.qgemm_w4a8, qg.qgemm_w4a8_g32)
        for fn in fns:
            for split in (1, 2):
                y13 = fn(x13.to(dev), packed, n, split_k=split, out_dtype=torch.float32)
                y16 = fn(x16.to(dev), packed, n, split_k=split, out_dtype=torch.float32)
                assert torch.equal(y13, y16[:13]), (fn.__name__, split)


def test_graph_replay_bit_identical_m16(dev):
    n, k = 768, 512
    w, _ = _weight(n, k, 5, False)
    packed = _packed(w, False, dev)
    x = si.activation(16, k, 6).to(dev)
    for fn in (qg.qgemm_w4a8, qg.qgemm_w4a8_g32):
        for split in (1, 2):
            eager = fn(x, packed, n, split_k=split)
            ws = torch.empty(max(qg.workspace_bytes(16, n, k, split), 1), dtype=torch.uint8, device=dev)
            out = torch.empty_like(eager)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(x, packed, n, split_k=split, out=out, workspace=ws)
            for _ in range(3):
                out.zero_()
                torch.cuda.synchronize()
                g.replay()
                torch.cuda.synchronize()
                assert torch.equal(out, eager), (fn.__name__, split)


def test_m_above_4_uses_every_split(dev):
    """Both paths at M > 4 (quantized rows on the matrix-core kernels; per-row
    scale after the split sum, per-group scales inside it) at every legal
    split, both forms of the kernel (5 and 16 rows: registers; 24 and 64:
    LDS-staged)."""
    n, k = 520, 2048
    for dq in (False, True):
        w, parts = _weight(n, k, 21, dq)
        packed = _packed(w, dq, dev)
        pairs = ((qg.qgemm_w4a8_dq, oracle.qgemm_w4a8_dq), (qg.qgemm_w4a8_g32_dq, oracle.qgemm_w4a8_g32_dq)) if dq \
            else ((qg.qgemm_w4a8, oracle.qgemm_w4a8), (qg.qgemm_w4a8_g32, oracle.qgemm_w4a8_g32))
        for fn, ref_fn in pairs:
            for m in (5, 16, 24, 64):
                x = si.activation(m, k, 40 + m)
                ref = ref_fn(si.bf16_bits(x), *parts)
                for split in si.SPLITS:
                    label = f"{fn.__name__} M={m} split={split}"
                    print(label, flush=True)
                    assert_w16(fn(x.to(dev), packed, n, split_k=split, out_dtype=torch.float32), ref, label)
