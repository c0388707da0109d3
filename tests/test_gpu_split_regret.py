"""The library's default split-K against exhaustive search, scored by regret.

executorch test_int4_quantized_gemm.py, Int4AutotunePickTest: on the guard
shapes (_GUARD_SHAPES) at buckets 1 and 4 (_GUARD_BUCKETS), the config
picked for each (shape, bucket) must be within MAX_REGRET = 1.10 of the
fastest one measured afterwards, and within MAX_MEAN_REGRET = 1.03 on
average.  Here the pick is the library's static default split (no tuning at
run time), and every legal split is timed the way bench.py times a call:
rotating weight copies (>= 1 GiB, so the Infinity Cache cannot serve a
weight twice), calls captured in a HIP graph, events on its stream, median
of several replays.  The decode layer shapes are timed and printed too.
"""
from __future__ import annotations

import math
import statistics

import pytest
import torch

import synthetic_inputs as si

import gemm_decode_qgemm_amd as qg

pytestmark = pytest.mark.gpu

GUARD_SHAPES = ((8192, 2048), (6144, 2048), (2048, 8192), (32000, 2048))
GUARD_BUCKETS = (1, 4)
MAX_REGRET = 1.10
MAX_MEAN_REGRET = 1.03


def _graph_us(fn, calls: int = 200, replays: int = 7) -> float:
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for i in range(calls):
                fn(i)
    torch.cuda.synchronize()
    times = []
    with torch.cuda.stream(s):
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        for _ in range(replays):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            g.replay()
            e1.record(s)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1) * 1e3 / calls)
    return statistics.median(times)


def _regrets(shapes, buckets, seed_of, quant=qg.quantize_int4_g32, gemm=qg.qgemm_w4a16, bits=4):
    dev = torch.device("cuda:0")
    rows = []
    for n, k in shapes:
        p0 = quant(si.int4_weight(n, k, seed_of(n, k)).to(dev))
        copies = max(2, math.ceil((1 << 30) / p0.numel()))
        packs = [p0] + [p0.clone() for _ in range(copies - 1)]
        for m in buckets:
            x = si.activation(m, k, 7 + m).to(dev)
            y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
            times = {}
            for split in [s for s in si.SPLITS if s <= k // 256]:
                ws = torch.empty(max(qg.workspace_bytes(m, n, k, split), 1), dtype=torch.uint8, device=dev)
                times[split] = _graph_us(
                    lambda i: gemm(x, packs[i % copies], n, split_k=split, out=y, workspace=ws))
            pick = qg.default_split_k(m, n, k, bits)
            best = min(times, key=times.get)
            rows.append(dict(n=n, k=k, m=m, pick=pick, best=best, times=times,
                             regret=times[pick] / times[best]))
            print(f"{n}x{k} M={m}: pick {pick} ({times[pick]:.2f} us), best {best} ({times[best]:.2f} us), "
                  f"regret {rows[-1]['regret']:.3f}; " +
                  " ".join(f"s{s}={t:.2f}" for s, t in times.items()), flush=True)
        del packs, p0
        torch.cuda.empty_cache()
    return rows


def test_default_split_regret_on_the_guard_shapes():
    rows = _regrets(GUARD_SHAPES, GUARD_BUCKETS, lambda n, k: 500 + GUARD_SHAPES.index((n, k)))
    worst = max(rows, key=lambda r: r["regret"])
    mean = statistics.mean(r["regret"] for r in rows)
    assert worst["regret"] <= MAX_REGRET, worst
    assert mean <= MAX_MEAN_REGRET, (mean, rows)


# Two more layer shapes of the 30B export the Triton tuning PR measures
# (1024 x 6656, 5376 x 4096).
EXTRA_SHAPES = ((1024, 6656), (5376, 4096))


def test_default_split_regret_on_the_layer_shapes():
    rows = _regrets(si.MODEL_SHAPES + EXTRA_SHAPES, GUARD_BUCKETS, lambda n, k: n ^ k)
    worst = max(rows, key=lambda r: r["regret"])
    assert worst["regret"] <= MAX_REGRET, worst


def test_default_split_regret_matrix_core_buckets():
    rows = _regrets(((39936, 6656), (8448, 6656), (6656, 19968)), (16, 32, 48, 64), lambda n, k: n ^ k)
    worst = max(rows, key=lambda r: r["regret"])
    assert worst["regret"] <= MAX_REGRET, worst


# The INT6 layers of the same pull request, tuned there at buckets 1, 4, 16 and 64.
INT6_SHAPES = ((4096, 5376), (5376, 21504), (6656, 19968), (1024, 6656))


def test_default_split_regret_int6_layers():
    rows = _regrets(INT6_SHAPES, (1, 4, 16, 64), lambda n, k: n ^ k,
                    quant=lambda w: qg.quantize_intn_g32(w, 6),
                    gemm=lambda x, p, n, **kw: qg.qgemm_wn_a16(x, p, n, 6, **kw), bits=6)
    worst = max(rows, key=lambda r: r["regret"])
    assert worst["regret"] <= MAX_REGRET, worst
