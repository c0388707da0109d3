"""Seeded synthetic inputs for the decode-time weight-only quantized linear layer.

This module is the only code that both the CPU oracle's callers and the HIP
path's callers share.  It draws random tensors and holds none of the layer's
arithmetic (no quantization, no packing, no dot products).

Recipe (shapes, seeds and distributions of executorch
``test_int4_quantized_gemm.py``: ``MODEL_SHAPES``, ``SMALL_SHAPES``,
``_packed_with_dense`` draws ``torch.randn(n, k, dtype=torch.bfloat16)`` after
``torch.manual_seed(seed)``; model-shape weights use seed ``n ^ k``;
``Int4QuantizedGemmPrecisionTest`` draws activations with seed
``9100 + 31 * shape_index + bucket``; gpt-fast issue #114 builds the int8
layer from ``randn(...).to(int8)`` weights and ``randn`` bf16 scales):

* INT4 weights: bf16 standard normal [N, K], ``torch.manual_seed(seed)``.
* activations: bf16 standard normal [M, K].
* INT8 layer: int8 uniform in [-127, 127], bf16 standard-normal scales, bf16
  standard-normal activations, drawn in that order from one seed.

Everything is drawn on the CPU with torch's generator, so the same seed gives
the same bits on every machine running the same torch build.
"""
from __future__ import annotations

import numpy as np
import torch

GROUP_SIZE = 32
# (N, K) of the INT4 decode layers (executorch test file, MODEL_SHAPES).
MODEL_SHAPES = ((8448, 6656), (6656, 4096), (39936, 6656), (6656, 19968), (256, 6656))
SMALL_SHAPES = ((768, 256), (256, 768), (1536, 512))
DECODE_M = (1, 2, 3, 4)          # W4A8_BUCKETS
LARGE_M = (16, 64)
SPLITS = (1, 2, 4, 8)
W8_SHAPE = (8192, 8192)          # gpt-fast issue #114, D = 8192
TINY_SHAPE = (768, 256)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """uint16 bit patterns of a bf16 CPU tensor (a view, no rounding)."""
    assert t.dtype == torch.bfloat16
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bits_to_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16)


def int4_weight(n: int, k: int, seed: int) -> torch.Tensor:
    torch.manual_seed(seed)
    return torch.randn(n, k, dtype=torch.bfloat16)


def activation(m: int, k: int, seed: int) -> torch.Tensor:
    torch.manual_seed(seed)
    return torch.randn(m, k, dtype=torch.bfloat16)


def model_weight_seed(n: int, k: int) -> int:
    return n ^ k


def model_activation_seed(shape_index: int, m: int) -> int:
    return 9100 + 31 * shape_index + m


def model_shape_index(n: int, k: int) -> int:
    return MODEL_SHAPES.index((n, k))


def tiny_inputs():
    """768x256 INT4 layer: W with seed 0, x [1, 256] with seed 1."""
    n, k = TINY_SHAPE
    return int4_weight(n, k, 0), activation(1, k, 1)


def decode_inputs(n: int, k: int, m: int):
    """A model-shape INT4 layer and an M-row activation (seeds as above)."""
    i = model_shape_index(n, k)
    return int4_weight(n, k, model_weight_seed(n, k)), activation(m, k, model_activation_seed(i, m))


def int8_layer(n: int = W8_SHAPE[0], k: int = W8_SHAPE[1], m: int = 1, seed: int = 0):
    """(W int8 [n,k] uniform in [-127,127], scales bf16 [n], x bf16 [m,k])."""
    torch.manual_seed(seed)
    w = torch.randint(-127, 128, (n, k), dtype=torch.int8)
    scales = torch.randn(n, dtype=torch.bfloat16)
    x = torch.randn(m, k, dtype=torch.bfloat16)
    return w, scales, x
