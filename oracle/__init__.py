"""Plain CPU oracle for the decode-time weight-only quantized linear layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``gemm_decode_qgemm_amd``) and neither imports the
other.

The arithmetic lives in ``qgemm_oracle.c`` (plain C, built with gcc by
``oracle/build.py``); this module only marshals numpy arrays through ctypes.
bf16 / fp16 arrays are passed as ``uint16`` bit patterns.

Sources: executorch ``test_int4_quantized_gemm.py`` (``_packed_with_dense``
for the quantizer recipe, ``_dequant_matmul`` and the module docstring for the
"dequant + F.linear" reference, ``Int4QuantizedGemmPrecisionTest`` for W4A8)
and gpt-fast issue #114 (``WeightOnlyInt8Linear.forward`` for W8A16).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# QGEMM_ORACLE_LIB lets the mutation test load a deliberately broken build of
# the oracle (tests/test_oracle_mutants.py); nothing else sets it.
LIB_PATH = os.environ.get("QGEMM_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build

        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    I = ctypes.c_int
    sig = {
        "orc_bf16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_fp16_to_double": (ctypes.c_double, [ctypes.c_uint16]),
        "orc_quantize_int4_g32": (I, [P, I64, I64, P, P, P]),
        "orc_quantize_group32": (I, [P, P, P, P]),
        "orc_int4_packed_bytes": (I64, [I64, I64]),
        "orc_pack_int4": (None, [P, P, P, I64, I64, P]),
        "orc_unpack_int4": (None, [P, I64, I64, P, P, P]),
        "orc_qgemm_w4a16": (None, [P, I64, I64, P, P, P, I64, P, I]),
        "orc_quantize_int8_rowwise": (I, [P, I64, I64, P, P]),
        "orc_qgemm_w8a16": (None, [P, I64, I64, P, P, I64, P, I]),
        "orc_actquant_int8": (None, [P, I64, I64, P, P]),
        "orc_qgemm_w4a8": (None, [P, I64, I64, P, P, P, I64, P, I]),
        "orc_actquant_int8_g32": (None, [P, I64, I64, P, P]),
        "orc_qgemm_w4a8_g32": (None, [P, I64, I64, P, P, P, I64, P, I]),
        "orc_quantize_int4_g32_dq": (I, [P, I64, I64, P, P, P, P]),
        "orc_int4_dq_packed_bytes": (I64, [I64, I64]),
        "orc_pack_int4_dq": (None, [P, P, P, P, I64, I64, P]),
        "orc_unpack_int4_dq": (None, [P, I64, I64, P, P, P, P]),
        "orc_qgemm_w4a16_dq": (None, [P, I64, I64, P, P, P, P, I64, P, I]),
        "orc_quantize_intn_g32": (I, [P, I64, I64, I, P, P, P]),
        "orc_quantize_group32_bits": (I, [P, I, P, P, P]),
        "orc_intn_packed_bytes": (I64, [I64, I64, I]),
        "orc_pack_intn": (None, [P, P, P, I64, I64, I, P]),
        "orc_unpack_intn": (None, [P, I64, I64, I, P, P, P]),
        "orc_qgemm_w4a8_dq": (None, [P, I64, I64, P, P, P, P, I64, P, I]),
        "orc_qgemm_w4a8_g32_dq": (None, [P, I64, I64, P, P, P, P, I64, P, I]),
        "orc_hardware_threads": (I, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, f"expected uint16 bit patterns, got {a.dtype}"
    return a


def hardware_threads() -> int:
    """Threads for the oracle's row-parallel driver: the host's online CPUs,
    capped by OMP_NUM_THREADS when set (a shared GPU host grants each GPU job
    a share of its cores)."""
    n = int(_load().orc_hardware_threads())
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def bf16_to_float64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (bf16 is the top half of binary32)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp16_to_float64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return b.view(np.float16).astype(np.float64)


# ---------------------------------------------------------------- INT4 g32
def quantize_group32(w32_bits):
    """One group: returns (scale_bits, zp, codes[32], flags)."""
    w = _u16(w32_bits).reshape(32)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint8)
    q = np.zeros(32, np.uint8)
    f = _load().orc_quantize_group32(_ptr(w), _ptr(s), _ptr(z), _ptr(q))
    return int(s[0]), int(z[0]), q, int(f)


def quantize_int4_g32(w_bits):
    """W bf16 bits [n, k] -> (codes u8 [n,k], scales u16 [n,k/32], zeros u8 [n,k/32], flags)."""
    w = _u16(w_bits)
    n, k = w.shape
    assert k % 32 == 0
    codes = np.empty((n, k), np.uint8)
    scales = np.empty((n, k // 32), np.uint16)
    zeros = np.empty((n, k // 32), np.uint8)
    f = _load().orc_quantize_int4_g32(_ptr(w), n, k, _ptr(codes), _ptr(scales), _ptr(zeros))
    return codes, scales, zeros, int(f)


def int4_packed_bytes(n: int, k: int) -> int:
    return int(_load().orc_int4_packed_bytes(n, k))


def pack_int4(codes, scales, zeros) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = _u16(scales)
    zeros = np.ascontiguousarray(zeros, np.uint8)
    n, k = codes.shape
    assert k % 256 == 0, "the packed layout needs K % 256 == 0"
    out = np.empty(int4_packed_bytes(n, k), np.uint8)
    _load().orc_pack_int4(_ptr(codes), _ptr(scales), _ptr(zeros), n, k, _ptr(out))
    return out


def unpack_int4(packed, n: int, k: int):
    packed = np.ascontiguousarray(packed, np.uint8)
    assert packed.size >= int4_packed_bytes(n, k)
    codes = np.empty((n, k), np.uint8)
    scales = np.empty((n, k // 32), np.uint16)
    zeros = np.empty((n, k // 32), np.uint8)
    _load().orc_unpack_int4(_ptr(packed), n, k, _ptr(codes), _ptr(scales), _ptr(zeros))
    return codes, scales, zeros


def dequant_int4(codes, scales, zeros) -> np.ndarray:
    """(q - zp) * s as float64 [n, k]; exact (4-bit integer times fp16)."""
    s = fp16_to_float64(scales)
    q = codes.astype(np.float64)
    z = zeros.astype(np.float64)
    return (q.reshape(q.shape[0], -1, 32) - z[:, :, None]).reshape(q.shape) * np.repeat(s, 32, axis=1)


def qgemm_w4a16(x_bits, codes, scales, zeros, threads: int = 1) -> np.ndarray:
    x = _u16(x_bits)
    m, k = x.shape
    n = codes.shape[0]
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = _u16(scales)
    zeros = np.ascontiguousarray(zeros, np.uint8)
    y = np.empty((m, n), np.float64)
    _load().orc_qgemm_w4a16(_ptr(x), m, k, _ptr(codes), _ptr(scales), _ptr(zeros), n, _ptr(y), threads)
    return y


# ------------------------------------------------------- INT5 / INT6 g32
def quantize_group32_bits(w32_bits, bits: int):
    """One group at 5 or 6 bits: returns (scale_bits, zp, codes[32], flags)."""
    w = _u16(w32_bits).reshape(32)
    s = np.zeros(1, np.uint16)
    z = np.zeros(1, np.uint8)
    q = np.zeros(32, np.uint8)
    f = _load().orc_quantize_group32_bits(_ptr(w), bits, _ptr(s), _ptr(z), _ptr(q))
    return int(s[0]), int(z[0]), q, int(f)


def quantize_intn_g32(w_bits, bits: int):
    """W bf16 bits [n, k] -> (codes u8 [n,k] in 0..2^bits-1, scales u16 [n,k/32], zeros u8, flags)."""
    w = _u16(w_bits)
    n, k = w.shape
    assert k % 32 == 0 and bits in (5, 6)
    codes = np.empty((n, k), np.uint8)
    scales = np.empty((n, k // 32), np.uint16)
    zeros = np.empty((n, k // 32), np.uint8)
    f = _load().orc_quantize_intn_g32(_ptr(w), n, k, bits, _ptr(codes), _ptr(scales), _ptr(zeros))
    return codes, scales, zeros, int(f)


def intn_packed_bytes(n: int, k: int, bits: int) -> int:
    return int(_load().orc_intn_packed_bytes(n, k, bits))


def pack_intn(codes, scales, zeros, bits: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = _u16(scales)
    zeros = np.ascontiguousarray(zeros, np.uint8)
    n, k = codes.shape
    assert k % 256 == 0 and bits in (5, 6)
    out = np.empty(intn_packed_bytes(n, k, bits), np.uint8)
    _load().orc_pack_intn(_ptr(codes), _ptr(scales), _ptr(zeros), n, k, bits, _ptr(out))
    return out


def unpack_intn(packed, n: int, k: int, bits: int):
    packed = np.ascontiguousarray(packed, np.uint8)
    assert packed.size >= intn_packed_bytes(n, k, bits)
    codes = np.empty((n, k), np.uint8)
    scales = np.empty((n, k // 32), np.uint16)
    zeros = np.empty((n, k // 32), np.uint8)
    _load().orc_unpack_intn(_ptr(packed), n, k, bits, _ptr(codes), _ptr(scales), _ptr(zeros))
    return codes, scales, zeros


# ------------------------------------------- INT4 g32 with scale codes
def quantize_int4_g32_dq(w_bits):
    """W bf16 bits [n, k] -> (codes u8 [n,k], scale codes u8 [n,k/32],
    row steps fp16 bits u16 [n], zeros u8 [n,k/32], flags)."""
    w = _u16(w_bits)
    n, k = w.shape
    assert k % 32 == 0
    codes = np.empty((n, k), np.uint8)
    scode = np.empty((n, k // 32), np.uint8)
    sstep = np.empty(n, np.uint16)
    zeros = np.empty((n, k // 32), np.uint8)
    f = _load().orc_quantize_int4_g32_dq(_ptr(w), n, k, _ptr(codes), _ptr(scode), _ptr(sstep), _ptr(zeros))
    return codes, scode, sstep, zeros, int(f)


def int4_dq_packed_bytes(n: int, k: int) -> int:
    return int(_load().orc_int4_dq_packed_bytes(n, k))


def pack_int4_dq(codes, scode, sstep, zeros) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scode = np.ascontiguousarray(scode, np.uint8)
    sstep = _u16(sstep)
    zeros = np.ascontiguousarray(zeros, np.uint8)
    n, k = codes.shape
    assert k % 256 == 0, "the packed layout needs K % 256 == 0"
    out = np.empty(int4_dq_packed_bytes(n, k), np.uint8)
    _load().orc_pack_int4_dq(_ptr(codes), _ptr(scode), _ptr(sstep), _ptr(zeros), n, k, _ptr(out))
    return out


def unpack_int4_dq(packed, n: int, k: int):
    packed = np.ascontiguousarray(packed, np.uint8)
    assert packed.size >= int4_dq_packed_bytes(n, k)
    codes = np.empty((n, k), np.uint8)
    scode = np.empty((n, k // 32), np.uint8)
    sstep = np.empty(n, np.uint16)
    zeros = np.empty((n, k // 32), np.uint8)
    _load().orc_unpack_int4_dq(_ptr(packed), n, k, _ptr(codes), _ptr(scode), _ptr(sstep), _ptr(zeros))
    return codes, scode, sstep, zeros


def qgemm_w4a16_dq(x_bits, codes, scode, sstep, zeros, threads: int = 1) -> np.ndarray:
    x = _u16(x_bits)
    m, k = x.shape
    n = codes.shape[0]
    codes = np.ascontiguousarray(codes, np.uint8)
    scode = np.ascontiguousarray(scode, np.uint8)
    sstep = _u16(sstep)
    zeros = np.ascontiguousarray(zeros, np.uint8)
    y = np.empty((m, n), np.float64)
    _load().orc_qgemm_w4a16_dq(_ptr(x), m, k, _ptr(codes), _ptr(scode), _ptr(sstep), _ptr(zeros), n,
                               _ptr(y), threads)
    return y


# ---------------------------------------------------------------- INT8
def quantize_int8_rowwise(w_bits):
    w = _u16(w_bits)
    n, k = w.shape
    q = np.empty((n, k), np.int8)
    s = np.empty(n, np.uint16)
    f = _load().orc_quantize_int8_rowwise(_ptr(w), n, k, _ptr(q), _ptr(s))
    return q, s, int(f)


def qgemm_w8a16(x_bits, w_i8, scale_bits, threads: int = 1) -> np.ndarray:
    x = _u16(x_bits)
    m, k = x.shape
    w = np.ascontiguousarray(w_i8, np.int8)
    n = w.shape[0]
    s = _u16(scale_bits)
    y = np.empty((m, n), np.float64)
    _load().orc_qgemm_w8a16(_ptr(x), m, k, _ptr(w), _ptr(s), n, _ptr(y), threads)
    return y


# ---------------------------------------------------------------- W4A8
def actquant_int8(x_bits):
    x = _u16(x_bits)
    m, k = x.shape
    xq = np.empty((m, k), np.int8)
    sx = np.empty(m, np.float32)
    _load().orc_actquant_int8(_ptr(x), m, k, _ptr(xq), _ptr(sx))
    return xq, sx


def actquant_int8_g32(x_bits):
    """Per-group-32 activation quantization: (xq [m, k] int8, sx [m, k/32] float32)."""
    x = _u16(x_bits)
    m, k = x.shape
    xq = np.empty((m, k), np.int8)
    sx = np.empty((m, k // 32), np.float32)
    _load().orc_actquant_int8_g32(_ptr(x), m, k, _ptr(xq), _ptr(sx))
    return xq, sx


def qgemm_w4a8_g32(x_bits, codes, scales, zeros, threads: int = 1) -> np.ndarray:
    x = _u16(x_bits)
    m, k = x.shape
    n = codes.shape[0]
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = _u16(scales)
    zeros = np.ascontiguousarray(zeros, np.uint8)
    y = np.empty((m, n), np.float64)
    _load().orc_qgemm_w4a8_g32(_ptr(x), m, k, _ptr(codes), _ptr(scales), _ptr(zeros), n, _ptr(y), threads)
    return y


def qgemm_w4a8(x_bits, codes, scales, zeros, threads: int = 1) -> np.ndarray:
    x = _u16(x_bits)
    m, k = x.shape
    n = codes.shape[0]
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = _u16(scales)
    zeros = np.ascontiguousarray(zeros, np.uint8)
    y = np.empty((m, n), np.float64)
    _load().orc_qgemm_w4a8(_ptr(x), m, k, _ptr(codes), _ptr(scales), _ptr(zeros), n, _ptr(y), threads)
    return y


def _w4a8_dq(fn, x_bits, codes, scode, sstep, zeros, threads):
    x = _u16(x_bits)
    m, k = x.shape
    n = codes.shape[0]
    codes = np.ascontiguousarray(codes, np.uint8)
    scode = np.ascontiguousarray(scode, np.uint8)
    sstep = _u16(sstep)
    zeros = np.ascontiguousarray(zeros, np.uint8)
    y = np.empty((m, n), np.float64)
    fn(_ptr(x), m, k, _ptr(codes), _ptr(scode), _ptr(sstep), _ptr(zeros), n, _ptr(y), threads)
    return y


def qgemm_w4a8_dq(x_bits, codes, scode, sstep, zeros, threads: int = 1) -> np.ndarray:
    """W4A8 (per-row int8 activations) on the scale-code weight."""
    return _w4a8_dq(_load().orc_qgemm_w4a8_dq, x_bits, codes, scode, sstep, zeros, threads)


def qgemm_w4a8_g32_dq(x_bits, codes, scode, sstep, zeros, threads: int = 1) -> np.ndarray:
    """W4A8 (int8 activations, one scale per group of 32) on the scale-code weight."""
    return _w4a8_dq(_load().orc_qgemm_w4a8_g32_dq, x_bits, codes, scode, sstep, zeros, threads)
