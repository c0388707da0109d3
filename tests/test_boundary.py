"""The C ABI on the host: the library loads, exports every function that
include/qgemm.h declares, and rejects every bad argument before launching
anything (executorch test_int4_quantized_gemm.py, Int4QuantizedGemmLegalityTest:
every rule is checked and the op "validates before launching";
Int4QuantizedGemmRulesTest.test_split_k_needs_one_k_tile_per_split).

No call here reaches a kernel: each one carries a definite argument error, so
these run on a machine without a GPU.
"""
from __future__ import annotations

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")
LIB = os.environ.get("QGEMM_LIB") or os.path.join(ROOT, "gemm_decode_qgemm_amd", "libqgemm.so")

OK, E_NULL, E_SHAPE, E_K, E_M, E_SPLIT, E_BUF, E_ALIGN, E_DTYPE, E_HIP = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
E_BITS = -10
E_SCRATCH = -11
SCRATCH_BYTES = 16 * 1024 * 1024
A = 0x10000          # a fake, 16-byte aligned "device" address (never dereferenced)
U = 0x10008          # 8-byte aligned only


@pytest.fixture(scope="module")
def lib():
    assert os.path.exists(LIB), "build the library first (__graft_entry__.build())"
    l = ctypes.CDLL(LIB)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sigs = {
        "qg_status_string": (ctypes.c_char_p, [I32]),
        "qg_int4_packed_bytes": (I64, [I64, I64]),
        "qg_default_split_k": (I32, [I64, I64, I64]),
        "qg_default_split_k_intn": (I32, [I64, I64, I64]),
        "qg_default_split_k_g32": (I32, [I64, I64, I64]),
        "qg_workspace_bytes": (I64, [I64, I64, I64, I32]),
        "qg_int4_dq_packed_bytes": (I64, [I64, I64]),
        "qg_intn_packed_bytes": (I64, [I64, I64, I32]),
        "quantize_intn_g32": (I32, [P, I64, I64, I32, P, I64, P, P]),
        "qgemm_wn_a16": (I32, [P, I64, I64, I32, P, I64, I64, P, I32, I32, P, I64, P]),
        "quantize_int4_g32": (I32, [P, I64, I64, P, I64, P, P]),
        "quantize_int4_g32_dq": (I32, [P, I64, I64, P, I64, P, P]),
        "qgemm_w4a16_dq": (I32, [P, I64, I64, P, I64, I64, P, I32, I32, P, I64, P]),
        "quantize_int8_rowwise": (I32, [P, I64, I64, P, P, P, P]),
        "qgemm_w4a16": (I32, [P, I64, I64, P, I64, I64, P, I32, I32, P, I64, P]),
        "qgemm_w4a16_noalloc": (I32, [P, I64, I64, P, I64, I64, P, I32, I32, P]),
        "qg_stream_read": (I32, [P, I64, P, I32, P]),
        "qgemm_w8a16": (I32, [P, I64, I64, P, P, I64, P, I32, P]),
        "qgemm_w4a8": (I32, [P, I64, I64, P, I64, I64, P, I32, I32, P, I64, P]),
        "qgemm_w4a8_g32": (I32, [P, I64, I64, P, I64, I64, P, I32, I32, P, I64, P]),
        "qgemm_w4a8_dq": (I32, [P, I64, I64, P, I64, I64, P, I32, I32, P, I64, P]),
        "qgemm_w4a8_g32_dq": (I32, [P, I64, I64, P, I64, I64, P, I32, I32, P, I64, P]),
    }
    for name, (res, args) in sigs.items():
        f = getattr(l, name)
        f.restype, f.argtypes = res, args
    return l


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"defined"})


def test_every_declared_function_is_exported(lib):
    names = declared_functions()
    assert len(names) >= 9, names
    for name in names:
        assert hasattr(lib, name), f"{name} declared in qgemm.h but not exported"


def test_status_strings(lib):
    for code in (OK, E_NULL, E_SHAPE, E_K, E_M, E_SPLIT, E_BUF, E_ALIGN, E_DTYPE, E_HIP, E_BITS, E_SCRATCH):
        s = lib.qg_status_string(code).decode()
        assert s and s != "unknown qgemm status"
    assert "multiple of 256" in lib.qg_status_string(E_K).decode()
    assert lib.qg_status_string(-99).decode() == "unknown qgemm status"


def test_packed_bytes_formula(lib):
    assert lib.qg_int4_packed_bytes(39936, 6656) == 39936 * 6656 // 2 + 39936 * 6656 // 32 * 5 // 2
    assert lib.qg_int4_packed_bytes(257, 512) == 5 * 2 * 9472          # padded to 5 row blocks
    assert lib.qg_int4_packed_bytes(64, 300) == E_K
    assert lib.qg_int4_packed_bytes(0, 256) == E_SHAPE
    # version 2 (scale codes): a 128-byte head of row steps per 64-row block,
    # then tiles of 8960 bytes: N*K/2 codes + N*K/32 * 1.5 + 2N when N % 64 == 0
    assert lib.qg_int4_dq_packed_bytes(39936, 6656) == 39936 * 6656 // 2 + 39936 * 6656 // 32 * 3 // 2 + 2 * 39936
    assert lib.qg_int4_dq_packed_bytes(257, 512) == 5 * (128 + 2 * 8960)
    assert lib.qg_int4_dq_packed_bytes(64, 300) == E_K
    assert lib.qg_int4_dq_packed_bytes(64, 0) == E_SHAPE
    # INT5 / INT6: tiles of 8192 + 2048 * (bits - 4) + 1536 bytes
    assert lib.qg_intn_packed_bytes(6656, 19968, 6) == 104 * 78 * 13824
    assert lib.qg_intn_packed_bytes(257, 512, 5) == 5 * 2 * 11776
    assert lib.qg_intn_packed_bytes(64, 256, 4) == E_BITS
    assert lib.qg_intn_packed_bytes(64, 300, 6) == E_K


def test_split_rule_one_k_tile_per_split(lib):
    for k in (256, 768, 4096):
        for split in (1, 2, 4, 8):
            expect = OK if split <= k // 256 else E_SPLIT
            ws = lib.qg_workspace_bytes(1, 256, k, split)
            assert (ws >= 0) == (expect == OK), (k, split, ws)
    assert lib.qg_workspace_bytes(1, 256, 4096, 3) == E_SPLIT
    assert lib.qg_workspace_bytes(4, 100, 4096, 4) == 4 * 4 * 100 * 4
    assert lib.qg_workspace_bytes(4, 100, 4096, 1) == 0


def test_default_split_table(lib):
    # M <= 4: one split from N = 4096 up; below, a workgroup of 32 rows per CU, at most 4
    for n, k in ((39936, 6656), (6656, 4096), (6656, 19968), (4096, 256),
                 (8192, 2048), (6144, 2048), (32000, 2048)):
        for m in (1, 4):
            assert lib.qg_default_split_k(m, n, k) == 1, (m, n, k)
    # a 32-row grid just past one round: M = 1 runs 64-row workgroups, M >= 2
    # the matrix-instruction GEMV, whose one-split time beats two splits there
    assert [lib.qg_default_split_k(m, 8448, 6656) for m in (1, 2, 3, 4)] == [1, 1, 1, 1]
    assert lib.qg_default_split_k(1, 2048, 8192) == 4
    assert lib.qg_default_split_k(1, 256, 6656) == 4
    assert lib.qg_default_split_k(3, 512, 6656) == 4
    assert lib.qg_default_split_k(1, 3072, 6656) == 4
    assert lib.qg_default_split_k(1, 256, 256) == 1       # capped by K / 256
    assert lib.qg_default_split_k(1, 256, 512) == 2
    # M > 4: row blocks of 64 x split >= 120 for the register-form kernel (up to
    # 16 rows), >= 300 for the LDS-staged one (17..64 rows), at most 8
    assert lib.qg_default_split_k(16, 39936, 6656) == 1
    assert lib.qg_default_split_k(16, 8448, 6656) == 1
    assert lib.qg_default_split_k(16, 6656, 19968) == 2
    assert lib.qg_default_split_k(64, 6656, 19968) == 4
    assert lib.qg_default_split_k(64, 256, 6656) == 8
    assert lib.qg_default_split_k(64, 39936, 6656) == 1
    assert lib.qg_default_split_k(32, 8448, 6656) == 4
    assert lib.qg_default_split_k(32, 39936, 6656) == 1
    assert lib.qg_default_split_k(48, 6656, 19968) == 4
    assert lib.qg_default_split_k(48, 6656, 4096) == 4
    assert lib.qg_default_split_k(17, 5376, 4096) == 4
    assert lib.qg_default_split_k(65, 256, 256) == E_M
    # INT5 / INT6, M > 4: ceil(N/64) * split >= 400, one step back under 4 tiles per split
    # while a workgroup per CU remains (measured on the INT6 layers)
    for m in (16, 64):
        assert lib.qg_default_split_k_intn(m, 5376, 21504) == 8
        assert lib.qg_default_split_k_intn(m, 6656, 19968) == 4
        assert lib.qg_default_split_k_intn(m, 4096, 5376) == 4
        assert lib.qg_default_split_k_intn(m, 1024, 6656) == 8
    assert lib.qg_default_split_k_intn(1, 5376, 21504) == lib.qg_default_split_k(1, 5376, 21504) == 1
    # W4A8 per group of 32: the W4A16 rule up to 32 rows; above, row blocks x
    # split >= 1200, at most 8, at least 3 tiles of 256 k per split
    for m in (1, 4, 16, 32):
        for n, k in ((39936, 6656), (8448, 6656), (6656, 19968), (6656, 4096)):
            assert lib.qg_default_split_k_g32(m, n, k) == lib.qg_default_split_k(m, n, k), (m, n, k)
    assert lib.qg_default_split_k_g32(64, 39936, 6656) == 2
    assert lib.qg_default_split_k_g32(64, 8448, 6656) == 8
    assert lib.qg_default_split_k_g32(48, 8448, 6656) == 8
    assert lib.qg_default_split_k_g32(64, 6656, 19968) == 8
    assert lib.qg_default_split_k_g32(64, 6656, 4096) == 4      # 3 tiles per split at most 8 / 2
    assert lib.qg_default_split_k_g32(64, 256, 512) == 1        # 2 tiles: no split keeps 3
    assert lib.qg_default_split_k_g32(65, 256, 256) == E_M
    assert lib.qg_default_split_k_intn(64, 256, 512) == 2                  # capped by K / 256
    # one workspace serves every default: here per-group W4A8 at its split 8
    # (quantized x, group scales, partials) needs the most
    assert lib.qg_workspace_bytes(64, 5376, 21504, 0) == 64 * 21504 * 2 + 8 * 21504 + 8 * 64 * 5376 * 4


@pytest.mark.parametrize("args,expect", [
    ((None, 1, 256, A, 1 << 20, 64, A, 0, 0, None, 0, None), E_NULL),      # x
    ((A, 1, 256, None, 1 << 20, 64, A, 0, 0, None, 0, None), E_NULL),      # packed
    ((A, 1, 256, A, 1 << 20, 64, None, 0, 0, None, 0, None), E_NULL),      # y
    ((A, 0, 256, A, 1 << 20, 64, A, 0, 0, None, 0, None), E_SHAPE),        # m < 1
    ((A, 1, 256, A, 1 << 20, 0, A, 0, 0, None, 0, None), E_SHAPE),         # n < 1
    ((A, 1, 288, A, 1 << 20, 64, A, 0, 0, None, 0, None), E_K),            # K % 256
    ((A, 65, 256, A, 1 << 20, 64, A, 0, 0, None, 0, None), E_M),           # M > 64
    ((A, 1, 256, A, 1 << 20, 64, A, 2, 0, None, 0, None), E_DTYPE),        # y_dtype
    ((A, 1, 768, A, 1 << 20, 64, A, 0, 4, A, 1 << 20, None), E_SPLIT),     # 4 > 768/256
    ((A, 1, 4096, A, 1 << 20, 64, A, 0, 3, A, 1 << 20, None), E_SPLIT),    # not a candidate
    ((A, 1, 256, A, 100, 64, A, 0, 0, None, 0, None), E_BUF),              # packed too small
    ((A, 2, 4096, A, 1 << 20, 64, A, 0, 4, A, 16, None), E_BUF),           # workspace too small
    ((A, 2, 4096, A, 1 << 20, 64, A, 0, 4, None, 0, None), E_NULL),        # workspace missing
    ((U, 1, 256, A, 1 << 20, 64, A, 0, 0, None, 0, None), E_ALIGN),        # x misaligned
    ((A, 1, 256, U, 1 << 20, 64, A, 0, 0, None, 0, None), E_ALIGN),        # packed misaligned
])
def test_qgemm_w4a16_and_w4a8_validate_before_launching(lib, args, expect):
    assert lib.qgemm_w4a16(*args) == expect
    # the scale-code layout shares the rules (its buffer size is checked against its own formula)
    assert lib.qgemm_w4a16_dq(*args) == expect
    # W4A8 (both activation granularities) shares the rules
    assert lib.qgemm_w4a8(*args) == expect
    assert lib.qgemm_w4a8_g32(*args) == expect
    assert lib.qgemm_w4a8_dq(*args) == expect
    assert lib.qgemm_w4a8_g32_dq(*args) == expect


def test_w4a8_m_range(lib):
    # W4A8 takes every bucket up to 64 rows (M > 4 on the matrix cores)
    assert lib.qgemm_w4a8(A, 65, 256, A, 1 << 20, 64, A, 0, 0, None, 0, None) == E_M
    assert lib.qgemm_w4a8_g32(A, 65, 256, A, 1 << 20, 64, A, 0, 0, None, 0, None) == E_M
    assert lib.qgemm_w4a16_dq(A, 65, 256, A, 1 << 20, 64, A, 0, 0, None, 0, None) == E_M
    assert lib.qgemm_w4a8_dq(A, 65, 256, A, 1 << 20, 64, A, 0, 0, None, 0, None) == E_M
    assert lib.qgemm_w4a8_g32_dq(A, 65, 256, A, 1 << 20, 64, A, 0, 0, None, 0, None) == E_M
    # above 4 rows every W4A8 entry point needs the workspace at any split
    # (quantized x, its scales -- per row 256 bytes, per group of 32 k/32 x 64
    # floats -- and partials): refused before any launch when missing or short
    need = lib.qg_workspace_bytes(5, 64, 256, 1)
    assert need == 5 * 256 * 2 + max(256, 256 // 32 * 64 * 4) + 5 * 64 * 4
    assert lib.qg_workspace_bytes(64, 64, 6656, 2) == 64 * 6656 * 2 + 6656 // 32 * 64 * 4 + 2 * 64 * 64 * 4
    for f in (lib.qgemm_w4a8, lib.qgemm_w4a8_dq, lib.qgemm_w4a8_g32, lib.qgemm_w4a8_g32_dq):
        assert f(A, 5, 256, A, 1 << 20, 64, A, 0, 1, None, 0, None) == E_NULL
        assert f(A, 5, 256, A, 1 << 20, 64, A, 0, 1, A, need - 1, None) == E_BUF
    assert lib.qgemm_w4a8_dq(A, 1, 256, A, 9087, 64, A, 0, 0, None, 0, None) == E_BUF
    # 9088 bytes hold a 64 x 256 scale-code weight, 9087 do not
    assert lib.qgemm_w4a16_dq(A, 1, 256, A, 9087, 64, A, 0, 0, None, 0, None) == E_BUF


@pytest.mark.parametrize("args,expect", [
    ((None, 1, 256, A, A, 64, A, 0, None), E_NULL),
    ((A, 1, 256, None, A, 64, A, 0, None), E_NULL),
    ((A, 1, 256, A, None, 64, A, 0, None), E_NULL),
    ((A, 1, 300, A, A, 64, A, 0, None), E_K),
    ((A, 65, 256, A, A, 64, A, 0, None), E_M),
    ((A, 5, 65536 + 256, A, A, 64, A, 7, None), E_DTYPE),      # M > 4 takes any K; dtype still checked
    ((A, 1, 256, A, A, 64, A, 7, None), E_DTYPE),
    ((A, 1, 256, A, A, 0, A, 0, None), E_SHAPE),
    ((A, 1, 65536 + 256, A, A, 64, A, 0, None), E_SHAPE),       # K above the VGPR-resident limit
    ((A, 1, 256, U, A, 64, A, 0, None), E_ALIGN),
    ((A, 1, 256, A, A + 1, 64, A, 0, None), E_ALIGN),            # scale must be 2-byte aligned
])
def test_qgemm_w8a16_validates_before_launching(lib, args, expect):
    assert lib.qgemm_w8a16(*args) == expect


@pytest.mark.parametrize("args,expect", [
    ((None, 64, 256, A, 1 << 20, None, None), E_NULL),
    ((A, 64, 256, None, 1 << 20, None, None), E_NULL),
    ((A, 64, 300, A, 1 << 20, None, None), E_K),
    ((A, 0, 256, A, 1 << 20, None, None), E_SHAPE),
    ((A, 64, 256, A, 9471, None, None), E_BUF),
    ((A, 64, 256, A, 9472, U + 2, None), E_ALIGN),               # status word misaligned
    ((U, 64, 256, A, 9472, None, None), E_ALIGN),
])
def test_quantize_int4_validates_before_launching(lib, args, expect):
    assert lib.quantize_int4_g32(*args) == expect


def test_intn_entry_points_validate_before_launching(lib):
    q = lib.quantize_intn_g32
    assert q(None, 64, 256, 6, A, 1 << 20, None, None) == E_NULL
    assert q(A, 64, 256, 7, A, 1 << 20, None, None) == E_BITS
    assert q(A, 64, 300, 6, A, 1 << 20, None, None) == E_K
    assert q(A, 64, 256, 6, A, 13823, None, None) == E_BUF
    assert q(A, 64, 256, 5, A, 11776, U + 2, None) == E_ALIGN
    g = lib.qgemm_wn_a16
    assert g(None, 1, 256, 6, A, 1 << 20, 64, A, 0, 0, None, 0, None) == E_NULL
    assert g(A, 1, 256, 4, A, 1 << 20, 64, A, 0, 0, None, 0, None) == E_BITS
    assert g(A, 65, 256, 6, A, 1 << 20, 64, A, 0, 0, None, 0, None) == E_M
    assert g(A, 1, 288, 6, A, 1 << 20, 64, A, 0, 0, None, 0, None) == E_K
    assert g(A, 1, 256, 6, A, 1 << 20, 64, A, 2, 0, None, 0, None) == E_DTYPE
    assert g(A, 1, 768, 6, A, 1 << 20, 64, A, 0, 4, A, 1 << 20, None) == E_SPLIT
    assert g(A, 1, 256, 5, A, 11775, 64, A, 0, 0, None, 0, None) == E_BUF
    assert g(A, 1, 4096, 6, A, 1 << 20, 64, A, 0, 4, None, 0, None) == E_NULL   # workspace missing
    assert g(U, 1, 256, 6, A, 1 << 20, 64, A, 0, 0, None, 0, None) == E_ALIGN


def test_quantize_int4_dq_validates_before_launching(lib):
    assert lib.quantize_int4_g32_dq(None, 64, 256, A, 1 << 20, None, None) == E_NULL
    assert lib.quantize_int4_g32_dq(A, 64, 256, None, 1 << 20, None, None) == E_NULL
    assert lib.quantize_int4_g32_dq(A, 64, 300, A, 1 << 20, None, None) == E_K
    assert lib.quantize_int4_g32_dq(A, 0, 256, A, 1 << 20, None, None) == E_SHAPE
    assert lib.quantize_int4_g32_dq(A, 64, 256, A, 9087, None, None) == E_BUF
    assert lib.quantize_int4_g32_dq(A, 64, 256, A, 9088, U + 2, None) == E_ALIGN
    assert lib.quantize_int4_g32_dq(U, 64, 256, A, 9088, None, None) == E_ALIGN


@pytest.mark.parametrize("args,expect", [
    ((None, 4, 256, A, A, None, None), E_NULL),
    ((A, 4, 256, None, A, None, None), E_NULL),
    ((A, 4, 256, A, None, None, None), E_NULL),
    ((A, 4, 100, A, A, None, None), E_K),
    ((A, -1, 256, A, A, None, None), E_SHAPE),
    ((A, 4, 256, U, A, None, None), E_ALIGN),
])
def test_quantize_int8_validates_before_launching(lib, args, expect):
    assert lib.quantize_int8_rowwise(*args) == expect


def test_python_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The binding raises instead of falling back to anything when the .so is missing."""
    import importlib.util

    monkeypatch.delenv("QGEMM_LIB", raising=False)   # a run that points at another build

    src = os.path.join(ROOT, "gemm_decode_qgemm_amd", "binding.py")
    copy = tmp_path / "binding.py"
    copy.write_text(open(src).read())
    spec = importlib.util.spec_from_file_location("binding_copy", copy)
    mod = importlib.util.module_from_spec(spec)
    with pytest.raises(ImportError, match="missing"):
        spec.loader.exec_module(mod)


@pytest.mark.parametrize("m", [5, 8, 16, 33, 64])
@pytest.mark.parametrize("n,k", [(8448, 6656), (6656, 19968), (6656, 4096), (256, 6656), (768, 256)])
def test_default_workspace_covers_w4a8_above_4_rows(lib, m, n, k):
    """At M > 4 both W4A8 forms put quantized x (bf16), the activation scales
    (max(256, 8k) bytes) and the partial sums at their own default split in
    the workspace; the split_k = 0 size must hold either."""
    ws = lib.qg_workspace_bytes(m, n, k, 0)
    scales = max(256, 8 * k)
    assert ws >= m * k * 2 + scales + lib.qg_default_split_k(m, n, k) * m * n * 4
    assert ws >= m * k * 2 + scales + lib.qg_default_split_k_g32(m, n, k) * m * n * 4
    for split in (1, 2, 4, 8):
        if split <= k // 256:
            assert lib.qg_workspace_bytes(m, n, k, split) >= m * k * 2 + scales + split * m * n * 4


def test_noalloc_checks_before_anything(lib):
    """qgemm_w4a16_noalloc: qgemm_w4a16's argument rules, and an explicit split
    whose partial sums exceed the static scratch is refused (QG_E_SCRATCH)
    before any HIP call; the default split always fits the scratch."""
    f = lib.qgemm_w4a16_noalloc
    n, k = 39936, 6656
    pb = lib.qg_int4_packed_bytes(n, k)
    assert f(A, 64, k, A, pb, n, A, 0, 8, None) == E_SCRATCH          # 8 * 64 * 39936 * 4 > 16 MiB
    assert f(A, 1, k, A, pb, n, A, 0, 3, None) == E_SPLIT
    assert f(None, 1, k, A, pb, n, A, 0, 0, None) == E_NULL
    assert f(A, 65, k, A, pb, n, A, 0, 0, None) == E_M
    assert f(A, 1, 300, A, pb, n, A, 0, 0, None) == E_K
    assert f(A, 1, k, A, pb - 1, n, A, 0, 0, None) == E_BUF
    assert f(U, 1, k, A, pb, n, A, 0, 0, None) == E_ALIGN
    assert f(A, 1, k, A, pb, n, A, 7, 0, None) == E_DTYPE
    assert "QG_SCRATCH_BYTES" in lib.qg_status_string(E_SCRATCH).decode()
    # the default split's partials always fit
    for m in (1, 2, 4, 5, 16, 17, 33, 48, 64):
        for n2 in (1, 63, 256, 768, 2048, 2431, 4096, 6656, 8448, 16384, 39936):
            for k2 in (256, 2048, 6656, 19968, 131072):
                s = lib.qg_default_split_k(m, n2, k2)
                need = s * m * n2 * 4 if s > 1 else 0
                assert need <= SCRATCH_BYTES, (m, n2, k2, s)
