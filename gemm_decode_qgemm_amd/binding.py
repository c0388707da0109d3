"""ctypes binding of libqgemm.so (the C ABI in include/qgemm.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in the library's
kernels.  Importing this module fails loudly if the library is not built.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# QGEMM_LIB names another build of the same library (for comparing builds).
LIB_PATH = os.environ.get("QGEMM_LIB") or os.path.join(_PKG, "libqgemm.so")

QG_BF16 = 0
QG_F32 = 1
TILE_ROWS = 64
TILE_K = 256
TILE_BYTES = 9472
GROUP = 32
MAX_M = 64
SCRATCH_BYTES = 16 * 1024 * 1024      # QG_SCRATCH_BYTES of include/qgemm.h
FLAG_NONFINITE = 1
FLAG_OVERFLOW = 2


class QGemmError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the HIP library first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
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
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.qg_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        raise QGemmError(status, what)


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a CUDA (HIP) device")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be rank-{ndim}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def int4_packed_bytes(n: int, k: int) -> int:
    v = int(lib.qg_int4_packed_bytes(n, k))
    _check(min(v, 0), "qg_int4_packed_bytes")
    return v


def int4_dq_packed_bytes(n: int, k: int) -> int:
    v = int(lib.qg_int4_dq_packed_bytes(n, k))
    _check(min(v, 0), "qg_int4_dq_packed_bytes")
    return v


def intn_packed_bytes(n: int, k: int, bits: int) -> int:
    v = int(lib.qg_intn_packed_bytes(n, k, bits))
    _check(min(v, 0), "qg_intn_packed_bytes")
    return v


def default_split_k(m: int, n: int, k: int, bits: int = 4, group_scales: bool = False) -> int:
    """The library's split for split_k = 0: INT4 layouts (bits = 4; with
    group_scales, W4A8 with one activation scale per group of 32), or INT5 / INT6."""
    if bits != 4:
        v = int(lib.qg_default_split_k_intn(m, n, k))
    elif group_scales:
        v = int(lib.qg_default_split_k_g32(m, n, k))
    else:
        v = int(lib.qg_default_split_k(m, n, k))
    _check(min(v, 0), "qg_default_split_k")
    return v


def workspace_bytes(m: int, n: int, k: int, split_k: int = 0) -> int:
    v = int(lib.qg_workspace_bytes(m, n, k, split_k))
    _check(min(v, 0), "qg_workspace_bytes")
    return v


def quantize_int4_g32(w: torch.Tensor, status: torch.Tensor | None = None,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [n, k] -> packed INT4 g32 weight (uint8, layout v1)."""
    _dev(w, "w", torch.bfloat16, 2)
    n, k = w.shape
    nbytes = int4_packed_bytes(n, k)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    st = lib.quantize_int4_g32(w.data_ptr(), n, k, out.data_ptr(), out.numel(), _ptr(status),
                               _stream(w.device))
    _check(st, "quantize_int4_g32")
    return out


def quantize_int4_g32_dq(w: torch.Tensor, status: torch.Tensor | None = None,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [n, k] -> packed INT4 g32 weight with scale codes (uint8, layout v2)."""
    _dev(w, "w", torch.bfloat16, 2)
    n, k = w.shape
    nbytes = int4_dq_packed_bytes(n, k)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    st = lib.quantize_int4_g32_dq(w.data_ptr(), n, k, out.data_ptr(), out.numel(), _ptr(status),
                                  _stream(w.device))
    _check(st, "quantize_int4_g32_dq")
    return out


def quantize_intn_g32(w: torch.Tensor, bits: int, status: torch.Tensor | None = None,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """bf16 [n, k] -> packed INT5 / INT6 g32 weight (uint8; bits = 5 or 6)."""
    _dev(w, "w", torch.bfloat16, 2)
    n, k = w.shape
    nbytes = intn_packed_bytes(n, k, bits)
    if out is None:
        out = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    st = lib.quantize_intn_g32(w.data_ptr(), n, k, bits, out.data_ptr(), out.numel(), _ptr(status),
                               _stream(w.device))
    _check(st, "quantize_intn_g32")
    return out


def quantize_int8_rowwise(w: torch.Tensor, status: torch.Tensor | None = None,
                          out: tuple | None = None):
    """bf16 [n, k] -> (int8 [n, k], bf16 scale [n]); `out` = (q, scale) to write into."""
    _dev(w, "w", torch.bfloat16, 2)
    n, k = w.shape
    if out is None:
        q = torch.empty((n, k), dtype=torch.int8, device=w.device)
        s = torch.empty(n, dtype=torch.bfloat16, device=w.device)
    else:
        q, s = out
        _dev(q, "q", torch.int8, 2)
        if tuple(q.shape) != (n, k) or s.dtype != torch.bfloat16 or s.numel() != n or not s.is_contiguous():
            raise ValueError("out must be (int8 [n, k], contiguous bf16 [n])")
    st = lib.quantize_int8_rowwise(w.data_ptr(), n, k, q.data_ptr(), s.data_ptr(), _ptr(status),
                                   _stream(w.device))
    _check(st, "quantize_int8_rowwise")
    return q, s


def _out(m: int, n: int, out_dtype: torch.dtype, device, out: torch.Tensor | None) -> tuple:
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")
    if out is None:
        out = torch.empty((m, n), dtype=out_dtype, device=device)
    else:
        _dev(out, "out", out_dtype, 2)
    return out, (QG_F32 if out_dtype == torch.float32 else QG_BF16)


def _workspace(m, n, k, split_k, device, workspace):
    need = workspace_bytes(m, n, k, split_k)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def qgemm_w4a16(x: torch.Tensor, packed: torch.Tensor, n: int, *, split_k: int = 0,
                out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[m, n] = x . dequant(W)^T for a packed INT4 g32 weight."""
    _dev(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    y, yd = _out(m, n, out_dtype, x.device, out)
    ws, ws_bytes = _workspace(m, n, k, split_k, x.device, workspace)
    st = lib.qgemm_w4a16(x.data_ptr(), m, k, packed.data_ptr(), packed.numel(), n, y.data_ptr(),
                         yd, split_k, _ptr(ws), ws_bytes, _stream(x.device))
    _check(st, "qgemm_w4a16")
    return y


def qgemm_w4a16_noalloc(x: torch.Tensor, packed: torch.Tensor, n: int, *, split_k: int = 0,
                        out_dtype: torch.dtype = torch.bfloat16,
                        out: torch.Tensor | None = None) -> torch.Tensor:
    """qgemm_w4a16 with the split-K partial sums in the library's static device
    scratch (no workspace; the C call allocates nothing).  Pass `out` to keep
    the wrapper from allocating the output.  Calls that overlap on one device
    share the scratch and must not run concurrently."""
    _dev(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    y, yd = _out(m, n, out_dtype, x.device, out)
    st = lib.qgemm_w4a16_noalloc(x.data_ptr(), m, k, packed.data_ptr(), packed.numel(), n, y.data_ptr(),
                                 yd, split_k, _stream(x.device))
    _check(st, "qgemm_w4a16_noalloc")
    return y


def stream_read(src: torch.Tensor, nbytes: int, sink: torch.Tensor, blocks: int = 1024) -> None:
    """qg_stream_read: read the first `nbytes` bytes of `src` once (the plain
    streaming-read rate the GEMVs are compared with); `sink` receives
    blocks * 4 XOR words (int32, at least that many elements)."""
    if not src.is_cuda or not sink.is_cuda or sink.dtype != torch.int32 or sink.numel() < 4 * blocks:
        raise ValueError("src and sink must be device tensors, sink int32 with >= 4 * blocks elements")
    if nbytes > src.numel() * src.element_size():
        raise ValueError("nbytes exceeds src")
    _check(lib.qg_stream_read(src.data_ptr(), nbytes, sink.data_ptr(), blocks, _stream(src.device)),
           "qg_stream_read")


def qgemm_w4a16_dq(x: torch.Tensor, packed: torch.Tensor, n: int, *, split_k: int = 0,
                   out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[m, n] = x . dequant(W)^T for a packed INT4 g32 weight with scale codes (m <= 64)."""
    _dev(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    y, yd = _out(m, n, out_dtype, x.device, out)
    ws, ws_bytes = _workspace(m, n, k, split_k, x.device, workspace)
    st = lib.qgemm_w4a16_dq(x.data_ptr(), m, k, packed.data_ptr(), packed.numel(), n, y.data_ptr(),
                            yd, split_k, _ptr(ws), ws_bytes, _stream(x.device))
    _check(st, "qgemm_w4a16_dq")
    return y


def qgemm_wn_a16(x: torch.Tensor, packed: torch.Tensor, n: int, bits: int, *, split_k: int = 0,
                 out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[m, n] = x . dequant(W)^T for a packed INT5 / INT6 g32 weight (m <= 64)."""
    _dev(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    y, yd = _out(m, n, out_dtype, x.device, out)
    ws, ws_bytes = _workspace(m, n, k, split_k, x.device, workspace)
    st = lib.qgemm_wn_a16(x.data_ptr(), m, k, bits, packed.data_ptr(), packed.numel(), n, y.data_ptr(),
                          yd, split_k, _ptr(ws), ws_bytes, _stream(x.device))
    _check(st, "qgemm_wn_a16")
    return y


def qgemm_w8a16(x: torch.Tensor, w: torch.Tensor, scale: torch.Tensor, *,
                out_dtype: torch.dtype = torch.bfloat16,
                out: torch.Tensor | None = None) -> torch.Tensor:
    """y[m, n] = (x . W^T) * scale[n] for an int8 [n, k] weight."""
    _dev(x, "x", torch.bfloat16, 2)
    _dev(w, "w", torch.int8, 2)
    _dev(scale, "scale", torch.bfloat16, 1)
    m, k = x.shape
    n = w.shape[0]
    if w.shape[1] != k or scale.shape[0] != n:
        raise ValueError("w must be [n, k] and scale [n]")
    y, yd = _out(m, n, out_dtype, x.device, out)
    st = lib.qgemm_w8a16(x.data_ptr(), m, k, w.data_ptr(), scale.data_ptr(), n, y.data_ptr(), yd,
                         _stream(x.device))
    _check(st, "qgemm_w8a16")
    return y


def qgemm_w4a8(x: torch.Tensor, packed: torch.Tensor, n: int, *, split_k: int = 0,
               out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A8: per-row int8 activations (quantized inside the call) x packed INT4 g32."""
    _dev(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    y, yd = _out(m, n, out_dtype, x.device, out)
    ws, ws_bytes = _workspace(m, n, k, split_k, x.device, workspace)
    st = lib.qgemm_w4a8(x.data_ptr(), m, k, packed.data_ptr(), packed.numel(), n, y.data_ptr(),
                        yd, split_k, _ptr(ws), ws_bytes, _stream(x.device))
    _check(st, "qgemm_w4a8")
    return y


def qgemm_w4a8_g32(x: torch.Tensor, packed: torch.Tensor, n: int, *, split_k: int = 0,
                   out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """W4A8 with one int8 activation scale per group of 32 (quantized inside the call)."""
    _dev(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    y, yd = _out(m, n, out_dtype, x.device, out)
    ws, ws_bytes = _workspace(m, n, k, split_k, x.device, workspace)
    st = lib.qgemm_w4a8_g32(x.data_ptr(), m, k, packed.data_ptr(), packed.numel(), n, y.data_ptr(),
                            yd, split_k, _ptr(ws), ws_bytes, _stream(x.device))
    _check(st, "qgemm_w4a8_g32")
    return y


def _w4a8_call(fn, name, x, packed, n, split_k, out_dtype, out, workspace):
    _dev(x, "x", torch.bfloat16, 2)
    m, k = x.shape
    y, yd = _out(m, n, out_dtype, x.device, out)
    ws, ws_bytes = _workspace(m, n, k, split_k, x.device, workspace)
    st = fn(x.data_ptr(), m, k, packed.data_ptr(), packed.numel(), n, y.data_ptr(), yd, split_k, _ptr(ws),
            ws_bytes, _stream(x.device))
    _check(st, name)
    return y


def qgemm_w4a8_dq(x: torch.Tensor, packed: torch.Tensor, n: int, *, split_k: int = 0,
                  out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """qgemm_w4a8 (per-row int8 activations) on a scale-code packed weight (m <= 64)."""
    return _w4a8_call(lib.qgemm_w4a8_dq, "qgemm_w4a8_dq", x, packed, n, split_k, out_dtype, out, workspace)


def qgemm_w4a8_g32_dq(x: torch.Tensor, packed: torch.Tensor, n: int, *, split_k: int = 0,
                      out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """qgemm_w4a8_g32 (one activation scale per group of 32) on a scale-code packed weight (m <= 64)."""
    return _w4a8_call(lib.qgemm_w4a8_g32_dq, "qgemm_w4a8_g32_dq", x, packed, n, split_k, out_dtype, out,
                      workspace)
