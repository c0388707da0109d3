"""MI355X (gfx950) decode-time weight-only quantized linear layer.

y = x . dequant(W)^T (. per-row scale) for INT4 group-32 asymmetric weights
(W4A16, W4A8; fp16 group scales, or uint8 scale codes with a per-row
fp16 step as the pages store them), INT5 / INT6 group-32 weights and INT8 per-channel weights (W8A16), M = 1..64 activation rows.
The computation runs in the HIP library libqgemm.so (C ABI: include/qgemm.h);
this package only binds it.
"""
from .binding import (  # noqa: F401
    FLAG_NONFINITE,
    FLAG_OVERFLOW,
    QG_BF16,
    QG_F32,
    SCRATCH_BYTES,
    QGemmError,
    default_split_k,
    int4_dq_packed_bytes,
    int4_packed_bytes,
    intn_packed_bytes,
    qgemm_w4a8,
    qgemm_w4a8_dq,
    qgemm_w4a8_g32,
    qgemm_w4a8_g32_dq,
    qgemm_w4a16,
    qgemm_w4a16_dq,
    qgemm_w4a16_noalloc,
    qgemm_w8a16,
    qgemm_wn_a16,
    quantize_int4_g32,
    quantize_int4_g32_dq,
    quantize_int8_rowwise,
    quantize_intn_g32,
    status_string,
    stream_read,
    workspace_bytes,
)
