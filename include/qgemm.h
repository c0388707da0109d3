/*
 * qgemm.h -- C ABI of the MI355X (gfx950) decode-time weight-only quantized
 * linear layer:   y[m, n] = sum_k x[m, k] * dequant(W)[n, k]  (* scale[n]).
 *
 * Pages this library implements (cited by title and section):
 *  [P1] executorch "backends/cuda/tests/test_int4_quantized_gemm.py":
 *       `_packed_with_dense` (INT4, group 32, asymmetric, min-max),
 *       module docstring and `_dequant_matmul` (dequant + F.linear reference),
 *       `Int4QuantizedGemmLegalityTest` (validate before launching: dtype,
 *       shape, "K must be a multiple of 256", static M), `Int4QuantizedGemmRulesTest.
 *       test_split_k_needs_one_k_tile_per_split` (split <= K / 256),
 *       `SUPPORTED_BUCKETS` (decode M up to 64), `Int4QuantizedGemmTest.
 *       test_cuda_graph_replay_matches_eager` (bit-identical replays),
 *       `Int4QuantizedGemmPrecisionTest` (int8 activations, W4A8).
 *  [P3] gpt-fast issue #114 "Question about the generated code of
 *       WeightOnlyInt8Linear": `WeightOnlyInt8Linear.forward`
 *       (y = F.linear(x, W.to(bf16)) * scales; the int8->bf16 convert must be
 *       fused into the GEMV, never materialized).
 *
 * Conventions for every entry point:
 *  - All data pointers are DEVICE pointers (HIP global memory) on the current
 *    device, 16-byte aligned; arrays are row-major and contiguous.
 *    bf16 / fp16 values are their 16-bit IEEE patterns.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous on that stream; the library never allocates, never
 *    synchronizes, and keeps no mutable global state (calls are re-entrant),
 *    with one exception: qgemm_w4a16_noalloc, which uses the library's own
 *    static device scratch (see there).
 *  - The caller owns every buffer.  Outputs must not alias inputs.
 *  - On an argument error the call returns a negative qg_status and launches
 *    nothing (the checks run on the host before any launch).  A HIP launch
 *    failure returns QG_E_HIP.  Data-dependent conditions (non-finite
 *    weights, scale overflow) are reported through the optional device word
 *    `status_dev`: kernels OR flag bits into it; the caller zeroes it first.
 *  - Results are deterministic: identical inputs, split and device give
 *    bit-identical outputs, eager or replayed from a HIP graph (no floating
 *    point atomics anywhere).
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- packed INT4 group-32 weight layout, version 1 ----------------------
 * The weight is stored as tiles of 64 rows x 256 k (8 groups of 32 per row),
 * each exactly 9472 bytes = 74 lines of 128 bytes:
 *   [0, 8192)     codes: 16-byte chunk of (group j, row r) at (j*64 + r)*16;
 *                 LE dword d of a chunk holds k = 8d+e of the group at nibble
 *                 position p = (e & 1)*4 + (e >> 1), i.e. bits [4p, 4p+4).
 *                 (dword >> 4i) & 0x000F000F then yields the codes of
 *                 k = 8d+2i and 8d+2i+1 in its low and high 16-bit halves.
 *   [8192, 9216)  fp16 scales: row r's 8 scales at 8192 + 16r, group j at +2j
 *   [9216, 9472)  zero points: row r's LE 32-bit word at 9216 + 4r,
 *                 group j in bits [4j, 4j+4)
 * Tiles are row-block major: tile = (n / 64) * (K / 256) + k / 256.  Rows
 * n >= N of the last row block are zero.  A wavefront (64 lanes, lane = row)
 * reads each region as whole 128-byte lines with one 16-byte load per lane. */
#define QG_INT4_LAYOUT_VERSION 1
#define QG_TILE_ROWS 64
#define QG_TILE_K 256
#define QG_TILE_BYTES 9472

/* ---- packed INT4 layout, version 2: scale codes --------------------------
 * The stored form of [P1] `_packed_with_dense`: a group's scale is a uint8
 * code times a per-row fp16 step ([P1] legality rules "scale codes must be
 * uint8", "scale_step must be float16", step shape [N, 1]).  Each 64-row
 * block is a 128-byte head (row r's fp16 step at 2r) followed by K/256 tiles
 * of 8960 bytes = 70 lines:
 *   [0, 8192)     codes, exactly as version 1
 *   [8192, 8704)  scale codes: row r's 8 bytes at 8192 + 8r, group j at +j
 *   [8704, 8960)  zero points: row r's LE 32-bit word at 8704 + 4r, group j
 *                 in bits [4j, 4j+4)
 * Row blocks follow each other; rows n >= N of the last block are zero.
 * 0.546875 bytes per weight + 2 per row (version 1: 0.578125). */
#define QG_DQ_HEAD_BYTES 128
#define QG_DQ_TILE_BYTES 8960
#define QG_GROUP 32
#define QG_MAX_M 64

enum qg_dtype { QG_BF16 = 0, QG_F32 = 1 };

enum qg_status {
    QG_OK = 0,
    QG_E_NULL = -1,        /* a required pointer is NULL */
    QG_E_SHAPE = -2,       /* m, n or k < 1 */
    QG_E_K_MULTIPLE = -3,  /* K % 256 != 0 ([P1] "K must be a multiple of 256") */
    QG_E_M_RANGE = -4,     /* M > 64 ([P1] "static M must be within" the buckets) */
    QG_E_SPLIT = -5,       /* split_k not in {0,1,2,4,8} or split_k > K/256 */
    QG_E_BUFFER = -6,      /* packed_bytes or ws_bytes too small */
    QG_E_ALIGN = -7,       /* a data pointer is not 16-byte aligned */
    QG_E_DTYPE = -8,       /* y_dtype is not QG_BF16 / QG_F32 */
    QG_E_HIP = -9,         /* a HIP launch failed */
    QG_E_BITS = -10,       /* a code width other than 5 or 6 (INT5 / INT6 entry points) */
    QG_E_SCRATCH = -11     /* qgemm_w4a16_noalloc: the split's partial sums exceed QG_SCRATCH_BYTES */
};

/* status_dev flag bits */
#define QG_FLAG_NONFINITE 1u   /* a weight group/row held Inf or NaN */
#define QG_FLAG_OVERFLOW 2u    /* an INT4 group's range exceeded 15 * 65504 */

/* Human-readable name of a qg_status value (static string). */
const char *qg_status_string(int32_t status);

/* Bytes of the packed INT4 buffer for an N x K weight:
 * ceil(N/64) * (K/256) * 9472 (= N*K/2 codes + N*K/32 * 2.5 bytes of fp16
 * scale and 4-bit zero when N % 64 == 0).  Returns a negative qg_status for
 * N < 1, K < 1 or K % 256 != 0. */
int64_t qg_int4_packed_bytes(int64_t n, int64_t k);

/* The split-K factor the library uses when a qgemm call passes split_k = 0
 * (a static table keyed by the shape), or a negative qg_status. */
int32_t qg_default_split_k(int64_t m, int64_t n, int64_t k);

/* The split-K factor qgemm_wn_a16 (INT5 / INT6) uses for split_k = 0: the
 * table above for m <= 4; for m > 4 the smallest split with
 * ceil(n/64) * split >= 400 (at most 8, at most k/256), one step smaller when
 * that leaves under 4 tiles of 256 k per split while ceil(n/64) * split/2
 * still reaches 256.  Negative qg_status on bad arguments. */
int32_t qg_default_split_k_intn(int64_t m, int64_t n, int64_t k);

/* The split-K factor qgemm_w4a8_g32 and qgemm_w4a8_g32_dq use for
 * split_k = 0: qg_default_split_k up to 32 rows; above 32 rows the smallest
 * split with ceil(n/64) * split >= 1200, at most 8 and with at least 3 tiles
 * of 256 k per split (these kernels also multiply in each group's activation
 * scale, and more splits pay).  Negative qg_status on bad arguments. */
int32_t qg_default_split_k_g32(int64_t m, int64_t n, int64_t k);

/* Workspace bytes a qgemm call needs for (m, n, k, split_k): split * m * n * 4
 * (fp32 partial sums) when the split is above 1, else 0.  For split_k = 0
 * the largest need of the defaults is assumed (qg_default_split_k,
 * qg_default_split_k_intn and qg_default_split_k_g32 at m rows), so one
 * workspace serves every entry point's default.  For m > 4 it also holds what the W4A8 entry
 * points need there: m * k * 2 bytes of quantized activations, max(256,
 * 8 * k) bytes of activation scales (per row, or per group of 32 as
 * k/32 x 64 floats) and split * m * n * 4 bytes of partial sums (at split 1
 * too).  Negative qg_status on bad arguments. */
int64_t qg_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t split_k);

/* ---- quantize_int4_g32 ---------------------------------------------------
 * [P1] `_packed_with_dense`: QuantConfig(bits=4, group_size=32,
 * symmetric=False, method="min_max").  For each row n and each group g of 32
 * consecutive k:
 *   lo = min(0, min v), hi = max(0, max v), r = hi - lo  (binary64)
 *   s  = the smallest positive fp16 with 15*s >= r  (1.0 when r == 0)
 *   zp = clamp(rint(-lo / s), 0, 15)                  (binary32, half-even)
 *   q  = clamp(rint(v / s) + zp, 0, 15)
 * and writes (q, s, zp) in the layout above.  Every dequantized value
 * (q - zp) * s lies within s/2 of its input.
 *   w_bf16        in : bf16 [n, k]
 *   packed        out: qg_int4_packed_bytes(n, k) bytes (padding rows zeroed)
 *   packed_bytes  in : size of `packed`
 *   status_dev    in/out, may be NULL: ORed with QG_FLAG_NONFINITE (that
 *                 group: codes 0, scale NaN, zp 0) and QG_FLAG_OVERFLOW
 *                 (that group's scale saturates at 65504).
 * Errors: QG_E_NULL, QG_E_SHAPE, QG_E_K_MULTIPLE, QG_E_BUFFER, QG_E_ALIGN. */
int32_t quantize_int4_g32(const void *w_bf16, int64_t n, int64_t k, void *packed,
                          int64_t packed_bytes, uint32_t *status_dev, void *stream);

/* ---- quantize_int8_rowwise -----------------------------------------------
 * Per-output-channel symmetric int8, the weight format of [P3]
 * `WeightOnlyInt8Linear` (int8 [out, in] plus one scale per output row):
 *   a = max_k |w[n, k]|;  s = the smallest positive bf16 with 127*s >= a
 *   (1.0 when a == 0);  q = clamp(rint(w / s), -127, 127)  (binary32).
 *   w_bf16      in : bf16 [n, k]      q  out: int8 [n, k]
 *   scale_bf16  out: bf16 [n]
 *   status_dev  in/out, may be NULL: QG_FLAG_NONFINITE (that row: q 0, s NaN).
 * Errors: QG_E_NULL, QG_E_SHAPE, QG_E_K_MULTIPLE (K % 256), QG_E_ALIGN. */
int32_t quantize_int8_rowwise(const void *w_bf16, int64_t n, int64_t k, int8_t *q,
                              void *scale_bf16, uint32_t *status_dev, void *stream);

/* ---- qgemm_w4a16 ---------------------------------------------------------
 * [P1] module docstring / `_dequant_matmul`: y = x . dequant(W)^T with the
 * packed INT4 g32 weight above, dequantized in registers (no bf16 copy of W
 * is ever written).  Accumulation is fp32.
 *   x_bf16   in : bf16 [m, k], 1 <= m <= 64      packed  in: [n, k] weight
 *   y        out: [m, n], bf16 (round to nearest even) or fp32 per y_dtype
 *   split_k  0 (library table) or 1, 2, 4, 8 with split_k <= k/256
 *   ws       fp32 workspace of qg_workspace_bytes(m, n, k, split_k) bytes
 *            (NULL allowed when that is 0); contents on return unspecified.
 * M <= 4 runs the VALU GEMV; 5 <= M <= 64 the MFMA kernel (rows padded to
 * 16 and masked).  split_k > 1 adds a second, atomic-free pass that sums the
 * partials in ascending split order.
 * Errors: QG_E_NULL, QG_E_SHAPE, QG_E_K_MULTIPLE, QG_E_M_RANGE, QG_E_SPLIT,
 * QG_E_BUFFER, QG_E_ALIGN, QG_E_DTYPE, QG_E_HIP. */
int32_t qgemm_w4a16(const void *x_bf16, int64_t m, int64_t k, const void *packed,
                    int64_t packed_bytes, int64_t n, void *y, int32_t y_dtype,
                    int32_t split_k, void *ws, int64_t ws_bytes, void *stream);

/* ---- qgemm_w4a16_noalloc -------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): qgemm_w4a16
 * without a workspace argument.  The split-K partial sums (split * m * n * 4
 * bytes when the split is above 1) go to a static device array of
 * QG_SCRATCH_BYTES inside the library, one per device, which each device the
 * library runs on holds until the process ends.  The call allocates nothing
 * (no hipMalloc, no hipFree, no allocating library routine); its first call
 * on a device looks the array's address up once (hipGetSymbolAddress).
 * Every call on a device shares that device's array and leaves its
 * contents behind: calls that overlap on one device (concurrent streams,
 * threads) race and must be serialized by the caller.  Nothing in the array
 * needs to start at zero (each call writes every partial it reads).
 * Arguments, kernels, results (bit-identical to qgemm_w4a16 at the same
 * split) and errors as qgemm_w4a16, plus QG_E_SCRATCH when an explicit
 * split_k needs more than QG_SCRATCH_BYTES (nothing is launched); the
 * default split (split_k = 0) always fits. */
#define QG_SCRATCH_BYTES (16 * 1024 * 1024)
int32_t qgemm_w4a16_noalloc(const void *x_bf16, int64_t m, int64_t k, const void *packed,
                            int64_t packed_bytes, int64_t n, void *y, int32_t y_dtype,
                            int32_t split_k, void *stream);

/* Bytes of the version 2 (scale-code) buffer for an N x K weight:
 * ceil(N/64) * (128 + (K/256) * 8960), or a negative qg_status as above. */
int64_t qg_int4_dq_packed_bytes(int64_t n, int64_t k);

/* ---- quantize_int4_g32_dq ------------------------------------------------
 * [P1] `_packed_with_dense` in its stored form (uint8 scale codes with a
 * per-row fp16 `scale_step`).  Per row n, with lo, hi and r of each group as
 * in quantize_int4_g32:
 *   step = the smallest positive fp16 with 3825*step >= max_g r  (3825 =
 *          255*15; 1.0 when every r is 0)
 *   c    = the smallest integer in 1..255 with 15*c*step >= r, per group
 *   s    = c * step  (exact in binary32), then zp and q exactly as in
 *          quantize_int4_g32 with that s.
 * Zero points stay integers 0..15 (a zero_point_step of 1).  Every
 * dequantized value (q - zp) * s lies within s/2 of its input.
 *   w_bf16        in : bf16 [n, k]
 *   packed        out: qg_int4_dq_packed_bytes(n, k) bytes, layout version 2
 *   packed_bytes  in : size of `packed`
 *   status_dev    in/out, may be NULL: QG_FLAG_NONFINITE (that row: step
 *                 NaN, every code 0), QG_FLAG_OVERFLOW (max_g r above
 *                 3825 * 65504: step 65504, codes at most 255).
 * Two launches on `stream` (row steps, then tiles).
 * Errors: QG_E_NULL, QG_E_SHAPE, QG_E_K_MULTIPLE, QG_E_BUFFER, QG_E_ALIGN. */
int32_t quantize_int4_g32_dq(const void *w_bf16, int64_t n, int64_t k, void *packed,
                             int64_t packed_bytes, uint32_t *status_dev, void *stream);

/* ---- qgemm_w4a16_dq ------------------------------------------------------
 * qgemm_w4a16 on a version 2 (scale-code) weight:
 *   y[m, n] = sum_g c[n,g] * step[n] * sum_{k in g} x[m,k] * (q[n,k] - zp[n,g]),
 * dequantized in registers, fp32 accumulation, on the same kernels and
 * buckets as qgemm_w4a16 (1 <= m <= 64).  Arguments, workspace
 * (qg_workspace_bytes) and errors as qgemm_w4a16, with packed_bytes checked
 * against qg_int4_dq_packed_bytes. */
int32_t qgemm_w4a16_dq(const void *x_bf16, int64_t m, int64_t k, const void *packed,
                       int64_t packed_bytes, int64_t n, void *y, int32_t y_dtype,
                       int32_t split_k, void *ws, int64_t ws_bytes, void *stream);

/* ---- INT5 / INT6 group-32 (the pages' INT5/INT6 quantized-GEMM family) ---
 * Executorch pull request #23737 lists INT5 and INT6 layers next to INT4
 * (INT6: 4096x5376, 5376x21504, 6656x19968, 1024x6656); the quantizer
 * recipe is [P1] `_packed_with_dense` with 2^bits - 1 steps:
 *   s  = the smallest positive fp16 with L*s >= r, L = 31 (INT5) or 63 (INT6)
 *   zp = clamp(rint(-lo / s), 0, L);  q = clamp(rint(v / s) + zp, 0, L)
 * (lo, hi, r as in quantize_int4_g32).  Packed layout: tiles of 64 rows x
 * 256 k, row-block major, 8192 + 2048*hb + 1536 bytes (hb = bits - 4; 11776
 * for INT5, 13824 for INT6):
 *   [0, 8192)             the low 4 bits of every code, exactly as version 1
 *   [8192, +2048 hb)      high-bit planes: the (4 hb)-byte chunk of (group j,
 *                         row r) at 8192 + (j*64 + r)*4*hb.  For code dword d
 *                         and pair p (k = 8d+2p even, 8d+2p+1 odd) INT5 keeps
 *                         the even k's bit at 4d + p and the odd k's at
 *                         16 + 4d + p of the LE chunk; INT6 keeps in LE dword
 *                         d/2 the even k's bits b = 0, 1 at 8(d%2) + 2p + b,
 *                         the odd k's 16 higher
 *   [.., +1024)           fp16 scales: row r's 8 at +16r, group j at +2j
 *   [.., +512)            zero points, one byte each: row r at +8r, group j at +j
 * Rows n >= N of the last row block are zero. */
int64_t qg_intn_packed_bytes(int64_t n, int64_t k, int32_t bits);

/* bf16 [n, k] -> the INT5 / INT6 packed weight above.  Arguments, status
 * flags (per group, as quantize_int4_g32, with L*65504 for the overflow) and
 * errors as quantize_int4_g32, plus QG_E_BITS. */
int32_t quantize_intn_g32(const void *w_bf16, int64_t n, int64_t k, int32_t bits, void *packed,
                          int64_t packed_bytes, uint32_t *status_dev, void *stream);

/* y[m, n] = x . dequant(W)^T for an INT5 / INT6 packed weight, 1 <= m <= 64
 * (the INT4 kernels' buckets: M <= 4 GEMVs, 5..64 the matrix cores),
 * dequantized in registers, fp32 accumulation.
 * Arguments, workspace (qg_workspace_bytes) and errors as qgemm_w4a16, with
 * packed_bytes checked against qg_intn_packed_bytes, plus QG_E_BITS. */
int32_t qgemm_wn_a16(const void *x_bf16, int64_t m, int64_t k, int32_t bits, const void *packed,
                     int64_t packed_bytes, int64_t n, void *y, int32_t y_dtype, int32_t split_k,
                     void *ws, int64_t ws_bytes, void *stream);

/* ---- qgemm_w8a16 ---------------------------------------------------------
 * [P3] `WeightOnlyInt8Linear.forward`: y[m, n] = (sum_k x[m,k] * W[n,k]) *
 * scale[n], fp32 accumulation, the int8 -> float convert fused into the dot
 * product.  W int8 [n, k] row-major as given (no repacking, 16-byte aligned),
 * scale bf16 [n] (2-byte aligned).
 *   x_bf16 in: bf16 [m, k], 1 <= m <= 64;  y out: [m, n] bf16 or fp32.
 * M <= 4 runs the VALU GEMV (k <= 65536, QG_E_SHAPE above); 5 <= M <= 64 the
 * matrix cores (the [P3] question of a fused kernel above batch size 1):
 * bf16 products of x with the exact w + 128, accumulated over all of K, then
 * y = s * (sum - 128 * sum_k x).
 * Errors: QG_E_NULL, QG_E_SHAPE, QG_E_K_MULTIPLE, QG_E_M_RANGE, QG_E_ALIGN,
 * QG_E_DTYPE, QG_E_HIP. */
int32_t qgemm_w8a16(const void *x_bf16, int64_t m, int64_t k, const int8_t *w,
                    const void *scale_bf16, int64_t n, void *y, int32_t y_dtype,
                    void *stream);

/* ---- qgemm_w4a8 ----------------------------------------------------------
 * [P1] `Int4QuantizedGemmPrecisionTest`: the decode kernels run the packed
 * INT4 weight against int8 activations.  Each row of x is quantized inside
 * the call (per-row symmetric absmax: a = max|x|, inv = 127/a, sx = a/127,
 * xq = clamp(rint(x * inv), -127, 127) in binary32; a == 0, and a row so
 * small that 127/a overflows binary32 (a <= 127 * 2^-128), give a zero row;
 * a row holding a NaN or an infinity gives a NaN row),
 * then  y[m,n] = sx[m] * sum_g s[n,g] * sum_{k in g} xq[m,k] * (q[n,k] - zp[n,g])
 * with exact integer group dots.  Arguments and errors as qgemm_w4a16
 * (1 <= m <= 64).  For m > 4 the call quantizes x once into the workspace
 * (xq held exactly as bf16 integers), runs the bf16 matrix-core kernel of
 * qgemm_w4a16 on it (exact products, the same integer group dots), and
 * applies sx after the split-K sum; the workspace is required there at any
 * split (qg_workspace_bytes).  The per-row scale is
 * the pages' precision class on gaussian activations; rows with a few large
 * outlier channels lose precision (qgemm_w4a8_g32 below keeps it). */
int32_t qgemm_w4a8(const void *x_bf16, int64_t m, int64_t k, const void *packed,
                   int64_t packed_bytes, int64_t n, void *y, int32_t y_dtype,
                   int32_t split_k, void *ws, int64_t ws_bytes, void *stream);

/* ---- qgemm_w4a8_g32 ------------------------------------------------------
 * [P1] `Int4QuantizedGemmPrecisionTest` with its outlier activations
 * (channels 0, K/3, 2K/3, K-1 scaled by 50, 35, 25, 20): W4A8 with one
 * activation scale per group of 32 consecutive k of a row, so an outlier
 * only coarsens its own group.  Per row m and group g:
 *   a = max |x[m, 32g .. 32g+31]|, inv = 127/a, sx[m,g] = a/127 (binary32),
 *   xq = clamp(rint(x * inv), -127, 127); a == 0 or 127/a overflowing gives a
 *   zero group, a NaN or an infinity in the group a NaN row;
 *   y[m,n] = sum_g sx[m,g] * s[n,g] * sum_{k in g} xq[m,k] * (q[n,k] - zp[n,g]).
 * Arguments, buffers, workspace and errors as qgemm_w4a8.  For m = 5..64 the
 * call quantizes x once into the workspace (xq as exact bf16 integers, the
 * group scales group-major) and runs the matrix-core kernel of qgemm_w4a16
 * on xq, multiplying each group's exact integer dot by s[n,g] * sx[m,g]: one
 * pass over the weight; the workspace is required there at any split
 * (qg_workspace_bytes). */
int32_t qgemm_w4a8_g32(const void *x_bf16, int64_t m, int64_t k, const void *packed,
                       int64_t packed_bytes, int64_t n, void *y, int32_t y_dtype,
                       int32_t split_k, void *ws, int64_t ws_bytes, void *stream);

/* ---- qgemm_w4a8_dq / qgemm_w4a8_g32_dq -----------------------------------
 * qgemm_w4a8 and qgemm_w4a8_g32 on a version 2 (scale-code) weight: the
 * same activation quantization, a group's weight scale c[n,g] * step[n]:
 *   per row:      y = sx[m] * sum_g c*step * sum_{k in g} xq (q - zp)
 *   per group 32: y = sum_g sx[m,g] * c*step * sum_{k in g} xq (q - zp).
 * Arguments, workspace and errors as qgemm_w4a8 and qgemm_w4a8_g32
 * (1 <= m <= 64, the same two forms above 4 rows), with
 * packed_bytes checked against qg_int4_dq_packed_bytes. */
int32_t qgemm_w4a8_dq(const void *x_bf16, int64_t m, int64_t k, const void *packed,
                      int64_t packed_bytes, int64_t n, void *y, int32_t y_dtype,
                      int32_t split_k, void *ws, int64_t ws_bytes, void *stream);
int32_t qgemm_w4a8_g32_dq(const void *x_bf16, int64_t m, int64_t k, const void *packed,
                          int64_t packed_bytes, int64_t n, void *y, int32_t y_dtype,
                          int32_t split_k, void *ws, int64_t ws_bytes, void *stream);

/* ---- qg_stream_read (measurement helper, not part of the layer) ---------
 * Reads `bytes` bytes of device memory at `src` once, with one 16-byte
 * non-temporal load per lane per step over `blocks` workgroups of 256 lanes
 * (2 x 16 bytes per lane per step, grid-strided), and writes one XOR word per
 * wave to `sink` (blocks * 4 uint32).  The plain streaming-read rate of a
 * buffer, against which the GEMVs' effective bandwidth is compared.
 * bytes: a multiple of 16; src 16-byte aligned; 1 <= blocks <= 65536.
 * Errors: QG_E_NULL, QG_E_SHAPE, QG_E_ALIGN, QG_E_HIP. */
int32_t qg_stream_read(const void *src, int64_t bytes, uint32_t *sink, int32_t blocks, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QGEMM_H */
