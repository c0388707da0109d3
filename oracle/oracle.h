/*
 * oracle.h -- plain, slow CPU oracle for the decode-time weight-only
 * quantized linear layer  y = x . dequant(W)^T (. per-row scale).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or constant with the HIP library; neither includes the other.
 *
 * Sources (the pages):
 *  [P1] executorch "backends/cuda/tests/test_int4_quantized_gemm.py"
 *       (the decode-sized INT4 GEMM test file): `_packed_with_dense`
 *       (QuantConfig bits=4, group_size=32, symmetric=False, method="min_max"),
 *       the module docstring and `_dequant_matmul` ("dequant + F.linear"
 *       reference), `_check_close` (tolerance class), and
 *       `Int4QuantizedGemmPrecisionTest` (W4A8 against the W4A16 reference).
 *  [P3] gpt-fast issue #114 "Question about the generated code of
 *       WeightOnlyInt8Linear": `WeightOnlyInt8Linear.forward`
 *       (F.linear(x, W.to(x.dtype)) * scales).
 *
 * Arithmetic: IEEE-754 binary32/binary64, round-to-nearest-even, no FMA
 * contraction (built with -ffp-contract=off), no fast-math, denormals kept.
 * Products of a bf16 activation and a dequantized weight are exact in
 * binary64, so the GEMM results below are the exact dot products up to one
 * binary64 rounding per addition (ascending k).
 *
 * All arrays are host memory owned by the caller, row-major and contiguous.
 * bf16 and fp16 values travel as their uint16 bit patterns.
 */
#ifndef QGEMM_ORACLE_H
#define QGEMM_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- number formats, decoded from the IEEE-754 bit layout ---- */
double orc_bf16_to_double(uint16_t bits);
double orc_fp16_to_double(uint16_t bits);

/* ---- INT4 group-32 asymmetric min-max quantizer ([P1] _packed_with_dense) ----
 * w: bf16 [n, k], k % 32 == 0.  Outputs the canonical (unpacked) form:
 *   codes  uint8  [n, k]      q in 0..15
 *   scales fp16   [n, k/32]   bit patterns
 *   zeros  uint8  [n, k/32]   zp in 0..15
 * Returns the OR of the per-group flags: 1 = a non-finite weight (that group
 * gets codes 0, scale NaN 0x7E00, zp 0), 2 = range above 15*65504 (scale
 * saturated to 65504). */
int orc_quantize_int4_g32(const uint16_t *w, int64_t n, int64_t k,
                          uint8_t *codes, uint16_t *scales, uint8_t *zeros);

/* One group of 32 values (exposed for the hand-worked pins). */
int orc_quantize_group32(const uint16_t *w32, uint16_t *scale, uint8_t *zp,
                         uint8_t *q32);

/* ---- packed tile layout (own format, version 1) ----
 * Tile = 64 rows x 256 k = 8 groups per row, 9472 bytes:
 *   [0, 8192)     codes: the 16-byte chunk of (group j, row r) at (j*64 + r)*16
 *   [8192, 9216)  fp16 scales: row r at 8192 + r*16, group j at +2*j
 *   [9216, 9472)  zero points: row r's 32-bit LE word at 9216 + r*4,
 *                 group j in bits [4j, 4j+4)
 * Inside a chunk, LE dword d holds k_local = 8d+e at nibble position
 * p = (e & 1)*4 + (e >> 1) (bits [4p, 4p+4)).
 * Tiles are ordered row-block major: tile = rb*(k/256) + kt.
 * Rows n >= N of the last row block are zero (codes 0, scale +0, zp 0). */
int64_t orc_int4_packed_bytes(int64_t n, int64_t k);
void orc_pack_int4(const uint8_t *codes, const uint16_t *scales,
                   const uint8_t *zeros, int64_t n, int64_t k, uint8_t *packed);
void orc_unpack_int4(const uint8_t *packed, int64_t n, int64_t k,
                     uint8_t *codes, uint16_t *scales, uint8_t *zeros);

/* ---- W4A16: y[m, n] = sum_k x[m,k] * (q[n,k] - zp[n,g]) * s[n,g] ----
 * ([P1] module docstring and `_dequant_matmul`: dequant then F.linear.)
 * x bf16 [m, k]; y double [m, n]; rows of W split over `threads` threads. */
void orc_qgemm_w4a16(const uint16_t *x, int64_t m, int64_t k,
                     const uint8_t *codes, const uint16_t *scales,
                     const uint8_t *zeros, int64_t n, double *y, int threads);

/* ---- INT8 per-output-channel symmetric quantizer ----
 * s[n] = smallest bf16 with 127*s >= max_k |w[n,k]| (1.0 for an all-zero
 * row); q = clamp(rint(w / s), -127, 127) in binary32.  Returns flag 1 if a
 * row held a non-finite value (that row: q 0, scale NaN 0x7FC0). */
int orc_quantize_int8_rowwise(const uint16_t *w, int64_t n, int64_t k,
                              int8_t *q, uint16_t *scales);

/* ---- W8A16 ([P3] WeightOnlyInt8Linear.forward):
 * y[m, n] = (sum_k x[m,k] * W[n,k]) * scale[n];  W int8 [n, k], scale bf16 [n]. */
void orc_qgemm_w8a16(const uint16_t *x, int64_t m, int64_t k, const int8_t *w,
                     const uint16_t *scales, int64_t n, double *y, int threads);

/* ---- W4A8: per-row symmetric absmax int8 activations ----
 * a = max_k |x[m,k]|; a == 0 gives xq = 0, sx = 0.  Otherwise
 * inv = 127/a and sx = a/127 (binary32 divisions), xq = clamp(rint(x*inv),
 * -127, 127) with a single binary32 multiply. */
void orc_actquant_int8(const uint16_t *x, int64_t m, int64_t k, int8_t *xq,
                       float *sx);
/* y[m,n] = sx[m] * sum_g s[n,g] * I[m,n,g],
 * I[m,n,g] = sum_{k in g} xq[m,k] * (q[n,k] - zp[n,g])  (exact integer). */
void orc_qgemm_w4a8(const uint16_t *x, int64_t m, int64_t k,
                    const uint8_t *codes, const uint16_t *scales,
                    const uint8_t *zeros, int64_t n, double *y, int threads);

/* ---- W4A8 with per-group-32 activation scales ----
 * The per-row rule above applied to each group of 32 consecutive k of a row
 * (sx is [m, k/32]); y[m,n] = sum_g sx[m,g] * s[n,g] * I[m,n,g]. */
void orc_actquant_int8_g32(const uint16_t *x, int64_t m, int64_t k, int8_t *xq,
                           float *sx);
void orc_qgemm_w4a8_g32(const uint16_t *x, int64_t m, int64_t k,
                        const uint8_t *codes, const uint16_t *scales,
                        const uint8_t *zeros, int64_t n, double *y, int threads);

/* ---- INT4 group-32 with scale codes ([P1] `_packed_with_dense` storage:
 * `scale` uint8 codes [N, K/32] times `scale_step` fp16 [N, 1]) ----
 * Per row: step = smallest fp16 with 3825*step >= the largest group range
 * (ranges widened to hold 0, as above; 1.0 for an all-zero row; 65504 and
 * flag 2 above 3825*65504).  Per group: c = smallest integer in 1..255 with
 * 15*c*step >= the group's range, s = c*step (exact in binary32), then zp and
 * the codes exactly as orc_quantize_group32 with that s.  Zero points are the
 * integers 0..15 (a zero_point_step of 1).  A row holding a non-finite value
 * gets step NaN 0x7E00 and all codes 0 (flag 1).
 *   codes u8 [n,k], scode u8 [n,k/32], sstep fp16 [n], zeros u8 [n,k/32]. */
int orc_quantize_int4_g32_dq(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes,
                             uint8_t *scode, uint16_t *sstep, uint8_t *zeros);

/* ---- packed layout, version 2 (scale codes) ----
 * Row block of 64 rows = a 128-byte head (row r's fp16 step at 2r) followed
 * by K/256 tiles of 8960 bytes:
 *   [0, 8192)     codes, exactly as version 1
 *   [8192, 8704)  scale codes: row r's 8 bytes at 8192 + 8r, group j at +j
 *   [8704, 8960)  zero points: row r's 32-bit LE word at 8704 + 4r, group j
 *                 in bits [4j, 4j+4)
 * Row blocks follow each other; rows n >= N are zero. */
int64_t orc_int4_dq_packed_bytes(int64_t n, int64_t k);
void orc_pack_int4_dq(const uint8_t *codes, const uint8_t *scode, const uint16_t *sstep,
                      const uint8_t *zeros, int64_t n, int64_t k, uint8_t *packed);
void orc_unpack_int4_dq(const uint8_t *packed, int64_t n, int64_t k, uint8_t *codes,
                        uint8_t *scode, uint16_t *sstep, uint8_t *zeros);

/* y[m, n] = sum_k x[m,k] * (q[n,k] - zp[n,g]) * scode[n,g] * sstep[n]. */
void orc_qgemm_w4a16_dq(const uint16_t *x, int64_t m, int64_t k, const uint8_t *codes,
                        const uint8_t *scode, const uint16_t *sstep, const uint8_t *zeros,
                        int64_t n, double *y, int threads);

/* ---- W4A8 on the scale-code form: the activation quantizers above, a
 * group's scale c * step:  per row y = sx[m] * sum_g c*step * I,
 * per group of 32 y = sum_g sx[m,g] * c*step * I. ---- */
void orc_qgemm_w4a8_dq(const uint16_t *x, int64_t m, int64_t k, const uint8_t *codes,
                       const uint8_t *scode, const uint16_t *sstep, const uint8_t *zeros,
                       int64_t n, double *y, int threads);
void orc_qgemm_w4a8_g32_dq(const uint16_t *x, int64_t m, int64_t k, const uint8_t *codes,
                           const uint8_t *scode, const uint16_t *sstep, const uint8_t *zeros,
                           int64_t n, double *y, int threads);

/* ---- INT5 / INT6 group-32 (the pages' INT5/INT6 quantized-GEMM family) ----
 * The INT4 reading with L = 2^bits - 1 steps: s = smallest positive fp16
 * with L*s >= r (1.0 for r == 0; 65504 and flag 2 above L*65504),
 * zp = clamp(rint(-lo/s), 0, L), q = clamp(rint(v/s) + zp, 0, L).
 * bits is 5 or 6; outputs as orc_quantize_int4_g32 (codes up to L).  The
 * dequant-then-dot reference orc_qgemm_w4a16 takes these codes unchanged. */
int orc_quantize_intn_g32(const uint16_t *w, int64_t n, int64_t k, int bits,
                          uint8_t *codes, uint16_t *scales, uint8_t *zeros);
int orc_quantize_group32_bits(const uint16_t *w32, int bits, uint16_t *scale, uint8_t *zp,
                              uint8_t *q32);

/* ---- packed layout for 5 / 6 bits (hb = bits - 4 high bits per code) ----
 * Tiles of 64 rows x 256 k, row-block major, 8192 + 2048*hb + 1536 bytes
 * (11776 for INT5, 13824 for INT6):
 *   [0, 8192)                 the low 4 bits of every code, exactly as v1
 *   [8192, 8192 + 2048 hb)    high planes: the (4 hb)-byte chunk of (group j,
 *                             row r) at 8192 + (j*64 + r)*4*hb; bit order
 *                             in the chunk: see high_bit_position
 *   [.., + 1024)              fp16 scales: row r at +16r, group j at +2j
 *   [.., + 512)               zero points, one byte each: row r at +8r, group j at +j
 * Rows n >= N of the last row block are zero. */
int64_t orc_intn_packed_bytes(int64_t n, int64_t k, int bits);
void orc_pack_intn(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                   int64_t n, int64_t k, int bits, uint8_t *packed);
void orc_unpack_intn(const uint8_t *packed, int64_t n, int64_t k, int bits,
                     uint8_t *codes, uint16_t *scales, uint8_t *zeros);

/* Thread count the machine offers (for the CPU baseline). */
int orc_hardware_threads(void);

#ifdef __cplusplus
}
#endif
#endif
