/*
 * qgemm_oracle.c -- plain CPU oracle (see oracle.h for the contract).
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg; never by the product path.  Parity of the
 * functions below is pinned by tests/test_oracle_*.py against hand-worked
 * groups, closed forms, invariants and exact brute force.
 *
 * Written for obviousness, not speed: one element at a time, ascending k,
 * binary64 accumulation.  Build: gcc -O2 -std=c11 -ffp-contract=off.
 */
#include "oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------ */
/* Number formats, from the IEEE-754 bit layouts.                      */
/* ------------------------------------------------------------------ */

/* bf16: 1 sign, 8 exponent (bias 127), 7 fraction bits = the top half of a
 * binary32 pattern, so the conversion is exact. */
double orc_bf16_to_double(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static float bf16_to_float(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp16 (binary16): 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_fp16_to_double(uint16_t bits) {
    int sign = bits >> 15;
    int e = (bits >> 10) & 0x1f;
    int frac = bits & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)frac, -24);               /* zero / subnormal */
    else if (e == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), e - 25);   /* 1.frac * 2^(e-15) */
    return sign ? -v : v;
}

#define FP16_MAX_BITS 0x7BFFu   /* 65504 */
#define FP16_ONE_BITS 0x3C00u
#define FP16_NAN_BITS 0x7E00u
#define BF16_MAX_BITS 0x7F7Fu
#define BF16_ONE_BITS 0x3F80u
#define BF16_NAN_BITS 0x7FC0u

/* Smallest positive finite fp16 s with mult*s >= r (r > 0, r <= mult*65504).
 * Positive finite fp16 patterns 0x0001..0x7BFF increase with their value,
 * so a binary search over the patterns finds it; mult*s is exact in binary64. */
static uint16_t smallest_fp16_covering(double r, double mult) {
    uint32_t lo = 1, hi = FP16_MAX_BITS;
    while (lo < hi) {
        uint32_t mid = (lo + hi) / 2;
        if (mult * orc_fp16_to_double((uint16_t)mid) >= r)
            hi = mid;
        else
            lo = mid + 1;
    }
    return (uint16_t)lo;
}

/* Same for bf16 (positive finite patterns 0x0001..0x7F7F). */
static uint16_t smallest_bf16_covering(double r, double mult) {
    uint32_t lo = 1, hi = BF16_MAX_BITS;
    while (lo < hi) {
        uint32_t mid = (lo + hi) / 2;
        if (mult * orc_bf16_to_double((uint16_t)mid) >= r)
            hi = mid;
        else
            lo = mid + 1;
    }
    return (uint16_t)lo;
}

static float clampf(float v, float lo, float hi) {
    return v < lo ? lo : (v > hi ? hi : v);
}

/* ------------------------------------------------------------------ */
/* INT4 group-32 asymmetric min-max quantizer.                         */
/* [P1] `_packed_with_dense`: QuantConfig(bits=4, group_size=32,        */
/* symmetric=False, method="min_max").  The pages print no formula;    */
/* this is the plainest reading of those settings: range widened to     */
/* hold 0, 15 steps, fp16 scale rounded up so every dequantized value   */
/* is within half a step, integer zero point, round-half-even, round    */
/* then add the zero point.                                             */
/* ------------------------------------------------------------------ */
/* One group of 32 with `levels` steps (15 for INT4, 31 for INT5, 63 for
 * INT6): the same reading with 2^bits - 1 in place of 15. */
static int quantize_group_levels(const uint16_t *w32, int levels, uint16_t *scale,
                                 uint8_t *zp, uint8_t *q32) {
    float v[32];
    float lo = 0.0f, hi = 0.0f;   /* the range always holds 0 */
    int nonfinite = 0;
    for (int i = 0; i < 32; i++) {
        v[i] = bf16_to_float(w32[i]);
        if (!isfinite(v[i])) nonfinite = 1;
        if (v[i] < lo) lo = v[i];
        if (v[i] > hi) hi = v[i];
    }
    if (nonfinite) {
        *scale = FP16_NAN_BITS;
        *zp = 0;
        for (int i = 0; i < 32; i++) q32[i] = 0;
        return 1;
    }
    int flags = 0;
    double r = (double)hi - (double)lo;   /* binary64 range */
    uint16_t sbits;
    if (r == 0.0) {
        sbits = FP16_ONE_BITS;            /* all-zero group */
    } else if (r > levels * 65504.0) {
        sbits = FP16_MAX_BITS;            /* saturate, flag it */
        flags |= 2;
    } else {
        sbits = smallest_fp16_covering(r, (double)levels);
    }
    float s = (float)orc_fp16_to_double(sbits);
    float top = (float)levels;
    float z = clampf(rintf(-lo / s), 0.0f, top);
    for (int i = 0; i < 32; i++) {
        float t = rintf(v[i] / s) + z;    /* round first, then add zp */
        q32[i] = (uint8_t)clampf(t, 0.0f, top);
    }
    *scale = sbits;
    *zp = (uint8_t)z;
    return flags;
}

int orc_quantize_group32(const uint16_t *w32, uint16_t *scale, uint8_t *zp,
                         uint8_t *q32) {
    return quantize_group_levels(w32, 15, scale, zp, q32);
}

int orc_quantize_group32_bits(const uint16_t *w32, int bits, uint16_t *scale, uint8_t *zp,
                              uint8_t *q32) {
    return quantize_group_levels(w32, (1 << bits) - 1, scale, zp, q32);
}

int orc_quantize_int4_g32(const uint16_t *w, int64_t n, int64_t k,
                          uint8_t *codes, uint16_t *scales, uint8_t *zeros) {
    int flags = 0;
    int64_t groups = k / 32;
    for (int64_t row = 0; row < n; row++)
        for (int64_t g = 0; g < groups; g++)
            flags |= orc_quantize_group32(w + row * k + g * 32,
                                          scales + row * groups + g,
                                          zeros + row * groups + g,
                                          codes + row * k + g * 32);
    return flags;
}

/* ------------------------------------------------------------------ */
/* Packed tile layout, version 1 (our own format; see oracle.h).       */
/* ------------------------------------------------------------------ */
enum { T_ROWS = 64, T_GROUPS = 8, T_K = 256, T_CODE_BYTES = 8192,
       T_SCALE_OFF = 8192, T_ZERO_OFF = 9216, T_BYTES = 9472 };

int64_t orc_int4_packed_bytes(int64_t n, int64_t k) {
    int64_t row_blocks = (n + T_ROWS - 1) / T_ROWS;
    return row_blocks * (k / T_K) * (int64_t)T_BYTES;
}

/* Byte offset and nibble shift of code (row r, k-in-tile kk) inside a tile. */
static void code_position(int r, int kk, int64_t *byte, int *shift) {
    int j = kk / 32;          /* group in tile */
    int kl = kk % 32;         /* k in group */
    int d = kl / 8;           /* dword in chunk */
    int e = kl % 8;
    int p = (e & 1) * 4 + (e >> 1);   /* nibble position in the dword */
    *byte = (int64_t)(j * T_ROWS + r) * 16 + d * 4 + p / 2;
    *shift = (p % 2) * 4;
}

void orc_pack_int4(const uint8_t *codes, const uint16_t *scales,
                   const uint8_t *zeros, int64_t n, int64_t k, uint8_t *packed) {
    int64_t kt_count = k / T_K, groups = k / 32;
    int64_t total = orc_int4_packed_bytes(n, k);
    memset(packed, 0, (size_t)total);
    for (int64_t row = 0; row < n; row++) {
        int64_t rb = row / T_ROWS;
        int r = (int)(row % T_ROWS);
        for (int64_t kt = 0; kt < kt_count; kt++) {
            uint8_t *tile = packed + (rb * kt_count + kt) * T_BYTES;
            for (int kk = 0; kk < T_K; kk++) {
                int64_t byte; int shift;
                code_position(r, kk, &byte, &shift);
                tile[byte] |= (uint8_t)((codes[row * k + kt * T_K + kk] & 0xF) << shift);
            }
            for (int j = 0; j < T_GROUPS; j++) {
                int64_t g = kt * T_GROUPS + j;
                uint16_t s = scales[row * groups + g];
                tile[T_SCALE_OFF + r * 16 + j * 2] = (uint8_t)(s & 0xFF);
                tile[T_SCALE_OFF + r * 16 + j * 2 + 1] = (uint8_t)(s >> 8);
                tile[T_ZERO_OFF + r * 4 + j / 2] |=
                    (uint8_t)((zeros[row * groups + g] & 0xF) << ((j % 2) * 4));
            }
        }
    }
}

void orc_unpack_int4(const uint8_t *packed, int64_t n, int64_t k,
                     uint8_t *codes, uint16_t *scales, uint8_t *zeros) {
    int64_t kt_count = k / T_K, groups = k / 32;
    for (int64_t row = 0; row < n; row++) {
        int64_t rb = row / T_ROWS;
        int r = (int)(row % T_ROWS);
        for (int64_t kt = 0; kt < kt_count; kt++) {
            const uint8_t *tile = packed + (rb * kt_count + kt) * T_BYTES;
            for (int kk = 0; kk < T_K; kk++) {
                int64_t byte; int shift;
                code_position(r, kk, &byte, &shift);
                codes[row * k + kt * T_K + kk] = (tile[byte] >> shift) & 0xF;
            }
            for (int j = 0; j < T_GROUPS; j++) {
                int64_t g = kt * T_GROUPS + j;
                scales[row * groups + g] =
                    (uint16_t)(tile[T_SCALE_OFF + r * 16 + j * 2] |
                               (tile[T_SCALE_OFF + r * 16 + j * 2 + 1] << 8));
                zeros[row * groups + g] =
                    (tile[T_ZERO_OFF + r * 4 + j / 2] >> ((j % 2) * 4)) & 0xF;
            }
        }
    }
}

/* ------------------------------------------------------------------ */
/* A tiny row-parallel driver: rows of W split into contiguous ranges.  */
/* ------------------------------------------------------------------ */
typedef void (*row_fn)(void *ctx, int64_t row_begin, int64_t row_end);
struct job { row_fn fn; void *ctx; int64_t begin, end; };

static void *run_job(void *arg) {
    struct job *j = (struct job *)arg;
    j->fn(j->ctx, j->begin, j->end);
    return NULL;
}

static void parallel_rows(row_fn fn, void *ctx, int64_t n, int threads) {
    if (threads < 1) threads = 1;
    if (threads > 512) threads = 512;
    if (threads == 1 || n < 2 * threads) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t tid[512];
    struct job jobs[512];
    int started = 0;
    for (int t = 0; t < threads; t++) {
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].begin = n * t / threads;
        jobs[t].end = n * (t + 1) / threads;
        if (pthread_create(&tid[t], NULL, run_job, &jobs[t]) == 0)
            started = t + 1;
        else
            break;
    }
    /* Whatever could not be started runs here. */
    if (started < threads) fn(ctx, jobs[started].begin, n);
    for (int t = 0; t < started; t++) pthread_join(tid[t], NULL);
}

int orc_hardware_threads(void) {
    long c = sysconf(_SC_NPROCESSORS_ONLN);
    return c > 0 ? (int)c : 1;
}

/* ------------------------------------------------------------------ */
/* W4A16: dequant, then the plain dot product ([P1] `_dequant_matmul`). */
/* ------------------------------------------------------------------ */
struct w4_ctx {
    const uint16_t *x; int64_t m, k;
    const uint8_t *codes; const uint16_t *scales; const uint8_t *zeros;
    int64_t n; double *y;
};

static void w4a16_rows(void *p, int64_t b, int64_t e) {
    struct w4_ctx *c = (struct w4_ctx *)p;
    int64_t groups = c->k / 32;
    for (int64_t row = b; row < e; row++)
        for (int64_t mi = 0; mi < c->m; mi++) {
            double acc = 0.0;
            for (int64_t g = 0; g < groups; g++) {
                double s = orc_fp16_to_double(c->scales[row * groups + g]);
                int z = c->zeros[row * groups + g];
                for (int64_t i = 0; i < 32; i++) {
                    int64_t kk = g * 32 + i;
                    int q = c->codes[row * c->k + kk];
                    double wdq = (double)(q - z) * s;        /* dequant */
                    acc += orc_bf16_to_double(c->x[mi * c->k + kk]) * wdq;
                }
            }
            c->y[mi * c->n + row] = acc;
        }
}

void orc_qgemm_w4a16(const uint16_t *x, int64_t m, int64_t k,
                     const uint8_t *codes, const uint16_t *scales,
                     const uint8_t *zeros, int64_t n, double *y, int threads) {
    struct w4_ctx c = {x, m, k, codes, scales, zeros, n, y};
    parallel_rows(w4a16_rows, &c, n, threads);
}

/* ------------------------------------------------------------------ */
/* INT8 per-output-channel symmetric quantizer.                        */
/* ------------------------------------------------------------------ */
int orc_quantize_int8_rowwise(const uint16_t *w, int64_t n, int64_t k,
                              int8_t *q, uint16_t *scales) {
    int flags = 0;
    for (int64_t row = 0; row < n; row++) {
        const uint16_t *wr = w + row * k;
        double amax = 0.0;
        int nonfinite = 0;
        for (int64_t i = 0; i < k; i++) {
            double v = orc_bf16_to_double(wr[i]);
            if (!isfinite(v)) nonfinite = 1;
            if (fabs(v) > amax) amax = fabs(v);
        }
        if (nonfinite) {
            flags |= 1;
            scales[row] = BF16_NAN_BITS;
            for (int64_t i = 0; i < k; i++) q[row * k + i] = 0;
            continue;
        }
        uint16_t sbits = amax == 0.0 ? BF16_ONE_BITS
                                     : smallest_bf16_covering(amax, 127.0);
        float s = bf16_to_float(sbits);
        for (int64_t i = 0; i < k; i++) {
            float t = rintf(bf16_to_float(wr[i]) / s);
            q[row * k + i] = (int8_t)clampf(t, -127.0f, 127.0f);
        }
        scales[row] = sbits;
    }
    return flags;
}

/* ------------------------------------------------------------------ */
/* W8A16 ([P3] WeightOnlyInt8Linear.forward).                          */
/* ------------------------------------------------------------------ */
struct w8_ctx {
    const uint16_t *x; int64_t m, k; const int8_t *w; const uint16_t *scales;
    int64_t n; double *y;
};

static void w8a16_rows(void *p, int64_t b, int64_t e) {
    struct w8_ctx *c = (struct w8_ctx *)p;
    for (int64_t row = b; row < e; row++)
        for (int64_t mi = 0; mi < c->m; mi++) {
            double acc = 0.0;
            for (int64_t kk = 0; kk < c->k; kk++)
                acc += orc_bf16_to_double(c->x[mi * c->k + kk]) *
                       (double)c->w[row * c->k + kk];
            c->y[mi * c->n + row] = acc * orc_bf16_to_double(c->scales[row]);
        }
}

void orc_qgemm_w8a16(const uint16_t *x, int64_t m, int64_t k, const int8_t *w,
                     const uint16_t *scales, int64_t n, double *y, int threads) {
    struct w8_ctx c = {x, m, k, w, scales, n, y};
    parallel_rows(w8a16_rows, &c, n, threads);
}

/* ------------------------------------------------------------------ */
/* W4A8 ([P1] Int4QuantizedGemmPrecisionTest: int8 activations held to */
/* the W4A16 reference's precision class).                             */
/* ------------------------------------------------------------------ */
/* Symmetric absmax int8 quantization of one span of activations:
 * a = max |x|; a == 0 gives xq = 0, sx = 0; otherwise inv = 127/a and
 * sx = a/127 (binary32 divisions), xq = clamp(rint(x * inv), -127, 127).
 * A span holding a NaN or an infinity has no finite scale: it gets sx = NaN
 * and codes 0, so every output it contributes to is NaN.
 * A span so small that 127/a overflows binary32 (a <= 127 * 2^-128, the
 * largest such bf16 value; every |x| in it is below 3.8e-37) has no finite
 * inverse scale either; it is read as a zero span: sx = 0 and codes 0. */
static void quant_span(const uint16_t *xr, int64_t len, int8_t *xq, float *sx) {
    float a = 0.0f;
    int finite = 1;
    for (int64_t i = 0; i < len; i++) {
        float v = fabsf(bf16_to_float(xr[i]));
        if (!isfinite(v)) finite = 0;
        else if (v > a) a = v;
    }
    if (!finite || a == 0.0f) {
        *sx = finite ? 0.0f : NAN;
        for (int64_t i = 0; i < len; i++) xq[i] = 0;
        return;
    }
    float inv = 127.0f / a;
    if (isinf(inv)) {
        *sx = 0.0f;
        for (int64_t i = 0; i < len; i++) xq[i] = 0;
        return;
    }
    *sx = a / 127.0f;
    for (int64_t i = 0; i < len; i++) {
        float t = rintf(bf16_to_float(xr[i]) * inv);
        xq[i] = (int8_t)clampf(t, -127.0f, 127.0f);
    }
}

void orc_actquant_int8(const uint16_t *x, int64_t m, int64_t k, int8_t *xq,
                       float *sx) {
    for (int64_t mi = 0; mi < m; mi++) quant_span(x + mi * k, k, xq + mi * k, sx + mi);
}

/* The same rule per group of 32 consecutive k of a row: sx is [m, k/32]. */
void orc_actquant_int8_g32(const uint16_t *x, int64_t m, int64_t k, int8_t *xq,
                           float *sx) {
    int64_t groups = k / 32;
    for (int64_t mi = 0; mi < m; mi++)
        for (int64_t g = 0; g < groups; g++)
            quant_span(x + mi * k + g * 32, 32, xq + mi * k + g * 32, sx + mi * groups + g);
}

struct w4a8_ctx {
    const int8_t *xq; const float *sx; int64_t m, k;
    const uint8_t *codes; const uint16_t *scales; const uint8_t *zeros;
    int64_t n; double *y;
};

static void w4a8_rows(void *p, int64_t b, int64_t e) {
    struct w4a8_ctx *c = (struct w4a8_ctx *)p;
    int64_t groups = c->k / 32;
    for (int64_t row = b; row < e; row++)
        for (int64_t mi = 0; mi < c->m; mi++) {
            double acc = 0.0;
            for (int64_t g = 0; g < groups; g++) {
                int64_t isum = 0;     /* exact integer group dot */
                int z = c->zeros[row * groups + g];
                for (int64_t i = 0; i < 32; i++) {
                    int64_t kk = g * 32 + i;
                    isum += (int64_t)c->xq[mi * c->k + kk] *
                            (int64_t)(c->codes[row * c->k + kk] - z);
                }
                acc += orc_fp16_to_double(c->scales[row * groups + g]) * (double)isum;
            }
            c->y[mi * c->n + row] = (double)c->sx[mi] * acc;
        }
}

void orc_qgemm_w4a8(const uint16_t *x, int64_t m, int64_t k,
                    const uint8_t *codes, const uint16_t *scales,
                    const uint8_t *zeros, int64_t n, double *y, int threads) {
    int8_t *xq = (int8_t *)malloc((size_t)(m * k));
    float *sx = (float *)malloc((size_t)m * sizeof(float));
    if (!xq || !sx) { free(xq); free(sx); abort(); }
    orc_actquant_int8(x, m, k, xq, sx);
    struct w4a8_ctx c = {xq, sx, m, k, codes, scales, zeros, n, y};
    parallel_rows(w4a8_rows, &c, n, threads);
    free(xq);
    free(sx);
}

/* W4A8 with one activation scale per group of 32:
 * y[m,n] = sum_g sx[m,g] * s[n,g] * I[m,n,g]; every product is exact in
 * binary64 (24 + 11 + 16 significant bits), the sum over g is in binary64. */
static void w4a8_g32_rows(void *p, int64_t b, int64_t e) {
    struct w4a8_ctx *c = (struct w4a8_ctx *)p;
    int64_t groups = c->k / 32;
    for (int64_t row = b; row < e; row++)
        for (int64_t mi = 0; mi < c->m; mi++) {
            double acc = 0.0;
            for (int64_t g = 0; g < groups; g++) {
                int64_t isum = 0;
                int zg = c->zeros[row * groups + g];
                for (int64_t i = 0; i < 32; i++) {
                    int64_t kk = g * 32 + i;
                    isum += (int64_t)c->xq[mi * c->k + kk] *
                            (int64_t)(c->codes[row * c->k + kk] - zg);
                }
                acc += (double)c->sx[mi * groups + g] *
                       orc_fp16_to_double(c->scales[row * groups + g]) * (double)isum;
            }
            c->y[mi * c->n + row] = acc;
        }
}

void orc_qgemm_w4a8_g32(const uint16_t *x, int64_t m, int64_t k,
                        const uint8_t *codes, const uint16_t *scales,
                        const uint8_t *zeros, int64_t n, double *y, int threads) {
    int64_t groups = k / 32;
    int8_t *xq = (int8_t *)malloc((size_t)(m * k));
    float *sx = (float *)malloc((size_t)(m * groups) * sizeof(float));
    if (!xq || !sx) { free(xq); free(sx); abort(); }
    orc_actquant_int8_g32(x, m, k, xq, sx);
    struct w4a8_ctx c = {xq, sx, m, k, codes, scales, zeros, n, y};
    parallel_rows(w4a8_g32_rows, &c, n, threads);
    free(xq);
    free(sx);
}

/* ------------------------------------------------------------------ */
/* INT4 group-32 with scale codes: the stored form of [P1]              */
/* `_packed_with_dense` (`scale` uint8 codes, `scale_step` fp16 per     */
/* row; legality rules "scale codes must be uint8", "scale_step must be */
/* float16", step shape [N, 1]).  A group's scale is code x row step.   */
/* Where the pages are silent, the reading taken: the row step is the   */
/* smallest fp16 with 255 x 15 x step >= the row's largest group range, */
/* a group's code the smallest c in 1..255 with 15 x c x step >= its    */
/* range, so every group still spans its range in 15 steps; zero points */
/* stay integers 0..15 (zero_point_step 1); then the codes exactly as   */
/* in orc_quantize_group32, with the scale c x step.                    */
/* ------------------------------------------------------------------ */
static void group_range(const uint16_t *w32, float *lo, float *hi, int *nonfinite) {
    *lo = 0.0f;
    *hi = 0.0f;
    for (int i = 0; i < 32; i++) {
        float v = bf16_to_float(w32[i]);
        if (!isfinite(v)) *nonfinite = 1;
        if (v < *lo) *lo = v;
        if (v > *hi) *hi = v;
    }
}

int orc_quantize_int4_g32_dq(const uint16_t *w, int64_t n, int64_t k, uint8_t *codes,
                             uint8_t *scode, uint16_t *sstep, uint8_t *zeros) {
    int flags = 0;
    int64_t groups = k / 32;
    for (int64_t row = 0; row < n; row++) {
        const uint16_t *wr = w + row * k;
        /* pass 1: the largest group range of the row */
        int nonfinite = 0;
        double rmax = 0.0;
        for (int64_t g = 0; g < groups; g++) {
            float lo, hi;
            group_range(wr + g * 32, &lo, &hi, &nonfinite);
            double r = (double)hi - (double)lo;
            if (r > rmax) rmax = r;
        }
        if (nonfinite) {   /* the whole row: NaN step, codes 0 */
            flags |= 1;
            sstep[row] = FP16_NAN_BITS;
            for (int64_t g = 0; g < groups; g++) {
                scode[row * groups + g] = 0;
                zeros[row * groups + g] = 0;
            }
            for (int64_t i = 0; i < k; i++) codes[row * k + i] = 0;
            continue;
        }
        uint16_t step;
        if (rmax == 0.0) {
            step = FP16_ONE_BITS;
        } else if (rmax > 3825.0 * 65504.0) {
            step = FP16_MAX_BITS;
            flags |= 2;
        } else {
            step = smallest_fp16_covering(rmax, 3825.0);   /* 3825 = 255 x 15 */
        }
        sstep[row] = step;
        double ds = orc_fp16_to_double(step);
        /* pass 2: per group, its scale code, zero point and codes */
        for (int64_t g = 0; g < groups; g++) {
            const uint16_t *w32 = wr + g * 32;
            float lo, hi;
            int dummy = 0;
            group_range(w32, &lo, &hi, &dummy);
            double r = (double)hi - (double)lo;
            int c = 1;
            while (c < 255 && 15.0 * c * ds < r) c++;     /* 15 c ds is exact in binary64 */
            float s = (float)(c * ds);                      /* exact: 8 x 11 significant bits */
            float z = clampf(rintf(-lo / s), 0.0f, 15.0f);
            for (int i = 0; i < 32; i++) {
                float t = rintf(bf16_to_float(w32[i]) / s) + z;
                codes[row * k + g * 32 + i] = (uint8_t)clampf(t, 0.0f, 15.0f);
            }
            scode[row * groups + g] = (uint8_t)c;
            zeros[row * groups + g] = (uint8_t)z;
        }
    }
    return flags;
}

/* Packed layout, version 2 (scale codes; see oracle.h). */
enum { D_ROWS = 64, D_HEAD = 128, D_TILE = 8960, D_SCODE_OFF = 8192, D_ZERO_OFF = 8704 };

int64_t orc_int4_dq_packed_bytes(int64_t n, int64_t k) {
    int64_t row_blocks = (n + D_ROWS - 1) / D_ROWS;
    return row_blocks * (D_HEAD + (k / T_K) * (int64_t)D_TILE);
}

void orc_pack_int4_dq(const uint8_t *codes, const uint8_t *scode, const uint16_t *sstep,
                      const uint8_t *zeros, int64_t n, int64_t k, uint8_t *packed) {
    int64_t kt_count = k / T_K, groups = k / 32;
    int64_t block_bytes = D_HEAD + kt_count * D_TILE;
    memset(packed, 0, (size_t)orc_int4_dq_packed_bytes(n, k));
    for (int64_t row = 0; row < n; row++) {
        uint8_t *block = packed + (row / D_ROWS) * block_bytes;
        int r = (int)(row % D_ROWS);
        block[2 * r] = (uint8_t)(sstep[row] & 0xFF);
        block[2 * r + 1] = (uint8_t)(sstep[row] >> 8);
        for (int64_t kt = 0; kt < kt_count; kt++) {
            uint8_t *tile = block + D_HEAD + kt * D_TILE;
            for (int kk = 0; kk < T_K; kk++) {
                int64_t byte; int shift;
                code_position(r, kk, &byte, &shift);
                tile[byte] |= (uint8_t)((codes[row * k + kt * T_K + kk] & 0xF) << shift);
            }
            for (int j = 0; j < T_GROUPS; j++) {
                int64_t g = kt * T_GROUPS + j;
                tile[D_SCODE_OFF + r * 8 + j] = scode[row * groups + g];
                tile[D_ZERO_OFF + r * 4 + j / 2] |=
                    (uint8_t)((zeros[row * groups + g] & 0xF) << ((j % 2) * 4));
            }
        }
    }
}

void orc_unpack_int4_dq(const uint8_t *packed, int64_t n, int64_t k, uint8_t *codes,
                        uint8_t *scode, uint16_t *sstep, uint8_t *zeros) {
    int64_t kt_count = k / T_K, groups = k / 32;
    int64_t block_bytes = D_HEAD + kt_count * D_TILE;
    for (int64_t row = 0; row < n; row++) {
        const uint8_t *block = packed + (row / D_ROWS) * block_bytes;
        int r = (int)(row % D_ROWS);
        sstep[row] = (uint16_t)(block[2 * r] | (block[2 * r + 1] << 8));
        for (int64_t kt = 0; kt < kt_count; kt++) {
            const uint8_t *tile = block + D_HEAD + kt * D_TILE;
            for (int kk = 0; kk < T_K; kk++) {
                int64_t byte; int shift;
                code_position(r, kk, &byte, &shift);
                codes[row * k + kt * T_K + kk] = (tile[byte] >> shift) & 0xF;
            }
            for (int j = 0; j < T_GROUPS; j++) {
                int64_t g = kt * T_GROUPS + j;
                scode[row * groups + g] = tile[D_SCODE_OFF + r * 8 + j];
                zeros[row * groups + g] = (tile[D_ZERO_OFF + r * 4 + j / 2] >> ((j % 2) * 4)) & 0xF;
            }
        }
    }
}

/* W4A16 on the scale-code form: dequant (q - zp) * (c * step), then the dot. */
struct w4dq_ctx {
    const uint16_t *x; int64_t m, k;
    const uint8_t *codes, *scode; const uint16_t *sstep; const uint8_t *zeros;
    int64_t n; double *y;
};

static void w4a16_dq_rows(void *p, int64_t b, int64_t e) {
    struct w4dq_ctx *c = (struct w4dq_ctx *)p;
    int64_t groups = c->k / 32;
    for (int64_t row = b; row < e; row++) {
        double step = orc_fp16_to_double(c->sstep[row]);
        for (int64_t mi = 0; mi < c->m; mi++) {
            double acc = 0.0;
            for (int64_t g = 0; g < groups; g++) {
                double s = (double)c->scode[row * groups + g] * step;
                int z = c->zeros[row * groups + g];
                for (int64_t i = 0; i < 32; i++) {
                    int64_t kk = g * 32 + i;
                    double wdq = (double)(c->codes[row * c->k + kk] - z) * s;
                    acc += orc_bf16_to_double(c->x[mi * c->k + kk]) * wdq;
                }
            }
            c->y[mi * c->n + row] = acc;
        }
    }
}

void orc_qgemm_w4a16_dq(const uint16_t *x, int64_t m, int64_t k, const uint8_t *codes,
                        const uint8_t *scode, const uint16_t *sstep, const uint8_t *zeros,
                        int64_t n, double *y, int threads) {
    struct w4dq_ctx c = {x, m, k, codes, scode, sstep, zeros, n, y};
    parallel_rows(w4a16_dq_rows, &c, n, threads);
}

/* ------------------------------------------------------------------ */
/* INT5 / INT6 group-32 (the pages' INT5/INT6 family): the INT4 reading */
/* with 31 / 63 steps, fp16 scale, integer zero point 0..2^bits-1.      */
/* ------------------------------------------------------------------ */
int orc_quantize_intn_g32(const uint16_t *w, int64_t n, int64_t k, int bits,
                          uint8_t *codes, uint16_t *scales, uint8_t *zeros) {
    int flags = 0;
    int64_t groups = k / 32;
    for (int64_t row = 0; row < n; row++)
        for (int64_t g = 0; g < groups; g++)
            flags |= orc_quantize_group32_bits(w + row * k + g * 32, bits,
                                               scales + row * groups + g,
                                               zeros + row * groups + g,
                                               codes + row * k + g * 32);
    return flags;
}

/* Packed layout for 5 and 6 bits (see oracle.h): the low 4 bits of every
 * code exactly as version 1, the high bits in a plane of hb = bits - 4 bits
 * per code. */
static int64_t intn_tile_bytes(int bits) { return 8192 + 2048 * (bits - 4) + 1024 + 512; }

int64_t orc_intn_packed_bytes(int64_t n, int64_t k, int bits) {
    int64_t row_blocks = (n + T_ROWS - 1) / T_ROWS;
    return row_blocks * (k / T_K) * intn_tile_bytes(bits);
}

/* Bit of the high plane (counted from the row's (4*hb)-byte group chunk,
 * little-endian) that holds high bit b of k-in-group kl.  Code dword d of
 * the low chunk holds k = 8d+e, pair p = e/2 being k = 8d+2p (even) and
 * 8d+2p+1 (odd).  INT5 (hb = 1): one plane dword; the even k's bit at
 * 4d + p, the odd k's at 16 + 4d + p.  INT6 (hb = 2): plane dword d/2; in
 * it the even k's two bits at 8(d%2) + 2p + b, the odd k's 16 higher.  So
 * (plane >> shift) & mask puts a pair's high bits where
 * (dword >> 4p) & 0x000F000F puts its low bits, 4 places lower. */
static int high_bit_position(int kl, int b, int hb) {
    int d = kl / 8, p = (kl % 8) / 2, odd = kl % 2;
    if (hb == 1) return 16 * odd + 4 * d + p;
    return 32 * (d / 2) + 16 * odd + 8 * (d % 2) + 2 * p + b;
}

void orc_pack_intn(const uint8_t *codes, const uint16_t *scales, const uint8_t *zeros,
                   int64_t n, int64_t k, int bits, uint8_t *packed) {
    int hb = bits - 4;
    int64_t tb = intn_tile_bytes(bits), kt_count = k / T_K, groups = k / 32;
    int64_t hi_off = 8192, s_off = 8192 + 2048 * hb, z_off = s_off + 1024;
    memset(packed, 0, (size_t)orc_intn_packed_bytes(n, k, bits));
    for (int64_t row = 0; row < n; row++) {
        int64_t rb = row / T_ROWS;
        int r = (int)(row % T_ROWS);
        for (int64_t kt = 0; kt < kt_count; kt++) {
            uint8_t *tile = packed + (rb * kt_count + kt) * tb;
            for (int kk = 0; kk < T_K; kk++) {
                int q = codes[row * k + kt * T_K + kk];
                int64_t byte; int shift;
                code_position(r, kk, &byte, &shift);
                tile[byte] |= (uint8_t)((q & 0xF) << shift);
                int j = kk / 32, kl = kk % 32;
                uint8_t *chunk = tile + hi_off + (int64_t)(j * T_ROWS + r) * 4 * hb;
                for (int b = 0; b < hb; b++) {
                    int pos = high_bit_position(kl, b, hb);
                    chunk[pos / 8] |= (uint8_t)(((q >> (4 + b)) & 1) << (pos % 8));
                }
            }
            for (int j = 0; j < T_GROUPS; j++) {
                int64_t g = kt * T_GROUPS + j;
                uint16_t sc = scales[row * groups + g];
                tile[s_off + r * 16 + j * 2] = (uint8_t)(sc & 0xFF);
                tile[s_off + r * 16 + j * 2 + 1] = (uint8_t)(sc >> 8);
                tile[z_off + r * 8 + j] = zeros[row * groups + g];
            }
        }
    }
}

void orc_unpack_intn(const uint8_t *packed, int64_t n, int64_t k, int bits,
                     uint8_t *codes, uint16_t *scales, uint8_t *zeros) {
    int hb = bits - 4;
    int64_t tb = intn_tile_bytes(bits), kt_count = k / T_K, groups = k / 32;
    int64_t hi_off = 8192, s_off = 8192 + 2048 * hb, z_off = s_off + 1024;
    for (int64_t row = 0; row < n; row++) {
        int64_t rb = row / T_ROWS;
        int r = (int)(row % T_ROWS);
        for (int64_t kt = 0; kt < kt_count; kt++) {
            const uint8_t *tile = packed + (rb * kt_count + kt) * tb;
            for (int kk = 0; kk < T_K; kk++) {
                int64_t byte; int shift;
                code_position(r, kk, &byte, &shift);
                int q = (tile[byte] >> shift) & 0xF;
                int j = kk / 32, kl = kk % 32;
                const uint8_t *chunk = tile + hi_off + (int64_t)(j * T_ROWS + r) * 4 * hb;
                for (int b = 0; b < hb; b++) {
                    int pos = high_bit_position(kl, b, hb);
                    q |= ((chunk[pos / 8] >> (pos % 8)) & 1) << (4 + b);
                }
                codes[row * k + kt * T_K + kk] = (uint8_t)q;
            }
            for (int j = 0; j < T_GROUPS; j++) {
                int64_t g = kt * T_GROUPS + j;
                scales[row * groups + g] =
                    (uint16_t)(tile[s_off + r * 16 + j * 2] | (tile[s_off + r * 16 + j * 2 + 1] << 8));
                zeros[row * groups + g] = tile[z_off + r * 8 + j];
            }
        }
    }
}

/* W4A8 on the scale-code form: the activations quantized exactly as in
 * orc_qgemm_w4a8 / orc_qgemm_w4a8_g32, a group's scale c * step.
 *   per row:      y[m,n] = sx[m] * sum_g (c[n,g] * step[n]) * I[m,n,g]
 *   per group 32: y[m,n] = sum_g sx[m,g] * (c[n,g] * step[n]) * I[m,n,g]
 * with I the exact integer group dot; c * step is exact in binary64, the
 * products and the sum over g are binary64. */
struct w4a8dq_ctx {
    const int8_t *xq; const float *sx; int64_t m, k;
    const uint8_t *codes, *scode; const uint16_t *sstep; const uint8_t *zeros;
    int64_t n; double *y; int per_group;
};

static void w4a8_dq_rows(void *p, int64_t b, int64_t e) {
    struct w4a8dq_ctx *c = (struct w4a8dq_ctx *)p;
    int64_t groups = c->k / 32;
    for (int64_t row = b; row < e; row++) {
        double step = orc_fp16_to_double(c->sstep[row]);
        for (int64_t mi = 0; mi < c->m; mi++) {
            double acc = 0.0;
            for (int64_t g = 0; g < groups; g++) {
                int64_t isum = 0;
                int zg = c->zeros[row * groups + g];
                for (int64_t i = 0; i < 32; i++) {
                    int64_t kk = g * 32 + i;
                    isum += (int64_t)c->xq[mi * c->k + kk] *
                            (int64_t)(c->codes[row * c->k + kk] - zg);
                }
                double s = (double)c->scode[row * groups + g] * step;
                if (c->per_group)
                    acc += (double)c->sx[mi * groups + g] * s * (double)isum;
                else
                    acc += s * (double)isum;
            }
            c->y[mi * c->n + row] = c->per_group ? acc : (double)c->sx[mi] * acc;
        }
    }
}

static void w4a8_dq_common(const uint16_t *x, int64_t m, int64_t k, const uint8_t *codes,
                           const uint8_t *scode, const uint16_t *sstep, const uint8_t *zeros,
                           int64_t n, double *y, int threads, int per_group) {
    int64_t groups = k / 32;
    int8_t *xq = (int8_t *)malloc((size_t)(m * k));
    float *sx = (float *)malloc((size_t)(m * (per_group ? groups : 1)) * sizeof(float));
    if (!xq || !sx) { free(xq); free(sx); abort(); }
    if (per_group)
        orc_actquant_int8_g32(x, m, k, xq, sx);
    else
        orc_actquant_int8(x, m, k, xq, sx);
    struct w4a8dq_ctx c = {xq, sx, m, k, codes, scode, sstep, zeros, n, y, per_group};
    parallel_rows(w4a8_dq_rows, &c, n, threads);
    free(xq);
    free(sx);
}

void orc_qgemm_w4a8_dq(const uint16_t *x, int64_t m, int64_t k, const uint8_t *codes,
                       const uint8_t *scode, const uint16_t *sstep, const uint8_t *zeros,
                       int64_t n, double *y, int threads) {
    w4a8_dq_common(x, m, k, codes, scode, sstep, zeros, n, y, threads, 0);
}

void orc_qgemm_w4a8_g32_dq(const uint16_t *x, int64_t m, int64_t k, const uint8_t *codes,
                           const uint8_t *scode, const uint16_t *sstep, const uint8_t *zeros,
                           int64_t n, double *y, int threads) {
    w4a8_dq_common(x, m, k, codes, scode, sstep, zeros, n, y, threads, 1);
}
