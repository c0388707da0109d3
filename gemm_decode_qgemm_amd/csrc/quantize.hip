// quantize.hip -- offline weight quantizers (gfx950).
//
// quantize_int4_g32: executorch test_int4_quantized_gemm.py, `_packed_with_dense`
//   (QuantConfig bits=4, group_size=32, symmetric=False, method="min_max").
// quantize_int8_rowwise: gpt-fast issue #114, `WeightOnlyInt8Linear` (int8
//   weight with one scale per output channel).
//
// Both must agree bit for bit with the CPU reference, so every decision that
// turns a float into an integer is taken with IEEE binary32/binary64
// operations in a fixed order: correctly rounded division, rint (half to
// even), no FMA contraction (built with -ffp-contract=off), denormals kept.
#include "qg_common.h"

namespace qg {

// Exact value of an fp16 pattern in binary64.
__device__ __forceinline__ double fp16_value(uint32_t bits) {
  return (double)fp16_to_f32(bits);
}

// Smallest positive finite fp16 s with mult*s >= r, for 0 < r <= mult*65504
// (mult = 15 for a group scale, 3825 = 255 x 15 for a row step).  Start from
// r/mult truncated to fp16, then step to the answer; mult*s is exact in
// binary64, so each comparison is exact.
__device__ uint32_t fp16_covering(double r, double mult) {
  double t = r / mult;
  uint32_t b;
  if (t >= 65504.0) {
    b = 0x7bffu;
  } else if (t < 6.103515625e-05) {           // below 2^-14: subnormal range
    b = (uint32_t)(t * 16777216.0);            // floor(t / 2^-24)
  } else {
    int e;
    double m = frexp(t, &e);                   // t = m * 2^e, m in [0.5, 1)
    uint32_t f = (uint32_t)((2.0 * m - 1.0) * 1024.0);
    b = ((uint32_t)(e + 14) << 10) | f;        // exponent field (e-1)+15
  }
  if (b == 0u) b = 1u;
  while (mult * fp16_value(b) < r) ++b;
  while (b > 1u && mult * fp16_value(b - 1u) >= r) --b;
  return b;
}

__device__ uint32_t fp16_scale_covering(double r) { return fp16_covering(r, 15.0); }

// Zero point and codes of a group for scale s: zp = clamp(rint(-lo/s), 0, 15),
// q = clamp(rint(v/s) + zp, 0, 15) (IEEE division, round half to even).
__device__ __forceinline__ uint32_t group_codes(const float (&v)[32], float lo, float s, uint32_t (&q)[32],
                                                float top = 15.0f) {
  float z = rintf(-lo / s);
  z = z < 0.0f ? 0.0f : (z > top ? top : z);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float t = rintf(v[i] / s) + z;
    t = t < 0.0f ? 0.0f : (t > top ? top : t);
    q[i] = (uint32_t)t;
  }
  return (uint32_t)z;
}

__device__ __forceinline__ void unpack_bf16x32(const uint32_t (&wb)[16], float (&v)[32]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = bf16_to_f32(wb[i] & 0xffffu);
    v[2 * i + 1] = bf16_to_f32(wb[i] >> 16);
  }
}

// The group's range widened to hold 0; false if a value is not finite.
__device__ __forceinline__ bool group_range(const float (&v)[32], float& lo, float& hi) {
  lo = 0.0f;
  hi = 0.0f;
  bool finite = true;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    finite &= __builtin_isfinite(v[i]);
    lo = v[i] < lo ? v[i] : lo;
    hi = v[i] > hi ? v[i] : hi;
  }
  return finite;
}

__device__ __forceinline__ void load_group(const uint16_t* src16, uint32_t (&wb)[16]) {
  const uint4* src = reinterpret_cast<const uint4*>(src16);
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 u = src[c];
    wb[4 * c] = u.x; wb[4 * c + 1] = u.y; wb[4 * c + 2] = u.z; wb[4 * c + 3] = u.w;
  }
}

// The 4 code dwords of a group in the packed nibble order (k = 8d+e at
// nibble position (e & 1)*4 + (e >> 1) of dword d).
__device__ __forceinline__ uint4 pack_chunk(const uint32_t (&q)[32]) {
  uint32_t dw[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t acc = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc |= q[8 * d + e] << (4 * ((e & 1) * 4 + (e >> 1)));
    dw[d] = acc;
  }
  return make_uint4(dw[0], dw[1], dw[2], dw[3]);
}

// One group of 32 bf16 weights -> scale bits, zero point, codes; returns flags.
__device__ uint32_t quantize_group(const uint32_t (&wb)[16], uint32_t& sbits,
                                   uint32_t& zp, uint32_t (&q)[32]) {
  float v[32];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = bf16_to_f32(wb[i] & 0xffffu);
    v[2 * i + 1] = bf16_to_f32(wb[i] >> 16);
  }
  float lo = 0.0f, hi = 0.0f;
  bool nonfinite = false;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    nonfinite |= !__builtin_isfinite(v[i]);
    lo = v[i] < lo ? v[i] : lo;
    hi = v[i] > hi ? v[i] : hi;
  }
  if (nonfinite) {
    sbits = 0x7e00u;
    zp = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) q[i] = 0;
    return QG_FLAG_NONFINITE;
  }
  uint32_t flags = 0;
  double r = (double)hi - (double)lo;
  if (r == 0.0) {
    sbits = 0x3c00u;
  } else if (r > 15.0 * 65504.0) {
    sbits = 0x7bffu;
    flags = QG_FLAG_OVERFLOW;
  } else {
    sbits = fp16_scale_covering(r);
  }
  zp = group_codes(v, lo, fp16_to_f32(sbits), q);
  return flags;
}

// One thread per (row, 256-k tile): quantizes 8 groups of its row and writes
// its 8 code chunks, its 8 scales (16 B) and its zero word (4 B).  A wave is
// 64 consecutive rows of one tile, so every store is a whole-line stream.
__global__ __launch_bounds__(256) void quantize_int4_g32_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, uint8_t* __restrict__ packed,
    int64_t tiles, uint32_t* __restrict__ status) {
  const int64_t wave_global = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave_global >= tiles) return;
  const int64_t kt_count = k / kTileK;
  const int64_t rb = wave_global / kt_count;
  const int64_t kt = wave_global % kt_count;
  const int r = threadIdx.x & 63;
  const int64_t row = rb * kTileRows + r;
  uint8_t* tile = packed + wave_global * kTileBytes;

  uint32_t flags = 0;
  uint32_t zword = 0;
  uint32_t sword[4] = {0, 0, 0, 0};
  for (int j = 0; j < kGroupsPerTile; ++j) {
    uint4 chunk = make_uint4(0, 0, 0, 0);
    if (row < n) {
      const uint4* src = reinterpret_cast<const uint4*>(w + row * k + kt * kTileK + j * 32);
      uint32_t wb[16];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        uint4 u = src[c];
        wb[4 * c] = u.x; wb[4 * c + 1] = u.y; wb[4 * c + 2] = u.z; wb[4 * c + 3] = u.w;
      }
      uint32_t sbits, zp, q[32];
      flags |= quantize_group(wb, sbits, zp, q);
      uint32_t dw[4];
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint32_t acc = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int p = (e & 1) * 4 + (e >> 1);   // nibble position of k = 8d+e
          acc |= q[8 * d + e] << (4 * p);
        }
        dw[d] = acc;
      }
      chunk = make_uint4(dw[0], dw[1], dw[2], dw[3]);
      sword[j >> 1] |= sbits << (16 * (j & 1));
      zword |= zp << (4 * j);
    }
    *reinterpret_cast<uint4*>(tile + (j * kTileRows + r) * 16) = chunk;
  }
  *reinterpret_cast<uint4*>(tile + kScaleOff + r * 16) =
      make_uint4(sword[0], sword[1], sword[2], sword[3]);
  *reinterpret_cast<uint32_t*>(tile + kZeroOff + r * 4) = zword;
  if (flags != 0 && status != nullptr) atomicOr(status, flags);
}

// ---- scale-code layout (version 2) -----------------------------------
// Same reading as above, with a group's scale stored as a uint8 code times a
// per-row fp16 step: step = smallest fp16 with 3825*step >= the row's
// largest group range; code = smallest c in 1..255 with 15*c*step >= the
// group's range; then zero point and codes as above with s = c*step.  A row
// holding a non-finite value gets step NaN and all codes 0 (flag 1).

// Pass 1: one wave per row (rows of the padded last block too): the largest
// group range, then the row's step into the block's head.
__global__ __launch_bounds__(256) void quantize_int4_dq_step_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, uint8_t* __restrict__ packed,
    int64_t block_bytes, int64_t rows_padded, uint32_t* __restrict__ status) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows_padded) return;                 // whole waves leave together
  const int lane = threadIdx.x & 63;
  double rmax = 0.0;
  bool finite = true;
  if (row < n) {
    for (int64_t g = lane; g < k / 32; g += 64) {
      uint32_t wb[16];
      load_group(w + row * k + g * 32, wb);
      float v[32], lo, hi;
      unpack_bf16x32(wb, v);
      finite &= group_range(v, lo, hi);
      const double r = (double)hi - (double)lo;
      rmax = r > rmax ? r : rmax;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const double o = __shfl_xor(rmax, off);
    rmax = o > rmax ? o : rmax;
  }
  const bool all_finite = __all(finite);
  if (lane == 0) {
    uint32_t bits = 0, flags = 0;
    if (row < n) {
      if (!all_finite) {
        bits = 0x7e00u;
        flags = QG_FLAG_NONFINITE;
      } else if (rmax == 0.0) {
        bits = 0x3c00u;
      } else if (rmax > 3825.0 * 65504.0) {
        bits = 0x7bffu;
        flags = QG_FLAG_OVERFLOW;
      } else {
        bits = fp16_covering(rmax, 3825.0);
      }
    }
    *reinterpret_cast<uint16_t*>(packed + (row / kTileRows) * block_bytes + 2 * (row % kTileRows)) =
        (uint16_t)bits;
    if (flags != 0 && status != nullptr) atomicOr(status, flags);
  }
}

// Smallest c in 1..255 with 15*c*step >= r (255 if none): start from the
// quotient, then step to the answer with exact binary64 comparisons.
__device__ uint32_t dq_scale_code(double r, double step) {
  const double t = r / (15.0 * step);
  uint32_t c = t >= 255.0 ? 255u : (t <= 1.0 ? 1u : (uint32_t)ceil(t));
  while (c < 255u && 15.0 * (double)c * step < r) ++c;
  while (c > 1u && 15.0 * (double)(c - 1u) * step >= r) --c;
  return c;
}

// Pass 2: one thread per (row, 256-k tile), as quantize_int4_g32_kernel:
// 8 code chunks, 8 scale codes (8 B) and the zero word (4 B) of its row.
__global__ __launch_bounds__(256) void quantize_int4_dq_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, uint8_t* __restrict__ packed,
    int64_t block_bytes, int64_t tiles) {
  const int64_t wave_global = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave_global >= tiles) return;
  const int64_t kt_count = k / kTileK;
  const int64_t rb = wave_global / kt_count;
  const int64_t kt = wave_global % kt_count;
  const int r = threadIdx.x & 63;
  const int64_t row = rb * kTileRows + r;
  uint8_t* block = packed + rb * block_bytes;
  uint8_t* tile = block + kDqHeadBytes + kt * kDqTileBytes;
  const uint32_t sbits = *reinterpret_cast<const uint16_t*>(block + 2 * r);   // written by pass 1
  // padding rows and rows with a non-finite value keep all-zero codes
  const bool live = row < n && (sbits & 0x7c00u) != 0x7c00u;
  const double step = fp16_value(sbits);

  uint32_t zword = 0;
  uint32_t cword[2] = {0, 0};
  for (int j = 0; j < kGroupsPerTile; ++j) {
    uint4 chunk = make_uint4(0, 0, 0, 0);
    if (live) {
      uint32_t wb[16];
      load_group(w + row * k + kt * kTileK + j * 32, wb);
      float v[32], lo, hi;
      unpack_bf16x32(wb, v);
      group_range(v, lo, hi);
      const uint32_t c = dq_scale_code((double)hi - (double)lo, step);
      const float s = (float)((double)c * step);     // exact: 8 x 11 significant bits
      uint32_t q[32];
      const uint32_t zp = group_codes(v, lo, s, q);
      chunk = pack_chunk(q);
      cword[j >> 2] |= c << (8 * (j & 3));
      zword |= zp << (4 * j);
    }
    *reinterpret_cast<uint4*>(tile + (j * kTileRows + r) * 16) = chunk;
  }
  *reinterpret_cast<uint2*>(tile + kDqScodeOff + r * 8) = make_uint2(cword[0], cword[1]);
  *reinterpret_cast<uint32_t*>(tile + kDqZeroOff + r * 4) = zword;
}

hipError_t launch_quantize_int4_g32_dq(const void* w, int64_t n, int64_t k, void* packed,
                                       uint32_t* status, hipStream_t stream) {
  const int64_t rbs = (n + kTileRows - 1) / kTileRows;
  const int64_t kt_count = k / kTileK;
  const int64_t block_bytes = kDqHeadBytes + kt_count * kDqTileBytes;
  const int64_t rows_padded = rbs * kTileRows;
  hipLaunchKernelGGL(quantize_int4_dq_step_kernel, dim3((unsigned)((rows_padded + 3) / 4)), dim3(256),
                     0, stream, static_cast<const uint16_t*>(w), n, k, static_cast<uint8_t*>(packed),
                     block_bytes, rows_padded, status);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t tiles = rbs * kt_count;
  hipLaunchKernelGGL(quantize_int4_dq_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(w), n, k, static_cast<uint8_t*>(packed), block_bytes,
                     tiles);
  return hipGetLastError();
}

// ---- INT5 / INT6 (the pages' INT5/INT6 family) ----------------------------
// The INT4 reading with L = 2^bits - 1 steps: s = smallest fp16 with L*s >= r,
// zp = clamp(rint(-lo/s), 0, L), q = clamp(rint(v/s) + zp, 0, L).  Layout:
// the low 4 bits of each code as the INT4 tile, then HB = bits - 4 high-bit
// planes, fp16 scales and one zero-point byte per group (tile of 8192 +
// 2048 HB + 1536 bytes).  A plane chunk (4 HB bytes per group and row) holds,
// for code dword d and pair p (k = 8d+2p even, 8d+2p+1 odd): INT5 the even
// k's bit at 4d + p and the odd k's at 16 + 4d + p; INT6 in dword d/2 the
// even k's two bits at 8(d%2) + 2p + b, the odd k's 16 higher.
template <int HB>
__global__ __launch_bounds__(256) void quantize_intn_g32_kernel(
    const uint16_t* __restrict__ w, int64_t n, int64_t k, uint8_t* __restrict__ packed,
    int64_t tiles, uint32_t* __restrict__ status) {
  constexpr int L = (1 << (HB + 4)) - 1;
  constexpr int64_t kTile = 8192 + 2048 * HB + 1536;
  constexpr int kS = 8192 + 2048 * HB, kZ = kS + 1024;
  const int64_t wave_global = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wave_global >= tiles) return;
  const int64_t kt_count = k / kTileK;
  const int64_t rb = wave_global / kt_count;
  const int64_t kt = wave_global % kt_count;
  const int r = threadIdx.x & 63;
  const int64_t row = rb * kTileRows + r;
  uint8_t* tile = packed + wave_global * kTile;

  uint32_t flags = 0;
  uint32_t sword[4] = {0, 0, 0, 0};
  uint32_t zword[2] = {0, 0};
  for (int j = 0; j < kGroupsPerTile; ++j) {
    uint4 chunk = make_uint4(0, 0, 0, 0);
    uint32_t plane[HB];
#pragma unroll
    for (int h = 0; h < HB; ++h) plane[h] = 0;
    if (row < n) {
      uint32_t wb[16];
      load_group(w + row * k + kt * kTileK + j * 32, wb);
      float v[32], lo, hi;
      unpack_bf16x32(wb, v);
      uint32_t q[32], sbits, zp;
      if (!group_range(v, lo, hi)) {
        sbits = 0x7e00u;
        zp = 0;
#pragma unroll
        for (int i = 0; i < 32; ++i) q[i] = 0;
        flags |= QG_FLAG_NONFINITE;
      } else {
        const double rng = (double)hi - (double)lo;
        if (rng == 0.0) {
          sbits = 0x3c00u;
        } else if (rng > (double)L * 65504.0) {
          sbits = 0x7bffu;
          flags |= QG_FLAG_OVERFLOW;
        } else {
          sbits = fp16_covering(rng, (double)L);
        }
        zp = group_codes(v, lo, fp16_to_f32(sbits), q, (float)L);
      }
      uint32_t lowq[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) lowq[i] = q[i] & 15u;
      chunk = pack_chunk(lowq);
#pragma unroll
      for (int kl = 0; kl < 32; ++kl) {
        const int d = kl >> 3, pp = (kl & 7) >> 1, odd = kl & 1;
        if constexpr (HB == 1) {
          plane[0] |= ((q[kl] >> 4) & 1u) << (16 * odd + 4 * d + pp);
        } else {
#pragma unroll
          for (int b = 0; b < 2; ++b)
            plane[d >> 1] |= ((q[kl] >> (4 + b)) & 1u) << (16 * odd + 8 * (d & 1) + 2 * pp + b);
        }
      }
      sword[j >> 1] |= sbits << (16 * (j & 1));
      zword[j >> 2] |= zp << (8 * (j & 3));
    }
    *reinterpret_cast<uint4*>(tile + (j * kTileRows + r) * 16) = chunk;
    if constexpr (HB == 1)
      *reinterpret_cast<uint32_t*>(tile + 8192 + (j * kTileRows + r) * 4) = plane[0];
    else
      *reinterpret_cast<uint2*>(tile + 8192 + (j * kTileRows + r) * 8) = make_uint2(plane[0], plane[1]);
  }
  *reinterpret_cast<uint4*>(tile + kS + r * 16) = make_uint4(sword[0], sword[1], sword[2], sword[3]);
  *reinterpret_cast<uint2*>(tile + kZ + r * 8) = make_uint2(zword[0], zword[1]);
  if (flags != 0 && status != nullptr) atomicOr(status, flags);
}

hipError_t launch_quantize_intn_g32(const void* w, int64_t n, int64_t k, int bits, void* packed,
                                    uint32_t* status, hipStream_t stream) {
  const int64_t tiles = ((n + kTileRows - 1) / kTileRows) * (k / kTileK);
  const dim3 grid((unsigned)((tiles + 3) / 4)), block(256);
  if (bits == 5)
    hipLaunchKernelGGL(quantize_intn_g32_kernel<1>, grid, block, 0, stream, static_cast<const uint16_t*>(w),
                       n, k, static_cast<uint8_t*>(packed), tiles, status);
  else if (bits == 6)
    hipLaunchKernelGGL(quantize_intn_g32_kernel<2>, grid, block, 0, stream, static_cast<const uint16_t*>(w),
                       n, k, static_cast<uint8_t*>(packed), tiles, status);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Smallest positive finite bf16 s with 127*s >= a, for a > 0 finite.
__device__ uint32_t bf16_scale_covering(double a) {
  float t = (float)(a / 127.0);
  uint32_t b = __float_as_uint(t) >> 16;       // truncate to bf16
  while (127.0 * (double)bf16_to_f32(b) < a) ++b;
  while (b > 1u && 127.0 * (double)bf16_to_f32(b - 1u) >= a) --b;
  return b;
}

// One 256-thread block per row: absmax reduction, then scale and codes.
// Threads take 16-byte pieces (8 values) of the row, piece p = tid + 256 j;
// the first kQ8Held pieces of each thread stay in registers between the two
// passes (all of them for K <= 8192), later ones are read again; codes are
// written 8 bytes per piece.
constexpr int kQ8Held = 4;

__device__ __forceinline__ void absmax8_flag(const uint4& u, float& amax, int& bad) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float v = bf16_to_f32(h ? (w[j] >> 16) : (w[j] & 0xffffu));
      bad |= !__builtin_isfinite(v);
      const float a = fabsf(v);
      amax = a > amax ? a : amax;
    }
}

// 8 codes rint(v / s) clamped to [-127, 127], packed little-endian.
__device__ __forceinline__ uint2 codes8(const uint4& u, float s) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float t = rintf(bf16_to_f32(h ? (w[j] >> 16) : (w[j] & 0xffffu)) / s);
      t = t < -127.0f ? -127.0f : (t > 127.0f ? 127.0f : t);
      const int e = 2 * j + h;
      out[e >> 2] |= ((uint32_t)(int)t & 0xffu) << (8 * (e & 3));
    }
  return make_uint2(out[0], out[1]);
}

__global__ __launch_bounds__(256) void quantize_int8_rowwise_kernel(
    const uint16_t* __restrict__ w, int64_t k, int8_t* __restrict__ q,
    uint16_t* __restrict__ scales, uint32_t* __restrict__ status) {
  __shared__ float red_max[4];
  __shared__ int red_bad[4];
  const int64_t row = blockIdx.x;
  const uint4* wr = reinterpret_cast<const uint4*>(w + row * k);
  uint2* qr = reinterpret_cast<uint2*>(q + row * k);
  const int pieces = (int)(k >> 3);
  const int tid = threadIdx.x;
  uint4 held[kQ8Held];
  float amax = 0.0f;
  int bad = 0;
#pragma unroll
  for (int j = 0; j < kQ8Held; ++j) {
    const int p = tid + 256 * j;
    held[j] = make_uint4(0u, 0u, 0u, 0u);
    if (p < pieces) held[j] = wr[p];
  }
#pragma unroll
  for (int j = 0; j < kQ8Held; ++j) absmax8_flag(held[j], amax, bad);   // zeros change nothing
  for (int p = tid + 256 * kQ8Held; p < pieces; p += 256) absmax8_flag(wr[p], amax, bad);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    float o = __shfl_xor(amax, off, 64);
    amax = o > amax ? o : amax;
    bad |= __shfl_xor(bad, off, 64);
  }
  if ((tid & 63) == 0) {
    red_max[tid >> 6] = amax;
    red_bad[tid >> 6] = bad;
  }
  __syncthreads();
  amax = red_max[0];
  bad = red_bad[0];
  for (int i = 1; i < 4; ++i) {
    amax = red_max[i] > amax ? red_max[i] : amax;
    bad |= red_bad[i];
  }
  if (bad) {
    for (int p = tid; p < pieces; p += 256) qr[p] = make_uint2(0u, 0u);
    if (tid == 0) {
      scales[row] = 0x7fc0u;
      if (status != nullptr) atomicOr(status, QG_FLAG_NONFINITE);
    }
    return;
  }
  const uint32_t sbits = amax == 0.0f ? 0x3f80u : bf16_scale_covering((double)amax);
  const float s = bf16_to_f32(sbits);
#pragma unroll
  for (int j = 0; j < kQ8Held; ++j) {
    const int p = tid + 256 * j;
    if (p < pieces) qr[p] = codes8(held[j], s);
  }
  for (int p = tid + 256 * kQ8Held; p < pieces; p += 256) qr[p] = codes8(wr[p], s);
  if (tid == 0) scales[row] = (uint16_t)sbits;
}

// ---- host launchers (called by the C ABI after validation) ----
hipError_t launch_quantize_int4_g32(const void* w, int64_t n, int64_t k, void* packed,
                                    uint32_t* status, hipStream_t stream) {
  const int64_t tiles = ((n + kTileRows - 1) / kTileRows) * (k / kTileK);
  const int64_t blocks = (tiles + 3) / 4;
  hipLaunchKernelGGL(quantize_int4_g32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(w), n, k, static_cast<uint8_t*>(packed),
                     tiles, status);
  return hipGetLastError();
}

hipError_t launch_quantize_int8_rowwise(const void* w, int64_t n, int64_t k, int8_t* q,
                                        void* scales, uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(quantize_int8_rowwise_kernel, dim3((unsigned)n), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(w), k, q, static_cast<uint16_t*>(scales),
                     status);
  return hipGetLastError();
}

}  // namespace qg
