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

// Smallest positive finite fp16 s with 15*s >= r, for 0 < r <= 15*65504.
// Start from r/15 truncated to fp16, then step to the answer; 15*s is exact
// in binary64, so each comparison is exact.
__device__ uint32_t fp16_scale_covering(double r) {
  double t = r / 15.0;
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
  while (15.0 * fp16_value(b) < r) ++b;
  while (b > 1u && 15.0 * fp16_value(b - 1u) >= r) --b;
  return b;
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
  float s = fp16_to_f32(sbits);
  float z = rintf(-lo / s);
  z = z < 0.0f ? 0.0f : (z > 15.0f ? 15.0f : z);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    float t = rintf(v[i] / s) + z;
    t = t < 0.0f ? 0.0f : (t > 15.0f ? 15.0f : t);
    q[i] = (uint32_t)t;
  }
  zp = (uint32_t)z;
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
