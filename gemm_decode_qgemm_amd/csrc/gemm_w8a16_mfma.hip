// gemm_w8a16_mfma.hip -- int8 weight-only linear layer for M = 5..64 rows on
// the matrix cores: y[m, n] = (sum_k x[m,k] W[n,k]) * s[n].
//
// gpt-fast issue #114 ("Question about the generated code of
// WeightOnlyInt8Linear"): the layer is F.linear(x, W.to(bf16)) * scales on
// the caller's row-major int8 [N, K] weight; the thread closes by asking how
// to fuse it for batch sizes above 1.  Here, as in the decode GEMV, the int8
// -> float convert stays in registers and W is read once; with 5..64
// activation rows each weight feeds enough products for the matrix cores.
//
// Arithmetic, v_mfma_f32_16x16x32_bf16 on exact operands:
//   B = w + 128 in 0..255 (a byte XORed with 0x80, converted exactly to bf16),
//   D = x . B accumulated over the whole K range in the matrix unit,
//   X = x . ones (the activation row sums, one more product per m-tile),
//   y = s * (D - 128 X),
// so every product is exact and the sums are fp32 (integer activations with
// sum |x| * 255 below 2^24 give the exact integer result).  The scale is per
// output row, so nothing is applied per group and the accumulators stay in
// the matrix unit from the first k to the last.
//
// Mapping (gfx950, wave64): a workgroup owns 32 weight rows (2 n-tiles of
// 16) and all M rows (MT m-tiles of 16); its KW waves take the 128-k blocks of
// K round robin.  In a block, lane (i, a) = (lane % 16, lane / 16) loads 32
// contiguous weight bytes of row 16 t + i (k = 128 b + 32 a .. + 32) and the
// same 32 k of x row 16 mt + i; step j of 4 uses k = 128 b + 32 a + 8 j .. + 8
// in lane group a, the same for A and B, so the 4 steps cover the block's 128 k
// once.  The next block's weights are loaded while the current one computes.
// The KW partial sums meet in LDS and are added in wave order.
#include "qg_common.h"

namespace qg {

constexpr int kW8NT = 2;    // n-tiles (16 weight rows each) per workgroup
constexpr int kW8KW = 8;    // waves per workgroup, along K

// 8 int8 weights (two dwords, k ascending) as the bf16 pairs (w + 128) of a
// B operand: each byte XORed with 0x80 is w + 128, converted exactly to fp32
// (v_cvt_f32_ubyte*), whose upper half is the exact bf16; v_perm_b32 joins two
// upper halves.  Plain C: the results feed a matrix instruction directly.
__device__ __forceinline__ bf16x8_t w8_operand(uint32_t d0, uint32_t d1, uint32_t sel_hi) {
  const uint32_t u[2] = {d0 ^ 0x80808080u, d1 ^ 0x80808080u};
  uint32_t b[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t v = u[h >> 1] >> (16 * (h & 1));
    const float lo = (float)(v & 0xffu);
    const float hi = (float)((v >> 8) & 0xffu);
    b[h] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), sel_hi);
  }
  return __builtin_bit_cast(bf16x8_t, u32x4_t{b[0], b[1], b[2], b[3]});
}

template <int MT>
__global__ __launch_bounds__(kW8KW * 64) void w8a16_mfma_kernel(
    const uint16_t* __restrict__ x, int m, const int8_t* __restrict__ w,
    const uint16_t* __restrict__ scale, int n, int k, void* __restrict__ y, int y_f32) {
  constexpr int NACC = kW8NT * MT + MT;            // per wave: the products, then X
  __shared__ f32x4_t red[kW8KW][NACC][64];
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, a = lane >> 4;
  const int wave = wave_id_uniform();
  const int row0 = blockIdx.x * (16 * kW8NT);
  const int nblk = k >> 7;
  const uint32_t sel_hi = __builtin_amdgcn_readfirstlane(0x07060302u);   // upper halves of (S1, S0)
  uint32_t one2 = 0x3f803f80u;           // bf16 pair (1, 1), kept in a VGPR
  asm volatile("" : "+v"(one2));
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{one2, one2, one2, one2});

  // Rows past n or m read the last row instead (a valid address); their
  // results are never stored.
  const int8_t* wr[kW8NT];
#pragma unroll
  for (int t = 0; t < kW8NT; ++t) wr[t] = w + (size_t)min(row0 + 16 * t + i, n - 1) * k + 32 * a;
  const uint16_t* xr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xr[mt] = x + (size_t)min(16 * mt + i, m - 1) * k + 32 * a;

  f32x4_t acc[kW8NT][MT], xs[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    xs[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < kW8NT; ++t) acc[t][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  auto load_w = [&](u32x4_t (&wv)[kW8NT][2], int b) {
#pragma unroll
    for (int t = 0; t < kW8NT; ++t) {
      const u32x4_t* p = reinterpret_cast<const u32x4_t*>(wr[t] + 128 * (size_t)b);
      wv[t][0] = load_stream<true>(p);
      wv[t][1] = load_stream<true>(p + 1);
    }
  };
  auto compute = [&](const u32x4_t (&wv)[kW8NT][2], int b) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bf16x8_t av[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        av[mt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(xr[mt] + 128 * (size_t)b + 8 * j));
#pragma unroll
      for (int t = 0; t < kW8NT; ++t) {
        const u32x4_t& q = wv[t][j >> 1];
        const bf16x8_t bv = (j & 1) ? w8_operand(q.z, q.w, sel_hi) : w8_operand(q.x, q.y, sel_hi);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bv, acc[t][mt], 0, 0, 0);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xs[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], ones, xs[mt], 0, 0, 0);
    }
  };

  // Two register sets used in turn: the next block's weights are loaded
  // before the current block computes (the loop conditions are uniform).
  int b = wave;
  if (b < nblk) {
    u32x4_t wa[kW8NT][2], wb[kW8NT][2];
    load_w(wa, b);
    while (true) {
      if (b + kW8KW >= nblk) { compute(wa, b); break; }
      load_w(wb, b + kW8KW);
      compute(wa, b);
      b += kW8KW;
      if (b + kW8KW >= nblk) { compute(wb, b); break; }
      load_w(wa, b + kW8KW);
      compute(wb, b);
      b += kW8KW;
    }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int t = 0; t < kW8NT; ++t) red[wave][t * MT + mt][lane] = acc[t][mt];
    red[wave][kW8NT * MT + mt][lane] = xs[mt];
  }
  __syncthreads();
  // One thread per (n-tile, m-tile, lane): the wave partials in wave order.
  for (int q = threadIdx.x; q < kW8NT * MT * 64; q += kW8KW * 64) {
    const int l = q & 63, tm = q >> 6;             // tm = t * MT + mt
    const int t = tm / MT, mt = tm % MT;
    f32x4_t d = red[0][tm][l], xsum = red[0][kW8NT * MT + mt][l];
    for (int ww = 1; ww < kW8KW; ++ww) {
      const f32x4_t r = red[ww][tm][l], rx = red[ww][kW8NT * MT + mt][l];
      d = f32x4_t{d[0] + r[0], d[1] + r[1], d[2] + r[2], d[3] + r[3]};
      xsum = f32x4_t{xsum[0] + rx[0], xsum[1] + rx[1], xsum[2] + rx[2], xsum[3] + rx[3]};
    }
    // lane l of n-tile t holds rows 16 mt + 4 (l / 16) + e of column 16 t + l % 16
    const int col = row0 + 16 * t + (l & 15);
    if (col >= n) continue;
    const float s = bf16_to_f32(scale[col]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * mt + 4 * (l >> 4) + e;
      if (row >= m) continue;
      const float v = (d[e] - 128.0f * xsum[e]) * s;
      if (y_f32)
        static_cast<float*>(y)[(size_t)row * n + col] = v;
      else
        static_cast<uint16_t*>(y)[(size_t)row * n + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

template <int MT>
static hipError_t launch_w8_mfma_t(const void* x, int m, const int8_t* w, const void* scale, int n, int k,
                                   void* y, int y_f32, hipStream_t stream) {
  hipLaunchKernelGGL((w8a16_mfma_kernel<MT>), dim3((n + 16 * kW8NT - 1) / (16 * kW8NT)), dim3(kW8KW * 64), 0,
                     stream, static_cast<const uint16_t*>(x), m, w, static_cast<const uint16_t*>(scale), n, k, y,
                     y_f32);
  return hipGetLastError();
}

// 5..64 rows: MT = ceil(m / 16) m-tiles, rows past m masked.
hipError_t launch_w8a16_mfma(int m, const void* x, const int8_t* w, const void* scale, int n, int k, void* y,
                             int y_f32, hipStream_t stream) {
  switch ((m + 15) / 16) {
    case 1: return launch_w8_mfma_t<1>(x, m, w, scale, n, k, y, y_f32, stream);
    case 2: return launch_w8_mfma_t<2>(x, m, w, scale, n, k, y, y_f32, stream);
    case 3: return launch_w8_mfma_t<3>(x, m, w, scale, n, k, y, y_f32, stream);
    case 4: return launch_w8_mfma_t<4>(x, m, w, scale, n, k, y, y_f32, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
