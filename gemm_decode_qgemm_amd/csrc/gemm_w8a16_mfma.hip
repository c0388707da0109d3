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
// Mapping (gfx950, wave64): a workgroup owns NT n-tiles of 16 weight rows
// and all M rows (MT m-tiles of 16); its KW waves take the BK-k blocks of
// K round robin.  In a block, lane (i, a) = (lane % 16, lane / 16) loads BK/4
// contiguous weight bytes of row 16 t + i (k = BK b + (BK/4) a .. + BK/4) and
// the same k of x row 16 mt + i; step j of BK/32 uses k = BK b + (BK/4) a +
// 8 j .. + 8 in lane group a, the same for A and B, so the steps cover the
// block's k once.  The next block's weights and activations are loaded while
// the current one computes.
// The KW partial sums meet in LDS and are added in wave order.
#include "qg_common.h"

namespace qg {

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

// One block of BK k: a lane's weight bytes (BK / 4 contiguous k of each of
// the 2 rows 16 t + i it owns) and activations (the same k of its MT rows).
template <int MT, int NT, int BK, bool PX>
struct W8Blk {
  u32x4_t w[NT][BK / 64];                        // 16 bytes = 16 k each
  u32x4_t xa[PX ? MT : 1][PX ? BK / 32 : 1];     // 8 bf16 = 8 k each (PX: loaded ahead)
};

// PX: the activations are loaded a block ahead with the weights (registers
// permitting); otherwise at the start of their block.
template <int MT, int NT, int BK, bool PX>
__global__ __launch_bounds__(kW8KW * 64) void w8a16_mfma_kernel(
    const uint16_t* __restrict__ x, int m, const int8_t* __restrict__ w,
    const uint16_t* __restrict__ scale, int n, int k, void* __restrict__ y, int y_f32) {
  constexpr int NACC = NT * MT + MT;            // per wave: the products, then X
  constexpr int KL = BK / 4;                       // k per lane group and block
  __shared__ f32x4_t red[kW8KW][NACC][64];
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, a = lane >> 4;
  const int wave = wave_id_uniform();
  const int row0 = blockIdx.x * (16 * NT);
  const int nblk = k / BK;
  const uint32_t sel_hi = __builtin_amdgcn_readfirstlane(0x07060302u);   // upper halves of (S1, S0)
  uint32_t one2 = 0x3f803f80u;           // bf16 pair (1, 1), kept in a VGPR
  asm volatile("" : "+v"(one2));
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{one2, one2, one2, one2});

  // Rows past n or m read the last row instead (a valid address); their
  // results are never stored.
  const int8_t* wr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wr[t] = w + (size_t)min(row0 + 16 * t + i, n - 1) * k + KL * a;
  const uint16_t* xr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xr[mt] = x + (size_t)min(16 * mt + i, m - 1) * k + KL * a;

  f32x4_t acc[NT][MT], xs[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    xs[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  auto load = [&](W8Blk<MT, NT, BK, PX>& u, int b) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < BK / 64; ++q)
        u.w[t][q] = load_stream<true>(reinterpret_cast<const u32x4_t*>(wr[t] + (size_t)b * BK) + q);
    if constexpr (PX) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < BK / 32; ++j)
          u.xa[mt][j] = *reinterpret_cast<const u32x4_t*>(xr[mt] + (size_t)b * BK + 8 * j);
    }
  };
  // step j: k = BK b + KL a + 8 j .. + 8 in lane group a, for A and B alike
  auto compute = [&](const W8Blk<MT, NT, BK, PX>& u, int b) {
    u32x4_t xl[PX ? 1 : MT][PX ? 1 : BK / 32];
    if constexpr (!PX) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < BK / 32; ++j)
          xl[mt][j] = *reinterpret_cast<const u32x4_t*>(xr[mt] + (size_t)b * BK + 8 * j);
    }
    auto xa = [&](int mt, int j) { return __builtin_bit_cast(bf16x8_t, PX ? u.xa[mt][j] : xl[mt][j]); };
#pragma unroll
    for (int j = 0; j < BK / 32; ++j) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4_t& q = u.w[t][j >> 1];
        const bf16x8_t bv = (j & 1) ? w8_operand(q.z, q.w, sel_hi) : w8_operand(q.x, q.y, sel_hi);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa(mt, j), bv, acc[t][mt], 0, 0, 0);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xs[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa(mt, j), ones, xs[mt], 0, 0, 0);
    }
  };

  // Two register sets used in turn: the next block's weights and activations
  // are loaded before the current block computes (uniform loop conditions).
  int b = wave;
  if (b < nblk) {
    W8Blk<MT, NT, BK, PX> ua, ub;
    load(ua, b);
    while (true) {
      if (b + kW8KW >= nblk) { compute(ua, b); break; }
      load(ub, b + kW8KW);
      compute(ua, b);
      b += kW8KW;
      if (b + kW8KW >= nblk) { compute(ub, b); break; }
      load(ua, b + kW8KW);
      compute(ub, b);
      b += kW8KW;
    }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][t * MT + mt][lane] = acc[t][mt];
    red[wave][NT * MT + mt][lane] = xs[mt];
  }
  __syncthreads();
  // One thread per (n-tile, m-tile, lane): the wave partials in wave order.
  for (int q = threadIdx.x; q < NT * MT * 64; q += kW8KW * 64) {
    const int l = q & 63, tm = q >> 6;             // tm = t * MT + mt
    const int t = tm / MT, mt = tm % MT;
    f32x4_t d = red[0][tm][l], xsum = red[0][NT * MT + mt][l];
    for (int ww = 1; ww < kW8KW; ++ww) {
      const f32x4_t r = red[ww][tm][l], rx = red[ww][NT * MT + mt][l];
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

template <int MT, int NT, int BK, bool PX>
static hipError_t launch_w8_mfma_t(const void* x, int m, const int8_t* w, const void* scale, int n, int k,
                                   void* y, int y_f32, hipStream_t stream) {
  hipLaunchKernelGGL((w8a16_mfma_kernel<MT, NT, BK, PX>), dim3((n + 16 * NT - 1) / (16 * NT)), dim3(kW8KW * 64), 0,
                     stream, static_cast<const uint16_t*>(x), m, w, static_cast<const uint16_t*>(scale), n, k, y,
                     y_f32);
  return hipGetLastError();
}

// 5..64 rows: MT = ceil(m / 16) m-tiles, rows past m masked; blocks of 128
// k.  Loading the activations a block ahead pays at 17..32 rows only
// (8192 x 8192: 28.8 us against 33.3 at 32 rows, but 30.7 against 25.0 at 16;
// 256-k blocks at 16 rows: 30.7); above 32 rows two register sets of them
// would spill.  Two n-tiles (32 weight rows) per workgroup, except at 17..32
// rows on layers of at least 32768 rows, where 64 rows per workgroup halve
// the activation reads and still leave 512 workgroups (39936 x 6656, 32 rows:
// 95.9 us against 113.9; at 8192 x 8192 the 128 workgroups of 64 rows lose at
// every M, 36.8 against 28.9 at 32 rows).  Four n-tiles above 32 rows would
// spill (256 registers per wave at 8 waves per workgroup).
hipError_t launch_w8a16_mfma(int m, const void* x, const int8_t* w, const void* scale, int n, int k, void* y,
                             int y_f32, hipStream_t stream) {
  switch ((m + 15) / 16) {
    case 1: return launch_w8_mfma_t<1, 2, 128, false>(x, m, w, scale, n, k, y, y_f32, stream);
    case 2:
      if (n >= 32768) return launch_w8_mfma_t<2, 4, 128, true>(x, m, w, scale, n, k, y, y_f32, stream);
      return launch_w8_mfma_t<2, 2, 128, true>(x, m, w, scale, n, k, y, y_f32, stream);
    case 3: return launch_w8_mfma_t<3, 2, 128, false>(x, m, w, scale, n, k, y, y_f32, stream);
    case 4: return launch_w8_mfma_t<4, 2, 128, false>(x, m, w, scale, n, k, y, y_f32, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
