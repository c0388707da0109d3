// gemm_w4a16_mfma.hip -- packed INT4 group-32 weight x bf16 activations for
// M = 5..64 rows, on the matrix cores.
//
// executorch test_int4_quantized_gemm.py: buckets 8..64 run a W4A16 kernel
// (the `_W4A16_DIRECT_KERNELS` / `_W4A16_SPLIT_KERNELS` of the bucket tests);
// the result is the same "dequant + F.linear" sum as the decode GEMV.  With
// 16..64 activation rows each weight feeds enough products for the matrix
// cores to pay off.
//
// Mapping (gfx950): a workgroup = one 64-row block of the weight, 4 waves, one
// 16-row n-tile each; M is padded to MT 16-row m-tiles.  Per half tile (4
// groups, 128 k) the workgroup stages x[0:16*MT, 128 k] into LDS (double
// buffered) together with each row's 4 group sums X[m][g]; each wave then
// runs, per group, one v_mfma_f32_16x16x32_bf16 per m-tile:
//   A = x (16 m x 32 k, exact bf16), B = 128 + q (32 k x 16 n, exact bf16,
//   built from the nibbles with one shift and one and-or per pair),
// into a fresh accumulator P, and folds P into fp32 results as
//   y[m][n] += s[n,g] * (P[m][n] - (128 + zp[n,g]) * X[m][g]).
// The products are exact and the fp32 accumulation matches the decode path,
// so no bf16 rounding of dequantized weights enters the result.
#include "qg_common.h"
#include "w4_common.h"

namespace qg {

constexpr int kXRow = 128 + 8;   // LDS row of 128 bf16 plus 16 bytes of padding

template <int MT>
__global__ __launch_bounds__(256) void w4a16_mfma_kernel(
    const uint16_t* __restrict__ x, int m, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][MT * 16][kXRow];
  __shared__ __attribute__((aligned(16))) float xsum[2][4][MT * 16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = wave_id_uniform();        // n-tile of this wave
  const int b = lane & 15, a = lane >> 4;
  const int rb = blockIdx.x;
  const int kt_count = k >> 8;
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  const int s0 = 2 * t0, s1 = 2 * t1;        // half-tile range
  const uint8_t* tiles = packed + (size_t)rb * kt_count * kTileBytes;
  const int nrow = 16 * wave + b;            // this lane's weight row within the block
  const uint32_t mask_s = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t magic_v = 0x43004300u;
  asm volatile("" : "+v"(magic_v));

  // ---- x staging: chunk c = (row, 16-byte piece) of the half tile; 4
  // consecutive threads hold one group of one row.
  constexpr int kPasses = MT;                // 16*MT rows x 16 pieces / 256 threads
  u32x4_t xr[kPasses];
  auto stage_load = [&](int hs) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int c = p * 256 + tid;
      const int row = c >> 4, piece = c & 15;
      xr[p] = u32x4_t{0, 0, 0, 0};
      if (row < m)
        xr[p] = *reinterpret_cast<const u32x4_t*>(x + (size_t)row * k + (size_t)hs * 128 + piece * 8);
    }
  };
  auto stage_store = [&](int bf) {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int c = p * 256 + tid;
      const int row = c >> 4, piece = c & 15;
      *reinterpret_cast<u32x4_t*>(&xs[bf][row][piece * 8]) = xr[p];
      const u32x4_t v = xr[p];
      float sum = 0.0f;
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) sum += bf16_to_f32(w[i] & 0xffffu) + bf16_to_f32(w[i] >> 16);
      sum += dpp_mov<0xB1>(sum);             // the 4 pieces of a group: quad reduction
      sum += dpp_mov<0x4E>(sum);
      if ((piece & 3) == 0) xsum[bf][piece >> 2][row] = sum;
    }
  };

  // ---- weights of one half tile for this lane: the code dword of its
  // k-slice a for each of the 4 groups, and its row's scales / zero points.
  struct WRegs {
    uint32_t c[4];
    u32x2_t sc;
    uint32_t zw;
  };
  auto load_w = [&](WRegs& r, int hs) {
    const uint8_t* tile = tiles + (size_t)(hs >> 1) * kTileBytes;
    const int half = hs & 1;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      r.c[jj] = load_stream<true>(reinterpret_cast<const uint32_t*>(
          tile + ((4 * half + jj) * kTileRows + nrow) * 16 + 4 * a));
    r.sc = load_stream<false>(reinterpret_cast<const u32x2_t*>(tile + kScaleOff + nrow * 16 + 8 * half));
    r.zw = load_stream<false>(reinterpret_cast<const uint16_t*>(tile + kZeroOff + nrow * 4 + 2 * half));
  };

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int bf, const WRegs& r) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      uint32_t bp[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) bp[i] = nibble_pair_bf16(r.c[jj], i, mask_s, magic_v);
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, u32x4_t{bp[0], bp[1], bp[2], bp[3]});
      const uint32_t sw = (jj < 2) ? r.sc.x : r.sc.y;
      const float s = fp16_to_f32((sw >> (16 * (jj & 1))) & 0xffffu);
      const float zb = (float)(((r.zw >> (4 * jj)) & 15u) + 128u);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const u32x4_t av = *reinterpret_cast<const u32x4_t*>(&xs[bf][16 * mt + b][32 * jj + 8 * a]);
        const f32x4_t xg = *reinterpret_cast<const f32x4_t*>(&xsum[bf][jj][16 * mt + 4 * a]);
        const f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, av), bv, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[mt][e] = __builtin_fmaf(s, __builtin_fmaf(-zb, xg[e], p[e]), acc[mt][e]);
      }
    }
  };

  WRegs wc, wn;
  stage_load(s0);
  stage_store(0);
  load_w(wc, s0);
  __syncthreads();
  for (int hs = s0; hs < s1; ++hs) {
    const int bf = (hs - s0) & 1;
    const bool next = hs + 1 < s1;
    if (next) {
      stage_load(hs + 1);
      load_w(wn, hs + 1);
    }
    compute(bf, wc);
    if (next) stage_store(bf ^ 1);
    __syncthreads();
    if (next) wc = wn;
  }

  // ---- results: lane (b, a) holds rows 16*mt + 4a + e of column nrow.
  const int col = rb * kTileRows + nrow;
  if (col < n) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * mt + 4 * a + e;
        if (row < m) {
          const float v = acc[mt][e];
          if (partial != nullptr)
            partial[((size_t)blockIdx.y * m + row) * n + col] = v;
          else if (y_f32)
            static_cast<float*>(y)[(size_t)row * n + col] = v;
          else
            static_cast<uint16_t*>(y)[(size_t)row * n + col] = (uint16_t)f32_to_bf16_rne(v);
        }
      }
  }
}

template <int MT>
static hipError_t launch_mfma_t(const void* x, int m, const void* packed, int n, int k, void* y,
                                int y_f32, float* partial, int split, hipStream_t stream) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  hipLaunchKernelGGL((w4a16_mfma_kernel<MT>), dim3(rbs, split), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), m, static_cast<const uint8_t*>(packed), n, k,
                     y, y_f32, partial, split);
  return hipGetLastError();
}

hipError_t launch_w4a16_mfma(int m, const void* x, const void* packed, int n, int k, void* y,
                             int y_f32, float* partial, int split, hipStream_t stream) {
  const int mt = (m + 15) / 16;
  switch (mt) {
    case 1: return launch_mfma_t<1>(x, m, packed, n, k, y, y_f32, partial, split, stream);
    case 2: return launch_mfma_t<2>(x, m, packed, n, k, y, y_f32, partial, split, stream);
    case 3: return launch_mfma_t<3>(x, m, packed, n, k, y, y_f32, partial, split, stream);
    case 4: return launch_mfma_t<4>(x, m, packed, n, k, y, y_f32, partial, split, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qg
