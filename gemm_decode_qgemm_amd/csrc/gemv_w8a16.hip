// gemv_w8a16.hip -- int8 weight-only GEMV, y[m, n] = (sum_k x[m,k] W[n,k]) * s[n].
//
// gpt-fast issue #114 ("Question about the generated code of
// WeightOnlyInt8Linear"): WeightOnlyInt8Linear.forward is
// F.linear(x, W.to(bf16)) * scales; the report there is that an unfused
// int8 -> bf16 convert materializes a bf16 weight and wrecks the GEMV's
// bandwidth, and Chillee's fused Inductor kernel reads int8 W once, casts in
// registers and reduces along K.  Here the weight is the caller's plain
// row-major int8 [N, K] (no repacking) and the convert is fused the same way.
//
// Mapping (gfx950, wave64), for M = 1..4:
//  * K is cut into 1024-byte chunks (64 lanes x 16 bytes: every wave load is
//    8 whole 128-byte lines of one row); wave w of a workgroup owns CPW
//    consecutive chunks, so a workgroup of W waves covers all of K;
//  * each lane keeps the 16 x values of its chunks in VGPRs as bf16 pairs and
//    reuses them for every row of the workgroup's block of rows (4 at M = 1,
//    8 otherwise);
//  * a weight dword (4 int8) is XORed with 0x80808080, so each byte is w+128
//    in 1..255, v_cvt_f32_ubyte0..3 turn the bytes into exact floats, and
//    v_perm_b32 packs the upper halves of two of them into an exact bf16 pair
//    for v_dot2c_f32_bf16 (products exact, fp32 accumulation); the +128 is
//    removed once per row with the lane's precomputed 128 * sum(x);
//  * the rows of the block are taken RB at a time: the RB weight loads of a
//    wave are all in flight before any of them is used (a wave holds RB KB in
//    flight; one row at a time left a CU ~16 KB in flight, half the HBM rate);
//  * per row, a 4-step DPP reduction sums each 16-lane row of the wave, and
//    the 4 row sums of every wave meet in LDS, added in a fixed order.
#include "qg_common.h"

namespace qg {

// Rows per workgroup and rows whose loads are in flight together (RB),
// measured on MI355X at 8192 x 8192: M = 1 12.2 us with (4, 4), 12.45 with
// (8, 4), 12.4 with (8, 2) or (16, 4), 13.4 with (16, 8), 15.3 with (16, 1);
// M = 4 17.3 us with (8, 4), 17.1-17.6 with (16, 4), 20.0 with (4, 4).  At
// 39936 x 6656 (M = 1) (4, 4) and (8, 4) both stream 6.6 TB/s.
template <int M>
constexpr int kW8Rows = M == 1 ? 4 : 8;
constexpr int kW8RB = 4;
constexpr int kW8MaxWaves = 16;

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xf, 0xf, true));
}

// Sum over the 16 lanes of each DPP row; every lane of the row gets it.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp_f<0x124>(v);   // row_ror:4
  v += dpp_f<0x128>(v);   // row_ror:8
  return v;
}

template <int M, int CPW>
__global__ __launch_bounds__(kW8MaxWaves * 64) void w8a16_gemv_kernel(
    const uint16_t* __restrict__ x, const int8_t* __restrict__ w,
    const uint16_t* __restrict__ scale, int n, int k, void* __restrict__ y, int y_f32) {
  constexpr int ROWS = kW8Rows<M>;
  __shared__ float red[kW8MaxWaves][ROWS][4 * M];
  const int lane = threadIdx.x & 63;
  const int wave = wave_id_uniform();
  const int nwaves = blockDim.x >> 6;
  const int row0 = blockIdx.x * ROWS;
  const int nch = (k + 1023) >> 10;

  bool valid[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int ch = wave * CPW + c;
    valid[c] = ch < nch && ch * 1024 + lane * 16 < k;
  }

  // Weight loads of RB rows.  Rows past n load nothing and use w = 0 (byte
  // 0x80 after the xor below); their sums are never stored.
  constexpr int RB = kW8RB;
  u32x4_t wv[RB][CPW];
  auto load_rows = [&](int r0) {
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      const int row = row0 + r0 + rr;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        wv[rr][c] = u32x4_t{0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
        if (valid[c] && row < n)
          wv[rr][c] = load_stream<true>(reinterpret_cast<const u32x4_t*>(
              w + (size_t)row * k + (size_t)(wave * CPW + c) * 1024 + lane * 16));
      }
    }
  };
  // At M <= 2 the first rows' weight loads go out before the x loads, so the
  // wait for x overlaps their HBM latency instead of preceding it (8192 x 8192:
  // M = 1 12.47 us against 12.78, M = 2 13.54 against 13.92).  With more
  // activation rows the weights held across the x loads and their sums cost
  // registers, and time (M = 3: 15.85 against 15.05, M = 4: 17.8 against
  // 16.8; all 8 rows of the block in flight at once was slower still), so
  // there x comes first.
  if constexpr (M <= 2) load_rows(0);

  // x of this lane's chunks as bf16 pairs, and 128 * (their sum).
  uint32_t xr[M][CPW][8];
  float bias[M];
#pragma unroll
  for (int m = 0; m < M; ++m) bias[m] = 0.0f;
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int kb = (wave * CPW + c) * 1024 + lane * 16;   // first k of this lane in the chunk
#pragma unroll
    for (int m = 0; m < M; ++m) {
      u32x4_t a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
      if (valid[c]) {
        const u32x4_t* p = reinterpret_cast<const u32x4_t*>(x + (size_t)m * k + kb);
        a = p[0];
        b = p[1];
      }
      const uint32_t v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xr[m][c][i] = v[i];
        bias[m] += bf16_to_f32(v[i] & 0xffffu) + bf16_to_f32(v[i] >> 16);
      }
    }
  }
#pragma unroll
  for (int m = 0; m < M; ++m) bias[m] *= 128.0f;

  const uint32_t sel_hi = __builtin_amdgcn_readfirstlane(0x07060302u);  // upper halves of (S1, S0)
  for (int r0 = 0; r0 < ROWS; r0 += RB) {
    if (M > 2 || r0 > 0) load_rows(r0);
#pragma unroll
    for (int rr = 0; rr < RB; ++rr) {
      float acc[M];
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = 0.0f;
#pragma unroll
      for (int c = 0; c < CPW; ++c) {
        const uint32_t dws[4] = {wv[rr][c].x, wv[rr][c].y, wv[rr][c].z, wv[rr][c].w};
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const uint32_t u = dws[d] ^ 0x80808080u;          // each byte: w + 128
          const float f0 = (float)(u & 0xffu);            // v_cvt_f32_ubyte0..3
          const float f1 = (float)((u >> 8) & 0xffu);
          const float f2 = (float)((u >> 16) & 0xffu);
          const float f3 = (float)(u >> 24);
          const uint32_t p01 = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), sel_hi);
          const uint32_t p23 = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), sel_hi);
#pragma unroll
          for (int m = 0; m < M; ++m) {
            acc[m] = dot2_bf16(xr[m][c][2 * d], p01, acc[m]);
            acc[m] = dot2_bf16(xr[m][c][2 * d + 1], p23, acc[m]);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float v = row16_sum(acc[m] - bias[m]);
        if ((lane & 15) == 0) red[wave][r0 + rr][(lane >> 4) * M + m] = v;
      }
    }
  }
  __syncthreads();
  // One thread per (row, m): waves in order, then the 4 DPP rows in order.
  const int t = threadIdx.x;
  if (t < ROWS * M) {
    const int r = t / M, m = t % M;
    const int row = row0 + r;
    if (row < n) {
      float v = 0.0f;
      for (int ww = 0; ww < nwaves; ++ww)
        for (int q = 0; q < 4; ++q) v += red[ww][r][q * M + m];
      v *= bf16_to_f32(scale[row]);
      if (y_f32)
        static_cast<float*>(y)[(size_t)m * n + row] = v;
      else
        static_cast<uint16_t*>(y)[(size_t)m * n + row] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// Chunks per wave: the smallest of 1..4 that covers K with at most 16 waves.
int w8a16_chunks_per_wave(int k) {
  const int nch = (k + 1023) / 1024;
  for (int cpw = 1; cpw <= 4; ++cpw)
    if ((nch + cpw - 1) / cpw <= kW8MaxWaves) return cpw;
  return -1;   // K above 4 * 16 * 1024
}

template <int M, int CPW>
static hipError_t launch_w8_t(const void* x, const int8_t* w, const void* scale, int n, int k,
                              void* y, int y_f32, hipStream_t stream) {
  const int nch = (k + 1023) / 1024;
  const int waves = (nch + CPW - 1) / CPW;
  hipLaunchKernelGGL((w8a16_gemv_kernel<M, CPW>), dim3((n + kW8Rows<M> - 1) / kW8Rows<M>),
                     dim3(waves * 64), 0, stream, static_cast<const uint16_t*>(x), w,
                     static_cast<const uint16_t*>(scale), n, k, y, y_f32);
  return hipGetLastError();
}

hipError_t launch_w8a16_gemv(int m, const void* x, const int8_t* w, const void* scale, int n,
                             int k, void* y, int y_f32, hipStream_t stream) {
  const int cpw = w8a16_chunks_per_wave(k);
#define QG_W8_CASE(MM, CC) \
  if (m == MM && cpw == CC) return launch_w8_t<MM, CC>(x, w, scale, n, k, y, y_f32, stream);
#define QG_W8_M(MM) QG_W8_CASE(MM, 1) QG_W8_CASE(MM, 2) QG_W8_CASE(MM, 3) QG_W8_CASE(MM, 4)
  QG_W8_M(1) QG_W8_M(2) QG_W8_M(3) QG_W8_M(4)
#undef QG_W8_M
#undef QG_W8_CASE
  return hipErrorInvalidValue;
}

}  // namespace qg
