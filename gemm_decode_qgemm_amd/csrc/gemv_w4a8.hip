// gemv_w4a8.hip -- decode GEMV of the packed INT4 group-32 weight against
// int8 activations, M = 1..4.
//
// executorch test_int4_quantized_gemm.py, Int4QuantizedGemmPrecisionTest:
// the decode buckets run the INT4 weight against int8 activations and are
// held to the W4A16 reference's precision class.  Each row of x is quantized
// inside the call, per row and symmetric:
//   a = max|x[m,:]|, inv = 127/a, sx = a/127 (binary32 divisions),
//   xq = clamp(rint(x * inv), -127, 127) (one binary32 multiply), a == 0 -> 0,
//   a row holding a NaN or an infinity gets sx = NaN (no finite scale), and a
//   row so small that 127/a overflows binary32 is a zero row (sx = 0, xq = 0);
// then y[m,n] = sx[m] * sum_g s[n,g] * I[m,n,g] with the exact integer group
// dot I = sum_{k in g} xq[m,k] * (q[n,k] - zp[n,g]).
//
// Kernels: M = 1 with per-row scales on the v_dot4c GEMVs below; M = 1 with
// one scale per group of 32 on w4a8_gemv_lds_kernel; M = 2..4 (both scale
// kinds) on w4a8_gemv_mx4_kernel, the 4x4x4 int8 matrix instruction.
//
// Mapping of the M = 1 v_dot4c GEMV (gfx950, wave64), as the W4A16 GEMV: one
// 64-row block per workgroup, lane = row, waves take half tiles (4 groups =
// 128 k) round robin (a 32-row variant below halves the block, as the W4A16
// one does).
//  * Prologue: the workgroup reads its x rows once for the absmax (L2-resident).
//  * Lane i of each 16-lane DPP row loads x[8i .. 8i+8) of the half tile and
//    quantizes it into two dwords of int8 in the byte order the nibbles need:
//    (w & 0x0F0F0F0F) holds the codes of k = 8d + {0,4,1,5}, ((w >> 4) &
//    0x0F0F0F0F) those of 8d + {2,6,3,7} -- so the dwords are exactly that.
//  * v_dot4c_i32_i8 multiplies a code dword by the xq dword broadcast from
//    the lane holding it (DPP row_newbcast), accumulating in int32; the zero
//    point comes off as zp * (group sum of xq), also broadcast by DPP.
#include "qg_common.h"
#include "dispatch.h"
#include "w4_common.h"

namespace qg {

// The trailing nop: a VALU read of a DPP dot result needs two wait states the
// compiler cannot see inside the asm (measured on MI355X for v_dot2c; applied
// to the integer dot as well).
#define QG_DPP_DOT4(acc, xr, wr, L) \
  "v_dot4c_i32_i8_dpp " acc ", " xr ", " wr " row_newbcast:" #L " row_mask:0xf bank_mask:0xf\n\t"
#define QG_DOT8(L0, L1, L2, L3)                                                               \
  "s_nop 1\n\t"                                                                              \
  QG_DPP_DOT4("%0", "%2", "%4", L0) QG_DPP_DOT4("%1", "%3", "%5", L0)                       \
  QG_DPP_DOT4("%0", "%2", "%6", L1) QG_DPP_DOT4("%1", "%3", "%7", L1)                       \
  QG_DPP_DOT4("%0", "%2", "%8", L2) QG_DPP_DOT4("%1", "%3", "%9", L2)                       \
  QG_DPP_DOT4("%0", "%2", "%10", L3) QG_DPP_DOT4("%1", "%3", "%11", L3)                     \
  "s_nop 2\n\t"
#define QG_DOT8_OPERANDS                                                                    \
  : "+v"(i0), "+v"(i1)                                                                      \
  : "v"(xlo), "v"(xhi), "v"(lo[0]), "v"(hi[0]), "v"(lo[1]), "v"(hi[1]), "v"(lo[2]),          \
    "v"(hi[2]), "v"(lo[3]), "v"(hi[3])

// i0 += sum_d dot4(lo[d], xq_lo @ lane 4*JJ+d); i1 likewise with the high nibbles.
template <int JJ>
__device__ __forceinline__ void group_dot4(int& i0, int& i1, uint32_t xlo, uint32_t xhi,
                                           const uint32_t (&lo)[4], const uint32_t (&hi)[4]) {
  if constexpr (JJ == 0) asm(QG_DOT8(0, 1, 2, 3) QG_DOT8_OPERANDS);
  if constexpr (JJ == 1) asm(QG_DOT8(4, 5, 6, 7) QG_DOT8_OPERANDS);
  if constexpr (JJ == 2) asm(QG_DOT8(8, 9, 10, 11) QG_DOT8_OPERANDS);
  if constexpr (JJ == 3) asm(QG_DOT8(12, 13, 14, 15) QG_DOT8_OPERANDS);
}

template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, true);
}

// The absmax keeps a NaN: nmax is the IEEE 754-2019 maximum (one
// v_maximum3_f32 on gfx950), which returns NaN when either input is NaN,
// where fmaxf would return the other input.  An infinity survives any max.
__device__ __forceinline__ float nmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// A span whose absmax is not finite (it holds a NaN or an infinity) has no
// finite scale: its absmax becomes NaN, which gives inv = 0 through
// a > 0 ? 127 / a : 0 and sx = a / 127 = NaN, so every output the span
// reaches is NaN.
__device__ __forceinline__ float finite_or_nan(float a) {
  return a < __builtin_inff() ? a : __builtin_nanf("");
}

// The span's scales from its absmax a (>= 0, or NaN as above): inv = 127 / a
// and sx = a / 127, both correctly rounded binary32 divisions.  Where 127 / a
// is not a finite binary32 number there is no inverse scale and inv = 0, so
// every code is 0: for a == 0 and for a span so small that the quotient
// overflows (a <= 127 * 2^-128), sx = 0 as well (a zero span, outputs 0); for
// a NaN absmax sx stays NaN.
__device__ __forceinline__ void span_scale(float a, float& inv, float& sx) {
  inv = 127.0f / a;
  sx = a / 127.0f;
  if (!(inv <= __FLT_MAX__)) {
    inv = 0.0f;
    if (a == a) sx = 0.0f;
  }
}

// Quantize 8 bf16 (one 16-byte load) to int8 with the row's inverse scale,
// packed as (q0,q4,q1,q5) and (q2,q6,q3,q7).
__device__ __forceinline__ void quant8(const u32x4_t& v, float inv, uint32_t& xlo, uint32_t& xhi) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  int q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float f = bf16_to_f32(h ? (w[i] >> 16) : (w[i] & 0xffffu));
      float t = rintf(f * inv);
      t = __builtin_amdgcn_fmed3f(t, -127.0f, 127.0f);
      q[2 * i + h] = (int)t;
    }
  }
  auto b = [&](int i) { return (uint32_t)q[i] & 0xffu; };
  xlo = b(0) | (b(4) << 8) | (b(1) << 16) | (b(5) << 24);
  xhi = b(2) | (b(6) << 8) | (b(3) << 16) | (b(7) << 24);
}

template <int M, int JJ>
__device__ __forceinline__ void do_group_a8(float (&acc)[M], const HalfRegs& cur,
                                            const uint32_t (&xlo)[M], const uint32_t (&xhi)[M],
                                            const int (&sxq)[M], uint32_t nib_s) {
  const u32x4_t cv = cur.c[JJ];
  const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    lo[d] = cw[d] & nib_s;
    hi[d] = (cw[d] >> 4) & nib_s;
  }
  const uint32_t sw = (JJ < 2) ? cur.sc.x : cur.sc.y;
  const float s = fp16_to_f32((sw >> (16 * (JJ & 1))) & 0xffffu);
  const int zp = (int)((cur.zw >> (4 * JJ)) & 15u);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    int i0 = 0, i1 = 0;
    group_dot4<JJ>(i0, i1, xlo[m], xhi[m], lo, hi);
    const int sg = dpp_i<0x150 + 4 * JJ>(sxq[m]);   // group sum of xq to every lane
    const int ig = i0 + i1 - zp * sg;                // exact: |ig| <= 32*127*15
    acc[m] = __builtin_fmaf(s, (float)ig, acc[m]);
  }
}

template <int M, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void w4a8_gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split) {
  __shared__ float red[WAVES * M * 64];
  __shared__ float amax_w[WAVES][M];
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int wave = wave_id_uniform();
  const int rb = blockIdx.x;
  const int kt_count = k >> 8;
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  const uint8_t* tiles = packed + (size_t)rb * kt_count * kTileBytes;

  // Per-row absmax of x over the whole K (every split needs the same scale).
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float a = 0.0f;
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (size_t)m * k);
    for (int i = threadIdx.x; i < (k >> 3); i += WAVES * 64) {
      const u32x4_t v = xr[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a = nmax(a, fabsf(bf16_to_f32(w[j] & 0xffffu)));
        a = nmax(a, fabsf(bf16_to_f32(w[j] >> 16)));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a = nmax(a, __shfl_xor(a, off, 64));
    if (lane == 0) amax_w[wave][m] = a;
  }
  __syncthreads();
  float inv[M], sx[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float a = amax_w[0][m];
    for (int ww = 1; ww < WAVES; ++ww) a = nmax(a, amax_w[ww][m]);
    span_scale(finite_or_nan(a), inv[m], sx[m]);
  }

  const uint32_t nib_s = __builtin_amdgcn_readfirstlane(0x0F0F0F0Fu);
  uint32_t ones_v = 0x01010101u;
  asm volatile("" : "+v"(ones_v));   // int8 ones in a VGPR, not a literal operand

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  for (int hs = 2 * t0 + wave; hs < 2 * t1; hs += WAVES) {
    HalfRegs r;
    load_half(r, tiles + (size_t)(hs >> 1) * kTileBytes, hs & 1, lane);
    uint32_t xlo[M], xhi[M];
    int sxq[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + (size_t)m * k + (size_t)hs * 128 + li * 8);
      quant8(v, inv[m], xlo[m], xhi[m]);
      // sum of this lane's 8 xq, then over the 4 lanes of its group
      int p = __builtin_amdgcn_sdot4((int)xlo[m], (int)ones_v, 0, false);
      p = __builtin_amdgcn_sdot4((int)xhi[m], (int)ones_v, p, false);
      p += dpp_i<0xB1>(p);
      p += dpp_i<0x4E>(p);
      sxq[m] = p;
    }
    do_group_a8<M, 0>(acc, r, xlo, xhi, sxq, nib_s);
    do_group_a8<M, 1>(acc, r, xlo, xhi, sxq, nib_s);
    do_group_a8<M, 2>(acc, r, xlo, xhi, sxq, nib_s);
    do_group_a8<M, 3>(acc, r, xlo, xhi, sxq, nib_s);
  }

#pragma unroll
  for (int m = 0; m < M; ++m) red[(wave * M + m) * 64 + lane] = acc[m];
  __syncthreads();
  for (int m = wave; m < M; m += WAVES) {
    float v = red[m * 64 + lane];
    for (int ww = 1; ww < WAVES; ++ww) v += red[(ww * M + m) * 64 + lane];
    const int row = rb * kTileRows + lane;
    if (row < n) {
      if (partial != nullptr) {
        // split partials stay in the unscaled integer-group domain times s;
        // the activation scale is the same for every split, applied here
        partial[((size_t)blockIdx.y * M + m) * n + row] = v * sx[m];
      } else {
        v *= sx[m];
        if (y_f32)
          static_cast<float*>(y)[(size_t)m * n + row] = v;
        else
          static_cast<uint16_t*>(y)[(size_t)m * n + row] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
  }
}

// 32-row variant (the mapping of Half32Regs): lanes 0-31 take groups {0,1}
// of each half tile, lanes 32-63 groups {2,3}, for the same 32 rows.  Each
// DPP row holds its lane half's 64 k: lane i quantizes the 8-k segment i % 8,
// so the code dword d of local group jj meets the xq of lane 4*jj + d, as in
// group_dot4<0> and group_dot4<1> above (lanes 8-15 repeat lanes 0-7).
template <int M, int JJ>
__device__ __forceinline__ void do_group_a8_32(float (&acc)[M], const Half32Regs& cur,
                                               const uint32_t (&xlo)[M], const uint32_t (&xhi)[M],
                                               const int (&sxq)[M], uint32_t nib_s, float s) {
  const u32x4_t cv = cur.c[JJ];
  const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
  uint32_t lo[4], hi[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    lo[d] = cw[d] & nib_s;
    hi[d] = (cw[d] >> 4) & nib_s;
  }
  const int zp = (int)((cur.zb >> (4 * JJ)) & 15u);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    int i0 = 0, i1 = 0;
    group_dot4<JJ>(i0, i1, xlo[m], xhi[m], lo, hi);
    const int sg = dpp_i<0x150 + 4 * JJ>(sxq[m]);   // group sum of xq to every lane
    const int ig = i0 + i1 - zp * sg;                // exact: |ig| <= 32*127*15
    acc[m] = __builtin_fmaf(s, (float)ig, acc[m]);
  }
}

template <int M, int WAVES, bool DQ = false>
__global__ __launch_bounds__(WAVES * 64) void w4a8_gemv32_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split) {
  __shared__ float red[WAVES * M * 64];
  __shared__ float amax_w[WAVES][M];
  const int lane = threadIdx.x & 63;
  const int seg = lane & 7;                        // 8-k segment of this lane's 64-k window
  const int lg = lane >> 5;                        // group pair of this lane
  const int wave = wave_id_uniform();
  const int rb = blockIdx.x >> 1;                  // 64-row block
  const int row = 32 * (blockIdx.x & 1) + (lane & 31);
  const int kt_count = k >> 8;
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  using L = W4Layout<DQ>;
  float step;
  const uint8_t* tiles = L::tiles(packed, rb, kt_count, row, step);

  // Per-row absmax of x over the whole K (every split needs the same scale).
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float a = 0.0f;
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (size_t)m * k);
    for (int i = threadIdx.x; i < (k >> 3); i += WAVES * 64) {
      const u32x4_t v = xr[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a = nmax(a, fabsf(bf16_to_f32(w[j] & 0xffffu)));
        a = nmax(a, fabsf(bf16_to_f32(w[j] >> 16)));
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) a = nmax(a, __shfl_xor(a, off, 64));
    if (lane == 0) amax_w[wave][m] = a;
  }
  __syncthreads();
  float inv[M], sx[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float a = amax_w[0][m];
    for (int ww = 1; ww < WAVES; ++ww) a = nmax(a, amax_w[ww][m]);
    span_scale(finite_or_nan(a), inv[m], sx[m]);
  }

  const uint32_t nib_s = __builtin_amdgcn_readfirstlane(0x0F0F0F0Fu);
  uint32_t ones_v = 0x01010101u;
  asm volatile("" : "+v"(ones_v));   // int8 ones in a VGPR, not a literal operand

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  for (int hs = 2 * t0 + wave; hs < 2 * t1; hs += WAVES) {
    Half32Regs r;
    L::load(r, tiles + (size_t)(hs >> 1) * L::kTile, hs & 1, lg, row);
    uint32_t xlo[M], xhi[M];
    int sxq[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + (size_t)m * k + (size_t)hs * 128 +
                                                          64 * lg + 8 * seg);
      quant8(v, inv[m], xlo[m], xhi[m]);
      // sum of this lane's 8 xq, then over the 4 lanes of its group
      int p = __builtin_amdgcn_sdot4((int)xlo[m], (int)ones_v, 0, false);
      p = __builtin_amdgcn_sdot4((int)xhi[m], (int)ones_v, p, false);
      p += dpp_i<0xB1>(p);
      p += dpp_i<0x4E>(p);
      sxq[m] = p;
    }
    do_group_a8_32<M, 0>(acc, r, xlo, xhi, sxq, nib_s, L::scale(r.sc, 0, step));
    do_group_a8_32<M, 1>(acc, r, xlo, xhi, sxq, nib_s, L::scale(r.sc, 1, step));
  }

  // Sum over waves and over the two lane halves (same row), in a fixed order.
#pragma unroll
  for (int m = 0; m < M; ++m) red[(wave * M + m) * 64 + lane] = acc[m];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 32 * M) {
    const int m = t >> 5, l = t & 31;
    float v = 0.0f;
    for (int w = 0; w < WAVES; ++w) {
      v += red[(w * M + m) * 64 + l];
      v += red[(w * M + m) * 64 + l + 32];
    }
    const int col = rb * kTileRows + 32 * (blockIdx.x & 1) + l;
    if (col < n) {
      // split partials carry the activation scale already (the same for every split)
      v *= sx[m];
      if (partial != nullptr)
        partial[((size_t)blockIdx.y * M + m) * n + col] = v;
      else if (y_f32)
        static_cast<float*>(y)[(size_t)m * n + col] = v;
      else
        static_cast<uint16_t*>(y)[(size_t)m * n + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------------------
// One activation scale per group of 32, M = 1: activations quantized once per
// workgroup, through LDS (32 rows, 16 waves).  The workgroup walks its K range
// in chunks of 16 half tiles (2048 k), one half tile per wave.  For each chunk
// every thread quantizes one 8-k segment of x into LDS (int8 in the byte
// order of the nibbles, as quant8): the 4 segments of a group are held by a
// lane quad, whose DPP max gives the group's absmax; then inv = 127 / a and
// sx = a / 127 (binary32 divisions).  After one barrier each wave runs the
// integer group dots of its half tile reading xq from LDS and scales each
// group's sum by sx * s.  The chunk buffers alternate, so one barrier per
// chunk orders both the writes before the reads and the reads before the
// rewrite.
constexpr int kA8Chunk = 16;                 // half tiles per chunk
constexpr int kA8Segs = kA8Chunk * 16;       // 8-k segments per chunk

template <int CTRL>
__device__ __forceinline__ float dpp_fa(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xf, 0xf, true));
}

template <int M, bool DQ = false>
__global__ __launch_bounds__(1024) void w4a8_gemv_lds_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split) {
  constexpr int WAVES = 16;
  __shared__ u32x2_t xq_s[2][M][kA8Segs];
  __shared__ float sx_s[2][M][kA8Segs / 4];
  __shared__ float red[WAVES * M * 64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int seg = lane & 7;
  const int lg = lane >> 5;
  const int wave = wave_id_uniform();
  const int rb = blockIdx.x >> 1;
  const int row = 32 * (blockIdx.x & 1) + (lane & 31);
  const int kt_count = k >> 8;
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  using L = W4Layout<DQ>;
  float step;
  const uint8_t* tiles = L::tiles(packed, rb, kt_count, row, step);

  const uint32_t nib_s = __builtin_amdgcn_readfirstlane(0x0F0F0F0Fu);
  uint32_t ones_v = 0x01010101u;
  asm volatile("" : "+v"(ones_v));

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  const int h0 = 2 * t0, h1 = 2 * t1;
  for (int cb = h0, buf = 0; cb < h1; cb += kA8Chunk, buf ^= 1) {
    const int nh = min(kA8Chunk, h1 - cb);       // half tiles in this chunk
    const int hs = cb + wave;                     // this wave's half tile
    Half32Regs r;
    if (wave < nh) L::load(r, tiles + (size_t)(hs >> 1) * L::kTile, hs & 1, lg, row);

    // ---- quantize the chunk: thread -> (m, segment); a chunk's segment count
    // is a multiple of 16, so lane quads are whole for the DPP max.
    {
      const int m = tid >> 8, sg = tid & (kA8Segs - 1);
      if (m < M && sg < nh * 16) {
        const u32x4_t v = *reinterpret_cast<const u32x4_t*>(x + (size_t)m * k + (size_t)cb * 128 + sg * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          a = nmax(a, fabsf(bf16_to_f32(w[j] & 0xffffu)));
          a = nmax(a, fabsf(bf16_to_f32(w[j] >> 16)));
        }
        a = nmax(a, dpp_fa<0xB1>(a));          // the lane quad holds one group of 32
        float inv, sxv;
        span_scale(finite_or_nan(nmax(a, dpp_fa<0x4E>(a))), inv, sxv);
        uint32_t lo, hi;
        quant8(v, inv, lo, hi);
        xq_s[buf][m][sg] = u32x2_t{lo, hi};
        if ((sg & 3) == 0) sx_s[buf][m][sg >> 2] = sxv;
      }
    }
    __syncthreads();

    if (wave < nh) {
      const int sl = wave * 16 + lg * 8 + seg;       // this lane's segment within the chunk
      uint32_t xlo[M], xhi[M];
      int sxq[M];
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const u32x2_t q = xq_s[buf][m][sl];
        xlo[m] = q.x;
        xhi[m] = q.y;
        int p = __builtin_amdgcn_sdot4((int)xlo[m], (int)ones_v, 0, false);
        p = __builtin_amdgcn_sdot4((int)xhi[m], (int)ones_v, p, false);
        p += dpp_i<0xB1>(p);
        p += dpp_i<0x4E>(p);
        sxq[m] = p;
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const u32x4_t cv = r.c[jj];
        const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          lo[d] = cw[d] & nib_s;
          hi[d] = (cw[d] >> 4) & nib_s;
        }
        const float s = L::scale(r.sc, jj, step);
        const int zp = (int)((r.zb >> (4 * jj)) & 15u);
#pragma unroll
        for (int m = 0; m < M; ++m) {
          int i0 = 0, i1 = 0;
          if (jj == 0)
            group_dot4<0>(i0, i1, xlo[m], xhi[m], lo, hi);
          else
            group_dot4<1>(i0, i1, xlo[m], xhi[m], lo, hi);
          const int sg = jj == 0 ? dpp_i<0x150>(sxq[m]) : dpp_i<0x154>(sxq[m]);
          const int ig = i0 + i1 - zp * sg;
          const float scale = s * sx_s[buf][m][wave * 4 + lg * 2 + jj];
          acc[m] = __builtin_fmaf(scale, (float)ig, acc[m]);
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < M; ++m) red[(wave * M + m) * 64 + lane] = acc[m];
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 32 * M) {
    const int m = t >> 5, l = t & 31;
    float v = 0.0f;
    for (int w = 0; w < WAVES; ++w) {
      v += red[(w * M + m) * 64 + l];
      v += red[(w * M + m) * 64 + l + 32];
    }
    const int col = rb * kTileRows + 32 * (blockIdx.x & 1) + l;
    if (col < n) {
      if (partial != nullptr)
        partial[((size_t)blockIdx.y * M + m) * n + col] = v;
      else if (y_f32)
        static_cast<float*>(y)[(size_t)m * n + col] = v;
      else
        static_cast<uint16_t*>(y)[(size_t)m * n + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ---------------------------------------------------------------------------
// Group dots on v_mfma_i32_4x4x4_16b_i8 (as gemv_w4a16_mx4.hip does for bf16),
// with the 32-row mapping of w4a8_gemv32_kernel and no barrier in the loop.
// Per half tile, a wave quantizes the M x 128 activations itself, one 8-k
// segment per lane (lane l < 16 M: row l / 16, segment l % 16, so each group
// of 32 is a lane quad), and leaves in a wave-private LDS slot the int8 codes
// (in quant8's byte order), each group's sum of xq and, per group of 32, its
// sx.  Then per group: A = xq (row i = activation row m, in lane 4b+i), B =
// the lane's own codes (lane 4b+j = weight row): a code dword gives two 4-k
// steps, (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F), whose byte order
// quant8 matches, so a group is 8 instructions with exact int32
// accumulation, D[m] in element m of the lane; the zero point is one integer
// multiply-add per activation row.  The cost per weight does not grow with M.
__device__ __forceinline__ i32x4_t mfma_i8_4x4x4(uint32_t a, uint32_t b, i32x4_t c) {
  return __builtin_amdgcn_mfma_i32_4x4x4i8((int)a, (int)b, c, 0, 0, 0);
}

// xq rows in a wave's slot are 144 bytes apart (16 segments of 8 bytes plus
// 16): an A-operand read touches (row i, group pair) chunks at 144 i + 64 pair
// bytes, distinct 16-byte positions modulo 128 and 256 bytes (disjoint banks).
constexpr int kA8XRowBytes = 144;

// max(a, |x|) over the 8 bf16 of a 16-byte load, keeping a NaN.
__device__ __forceinline__ float absmax8(const u32x4_t& v, float a) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    a = nmax(a, fabsf(bf16_to_f32(w[j] & 0xffffu)));
    a = nmax(a, fabsf(bf16_to_f32(w[j] >> 16)));
  }
  return a;
}

// R64: one 64-row block per workgroup (lane = row; each lane loads both group
// pairs of its row and takes the half tile's 4 groups in turn), one workgroup
// per CU, so 128 VGPRs and two register sets used in turn: the next half
// tile's loads are in flight while the current one is computed (the grids it
// is used on are in dispatch.h, gemv_shape).
template <int M, bool GS, bool DQ = false, bool R64 = false>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(R64 ? 4 : 8))) void w4a8_gemv_mx4_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split) {
  constexpr int WAVES = 16;
  __shared__ __attribute__((aligned(16))) uint8_t xq_s[WAVES][M * kA8XRowBytes];
  __shared__ __attribute__((aligned(16))) int gsum_s[WAVES][4][4];          // [group][m]
  __shared__ __attribute__((aligned(16))) float gsx_s[WAVES][GS ? 4 : 1][4];
  __shared__ float red[WAVES * M * 64];
  __shared__ float amax_w[WAVES][M];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int lg = R64 ? 0 : lane >> 5;              // group pair (R64: both, in turn)
  const int xrow = (lane & 3) < M ? (lane & 3) : M - 1;   // A row of this lane
  const int wave = wave_id_uniform();
  const int rb = R64 ? blockIdx.x : blockIdx.x >> 1;
  const int row = R64 ? lane : 32 * (blockIdx.x & 1) + (lane & 31);
  const int kt_count = k >> 8;
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  using L = W4Layout<DQ>;
  constexpr int NP = R64 ? 2 : 1;   // group pairs per lane
  float step;
  const uint8_t* tiles = L::tiles(packed, rb, kt_count, row, step);
  // Quantizing lanes: l < 16 M takes k = 8 (l % 16) .. + 8 of x row l / 16.
  const bool qlane = lane < 16 * M;
  const int qm = qlane ? lane >> 4 : 0, qs = lane & 15;
  const uint16_t* xsrc = x + (size_t)qm * k + 8 * qs;
  uint8_t* const slot = xq_s[wave];

  int hs = 2 * t0 + wave;
  const int h_end = 2 * t1;
  Half32Regs r[NP];
  auto load_w = [&](Half32Regs (&rr)[NP], int h) {   // tile h/2, half h%2
#pragma unroll
    for (int p = 0; p < NP; ++p) L::load(rr[p], tiles + (size_t)(h >> 1) * L::kTile, h & 1, lg + p, row);
  };
  auto load_x = [&](int h) {
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (qlane) v = *reinterpret_cast<const u32x4_t*>(xsrc + (size_t)h * 128);
    return v;
  };
  float inv_q = 0.0f, sx_row[M];
  if constexpr (!GS) {
    // Per-row absmax over the whole row (the workgroup reads x once from L2).
    // The first pass of x loads goes out first, then the first half tile's
    // weight loads, so the wait for x does not wait for HBM and the weight
    // loads stay in flight through the reduction and its barrier.
    const int k8 = k >> 3;
    u32x4_t v0[M];
    // Threads past the row's end re-read its first 8 values (k8 >= 32), which
    // leaves the maximum unchanged and needs no branch.
    const int i0 = tid < k8 ? tid : 0;
#pragma unroll
    for (int m = 0; m < M; ++m) v0[m] = reinterpret_cast<const u32x4_t*>(x + (size_t)m * k)[i0];
    // Unconditional (a branch here makes the compiler wait for these loads
    // with the x loads): a wave without a half tile loads the range's last
    // one, which another wave reads as well (an L2 hit), and discards it.
    load_w(r, hs < h_end ? hs : h_end - 1);
    float am[M];
#pragma unroll
    for (int m = 0; m < M; ++m) am[m] = absmax8(v0[m], 0.0f);
#pragma unroll
    for (int m = 0; m < M; ++m)
      for (int i = tid + WAVES * 64; i < k8; i += WAVES * 64)
        am[m] = absmax8(reinterpret_cast<const u32x4_t*>(x + (size_t)m * k)[i], am[m]);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      // wave max: the 16-lane rows by DPP, then the four row maxima
      float a = am[m];
      a = nmax(a, dpp_fa<0xB1>(a));    // quad_perm [1,0,3,2]
      a = nmax(a, dpp_fa<0x4E>(a));    // quad_perm [2,3,0,1]
      a = nmax(a, dpp_fa<0x124>(a));   // row_ror:4
      a = nmax(a, dpp_fa<0x128>(a));   // row_ror:8
      const int ai = __float_as_int(a);
      a = nmax(nmax(__int_as_float(__builtin_amdgcn_readlane(ai, 0)),
                      __int_as_float(__builtin_amdgcn_readlane(ai, 16))),
                nmax(__int_as_float(__builtin_amdgcn_readlane(ai, 32)),
                      __int_as_float(__builtin_amdgcn_readlane(ai, 48))));
      if (lane == 0) amax_w[wave][m] = a;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float a = amax_w[0][m];
      for (int ww = 1; ww < WAVES; ++ww) a = nmax(a, amax_w[ww][m]);
      float inv_m;
      span_scale(finite_or_nan(a), inv_m, sx_row[m]);
      if (m == qm) inv_q = inv_m;
    }
  } else {
    if (hs < h_end) load_w(r, hs);
  }

  const uint32_t nib_s = __builtin_amdgcn_readfirstlane(0x0F0F0F0Fu);
  uint32_t ones_v = 0x01010101u;
  asm volatile("" : "+v"(ones_v));

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  auto compute = [&](const Half32Regs (&rr)[NP], const u32x4_t& v) {
    // ---- quantize this lane's segment; the quad holds one group of 32.
    float inv = inv_q, sxv = 0.0f;
    if constexpr (GS) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        a = nmax(a, fabsf(bf16_to_f32(w[j] & 0xffffu)));
        a = nmax(a, fabsf(bf16_to_f32(w[j] >> 16)));
      }
      a = nmax(a, dpp_fa<0xB1>(a));
      span_scale(finite_or_nan(nmax(a, dpp_fa<0x4E>(a))), inv, sxv);
    }
    uint32_t lo, hi;
    quant8(v, inv, lo, hi);
    int p = __builtin_amdgcn_sdot4((int)lo, (int)ones_v, 0, false);
    p = __builtin_amdgcn_sdot4((int)hi, (int)ones_v, p, false);
    p += dpp_i<0xB1>(p);                           // group sum of xq over the quad
    p += dpp_i<0x4E>(p);
    // The slot is private to the wave and a wave's LDS operations complete in
    // order (see gemv_w4a16_mx4.hip); the fences keep the compiler from moving
    // LDS accesses across.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (qlane) {
      *reinterpret_cast<u32x2_t*>(slot + qm * kA8XRowBytes + 8 * qs) = u32x2_t{lo, hi};
      if ((qs & 3) == 0) {
        gsum_s[wave][qs >> 2][qm] = p;
        if constexpr (GS) gsx_s[wave][qs >> 2][qm] = sxv;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int g = 2 * (lg + p) + jj;             // group within the half tile
      const Half32Regs& r = rr[p];
      const uint8_t* xp = slot + xrow * kA8XRowBytes + 32 * g;
      const u32x4_t xa0 = *reinterpret_cast<const u32x4_t*>(xp);
      const u32x4_t xa1 = *reinterpret_cast<const u32x4_t*>(xp + 16);
      const uint32_t xa[8] = {xa0.x, xa0.y, xa0.z, xa0.w, xa1.x, xa1.y, xa1.z, xa1.w};
      const u32x4_t cv = r.c[jj];
      const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
      i32x4_t d = {0, 0, 0, 0};
#pragma unroll
      for (int dd = 0; dd < 4; ++dd) {
        d = mfma_i8_4x4x4(xa[2 * dd], cw[dd] & nib_s, d);
        d = mfma_i8_4x4x4(xa[2 * dd + 1], (cw[dd] >> 4) & nib_s, d);
      }
      const i32x4_t sg = *reinterpret_cast<const i32x4_t*>(&gsum_s[wave][g][0]);
      const float s = L::scale(r.sc, jj, step);
      const int zp = (int)((r.zb >> (4 * jj)) & 15u);
      f32x4_t sxg = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (GS) sxg = *reinterpret_cast<const f32x4_t*>(&gsx_s[wave][g][0]);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const int ig = d[m] - zp * sg[m];          // exact: |ig| <= 32*127*15
        const float scale = GS ? s * sxg[m] : s;
        acc[m] = __builtin_fmaf(scale, (float)ig, acc[m]);
      }
    }
  };

  if constexpr (!R64) {
    for (bool first = true; hs < h_end; hs += WAVES, first = false) {
      if (!first) load_w(r, hs);
      compute(r, load_x(hs));
    }
  } else if (hs < h_end) {                         // uniform; r holds half tile hs
    Half32Regs r2[NP];
    u32x4_t va = load_x(hs), vb;
    __builtin_amdgcn_sched_barrier(0);
    while (true) {
      if (hs + WAVES >= h_end) { compute(r, va); break; }
      load_w(r2, hs + WAVES);
      vb = load_x(hs + WAVES);
      __builtin_amdgcn_sched_barrier(0);
      compute(r, va);
      hs += WAVES;
      if (hs + WAVES >= h_end) { compute(r2, vb); break; }
      load_w(r, hs + WAVES);
      va = load_x(hs + WAVES);
      __builtin_amdgcn_sched_barrier(0);
      compute(r2, vb);
      hs += WAVES;
    }
  }

#pragma unroll
  for (int m = 0; m < M; ++m) red[(wave * M + m) * 64 + lane] = acc[m];
  __syncthreads();
  const int t = threadIdx.x;
  constexpr int RW = R64 ? 64 : 32;   // output rows of the workgroup
  if (t < RW * M) {
    const int m = t / RW, l = t % RW;
    float v = 0.0f;
    for (int w = 0; w < WAVES; ++w) {
      v += red[(w * M + m) * 64 + l];
      if constexpr (!R64) v += red[(w * M + m) * 64 + l + 32];
    }
    const int col = R64 ? rb * kTileRows + l : rb * kTileRows + 32 * (blockIdx.x & 1) + l;
    if (col < n) {
      if constexpr (!GS) v *= sx_row[m];
      if (partial != nullptr)
        partial[((size_t)blockIdx.y * M + m) * n + col] = v;
      else if (y_f32)
        static_cast<float*>(y)[(size_t)m * n + col] = v;
      else
        static_cast<uint16_t*>(y)[(size_t)m * n + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

template <int M, bool GS, bool DQ = false>
static hipError_t launch_w4a8_mx4_t(const void* x, const void* packed, int n, int k, void* y,
                                    int y_f32, float* partial, int split, hipStream_t stream) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  if (gemv_shape(M, n, split).rows == 64)
    hipLaunchKernelGGL((w4a8_gemv_mx4_kernel<M, GS, DQ, true>), dim3(rbs, split), dim3(1024), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(packed), n, k,
                       y, y_f32, partial, split);
  else
    hipLaunchKernelGGL((w4a8_gemv_mx4_kernel<M, GS, DQ>), dim3(2 * rbs, split), dim3(1024), 0, stream,
                       static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(packed), n, k,
                       y, y_f32, partial, split);
  return hipGetLastError();
}

hipError_t launch_w4a8_gemv_mx4(int m, bool group_scales, const void* x, const void* packed, int n,
                                int k, void* y, int y_f32, float* partial, int split,
                                hipStream_t stream) {
#define QG_A8X(MM)                                                                              \
  if (m == MM)                                                                                  \
    return group_scales ? launch_w4a8_mx4_t<MM, true>(x, packed, n, k, y, y_f32, partial, split, stream) \
                        : launch_w4a8_mx4_t<MM, false>(x, packed, n, k, y, y_f32, partial, split, stream);
  QG_A8X(2) QG_A8X(3) QG_A8X(4)
#undef QG_A8X
  return hipErrorInvalidValue;
}

template <int M, bool DQ = false>
static hipError_t launch_w4a8_lds_t(const void* x, const void* packed, int n, int k, void* y,
                                    int y_f32, float* partial, int split, hipStream_t stream) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  hipLaunchKernelGGL((w4a8_gemv_lds_kernel<M, DQ>), dim3(2 * rbs, split), dim3(1024), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(packed), n, k,
                     y, y_f32, partial, split);
  return hipGetLastError();
}

hipError_t launch_w4a8_gemv_lds(int m, bool group_scales, const void* x, const void* packed, int n,
                                int k, void* y, int y_f32, float* partial, int split,
                                hipStream_t stream) {
  // Only M = 1 with one scale per group runs here: M = 2..4 run on
  // w4a8_gemv_mx4_kernel, M = 1 per-row scales on w4a8_gemv32_kernel.
  if (m == 1 && group_scales) return launch_w4a8_lds_t<1>(x, packed, n, k, y, y_f32, partial, split, stream);
  return hipErrorInvalidValue;
}

template <int M, int WAVES, bool DQ = false>
static hipError_t launch_w4a8_32_t(const void* x, const void* packed, int n, int k, void* y,
                                   int y_f32, float* partial, int split, hipStream_t stream) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  hipLaunchKernelGGL((w4a8_gemv32_kernel<M, WAVES, DQ>), dim3(2 * rbs, split), dim3(WAVES * 64), 0,
                     stream, static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(packed),
                     n, k, y, y_f32, partial, split);
  return hipGetLastError();
}

template <int M, int WAVES>
static hipError_t launch_w4a8_t(const void* x, const void* packed, int n, int k, void* y,
                                int y_f32, float* partial, int split, hipStream_t stream) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  hipLaunchKernelGGL((w4a8_gemv_kernel<M, WAVES>), dim3(rbs, split), dim3(WAVES * 64), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(packed), n, k,
                     y, y_f32, partial, split);
  return hipGetLastError();
}

hipError_t launch_w4a8_gemv(int m, const void* x, const void* packed, int n, int k, void* y,
                            int y_f32, float* partial, int split, int rows, int waves,
                            hipStream_t stream) {
#define QG_A8_CASE(MM, WW)                                                                      \
  if (m == MM && waves == WW)                                                                   \
    return rows == 32 ? launch_w4a8_32_t<MM, WW>(x, packed, n, k, y, y_f32, partial, split, stream) \
                      : launch_w4a8_t<MM, WW>(x, packed, n, k, y, y_f32, partial, split, stream);
  // M = 1 only: M = 2..4 run on w4a8_gemv_mx4_kernel.
#define QG_A8_M(MM) QG_A8_CASE(MM, 16)
  QG_A8_M(1)
#undef QG_A8_M
#undef QG_A8_CASE
  return hipErrorInvalidValue;
}

// The scale-code layout (version 2): the 32-row kernels above reading it
// through W4Layout<true>; M = 1 per row on w4a8_gemv32_kernel, M = 1 per
// group on w4a8_gemv_lds_kernel, M = 2..4 on w4a8_gemv_mx4_kernel.
hipError_t launch_w4a8_dq(int m, bool group_scales, const void* x, const void* packed, int n, int k,
                          void* y, int y_f32, float* partial, int split, hipStream_t stream) {
  if (m == 1)
    return group_scales ? launch_w4a8_lds_t<1, true>(x, packed, n, k, y, y_f32, partial, split, stream)
                        : launch_w4a8_32_t<1, 16, true>(x, packed, n, k, y, y_f32, partial, split, stream);
#define QG_A8D(MM)                                                                                       \
  if (m == MM)                                                                                           \
    return group_scales ? launch_w4a8_mx4_t<MM, true, true>(x, packed, n, k, y, y_f32, partial, split, stream) \
                        : launch_w4a8_mx4_t<MM, false, true>(x, packed, n, k, y, y_f32, partial, split, stream);
  QG_A8D(2) QG_A8D(3) QG_A8D(4)
#undef QG_A8D
  return hipErrorInvalidValue;
}


// ---------------------------------------------------------------------------
// Per-row scales at 5..64 rows, on the bf16 matrix-core kernels.  xq is an
// integer in [-127, 127], exact in bf16, so the matrix-core kernel run on xq
// forms the same exact integer group dots (each product exact, a group's sum
// below 2^24) and scales them by s as the int8 kernels do; sx is applied
// after the split-K sum.
//
// Pass 1: a workgroup per (row, chunk of 2048 k).  Each workgroup takes the
// row's a = max|x| (the NaN-keeping max) from a full read of the row (an L2
// hit after the first), inv and sx as in the fused kernels, and writes
// xq = clamp(rint(x * inv), -127, 127) of its chunk as bf16 (the upper half
// of the binary32 value, exact for these integers); chunk 0 writes sx.
__global__ __launch_bounds__(256) void w4a8_actquant_bf16_kernel(const uint16_t* __restrict__ x,
                                                                  int k, uint16_t* __restrict__ xq,
                                                                  float* __restrict__ sx) {
  __shared__ float wmax[4];
  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (size_t)row * k);
  const int k8 = k >> 3;
  float a = 0.0f;
  for (int i = tid; i < k8; i += 256) a = absmax8(xr[i], a);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) a = nmax(a, __shfl_xor(a, off, 64));
  if ((tid & 63) == 0) wmax[tid >> 6] = a;
  __syncthreads();
  float inv, sxv;
  span_scale(finite_or_nan(nmax(nmax(wmax[0], wmax[1]), nmax(wmax[2], wmax[3]))), inv, sxv);
  if (blockIdx.x == 0 && tid == 0) sx[row] = sxv;
  const int i = blockIdx.x * 256 + tid;
  if (i >= k8) return;
  const u32x4_t v = xr[i];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t h[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float f = bf16_to_f32(e ? (w[j] >> 16) : (w[j] & 0xffffu));
      const float t = __builtin_amdgcn_fmed3f(rintf(f * inv), -127.0f, 127.0f);
      h[e] = __float_as_uint(t) >> 16;
    }
    o[j] = h[0] | (h[1] << 16);
  }
  reinterpret_cast<u32x4_t*>(xq + (size_t)row * k)[i] = u32x4_t{o[0], o[1], o[2], o[3]};
}

// One activation scale per group of 32 at 5..64 rows: the quantize pass of
// the M <= 4 per-group kernels, written out once for the matrix-core kernels.
// A workgroup takes 2048 k of one row, a thread 8 k, a lane quad one group:
// a = max|x| over the group (the NaN-keeping max, DPP over the quad), inv and
// sx as everywhere (span_scale), xq = clamp(rint(x * inv), -127, 127) stored
// as exact bf16 integers in xq [m, k], and sx of row r, group g stored
// group-major at sxg[64 g + r].
__global__ __launch_bounds__(256) void w4a8_actquant_g32_bf16_kernel(const uint16_t* __restrict__ x, int k,
                                                                      uint16_t* __restrict__ xq,
                                                                      float* __restrict__ sxg) {
  const int row = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;     // 16-byte piece of the row
  const int k8 = k >> 3;                             // a multiple of 32: quads stay whole
  const bool live = i < k8;
  const u32x4_t v = live ? reinterpret_cast<const u32x4_t*>(x + (size_t)row * k)[i] : u32x4_t{0u, 0u, 0u, 0u};
  float a = absmax8(v, 0.0f);
  a = nmax(a, dpp_fa<0xB1>(a));
  a = nmax(a, dpp_fa<0x4E>(a));
  float inv, sxv;
  span_scale(finite_or_nan(a), inv, sxv);
  if (!live) return;
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t h[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float f = bf16_to_f32(e ? (w[j] >> 16) : (w[j] & 0xffffu));
      const float t = __builtin_amdgcn_fmed3f(rintf(f * inv), -127.0f, 127.0f);
      h[e] = __float_as_uint(t) >> 16;
    }
    o[j] = h[0] | (h[1] << 16);
  }
  reinterpret_cast<u32x4_t*>(xq + (size_t)row * k)[i] = u32x4_t{o[0], o[1], o[2], o[3]};
  if ((i & 3) == 0) sxg[(size_t)(i >> 2) * 64 + row] = sxv;
}

// Pass 3: y[r, c] = sx[r] * sum over s (ascending) of partial[s, r, c]; a
// workgroup per (256 columns, row).
__global__ __launch_bounds__(256) void w4a8_rowscale_reduce_kernel(const float* __restrict__ partial,
                                                                    int split, int n, int64_t mn,
                                                                    const float* __restrict__ sx,
                                                                    void* __restrict__ y, int y_f32) {
  const int col = blockIdx.x * 256 + threadIdx.x;
  if (col >= n) return;
  const int row = blockIdx.y;
  const int64_t i = (int64_t)row * n + col;
  float v = partial[i];
  for (int s = 1; s < split; ++s) v += partial[(int64_t)s * mn + i];
  v *= sx[row];
  if (y_f32)
    static_cast<float*>(y)[i] = v;
  else
    static_cast<uint16_t*>(y)[i] = (uint16_t)f32_to_bf16_rne(v);
}

hipError_t launch_w4a8_actquant_bf16(int m, const void* x, int k, void* xq, float* sx,
                                     hipStream_t stream) {
  const int chunks = ((k >> 3) + 255) / 256;
  hipLaunchKernelGGL(w4a8_actquant_bf16_kernel, dim3(chunks, m), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), k, static_cast<uint16_t*>(xq), sx);
  return hipGetLastError();
}

hipError_t launch_w4a8_actquant_g32_bf16(int m, const void* x, int k, void* xq, float* sxg,
                                         hipStream_t stream) {
  const int chunks = ((k >> 3) + 255) / 256;
  hipLaunchKernelGGL(w4a8_actquant_g32_bf16_kernel, dim3(chunks, m), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), k, static_cast<uint16_t*>(xq), sxg);
  return hipGetLastError();
}

hipError_t launch_w4a8_rowscale_reduce(const float* partial, int split, int m, int n, const float* sx,
                                       void* y, int y_f32, hipStream_t stream) {
  hipLaunchKernelGGL(w4a8_rowscale_reduce_kernel, dim3((n + 255) / 256, m), dim3(256), 0, stream,
                     partial, split, n, (int64_t)m * n, sx, y, y_f32);
  return hipGetLastError();
}

}  // namespace qg
