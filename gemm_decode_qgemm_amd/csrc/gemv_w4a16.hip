// gemv_w4a16.hip -- decode GEMV for the packed INT4 group-32 weight, M = 1..4.
//
// Computes y[m, n] = sum_k x[m, k] * (q[n,k] - zp[n,g]) * s[n,g], the
// "dequant + F.linear" reference of executorch test_int4_quantized_gemm.py
// (module docstring, `_dequant_matmul`), without ever writing a dequantized
// weight: gpt-fast issue #114 (feiyuvl's report) shows an unfused int->bf16
// convert costs the GEMV its bandwidth.
//
// Mapping (gfx950, wave64):
//  * a workgroup owns one 64-row block and one split-K range of 256-k tiles;
//    lane r of every wave owns row r, waves take tiles round robin, so each
//    wave streams whole tiles: 10 loads of 16/4 B per lane, every one a run of
//    whole 128-byte lines;
//  * x is the same for all 64 lanes, so each lane keeps only 1/16 of a tile's
//    x in VGPRs (two 16-byte loads per row m per tile, L2-resident) and
//    v_dot2c_f32_bf16 takes the x pair it needs from the lane that holds it
//    through a DPP row broadcast: no LDS, no scalar registers, no extra
//    instruction per product;
//  * nibbles become exact bf16 pairs (128 + q) with one shift and one and-or
//    (see nibble_pair_bf16), v_dot2c accumulates x * (128 + q) in fp32, and a
//    per-group correction subtracts (128 + zp) * X_g, where X_g (the group sum
//    of x) comes from a 4-lane DPP reduction of the same registers;
//  * the waves' per-row partials are summed through LDS in wave order, and a
//    split-K launch writes fp32 partials that a second pass sums in split
//    order (no atomics: results are bit-reproducible).
#include "qg_common.h"
#include "w4_common.h"

namespace qg {

// x of one half tile (128 k = 64 dwords per row m) lives in VGPRs spread
// over the 16 lanes of each DPP row: lane i holds dwords 4i..4i+3; the four
// rows of the wave hold the same copy.  Dword q of the half's group jj is
// therefore register q % 4 of lane 4*jj + q / 4, read with DPP row_newbcast.
template <int M>
struct XHalf {
  u32x4_t v[M];
};

template <int M>
__device__ __forceinline__ void load_xhalf(XHalf<M>& xr, const uint32_t* x32, int k32, int hs, int li) {
#pragma unroll
  for (int m = 0; m < M; ++m)
    xr.v[m] = *reinterpret_cast<const u32x4_t*>(x32 + (size_t)m * k32 + (size_t)hs * 64 + li * 4);
}

// d0 += x . (128+q) over the even dwords and d1 over the odd dwords of one
// group: 16 v_dot2c_f32_bf16 whose x operand is broadcast by DPP from the lane
// that holds it.  The leading `s_nop 1` gives the two wait states a DPP read
// needs after a VALU write of its source register.  The trailing nop covers a
// hazard measured on MI355X: a VALU read of a v_dot2c_f32_bf16_dpp result less
// than two wait states after it sees the old value (the compiler cannot see
// into the asm to insert them); one-hot tests lose exactly the block's last
// product without it and are exact with one or more.
#define QG_DPP_DOT(acc, xr, pr, L) \
  "v_dot2c_f32_bf16_dpp " acc ", " xr ", " pr " row_newbcast:" #L " row_mask:0xf bank_mask:0xf\n\t"
#ifndef QG_DOT_TAIL_NOP
#define QG_DOT_TAIL_NOP 2
#endif
#define QG_STR2(x) #x
#define QG_STR(x) QG_STR2(x)
#define QG_DOT16(L0, L1, L2, L3)                                                              \
  "s_nop 1\n\t"                                                                              \
  QG_DPP_DOT("%0", "%2", "%6", L0) QG_DPP_DOT("%1", "%3", "%7", L0)                          \
  QG_DPP_DOT("%0", "%4", "%8", L0) QG_DPP_DOT("%1", "%5", "%9", L0)                          \
  QG_DPP_DOT("%0", "%2", "%10", L1) QG_DPP_DOT("%1", "%3", "%11", L1)                        \
  QG_DPP_DOT("%0", "%4", "%12", L1) QG_DPP_DOT("%1", "%5", "%13", L1)                        \
  QG_DPP_DOT("%0", "%2", "%14", L2) QG_DPP_DOT("%1", "%3", "%15", L2)                        \
  QG_DPP_DOT("%0", "%4", "%16", L2) QG_DPP_DOT("%1", "%5", "%17", L2)                        \
  QG_DPP_DOT("%0", "%2", "%18", L3) QG_DPP_DOT("%1", "%3", "%19", L3)                        \
  QG_DPP_DOT("%0", "%4", "%20", L3) QG_DPP_DOT("%1", "%5", "%21", L3)                        \
  "s_nop " QG_STR(QG_DOT_TAIL_NOP) "\n\t"
#define QG_DOT16_OPERANDS                                                                    \
  : "+v"(d0), "+v"(d1)                                                                       \
  : "v"(xv.x), "v"(xv.y), "v"(xv.z), "v"(xv.w), "v"(pr[0]), "v"(pr[1]), "v"(pr[2]),          \
    "v"(pr[3]), "v"(pr[4]), "v"(pr[5]), "v"(pr[6]), "v"(pr[7]), "v"(pr[8]), "v"(pr[9]),      \
    "v"(pr[10]), "v"(pr[11]), "v"(pr[12]), "v"(pr[13]), "v"(pr[14]), "v"(pr[15])

template <int JJ>
__device__ __forceinline__ void group_dot(float& d0, float& d1, const u32x4_t& xv,
                                          const uint32_t (&pr)[16]) {
  if constexpr (JJ == 0) asm(QG_DOT16(0, 1, 2, 3) QG_DOT16_OPERANDS);
  if constexpr (JJ == 1) asm(QG_DOT16(4, 5, 6, 7) QG_DOT16_OPERANDS);
  if constexpr (JJ == 2) asm(QG_DOT16(8, 9, 10, 11) QG_DOT16_OPERANDS);
  if constexpr (JJ == 3) asm(QG_DOT16(12, 13, 14, 15) QG_DOT16_OPERANDS);
}


template <int M, int JJ>
__device__ __forceinline__ void do_group(float (&acc)[M], const HalfRegs& cur, const XHalf<M>& xc,
                                         const float (&xq)[M], uint32_t mask_s, uint32_t magic_v) {
  const u32x4_t cv = cur.c[JJ];
  const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
  uint32_t pr[16];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[4 * d + i] = nibble_pair_bf16(cw[d], i, mask_s, magic_v);
  const uint32_t sw = (JJ < 2) ? cur.sc.x : cur.sc.y;
  const float s = fp16_to_f32((sw >> (16 * (JJ & 1))) & 0xffffu);
  const float zb = (float)(((cur.zw >> (4 * JJ)) & 15u) + 128u);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    float d0 = 0.0f, d1 = 0.0f;
    group_dot<JJ>(d0, d1, xc.v[m], pr);
    const float xg = dpp_mov<0x150 + 4 * JJ>(xq[m]);   // X of group JJ to every lane
    const float tg = __builtin_fmaf(-zb, xg, d0 + d1);
    acc[m] = __builtin_fmaf(s, tg, acc[m]);
  }
}

// One half tile: group sums of x, then 4 groups of dequant-dot-correct.
template <int M>
__device__ __forceinline__ void half_compute(float (&acc)[M], const HalfRegs& cur,
                                             const XHalf<M>& xc, uint32_t mask_s,
                                             uint32_t magic_v, uint32_t ones_v) {
  // X_g: lane i of a row sums its 4 dwords (group i/4 of the half), then the
  // quad of lanes sharing a group adds up (DPP quad_perm [1,0,3,2], [2,3,0,1]).
  float xq[M];
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const u32x4_t v = xc.v[m];
    float p = dot2_bf16(v.x, ones_v, 0.0f);
    p = dot2_bf16(v.y, ones_v, p);
    p = dot2_bf16(v.z, ones_v, p);
    p = dot2_bf16(v.w, ones_v, p);
    p += dpp_mov<0xB1>(p);
    p += dpp_mov<0x4E>(p);
    xq[m] = p;
  }
  do_group<M, 0>(acc, cur, xc, xq, mask_s, magic_v);
  do_group<M, 1>(acc, cur, xc, xq, mask_s, magic_v);
  do_group<M, 2>(acc, cur, xc, xq, mask_s, magic_v);
  do_group<M, 3>(acc, cur, xc, xq, mask_s, magic_v);
}

// Work unit = half tile.  Wave w of a workgroup takes half tiles w, w+WAVES,
// ... of its row block's split-K range.  LA = look-ahead: the loads of the
// next LA units are in flight while a unit computes (register sets used in a
// ring, unrolled, so no copies); LA = 0 loads, waits and computes.
template <int M, int WAVES, bool NT, int LA>
__global__ __launch_bounds__(WAVES * 64) void w4a16_gemv_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split) {
  __shared__ float red[WAVES * M * 64];
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int wave = wave_id_uniform();
  const int rb = blockIdx.x;
  const int kt_count = k >> 8;
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  const uint8_t* tiles = packed + (size_t)rb * kt_count * kTileBytes;
  const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
  const int k32 = k >> 1;
  const uint32_t mask_s = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t magic_v = 0x43004300u;
  asm volatile("" : "+v"(magic_v));   // keep the constant in a VGPR
  // The bf16 pair (1.0, 1.0) for the group sums, also held in a VGPR: as a
  // literal or inline constant in v_dot2c_f32_bf16 the pair is not read as
  // two bf16 halves on gfx950 (the inline constant 1.0 arrives as the f32
  // pattern 0x3F800000, i.e. the pair (0, 1.0)).
  uint32_t ones_v = 0x3f803f80u;
  asm volatile("" : "+v"(ones_v));

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  const int s1 = 2 * t1;
  int hs = 2 * t0 + wave;   // half-tile index along k (tile hs/2, half hs%2)
  auto load = [&](HalfRegs& r, XHalf<M>& xr, int h) {
    load_half<NT>(r, tiles + (size_t)(h >> 1) * kTileBytes, h & 1, lane);
    load_xhalf<M>(xr, x32, k32, h, li);
  };
  if constexpr (LA == 0) {
    for (; hs < s1; hs += WAVES) {
      HalfRegs r;
      XHalf<M> xr;
      load(r, xr, hs);
      half_compute<M>(acc, r, xr, mask_s, magic_v, ones_v);
    }
  } else if constexpr (LA == 1) {
    HalfRegs ra, rb2;
    XHalf<M> xa, xb;
    if (hs < s1) load(ra, xa, hs);
    while (hs < s1) {
      if (hs + WAVES < s1) load(rb2, xb, hs + WAVES);
      half_compute<M>(acc, ra, xa, mask_s, magic_v, ones_v);
      hs += WAVES;
      if (hs >= s1) break;
      if (hs + WAVES < s1) load(ra, xa, hs + WAVES);
      half_compute<M>(acc, rb2, xb, mask_s, magic_v, ones_v);
      hs += WAVES;
    }
  } else {
    HalfRegs r0, r1, r2;
    XHalf<M> x0, x1, x2;
    if (hs < s1) load(r0, x0, hs);
    if (hs + WAVES < s1) load(r1, x1, hs + WAVES);
    while (hs < s1) {
      if (hs + 2 * WAVES < s1) load(r2, x2, hs + 2 * WAVES);
      half_compute<M>(acc, r0, x0, mask_s, magic_v, ones_v);
      hs += WAVES;
      if (hs >= s1) break;
      if (hs + 2 * WAVES < s1) load(r0, x0, hs + 2 * WAVES);
      half_compute<M>(acc, r1, x1, mask_s, magic_v, ones_v);
      hs += WAVES;
      if (hs >= s1) break;
      if (hs + 2 * WAVES < s1) load(r1, x1, hs + 2 * WAVES);
      half_compute<M>(acc, r2, x2, mask_s, magic_v, ones_v);
      hs += WAVES;
    }
  }

  // Cross-wave sum in wave order (fixed, so repeat calls are bit-identical).
#pragma unroll
  for (int m = 0; m < M; ++m) red[(wave * M + m) * 64 + lane] = acc[m];
  __syncthreads();
  for (int m = wave; m < M; m += WAVES) {
    float v = red[m * 64 + lane];
    for (int w = 1; w < WAVES; ++w) v += red[(w * M + m) * 64 + lane];
    const int row = rb * kTileRows + lane;
    if (row < n) {
      if (partial != nullptr) {
        partial[((size_t)blockIdx.y * M + m) * n + row] = v;
      } else if (y_f32) {
        static_cast<float*>(y)[(size_t)m * n + row] = v;
      } else {
        static_cast<uint16_t*>(y)[(size_t)m * n + row] = (uint16_t)f32_to_bf16_rne(v);
      }
    }
  }
}

// Second split-K pass: y = sum over s (ascending) of partial[s], no atomics.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int split, int64_t mn,
                                                            void* __restrict__ y, int y_f32) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= mn) return;
  float v = partial[i];
  for (int s = 1; s < split; ++s) v += partial[(int64_t)s * mn + i];
  if (y_f32)
    static_cast<float*>(y)[i] = v;
  else
    static_cast<uint16_t*>(y)[i] = (uint16_t)f32_to_bf16_rne(v);
}

hipError_t launch_splitk_reduce(const float* partial, int split, int64_t mn, void* y, int y_f32,
                                hipStream_t stream) {
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0,
                     stream, partial, split, mn, y, y_f32);
  return hipGetLastError();
}

template <int M, int WAVES, bool NT, int LA>
static hipError_t launch_w4a16_t(const void* x, const void* packed, int n, int k, void* y,
                                 int y_f32, float* partial, int split, hipStream_t stream) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  const int kt = k / kTileK;
  (void)kt;
  hipLaunchKernelGGL((w4a16_gemv_kernel<M, WAVES, NT, LA>), dim3(rbs, split), dim3(WAVES * 64), 0,
                     stream, static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(packed),
                     n, k, y, y_f32, partial, split);
  return hipGetLastError();
}

// Shared-memory bytes the GEMV needs (the host checks it against the limit).
size_t w4a16_gemv_smem_bytes(int m, int k, int split, int waves) {
  (void)k; (void)split;
  return (size_t)(waves * m * 64) * sizeof(float);
}

hipError_t launch_w4a16_gemv(int m, const void* x, const void* packed, int n, int k, void* y,
                             int y_f32, float* partial, int split, int waves, int la,
                             hipStream_t stream) {
#define QG_W4_CASE(MM, WW, LAV)                                                                \
  if (m == MM && waves == WW && la == LAV)                                                     \
    return launch_w4a16_t<MM, WW, true, LAV>(x, packed, n, k, y, y_f32, partial, split, stream);
#define QG_W4_M(MM)                                                                            \
  QG_W4_CASE(MM, 4, 0) QG_W4_CASE(MM, 8, 0) QG_W4_CASE(MM, 16, 0)                             \
  QG_W4_CASE(MM, 4, 1) QG_W4_CASE(MM, 8, 1) QG_W4_CASE(MM, 16, 1)
  QG_W4_M(1) QG_W4_M(2) QG_W4_M(3) QG_W4_M(4)
#undef QG_W4_M
#undef QG_W4_CASE
  return hipErrorInvalidValue;
}

}  // namespace qg
