// gemv_w4a16.hip -- decode GEMV for the packed INT4 group-32 weight, M = 1
// (the kernels are written for any M <= 4, but M = 2..4 run faster on the
// matrix instruction, gemv_w4a16_mx4.hip, and only M = 1 is instantiated).
//
// Computes y[m, n] = sum_k x[m, k] * (q[n,k] - zp[n,g]) * s[n,g], the
// "dequant + F.linear" reference of executorch test_int4_quantized_gemm.py
// (module docstring, `_dequant_matmul`), without ever writing a dequantized
// weight: gpt-fast issue #114 (feiyuvl's report) shows an unfused int->bf16
// convert costs the GEMV its bandwidth.
//
// Mapping (gfx950, wave64):
//  * a workgroup owns one 64-row block (or, in the 32-row variant below, half
//    of one) and one split-K range of 256-k tiles; lane r of every wave owns
//    row r, waves take half tiles round robin: per half tile and lane 4 code
//    chunks of 16 B, the scales and the zero nibbles, each wave-wide load a
//    run of whole 128-byte lines, all through a buffer view of the tile (a
//    descriptor built in scalar registers from the tile's address, 32-bit
//    lane offsets: no vector address arithmetic);
//  * where the grid has at most one workgroup per CU a wave keeps two register
//    sets and loads the next half tile while it computes the current one;
//  * both packed layouts: fp16 scales (v1) or uint8 scale codes times the
//    row's fp16 step (v2, scale codes);
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
  for (int m = 0; m < M; ++m) {
    const BufView xb(x32 + (size_t)m * k32 + (size_t)hs * 64, 256);
    xr.v[m] = xb.b128<false>((uint32_t)li * 16u);
  }
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
  "s_nop 2\n\t"
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


// DQ: the group's scale is its uint8 code times the row's step.
template <int M, int JJ, bool DQ>
__device__ __forceinline__ void do_group(float (&acc)[M], const HalfRegs& cur, const XHalf<M>& xc,
                                         const float (&xq)[M], const float (&zb)[4],
                                         uint32_t mask_s, uint32_t magic_v, float step) {
  const u32x4_t cv = cur.c[JJ];
  const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
  uint32_t pr[16];
#pragma unroll
  for (int d = 0; d < 4; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) pr[4 * d + i] = nibble_pair_bf16(cw[d], i, mask_s, magic_v);
  float s;
  if constexpr (DQ) {
    s = (float)((cur.sc.x >> (8 * JJ)) & 0xffu) * step;
  } else {
    const uint32_t sw = (JJ < 2) ? cur.sc.x : cur.sc.y;
    s = fp16_to_f32((sw >> (16 * (JJ & 1))) & 0xffffu);
  }
#pragma unroll
  for (int m = 0; m < M; ++m) {
    // The dot starts from -(128 + zp) * X_g, so it ends at sum x * (q - zp).
    const float xg = dpp_mov<0x150 + 4 * JJ>(xq[m]);   // X of group JJ to every lane
    float d0 = -zb[JJ] * xg, d1 = 0.0f;
    group_dot<JJ>(d0, d1, xc.v[m], pr);
    acc[m] = __builtin_fmaf(s, d0 + d1, acc[m]);
  }
}

// One half tile: group sums of x, then 4 groups of dequant-dot-correct.
template <int M, bool DQ = false>
__device__ __forceinline__ void half_compute(float (&acc)[M], const HalfRegs& cur,
                                             const XHalf<M>& xc, uint32_t mask_s,
                                             uint32_t magic_v, uint32_t ones_v, float step = 1.0f) {
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
  // 128 + zp of the 4 groups: the zero nibbles spread to bytes with 0x80 set,
  // then one byte-to-float conversion each.
  const uint32_t z02 = (cur.zw & 0x0F0Fu) | 0x8080u;          // groups 0, 2
  const uint32_t z13 = ((cur.zw >> 4) & 0x0F0Fu) | 0x8080u;   // groups 1, 3
  const float zb[4] = {(float)(z02 & 0xffu), (float)(z13 & 0xffu), (float)(z02 >> 8),
                       (float)(z13 >> 8)};
  do_group<M, 0, DQ>(acc, cur, xc, xq, zb, mask_s, magic_v, step);
  do_group<M, 1, DQ>(acc, cur, xc, xq, zb, mask_s, magic_v, step);
  do_group<M, 2, DQ>(acc, cur, xc, xq, zb, mask_s, magic_v, step);
  do_group<M, 3, DQ>(acc, cur, xc, xq, zb, mask_s, magic_v, step);
}

// Work unit = half tile.  Wave w of a workgroup takes half tiles w, w+WAVES,
// ... of its row block's split-K range: load, wait, compute, the other
// resident waves keeping the memory system busy.  PF: the two-register-set
// loop, for grids of at most one workgroup per CU (8448 x 6656: 8.77 -> 8.69
// us; 12288 x 4096: 7.09 -> 6.92).  DQ: the scale-code layout.
template <int M, int WAVES, bool PF = false, bool DQ = false>
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
  constexpr int kTile = DQ ? kDqTileBytes : kTileBytes;
  const uint8_t* tiles;
  float step = 1.0f;
  if constexpr (DQ) {   // the block's head holds each row's fp16 step
    const uint8_t* block = packed + (size_t)rb * (kDqHeadBytes + (size_t)kt_count * kDqTileBytes);
    step = fp16_to_f32(*reinterpret_cast<const uint16_t*>(block + 2 * lane));
    tiles = block + kDqHeadBytes;
  } else {
    tiles = packed + (size_t)rb * kt_count * kTileBytes;
  }
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

  auto load = [&](HalfRegs& r, XHalf<M>& xr, int hs) {   // tile hs/2, half hs%2
    load_half<DQ>(r, tiles + (size_t)(hs >> 1) * kTile, hs & 1, lane);
    load_xhalf<M>(xr, x32, k32, hs, li);
  };
  if constexpr (!PF) {
    for (int hs = 2 * t0 + wave; hs < 2 * t1; hs += WAVES) {
      HalfRegs r;
      XHalf<M> xr;
      load(r, xr, hs);
      half_compute<M, DQ>(acc, r, xr, mask_s, magic_v, ones_v, step);
    }
  } else {
    const int h_end = 2 * t1;
    int hs = 2 * t0 + wave;
    if (hs < h_end) {
      HalfRegs ra, rb;
      XHalf<M> xa, xb;
      load(ra, xa, hs);
      __builtin_amdgcn_sched_barrier(0);
      while (true) {
        if (hs + WAVES >= h_end) { half_compute<M, DQ>(acc, ra, xa, mask_s, magic_v, ones_v, step); break; }
        load(rb, xb, hs + WAVES);
        __builtin_amdgcn_sched_barrier(0);
        half_compute<M, DQ>(acc, ra, xa, mask_s, magic_v, ones_v, step);
        hs += WAVES;
        if (hs + WAVES >= h_end) { half_compute<M, DQ>(acc, rb, xb, mask_s, magic_v, ones_v, step); break; }
        load(ra, xa, hs + WAVES);
        __builtin_amdgcn_sched_barrier(0);
        half_compute<M, DQ>(acc, rb, xb, mask_s, magic_v, ones_v, step);
        hs += WAVES;
      }
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

// ---------------------------------------------------------------------------
// 32-row variant.  A workgroup owns 32 rows of a 64-row block (the tile's
// 128-byte lines hold 8 rows each, so halves of a block never share a code
// line), which doubles the number of workgroups and evens out the work per CU
// when the row-block count is not a multiple of the CU count.  Lanes 0-31 take
// groups {0,1} of each half tile for rows 0-31, lanes 32-63 groups {2,3}; each
// wave-wide code load is two runs of 512 contiguous bytes.  x of a half tile
// sits 2 dwords per lane: DPP rows 0-1 hold groups {0,1}, rows 2-3 {2,3}
// (Half32Regs / W4Layout::load in w4_common.h).
#define QG_DOT16_2R(L0, L1, L2, L3, L4, L5, L6, L7)                                       \
  "s_nop 1\n\t"                                                                            \
  QG_DPP_DOT("%0", "%2", "%4", L0) QG_DPP_DOT("%1", "%3", "%5", L0)                        \
  QG_DPP_DOT("%0", "%2", "%6", L1) QG_DPP_DOT("%1", "%3", "%7", L1)                        \
  QG_DPP_DOT("%0", "%2", "%8", L2) QG_DPP_DOT("%1", "%3", "%9", L2)                        \
  QG_DPP_DOT("%0", "%2", "%10", L3) QG_DPP_DOT("%1", "%3", "%11", L3)                      \
  QG_DPP_DOT("%0", "%2", "%12", L4) QG_DPP_DOT("%1", "%3", "%13", L4)                      \
  QG_DPP_DOT("%0", "%2", "%14", L5) QG_DPP_DOT("%1", "%3", "%15", L5)                      \
  QG_DPP_DOT("%0", "%2", "%16", L6) QG_DPP_DOT("%1", "%3", "%17", L6)                      \
  QG_DPP_DOT("%0", "%2", "%18", L7) QG_DPP_DOT("%1", "%3", "%19", L7)                      \
  "s_nop 2\n\t"
#define QG_DOT16_2R_OPERANDS                                                               \
  : "+v"(d0), "+v"(d1)                                                                     \
  : "v"(xv.x), "v"(xv.y), "v"(pr[0]), "v"(pr[1]), "v"(pr[2]), "v"(pr[3]), "v"(pr[4]),      \
    "v"(pr[5]), "v"(pr[6]), "v"(pr[7]), "v"(pr[8]), "v"(pr[9]), "v"(pr[10]), "v"(pr[11]),  \
    "v"(pr[12]), "v"(pr[13]), "v"(pr[14]), "v"(pr[15])

template <int JJ>
__device__ __forceinline__ void group_dot_2r(float& d0, float& d1, const u32x2_t& xv,
                                             const uint32_t (&pr)[16]) {
  if constexpr (JJ == 0) asm(QG_DOT16_2R(0, 1, 2, 3, 4, 5, 6, 7) QG_DOT16_2R_OPERANDS);
  if constexpr (JJ == 1) asm(QG_DOT16_2R(8, 9, 10, 11, 12, 13, 14, 15) QG_DOT16_2R_OPERANDS);
}

// PF: two register sets used in turn, so that a wave has the next half
// tile's loads in flight while it computes the current one (for grids of at
// most one workgroup per CU, where nothing else hides the load latency).  The
// scheduling barriers keep the compiler from sinking the loads below the
// computation they are meant to overlap.
template <int M, int WAVES, bool DQ = false, bool PF = false>
__global__ __launch_bounds__(WAVES * 64) void w4a16_gemv32_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split) {
  __shared__ float red[WAVES * M * 64];
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int lg = lane >> 5;                       // group pair of this lane
  const int wave = wave_id_uniform();
  const int rb = blockIdx.x >> 1;                 // 64-row block
  const int row = 32 * (blockIdx.x & 1) + (lane & 31);   // row within the block
  const int kt_count = k >> 8;
  using L = W4Layout<DQ>;
  float step;
  const uint8_t* tiles = L::tiles(packed, rb, kt_count, row, step);
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
  const int k32 = k >> 1;
  const uint32_t mask_s = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t magic_v = 0x43004300u;
  asm volatile("" : "+v"(magic_v));
  uint32_t ones_v = 0x3f803f80u;   // bf16 (1, 1), kept out of literal operands
  asm volatile("" : "+v"(ones_v));

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  // Buffer views per half tile: of its weight tile and of its 128 k of x.
  auto load = [&](Half32Regs& r, u32x2_t (&xv)[M], int hs) {
    L::load(r, tiles + (size_t)(hs >> 1) * L::kTile, hs & 1, lg, row);
#pragma unroll
    for (int m = 0; m < M; ++m) {
      const BufView xb(x32 + (size_t)m * k32 + (size_t)hs * 64, 256);
      xv[m] = xb.b64((uint32_t)(32 * lg + 2 * li) * 4u);
    }
  };
  auto compute = [&](const Half32Regs& r, const u32x2_t (&xv)[M]) {
    // group sums: 8 lanes per group (quad_perm [1,0,3,2], [2,3,0,1], half-row mirror)
    float xq[M];
#pragma unroll
    for (int m = 0; m < M; ++m) {
      float p = dot2_bf16(xv[m].x, ones_v, 0.0f);
      p = dot2_bf16(xv[m].y, ones_v, p);
      p += dpp_mov<0xB1>(p);
      p += dpp_mov<0x4E>(p);
      p += dpp_mov<0x141>(p);
      xq[m] = p;
    }
    const float zb0 = (float)((r.zb & 15u) | 0x80u);          // 128 + zp
    const float zb1 = (float)(((r.zb >> 4) & 15u) | 0x80u);
    const float s0 = L::scale(r.sc, 0, step);
    const float s1 = L::scale(r.sc, 1, step);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const u32x4_t cv = r.c[jj];
      const uint32_t cw[4] = {cv.x, cv.y, cv.z, cv.w};
      uint32_t pr[16];
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[4 * d + i] = nibble_pair_bf16(cw[d], i, mask_s, magic_v);
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const float xg = jj == 0 ? dpp_mov<0x150>(xq[m]) : dpp_mov<0x158>(xq[m]);
        float d0 = -(jj == 0 ? zb0 : zb1) * xg, d1 = 0.0f;
        if (jj == 0)
          group_dot_2r<0>(d0, d1, xv[m], pr);
        else
          group_dot_2r<1>(d0, d1, xv[m], pr);
        acc[m] = __builtin_fmaf(jj == 0 ? s0 : s1, d0 + d1, acc[m]);
      }
    }
  };

  if constexpr (!PF) {
    for (int hs = 2 * t0 + wave; hs < 2 * t1; hs += WAVES) {
      Half32Regs r;
      u32x2_t xv[M];
      load(r, xv, hs);
      compute(r, xv);
    }
  } else {
    const int h_end = 2 * t1;
    int hs = 2 * t0 + wave;
    if (hs < h_end) {                                    // uniform
      Half32Regs ra, rb;
      u32x2_t xa[M], xb[M];
      load(ra, xa, hs);
      __builtin_amdgcn_sched_barrier(0);
      while (true) {
        if (hs + WAVES >= h_end) { compute(ra, xa); break; }
        load(rb, xb, hs + WAVES);
        __builtin_amdgcn_sched_barrier(0);
        compute(ra, xa);
        hs += WAVES;
        if (hs + WAVES >= h_end) { compute(rb, xb); break; }
        load(ra, xa, hs + WAVES);
        __builtin_amdgcn_sched_barrier(0);
        compute(rb, xb);
        hs += WAVES;
      }
    }
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
      if (partial != nullptr)
        partial[((size_t)blockIdx.y * M + m) * n + col] = v;
      else if (y_f32)
        static_cast<float*>(y)[(size_t)m * n + col] = v;
      else
        static_cast<uint16_t*>(y)[(size_t)m * n + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// ---- INT5 / INT6 (the pages' INT5/INT6 family), M = 1 ----------------------
// Layout and pair extraction: WnLayout (w4_common.h).  The low nibbles go
// through nibble_pair_bf16 as for INT4, the high bits are ORed in four places
// up; the arithmetic is then the INT4 GEMV's (128 + q stays exact for q <= 63).
template <int HB>
__device__ __forceinline__ uint32_t wide_pair(const WnRegs<HB>& r, int jj, int d, int i, uint32_t mask_s,
                                              uint32_t magic_v) {
  return nibble_pair_bf16(r.c[jj][d], i, mask_s, magic_v) | (WnLayout<HB>::high(r, jj, d, i) << 4);
}

// PF: the two-register-set loop of w4a16_gemv32_kernel, for grids of at most
// one workgroup per CU.
template <int HB, int WAVES, bool PF = false>
__global__ __launch_bounds__(WAVES * 64) void wn_a16_gemv32_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split) {
  __shared__ float red[WAVES * 64];
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int lg = lane >> 5;
  const int wave = wave_id_uniform();
  const int rb = blockIdx.x >> 1;
  const int row = 32 * (blockIdx.x & 1) + (lane & 31);
  const int kt_count = k >> 8;
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  using L = WnLayout<HB>;
  const uint8_t* tiles = packed + (size_t)rb * kt_count * L::kTile;
  const uint32_t* x32 = reinterpret_cast<const uint32_t*>(x);
  const uint32_t mask_s = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t magic_v = 0x43004300u;
  asm volatile("" : "+v"(magic_v));
  uint32_t ones_v = 0x3f803f80u;
  asm volatile("" : "+v"(ones_v));

  float acc = 0.0f;
  auto load = [&](WnRegs<HB>& r, u32x2_t& xv, int hs) {
    L::load(r, tiles + (size_t)(hs >> 1) * L::kTile, hs & 1, lg, row);
    xv = BufView(x32 + (size_t)hs * 64, 256).b64((uint32_t)(32 * lg + 2 * li) * 4u);
  };
  auto compute = [&](const WnRegs<HB>& r, const u32x2_t& xv) {
    float p = dot2_bf16(xv.x, ones_v, 0.0f);
    p = dot2_bf16(xv.y, ones_v, p);
    p += dpp_mov<0xB1>(p);
    p += dpp_mov<0x4E>(p);
    p += dpp_mov<0x141>(p);
    const float xq = p;
    const float zb0 = (float)((r.zb & 0xffu) | 0x80u);          // 128 + zp (zp <= 63)
    const float zb1 = (float)(((r.zb >> 8) & 0xffu) | 0x80u);
    const float s0 = fp16_to_f32(r.sc & 0xffffu);
    const float s1 = fp16_to_f32(r.sc >> 16);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      uint32_t pr[16];
#pragma unroll
      for (int d = 0; d < 4; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[4 * d + i] = wide_pair<HB>(r, jj, d, i, mask_s, magic_v);
      const float xg = jj == 0 ? dpp_mov<0x150>(xq) : dpp_mov<0x158>(xq);
      float d0 = -(jj == 0 ? zb0 : zb1) * xg, d1 = 0.0f;
      if (jj == 0)
        group_dot_2r<0>(d0, d1, xv, pr);
      else
        group_dot_2r<1>(d0, d1, xv, pr);
      acc = __builtin_fmaf(jj == 0 ? s0 : s1, d0 + d1, acc);
    }
  };

  if constexpr (!PF) {
    for (int hs = 2 * t0 + wave; hs < 2 * t1; hs += WAVES) {
      WnRegs<HB> r;
      u32x2_t xv;
      load(r, xv, hs);
      __builtin_amdgcn_sched_barrier(0);   // every load of the step issued before the first wait
      compute(r, xv);
    }
  } else {
    const int h_end = 2 * t1;
    int hs = 2 * t0 + wave;
    if (hs < h_end) {                                    // uniform
      WnRegs<HB> ra, rb;
      u32x2_t xa, xb;
      load(ra, xa, hs);
      __builtin_amdgcn_sched_barrier(0);
      while (true) {
        if (hs + WAVES >= h_end) { compute(ra, xa); break; }
        load(rb, xb, hs + WAVES);
        __builtin_amdgcn_sched_barrier(0);
        compute(ra, xa);
        hs += WAVES;
        if (hs + WAVES >= h_end) { compute(rb, xb); break; }
        load(ra, xa, hs + WAVES);
        __builtin_amdgcn_sched_barrier(0);
        compute(rb, xb);
        hs += WAVES;
      }
    }
  }

  red[wave * 64 + lane] = acc;
  __syncthreads();
  const int t = threadIdx.x;
  if (t < 32) {
    float v = 0.0f;
    for (int w = 0; w < WAVES; ++w) {
      v += red[w * 64 + t];
      v += red[w * 64 + t + 32];
    }
    const int col = rb * kTileRows + 32 * (blockIdx.x & 1) + t;
    if (col < n) {
      if (partial != nullptr)
        partial[(size_t)blockIdx.y * n + col] = v;
      else if (y_f32)
        static_cast<float*>(y)[col] = v;
      else
        static_cast<uint16_t*>(y)[col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

template <int HB>
static hipError_t launch_wn_t(const void* x, const void* packed, int n, int k, void* y, int y_f32,
                              float* partial, int split, hipStream_t stream) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  const dim3 grid(2 * rbs, split), block(16 * 64);
  const auto* xs = static_cast<const uint16_t*>(x);
  const auto* ps = static_cast<const uint8_t*>(packed);
  if (2 * rbs * split <= kCUs)
    hipLaunchKernelGGL((wn_a16_gemv32_kernel<HB, 16, true>), grid, block, 0, stream, xs, ps, n, k, y, y_f32,
                       partial, split);
  else
    hipLaunchKernelGGL((wn_a16_gemv32_kernel<HB, 16>), grid, block, 0, stream, xs, ps, n, k, y, y_f32, partial,
                       split);
  return hipGetLastError();
}

hipError_t launch_wn_a16_gemv32(int bits, const void* x, const void* packed, int n, int k, void* y,
                                int y_f32, float* partial, int split, hipStream_t stream) {
  if (bits == 5) return launch_wn_t<1>(x, packed, n, k, y, y_f32, partial, split, stream);
  if (bits == 6) return launch_wn_t<2>(x, packed, n, k, y, y_f32, partial, split, stream);
  return hipErrorInvalidValue;
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

template <int M, int WAVES, bool DQ = false>
static hipError_t launch_w4a16_t(const void* x, const void* packed, int n, int k, void* y,
                                 int y_f32, float* partial, int split, hipStream_t stream) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  if (rbs * split <= kCUs)
    hipLaunchKernelGGL((w4a16_gemv_kernel<M, WAVES, true, DQ>), dim3(rbs, split), dim3(WAVES * 64), 0,
                       stream, static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(packed),
                       n, k, y, y_f32, partial, split);
  else
    hipLaunchKernelGGL((w4a16_gemv_kernel<M, WAVES, false, DQ>), dim3(rbs, split), dim3(WAVES * 64), 0,
                       stream, static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(packed),
                       n, k, y, y_f32, partial, split);
  return hipGetLastError();
}

// M = 1 on the scale-code layout, one 64-row block per workgroup.
hipError_t launch_w4a16_gemv_dq(int m, const void* x, const void* packed, int n, int k, void* y,
                                int y_f32, float* partial, int split, hipStream_t stream) {
  if (m != 1) return hipErrorInvalidValue;
  return launch_w4a16_t<1, 16, true>(x, packed, n, k, y, y_f32, partial, split, stream);
}

// M = 1 on either layout: half a 64-row block per workgroup, with the
// two-register-set loop when the grid has at most one workgroup per CU.
template <bool DQ>
static hipError_t launch_gemv32_m1(const void* x, const void* packed, int n, int k, void* y, int y_f32,
                                   float* partial, int split, hipStream_t stream) {
  const auto* xs = static_cast<const uint16_t*>(x);
  const auto* ps = static_cast<const uint8_t*>(packed);
  const int rbs = (n + kTileRows - 1) / kTileRows;
  const dim3 grid(2 * rbs, split), block(16 * 64);
  if (2 * rbs * split <= kCUs)
    hipLaunchKernelGGL((w4a16_gemv32_kernel<1, 16, DQ, true>), grid, block, 0, stream, xs, ps, n, k, y, y_f32,
                       partial, split);
  else
    hipLaunchKernelGGL((w4a16_gemv32_kernel<1, 16, DQ>), grid, block, 0, stream, xs, ps, n, k, y, y_f32,
                       partial, split);
  return hipGetLastError();
}

// M = 1 on the scale-code layout (version 2).
hipError_t launch_w4a16_gemv32_dq(int m, const void* x, const void* packed, int n, int k, void* y,
                                  int y_f32, float* partial, int split, hipStream_t stream) {
  if (m != 1) return hipErrorInvalidValue;
  return launch_gemv32_m1<true>(x, packed, n, k, y, y_f32, partial, split, stream);
}

// M = 2..4 run on the matrix-instruction GEMV (gemv_w4a16_mx4.hip).
hipError_t launch_w4a16_gemv32(int m, const void* x, const void* packed, int n, int k, void* y,
                               int y_f32, float* partial, int split, int waves, hipStream_t stream) {
  if (m != 1 || waves != 16) return hipErrorInvalidValue;
  return launch_gemv32_m1<false>(x, packed, n, k, y, y_f32, partial, split, stream);
}

hipError_t launch_w4a16_gemv(int m, const void* x, const void* packed, int n, int k, void* y,
                             int y_f32, float* partial, int split, int waves, hipStream_t stream) {
#define QG_W4_CASE(MM, WW) \
  if (m == MM && waves == WW) return launch_w4a16_t<MM, WW>(x, packed, n, k, y, y_f32, partial, split, stream);
#define QG_W4_M(MM) QG_W4_CASE(MM, 16)
  QG_W4_M(1)
#undef QG_W4_M
#undef QG_W4_CASE
  return hipErrorInvalidValue;
}

}  // namespace qg
