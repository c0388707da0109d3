// gemm_w4a16_mfma.hip -- packed INT4 group-32 weight x bf16 activations for
// M = 5..64 rows, on the matrix cores.
//
// executorch test_int4_quantized_gemm.py: buckets 8..64 run a W4A16 kernel
// (the `_W4A16_DIRECT_KERNELS` / `_W4A16_SPLIT_KERNELS` of the bucket tests);
// the result is the same "dequant + F.linear" sum as the decode GEMV.  With
// 16..64 activation rows each weight feeds enough products for the matrix
// cores to pay off.
//
// Arithmetic, per group g and 16 x 16 output tile, with v_mfma_f32_16x16x32_bf16:
//   P = x (16 m x 32 k, exact bf16) . (128 + q) (32 k x 16 n, exact bf16),
//   X = x . ones (the group sums, landing in the accumulator layout),
//   y[m][n] += s[n,g] * (P[m][n] - (128 + zp[n,g]) * X[m]),
// so every product is exact and the sums are fp32, as in the decode GEMV.
//
// Two forms; mfma_lds_form() (qg_common.h) picks one per call.
//
// Register form (up to 16 rows), mapping (gfx950):
//  * a wave owns a whole 64-row block (4 n-tiles of 16 rows) and MT m-tiles
//    for a range of half tiles (4 groups = 128 k); a workgroup is KW x MG
//    waves: KW waves split the block's K range round robin, MG wave groups
//    take different m-tiles (each loads the block's weights: the second read
//    is an L2 hit), and the KW partial sums are added through LDS in wave
//    order at the end (no atomics, bit-reproducible);
//  * weights: lane (i, a) = (lane % 16, lane / 16) loads the whole 16-byte
//    chunk of group a, row 16t + i -- one wave-wide load is 4 runs of 256
//    contiguous bytes, and the 4 loads of a half tile cover its code lines
//    exactly -- then a 4 x 4 transpose across the wave's 16-lane rows
//    (v_permlane32_swap, v_permlane16_swap) leaves in register j the dword a
//    of group j, which is what the B operand of the MFMA wants from that lane;
//  * activations: the A operand comes straight from global memory (x is a
//    few hundred KB and stays in L2), 16 bytes per lane per group and m-tile,
//    and is reused by the 4 n-tiles;
//  * the next half tile's weights (and, for MT = 1, activations) are loaded
//    while the current one computes.
#include "qg_common.h"
#include "w4_common.h"

namespace qg {


// (row r, register j) -> (row j, register r) over the wave's four 16-lane rows:
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with the
// lower 32 of its second, v_permlane16_swap the odd 16-lane rows of the first
// with the even rows of the second (both checked on MI355X).
__device__ __forceinline__ void transpose_rows4(u32x4_t& v) {
  const auto s02 = __builtin_amdgcn_permlane32_swap(v.x, v.z, false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(v.y, v.w, false, false);
  const auto t01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
  const auto t23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
  v = u32x4_t{t01[0], t01[1], t23[0], t23[1]};
}

// bf16 pairs (128 + q) of nibbles 2e, 2e+1 of a code dword, in plain C: the
// result feeds an MFMA source operand, and the compiler must see the VALU op
// that writes it to insert the wait states the MFMA read needs (an inline-asm
// v_and_or_b32 here, invisible to it, gave corrupted products on MI355X).
// `mask_s` holds 0x000F000F in an SGPR and `magic_v` 0x43004300 in a VGPR, so
// the and + or select to one v_and_or_b32 (VOP3 takes no 32-bit literal).
__device__ __forceinline__ uint32_t nibble_pair_mfma(uint32_t w, int e, uint32_t mask_s,
                                                     uint32_t magic_v) {
  return ((w >> (4 * e)) & mask_s) | magic_v;
}

// Tile geometry of the packed weight: HB = 0 is the INT4 layout (version 1);
// HB = 1, 2 the INT5 / INT6 layout (low nibbles as INT4, then HB high-bit
// planes, fp16 scales, one zero-point byte per group; see WnLayout).
// DQ: the INT4 layout with scale codes (version 2): a 128-byte head of row
// steps per 64-row block, tiles of 8960 bytes, a group's scale = its uint8
// code times its row's step.
template <int HB, bool DQ = false>
struct MfmaTile {
  static constexpr int kBytes = DQ ? kDqTileBytes : (HB == 0 ? kTileBytes : WnLayout<HB>::kTile);
  static constexpr int kScale = DQ ? kDqScodeOff : (HB == 0 ? kScaleOff : WnLayout<HB>::kS);
  static constexpr int kZero = DQ ? kDqZeroOff : (HB == 0 ? kZeroOff : WnLayout<HB>::kZ);
  static constexpr int kHead = DQ ? kDqHeadBytes : 0;
  __device__ static const uint8_t* block(const uint8_t* packed, int rb, int kt_count) {
    return packed + (size_t)rb * (kHead + (size_t)kt_count * kBytes);
  }
};

// The high-bit plane of a (group a, row) chunk as the four registers whose
// transpose (transpose_rows4) leaves in lane (i, a) register j the plane dword
// holding the high bits of code dword a of group j: INT5 has one plane dword
// for all four code dwords, INT6 one per pair of them (dword a/2).
template <int HB>
__device__ __forceinline__ u32x4_t plane_for_transpose(const u32x2_t& p) {
  if constexpr (HB == 1)
    return u32x4_t{p.x, p.x, p.x, p.x};
  else
    return u32x4_t{p.x, p.x, p.y, p.y};
}

// bf16 pair (128 + q) of nibble pair e of code dword `dw` (this lane's code
// dword a of a group), with the high bits from that group's plane dword `pw`
// (plain C, as nibble_pair_mfma).
template <int HB>
__device__ __forceinline__ uint32_t wide_pair_mfma(uint32_t dw, uint32_t pw, int a, int e, uint32_t mask_s,
                                                   uint32_t magic_v) {
  const uint32_t lo = nibble_pair_mfma(dw, e, mask_s, magic_v);
  if constexpr (HB == 0) return lo;
  const uint32_t hi = HB == 1 ? (pw >> (4 * a + e)) & 0x00010001u
                              : (pw >> (8 * (a & 1) + 2 * e)) & 0x00030003u;
  return lo | (hi << 4);
}

constexpr int kNT = 4;   // n-tiles of 16 rows per wave: a whole 64-row block

template <int MT, int HB, bool AS = false>
struct MfmaUnit {
  u32x4_t w[kNT];      // code chunks (group a, row 16t + i), transposed after the load
  u32x2_t hp[HB > 0 ? kNT : 1];   // their high-bit planes (INT5 / INT6)
  u32x2_t scl;         // fp16 scales of row `lane` (the half tile's 4 groups)
  uint32_t zwl;        // zero points of row `lane` (16 bits of nibbles; INT5/6: 4 bytes)
  u32x4_t xa[MT][4];   // A operands: x[16 mt + i][32 g + 8 a .. + 8] per group g
  f32x4_t sxa[AS ? MT : 1][AS ? 4 : 1];   // activation scales of rows 16 mt + 4a + e, per group g
};

// A wave owns one 64-row block (the 4 n-tiles) for a range of half tiles.
// PIPE: software pipeline over two register sets (PFX: the next unit's
// activations too), or load-wait-compute per unit with the other resident
// waves covering the latency.
// AS (W4A8 with one activation scale per group of 32): x holds the int8 codes
// xq (exact bf16 integers), act_scale their scales group-major, sx of row r
// and group g at act_scale[64 g + r]; each group's integer dot is multiplied
// by s[n,g] * sx[m,g] before it is added.
template <int MT, int KW, int MG, bool PIPE, bool PFX, int HB = 0, bool DQ = false, bool RS = false,
          bool AS = false>
__global__ __launch_bounds__(KW * MG * 64) void w4a16_mfma_kernel(
    const uint16_t* __restrict__ x, int m, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split,
    const float* __restrict__ row_scale, const float* __restrict__ act_scale) {
  constexpr int WAVES = KW * MG;
  __shared__ f32x4_t red[WAVES][kNT][64];
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, a = lane >> 4;
  const int wave = wave_id_uniform();
  const int kw = wave % KW, mg = wave / KW;
  const int rb = blockIdx.x;
  const int kt_count = k >> 8;
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  using T = MfmaTile<HB, DQ>;
  const uint8_t* blk = T::block(packed, rb, kt_count);
  const uint8_t* tiles = blk + T::kHead;
  // scale codes: the steps of rows 16t + i, the rows this lane's scales belong to
  float stp[kNT];
#pragma unroll
  for (int t = 0; t < kNT; ++t)
    stp[t] = DQ ? fp16_to_f32(*reinterpret_cast<const uint16_t*>(blk + 2 * (16 * t + i))) : 1.0f;
  const uint32_t mask_s = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t magic_v = 0x43004300u;
  asm volatile("" : "+v"(magic_v));     // an empty asm: keeps the constant in a VGPR
  uint32_t one2 = 0x3f803f80u;          // bf16 pair (1, 1), kept in a VGPR
  asm volatile("" : "+v"(one2));
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{one2, one2, one2, one2});

  // Codes: lane (i, a) loads the chunk of group a, row 16t + i.  Scales and
  // zero points: lane l loads those of row l only (one 8-byte and one 2-byte
  // load per half tile; per n-tile loads with 4 lanes per row cost a quarter
  // of the kernel's time); compute() hands row 16t + i to lane (i, a).
  // Through a buffer view of the (wave-uniform) tile: 32-bit lane offsets.
  auto load_w = [&](MfmaUnit<MT, HB, AS>& u, int hs) {
    const BufView v(tiles + (size_t)(hs >> 1) * T::kBytes, T::kBytes);
    const int half = hs & 1;
#pragma unroll
    for (int t = 0; t < kNT; ++t) {
      const uint32_t r = (uint32_t)((4 * half + a) * kTileRows + 16 * t + i);
      u.w[t] = v.b128<true>(r * 16u);
      if constexpr (HB == 1) u.hp[t].x = v.b32<true>(8192u + r * 4u);
      if constexpr (HB == 2) u.hp[t] = v.b64<true>(8192u + r * 8u);
    }
    if constexpr (DQ)
      u.scl = u32x2_t{v.b32((uint32_t)(T::kScale + lane * 8 + 4 * half)), 0u};
    else
      u.scl = v.b64((uint32_t)(T::kScale + lane * 16 + 8 * half));
    if constexpr (HB == 0)
      u.zwl = v.b16((uint32_t)(T::kZero + lane * 4 + 2 * half));
    else
      u.zwl = v.b32((uint32_t)(T::kZero + lane * 8 + 4 * half));
  };
  // Rows of x at or past m read row m - 1 instead (a valid address, no
  // branch and no select): output row r of an MFMA depends on row r of its A
  // operand only, and those rows are never stored.
  auto load_x = [&](MfmaUnit<MT, HB, AS>& u, int hs) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int row = min(16 * (mg * MT + mt) + i, m - 1);
      const uint16_t* xr = x + (size_t)row * k + (size_t)hs * 128 + 8 * a;
#pragma unroll
      for (int g = 0; g < 4; ++g) u.xa[mt][g] = *reinterpret_cast<const u32x4_t*>(xr + 32 * g);
      if constexpr (AS) {
        // rows 16 mt + 4a .. + 3 of groups 4 hs .. 4 hs + 3 (rows past m are
        // read but never stored)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          u.sxa[mt][g] = *reinterpret_cast<const f32x4_t*>(act_scale + (size_t)(4 * hs + g) * 64 +
                                                           16 * (mg * MT + mt) + 4 * a);
      }
    }
  };

  f32x4_t acc[kNT][MT];
#pragma unroll
  for (int t = 0; t < kNT; ++t)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[t][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](MfmaUnit<MT, HB, AS>& u) {
#pragma unroll
    for (int t = 0; t < kNT; ++t) transpose_rows4(u.w[t]);
    u32x4_t hr[kNT];
    if constexpr (HB > 0) {
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        hr[t] = plane_for_transpose<HB>(u.hp[t]);
        transpose_rows4(hr[t]);
      }
    }
    // Row 16t + i's metadata to lane (i, a): the same transpose applied to
    // four copies of a register leaves row t of it, in register t, in every
    // 16-lane row.
    u32x4_t s0{u.scl.x, u.scl.x, u.scl.x, u.scl.x}, s1{u.scl.y, u.scl.y, u.scl.y, u.scl.y};
    u32x4_t zz{u.zwl, u.zwl, u.zwl, u.zwl};
    transpose_rows4(s0);
    transpose_rows4(s1);
    transpose_rows4(zz);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4_t xg[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xg[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, u.xa[mt][g]), ones,
                                                        f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        const uint32_t dw = u.w[t][g];
        const uint32_t pw = HB > 0 ? hr[t][g] : 0u;
        uint32_t bp[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) bp[e] = wide_pair_mfma<HB>(dw, pw, a, e, mask_s, magic_v);
        const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, u32x4_t{bp[0], bp[1], bp[2], bp[3]});
        const uint32_t sw = g < 2 ? s0[t] : s1[t];
        const float s = DQ ? (float)((s0[t] >> (8 * g)) & 0xffu) * stp[t]
                           : fp16_to_f32((sw >> (16 * (g & 1))) & 0xffffu);
        const uint32_t zp = HB == 0 ? (zz[t] >> (4 * g)) & 15u : (zz[t] >> (8 * g)) & 0xffu;
        const float zb = (float)(zp | 0x80u);   // 128 + zp (zp <= 63)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8_t, u.xa[mt][g]), bv, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float se = AS ? s * u.sxa[mt][g][e] : s;
            acc[t][mt][e] = __builtin_fmaf(se, __builtin_fmaf(-zb, xg[mt][e], p[e]), acc[t][mt][e]);
          }
        }
      }
      // keep each group's MFMA results from being hoisted into the next group
      // (their registers would all be live at once)
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Software pipeline over two register sets used in turn (no copies): the
  // next unit's loads are issued before the current unit computes.  The loop
  // conditions are wave-uniform.
  const int h_end = 2 * t1;
  int hs = 2 * t0 + kw;
  if constexpr (!PIPE) {
    for (; hs < h_end; hs += KW) {
      MfmaUnit<MT, HB, AS> u;
      load_w(u, hs);
      load_x(u, hs);
      compute(u);
    }
  } else if (hs < h_end) {
    MfmaUnit<MT, HB, AS> ua, ub;
    load_w(ua, hs);
    load_x(ua, hs);
    while (true) {
      if (hs + KW >= h_end) { compute(ua); break; }
      load_w(ub, hs + KW);
      if constexpr (PFX) load_x(ub, hs + KW);
      compute(ua);
      if constexpr (!PFX) load_x(ub, hs + KW);
      hs += KW;
      if (hs + KW >= h_end) { compute(ub); break; }
      load_w(ua, hs + KW);
      if constexpr (PFX) load_x(ua, hs + KW);
      compute(ub);
      if constexpr (!PFX) load_x(ua, hs + KW);
      hs += KW;
    }
  }

  // ---- the KW partial sums of each m-tile, in wave order; lane (i, a) of
  // n-tile t holds rows 4a + e of column 16t + i.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int t = 0; t < kNT; ++t) red[wave][t][lane] = acc[t][mt];
    __syncthreads();
    for (int q = threadIdx.x; q < MG * kNT * 64; q += WAVES * 64) {
      const int l = q & 63, t = (q >> 6) % kNT, g = q / (kNT * 64);
      f32x4_t v = red[g * KW][t][l];
      for (int w = 1; w < KW; ++w) {
        const f32x4_t r = red[g * KW + w][t][l];
        v = f32x4_t{v[0] + r[0], v[1] + r[1], v[2] + r[2], v[3] + r[3]};
      }
      const int col = rb * kTileRows + 16 * t + (l & 15);
      if (col < n) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * (g * MT + mt) + 4 * (l >> 4) + e;
          if (row < m) {
            if (partial != nullptr) {
              partial[((size_t)blockIdx.y * m + row) * n + col] = v[e];
            } else {
              float o = v[e];
              if constexpr (RS) o *= row_scale[row];
              if (y_f32)
                static_cast<float*>(y)[(size_t)row * n + col] = o;
              else
                static_cast<uint16_t*>(y)[(size_t)row * n + col] = (uint16_t)f32_to_bf16_rne(o);
            }
          }
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// LDS-staged form (17..64 rows): a workgroup is one 64-row block of 4 MG
// waves (wave w: n-tile w % 4, m-tiles MT (w / 4) .. + MT) and streams x
// through LDS one 256-k tile at a time, shared by all its waves; a wave keeps
// its MT m-tiles of its n-tile in registers, so a weight operand is expanded
// once for MT products (and by MG waves).  The launchers take MG = 1 (all
// m-tiles of a row block in one wave: the decode is the largest share of a
// wave's issue time, so it is spread over as many products as possible).
// The zero point rides in a
// second MFMA per product whose B operand is -(128 + zp) in every slot (an
// exact bf16), so each group ends with one FMA per output: y += s * D.
//
// Pipeline: while tile kt is computed, tile kt+1's activations are copied
// into the other LDS buffer by global_load_lds_dwordx4 (no VGPRs) and its
// codes and metadata are loaded into the other register set; one barrier per
// tile.  From 33 rows a single x buffer (copied between two barriers) leaves
// room for more workgroups per CU, which overlap each other's copies.  LDS layout: 16-byte piece c of x row r (k = 8c .. 8c+8 of the tile)
// sits at piece index 32 r + (c ^ (r & 15)), so the A-operand read of lanes
// (i, a) = (lane % 16, lane / 16) -- row 16 mt + i, piece 4 g + a -- hits 16
// distinct bank quads in any 16 consecutive lanes; the swizzle is applied on
// the global side of the copy, whose LDS side is 64 consecutive pieces.
template <int HB>
struct Mfma2W {
  u32x4_t c0, c1;   // code chunks of groups a and 4 + a, row 16t + i
  u32x2_t h0, h1;   // their high-bit planes (INT5 / INT6)
  u32x4_t sc;       // the row's 8 fp16 scales
  u32x2_t zw;       // the row's 8 zero points (nibbles in .x; INT5/6: 8 bytes)
};

// AS: as for the register form; the tile's 8 groups x 64 rows of activation
// scales are copied into LDS with its activations.
template <int MT, int MG, int HB = 0, bool DQ = false, bool RS = false, bool AS = false>
__global__ __launch_bounds__(256 * MG) void w4a16_mfma2_kernel(
    const uint16_t* __restrict__ x, int m, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split,
    const float* __restrict__ row_scale, const float* __restrict__ act_scale) {
  constexpr int MR = 16 * MT * MG;                 // staged x rows
  // x buffers: two (the next tile copied while this one computes) up to 32
  // rows; one from 33 rows, where a second 24-32 KB buffer would leave room
  // for only 2 workgroups per CU while the registers allow 3-4: the other
  // workgroups of the CU then fill each one's copy time (measured on MI355X,
  // us, one / two buffers: 64 rows 39936 x 6656 83.1 / 90.9, 8448 x 6656
  // 29.5 / 31.9, per-group W4A8 39936 x 6656 97.8 / 112.6; 48 rows 39936 x
  // 6656 66.8 / 71.5).
  constexpr int NB = MT >= 3 ? 1 : 2;
  __shared__ __attribute__((aligned(16))) uint8_t xs[NB][MR * 512];
  __shared__ __attribute__((aligned(16))) float sxs[AS ? NB : 1][AS ? 8 * 64 : 4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int i = lane & 15, a = lane >> 4;
  const int wv = wave_id_uniform();
  const int t = wv & 3;                            // n-tile: rows 16t .. 16t+15 of the block
  const int mg = wv >> 2;                          // m-tiles mg MT .. mg MT + MT - 1
  const int rb = blockIdx.x;
  const int kt_count = k >> 8;
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  using T = MfmaTile<HB, DQ>;
  const uint8_t* blk = T::block(packed, rb, kt_count);
  const uint8_t* tiles = blk + T::kHead;
  // scale codes: the step of this lane's row 16t + i
  const float stp = DQ ? fp16_to_f32(*reinterpret_cast<const uint16_t*>(blk + 2 * (16 * t + i))) : 1.0f;
  const uint32_t mask_s = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t magic_v = 0x43004300u;
  asm volatile("" : "+v"(magic_v));

  // Copy x[:, 256 kt .. +256] into xs[buf]: wave t issues pieces 64u .. 64u+63
  // for u = t, t + 4, ...; rows at or past m repeat row m - 1 (their outputs
  // are never stored).
  // (a fixed count per wave: with the bound on wv unknown to the compiler,
  // a loop to MR / 2 kept a branch per copy and 14 more VGPRs at 64 rows)
  constexpr int NJ = MR / 2 / (4 * MG);           // copies per wave and tile
  static_assert(NJ * 4 * MG * 2 == MR, "every wave issues the same number of copies");
  auto stage = [&](int kt, int buf) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int u = wv + 4 * MG * j;
      const int r = 2 * u + (lane >> 5);
      const int c = (lane & 31) ^ (r & 15);
      const int src = r < m ? r : m - 1;
      __builtin_amdgcn_global_load_lds(x + (size_t)src * k + (size_t)kt * 256 + 8 * c,
                                       (__attribute__((address_space(3))) void*)(xs[buf] + 1024 * u),
                                       16, 0, 0);
    }
    if constexpr (AS) {
      // groups 8 kt .. 8 kt + 7, 64 rows each: 2 KB, contiguous in act_scale
      if (wv < 2)
        __builtin_amdgcn_global_load_lds(act_scale + (size_t)kt * 512 + 256 * wv + 4 * lane,
                                         (__attribute__((address_space(3))) void*)(&sxs[buf][256 * wv]),
                                         16, 0, 0);
    }
  };
  // Through a buffer view of the (uniform) tile: 32-bit lane offsets.
  auto load_w = [&](Mfma2W<HB>& w, int kt) {
    const BufView v(tiles + (size_t)kt * T::kBytes, T::kBytes);
    const uint32_t r0 = (uint32_t)(a * kTileRows + 16 * t + i), r1 = r0 + 4 * kTileRows;
    const uint32_t row = (uint32_t)(16 * t + i);
    w.c0 = v.b128<true>(r0 * 16u);
    w.c1 = v.b128<true>(r1 * 16u);
    if constexpr (HB == 0) {
      // unused, but set: left undefined, the copies between the two register
      // sets kept a stack slot that the compiler moved into LDS
      w.h0 = u32x2_t{0u, 0u};
      w.h1 = u32x2_t{0u, 0u};
    }
    if constexpr (HB == 1) {
      w.h0.x = v.b32<true>(8192u + r0 * 4u);
      w.h1.x = v.b32<true>(8192u + r1 * 4u);
    }
    if constexpr (HB == 2) {
      w.h0 = v.b64<true>(8192u + r0 * 8u);
      w.h1 = v.b64<true>(8192u + r1 * 8u);
    }
    if constexpr (DQ) {
      const u32x2_t c8 = v.b64((uint32_t)T::kScale + row * 8u);
      w.sc = u32x4_t{c8.x, c8.y, 0u, 0u};
    } else {
      w.sc = v.b128<false>((uint32_t)T::kScale + row * 16u);
    }
    if constexpr (HB == 0)
      w.zw.x = v.b32((uint32_t)T::kZero + row * 4u);
    else
      w.zw = v.b64((uint32_t)T::kZero + row * 8u);
  };
  // Every wave's copies into LDS must have landed before the barrier that
  // hands the buffer to the other waves.
  auto sync = [&]() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Per group: 2 MT products (all code products first, then all zero-point
  // products, so dependent pairs are MT instructions apart), and the previous
  // group's scale FMAs while these are in flight.
  auto compute = [&](Mfma2W<HB>& w, int buf) {
    transpose_rows4(w.c0);
    transpose_rows4(w.c1);
    u32x4_t hr0{}, hr1{};
    if constexpr (HB > 0) {
      hr0 = plane_for_transpose<HB>(w.h0);
      hr1 = plane_for_transpose<HB>(w.h1);
      transpose_rows4(hr0);
      transpose_rows4(hr1);
    }
    const uint8_t* xb = xs[buf];
    f32x4_t dp[MT];
    float sp = 0.0f;
    f32x4_t sxp[AS ? MT : 1];     // the previous group's activation scales
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const uint32_t dw = g < 4 ? w.c0[g] : w.c1[g - 4];
      const uint32_t pw = HB > 0 ? (g < 4 ? hr0[g] : hr1[g - 4]) : 0u;
      uint32_t bp[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) bp[e] = wide_pair_mfma<HB>(dw, pw, a, e, mask_s, magic_v);
      const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, u32x4_t{bp[0], bp[1], bp[2], bp[3]});
      const uint32_t z = HB == 0 ? (w.zw.x >> (4 * g)) & 15u
                                 : ((g < 4 ? w.zw.x : w.zw.y) >> (8 * (g & 3))) & 0xffu;
      const uint32_t zn = (z | (z << 16)) | 0xC300C300u;     // bf16 pair -(128 + zp)
      const bf16x8_t bz = __builtin_bit_cast(bf16x8_t, u32x4_t{zn, zn, zn, zn});
      const float s = DQ ? (float)((w.sc[g >> 2] >> (8 * (g & 3))) & 0xffu) * stp
                         : fp16_to_f32((w.sc[g >> 1] >> (16 * (g & 1))) & 0xffffu);
      bf16x8_t av[MT];
      f32x4_t d[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = 16 * (mg * MT + mt) + i;
        av[mt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                  xb + 16 * (32 * r + ((4 * g + a) ^ (r & 15)))));
        d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bv, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        d[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bz, d[mt], 0, 0, 0);
      if (g > 0) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[mt][e] = __builtin_fmaf(AS ? sp * sxp[mt][e] : sp, dp[mt][e], acc[mt][e]);
            // pin the update here: left alone, the compiler sinks every
            // group's FMAs past the tile's barrier and keeps all 8 groups'
            // products live
            asm volatile("" : "+v"(acc[mt][e]));
          }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) dp[mt] = d[mt];
      sp = s;
      if constexpr (AS) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          sxp[mt] = *reinterpret_cast<const f32x4_t*>(&sxs[buf][64 * g + 16 * (mg * MT + mt) + 4 * a]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[mt][e] = __builtin_fmaf(AS ? sp * sxp[mt][e] : sp, dp[mt][e], acc[mt][e]);
        asm volatile("" : "+v"(acc[mt][e]));
      }
  };

  if (t0 < t1) {
    Mfma2W<HB> cur;
    stage(t0, 0);
    load_w(cur, t0);
    sync();
    for (int kt = t0; kt < t1; ++kt) {
      Mfma2W<HB> nxt = cur;
      const bool more = kt + 1 < t1;            // uniform
      if constexpr (NB == 2) {
        if (more) {
          stage(kt + 1, (kt + 1 - t0) & 1);
          load_w(nxt, kt + 1);
        }
        compute(cur, (kt - t0) & 1);
        cur = nxt;
        if (more) sync();
      } else {
        // one buffer: the codes still go a tile ahead; x is copied once
        // every wave is done with the tile before
        if (more) load_w(nxt, kt + 1);
        compute(cur, 0);
        cur = nxt;
        if (more) {
          __syncthreads();
          stage(kt + 1, 0);
          sync();
        }
      }
    }
  }

  // lane (i, a) holds rows 16 mt + 4a + e of column 16t + i of the block
  const int col = rb * kTileRows + 16 * t + i;
  if (col < n) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 16 * (mg * MT + mt) + 4 * a + e;
        if (row < m) {
          if (partial != nullptr) {
            partial[((size_t)blockIdx.y * m + row) * n + col] = acc[mt][e];
          } else {
            float o = acc[mt][e];
            if constexpr (RS) o *= row_scale[row];
            if (y_f32)
              static_cast<float*>(y)[(size_t)row * n + col] = o;
            else
              static_cast<uint16_t*>(y)[(size_t)row * n + col] = (uint16_t)f32_to_bf16_rne(o);
          }
        }
      }
  }
}

template <int MT, int MG = 1, int HB = 0, bool DQ = false, bool RS = false, bool AS = false>
static hipError_t launch_mfma2_t(const void* x, int m, const void* packed, int n, int k, void* y,
                                 int y_f32, float* partial, int split, hipStream_t stream,
                                 const float* row_scale = nullptr, const float* act_scale = nullptr) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  hipLaunchKernelGGL((w4a16_mfma2_kernel<MT, MG, HB, DQ, RS, AS>), dim3(rbs, split), dim3(256 * MG), 0, stream,
                     static_cast<const uint16_t*>(x), m, static_cast<const uint8_t*>(packed), n, k,
                     y, y_f32, partial, split, row_scale, act_scale);
  return hipGetLastError();
}

template <int MT, int KW, int MG, bool PIPE, bool PFX, int HB = 0, bool DQ = false, bool RS = false,
          bool AS = false>
static hipError_t launch_mfma_t(const void* x, int m, const void* packed, int n, int k, void* y,
                                int y_f32, float* partial, int split, hipStream_t stream,
                                const float* row_scale = nullptr, const float* act_scale = nullptr) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  hipLaunchKernelGGL((w4a16_mfma_kernel<MT, KW, MG, PIPE, PFX, HB, DQ, RS, AS>), dim3(rbs, split),
                     dim3(KW * MG * 64), 0, stream, static_cast<const uint16_t*>(x), m,
                     static_cast<const uint8_t*>(packed), n, k, y, y_f32, partial, split, row_scale,
                     act_scale);
  return hipGetLastError();
}

// Register form, up to 16 rows: one m-tile per wave, 4 waves along K,
// pipelined with activation prefetch (measured on MI355X at 39936 x 6656,
// 8448 x 6656 and 6656 x 19968).  The same template with 2 m-tiles per wave
// or wave groups along M ran 32..64 rows before the LDS-staged form, which
// is faster there (39936 x 6656: 32 rows 57.4 us against 52.7, 64 rows 115.5
// against 91.9 in the LDS form's 2 x 2 mapping of then, 87.5 in its 4 x 1).
template <bool RS>
static hipError_t launch_w4a16_mfma_rs(int m, const void* x, const void* packed, int n, int k, void* y,
                                      int y_f32, float* partial, int split, hipStream_t stream,
                                      const float* row_scale) {
#define QG_MF(MT, KW, MG, PIPE, PFX) \
  return launch_mfma_t<MT, KW, MG, PIPE, PFX, 0, false, RS>(x, m, packed, n, k, y, y_f32, partial, split, stream, row_scale)
  if (mfma_lds_form(m)) {
    // (m-tiles per wave, waves per n-tile): every m-tile in one wave, so that
    // each wave's weight decode serves them all.  Measured on MI355X against
    // the forms with wave groups along M (us; 4 x 1: 144 VGPRs, 2 waves per
    // SIMD): 64 rows as 4 x 1 against 2 x 2 (and 1 x 4), 39936 x 6656 87.5
    // against 95.7 (131.2), 8448 x 6656 31.4 against 32.9, 6656 x 19968 47.7
    // against 52.2, 32768 x 8192 80.0 against 87.5; 48 rows as 3 x 1 against
    // 1 x 3, 8448 x 6656 23.9 against 30.9, 6656 x 19968 40.2 against 52.0,
    // 6656 x 4096 15.4 against 18.1.
    switch ((m + 15) / 16) {
      case 2: return launch_mfma2_t<2, 1, 0, false, RS>(x, m, packed, n, k, y, y_f32, partial, split, stream, row_scale);
      case 3: return launch_mfma2_t<3, 1, 0, false, RS>(x, m, packed, n, k, y, y_f32, partial, split, stream, row_scale);
      case 4: return launch_mfma2_t<4, 1, 0, false, RS>(x, m, packed, n, k, y, y_f32, partial, split, stream, row_scale);
      default: return hipErrorInvalidValue;
    }
  }
  QG_MF(1, 4, 1, true, true);
#undef QG_MF
}

// row_scale (optional, [m] fp32): each row's result times its scale before
// the store; only where the kernel writes y itself (no partial sums).
hipError_t launch_w4a16_mfma(int m, const void* x, const void* packed, int n, int k, void* y,
                             int y_f32, float* partial, int split, hipStream_t stream,
                             const float* row_scale) {
  if (row_scale != nullptr && partial == nullptr)
    return launch_w4a16_mfma_rs<true>(m, x, packed, n, k, y, y_f32, partial, split, stream, row_scale);
  return launch_w4a16_mfma_rs<false>(m, x, packed, n, k, y, y_f32, partial, split, stream, nullptr);
}

// INT5 / INT6 and the scale-code INT4 layout on the same two forms and the
// same bucket choice as INT4.
template <int HB, bool DQ = false, bool RS = false, bool AS = false>
static hipError_t launch_wn_mfma_t(int m, const void* x, const void* packed, int n, int k, void* y,
                                   int y_f32, float* partial, int split, hipStream_t stream,
                                   const float* row_scale = nullptr, const float* act_scale = nullptr) {
#define QG_MF2(MT, MG) \
  launch_mfma2_t<MT, MG, HB, DQ, RS, AS>(x, m, packed, n, k, y, y_f32, partial, split, stream, row_scale, act_scale)
  if (mfma_lds_form(m)) {
    switch ((m + 15) / 16) {
      case 2: return QG_MF2(2, 1);
      case 3: return QG_MF2(3, 1);
      case 4: return QG_MF2(4, 1);
      default: return hipErrorInvalidValue;
    }
  }
#undef QG_MF2
  return launch_mfma_t<1, 4, 1, true, true, HB, DQ, RS, AS>(
      x, m, packed, n, k, y, y_f32, partial, split, stream, row_scale, act_scale);
}

hipError_t launch_wn_a16_mfma(int bits, int m, const void* x, const void* packed, int n, int k, void* y,
                              int y_f32, float* partial, int split, hipStream_t stream) {
  if (bits == 5) return launch_wn_mfma_t<1>(m, x, packed, n, k, y, y_f32, partial, split, stream);
  if (bits == 6) return launch_wn_mfma_t<2>(m, x, packed, n, k, y, y_f32, partial, split, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_w4a16_mfma_dq(int m, const void* x, const void* packed, int n, int k, void* y, int y_f32,
                                float* partial, int split, hipStream_t stream, const float* row_scale) {
  if (row_scale != nullptr && partial == nullptr)
    return launch_wn_mfma_t<0, true, true>(m, x, packed, n, k, y, y_f32, partial, split, stream, row_scale);
  return launch_wn_mfma_t<0, true>(m, x, packed, n, k, y, y_f32, partial, split, stream);
}

// W4A8 with one activation scale per group of 32, 5..64 rows: x holds the
// int8 codes as exact bf16 integers and act_scale their scales group-major
// (64 per group); both packed layouts, the W4A16 forms and bucket choice.
hipError_t launch_w4a8g_mfma(bool dq, int m, const void* xq, const float* act_scale, const void* packed, int n,
                             int k, void* y, int y_f32, float* partial, int split, hipStream_t stream) {
  if (dq)
    return launch_wn_mfma_t<0, true, false, true>(m, xq, packed, n, k, y, y_f32, partial, split, stream, nullptr,
                                                  act_scale);
  return launch_wn_mfma_t<0, false, false, true>(m, xq, packed, n, k, y, y_f32, partial, split, stream, nullptr,
                                                 act_scale);
}

}  // namespace qg
