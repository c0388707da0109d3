// w4_common.h -- pieces shared by the kernels that read the packed weights
// (include/qgemm.h: INT4 layout v1, scale codes v2, INT5 / INT6): the raw
// buffer view the loads go through, the per-lane half-tile loads of each
// layout, the split-K partition and a DPP move helper.  Internal header.
#pragma once

#include "qg_common.h"

namespace qg {

// One half tile (4 groups = 128 k) of one lane's row: 4 code chunks, the 4
// fp16 scales (8 B) and the 4 zero points (16 bits of the row's zero word).
struct HalfRegs {
  u32x4_t c[4];
  u32x2_t sc;
  uint32_t zw;
};

// A raw buffer over `bytes` bytes at a wave-uniform `base`: its loads take an
// unsigned 32-bit per-lane offset and no vector address arithmetic (the
// descriptor lives in scalar registers, built per tile from the scalar tile
// address), and a read at or past `bytes` returns zero.  Cache policy of the
// streaming loads: non-temporal (bit 1 of the policy operand on gfx950).
struct BufView {
  __amdgpu_buffer_rsrc_t r;
  __device__ __forceinline__ BufView(const void* base, int bytes)
      : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000)) {}
  template <bool NT>
  __device__ __forceinline__ u32x4_t b128(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, NT ? 2 : 0);
  }
  template <bool NT = false>
  __device__ __forceinline__ u32x2_t b64(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, NT ? 2 : 0);
  }
  template <bool NT = false>
  __device__ __forceinline__ uint32_t b32(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, NT ? 2 : 0);
  }
  __device__ __forceinline__ uint32_t b16(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
  }
  __device__ __forceinline__ uint32_t b8(uint32_t off) const {
    return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
  }
};

// One half tile of one lane's row (64-row mapping: lane = row), through a
// buffer view of the tile (`tile` wave-uniform).  Codes are streamed
// non-temporally.  Scales and zero points of the two half tiles share
// 128-byte lines, and the other half is read by another wave of the same
// workgroup moments later: those loads keep the default (temporal) policy so
// that wave hits in L2 instead of fetching the line from HBM again.
// DQ (scale-code layout): sc.x holds the half's 4 uint8 scale codes instead.
template <bool DQ = false>
__device__ __forceinline__ void load_half(HalfRegs& r, const uint8_t* tile, int half, int lane) {
  const BufView v(tile, DQ ? kDqTileBytes : kTileBytes);
  const uint32_t co = (uint32_t)((4 * half * kTileRows + lane) * 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) r.c[j] = v.b128<true>(co + j * (kTileRows * 16));
  if constexpr (DQ) {
    r.sc = u32x2_t{v.b32((uint32_t)(kDqScodeOff + lane * 8 + 4 * half)), 0u};
    r.zw = v.b16((uint32_t)(kDqZeroOff + lane * 4 + 2 * half));
  } else {
    r.sc = v.b64((uint32_t)(kScaleOff + lane * 16 + 8 * half));
    r.zw = v.b16((uint32_t)(kZeroOff + lane * 4 + 2 * half));
  }
}

// The 32-row mapping: a workgroup owns rows [32h, 32h + 32) of a 64-row block
// (h = blockIdx.x & 1).  Lane l holds row 32h + (l & 31) and the group pair
// lg = l >> 5 of each half tile: groups 2lg and 2lg + 1, i.e. 2 code chunks
// (32 B), their 2 fp16 scales (4 B) and zero points (1 byte).  A wave-wide
// code load is two runs of 512 contiguous bytes; the tile's 128-byte lines
// hold 8 rows each, so the two halves of a block never share a code line.
struct Half32Regs {
  u32x4_t c[2];
  uint32_t sc;
  uint32_t zb;
};

// The two packed layouts seen by the 32-row kernels.  Version 1: tiles of
// 9472 bytes with fp16 scales.  Version 2 (scale codes): each 64-row block
// starts with a 128-byte head of fp16 row steps, its tiles are 8960 bytes,
// and a group's scale is its uint8 code times the row's step (exact in
// binary32: 8 x 11 significant bits).  Codes sit at the same place in both.
template <bool DQ>
struct W4Layout;

// Also used by the matrix-instruction GEMV: `pair` gives the bf16 pair
// (128 + q(8d+2e), 128 + q(8d+2e+1)) of group jj in plain C (it may feed a
// matrix-instruction operand), `zero` the group's zero point.
template <>
struct W4Layout<false> {
  using Regs = Half32Regs;
  static constexpr int kTile = kTileBytes;
  __device__ static const uint8_t* tiles(const uint8_t* packed, int rb, int kt_count, int, float& step) {
    step = 1.0f;
    return packed + (size_t)rb * kt_count * kTileBytes;
  }
  // One half tile of one lane's row and group pair (32-row mapping), through
  // a buffer view of the tile (`tile` wave-uniform); policies as load_half.
  __device__ static void load(Half32Regs& r, const uint8_t* tile, int half, int lg, int row) {
    const BufView v(tile, kTileBytes);
    const uint32_t co = (uint32_t)(((4 * half + 2 * lg) * kTileRows + row) * 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) r.c[j] = v.b128<true>(co + j * (kTileRows * 16));
    r.sc = v.b32((uint32_t)(kScaleOff + row * 16 + 8 * half + 4 * lg));
    r.zb = v.b8((uint32_t)(kZeroOff + row * 4 + 2 * half + lg));
  }
  // scale of group 2 lg + jj of the half tile
  __device__ static float scale(uint32_t sc, int jj, float) {
    return fp16_to_f32((sc >> (16 * jj)) & 0xffffu);
  }
  __device__ static uint32_t pair(const Regs& r, int jj, int d, int e, uint32_t mask_s, uint32_t magic_v) {
    return ((r.c[jj][d] >> (4 * e)) & mask_s) | magic_v;
  }
  __device__ static uint32_t zero(const Regs& r, int jj) { return (r.zb >> (4 * jj)) & 15u; }
};

template <>
struct W4Layout<true> {
  using Regs = Half32Regs;
  static constexpr int kTile = kDqTileBytes;
  __device__ static const uint8_t* tiles(const uint8_t* packed, int rb, int kt_count, int row, float& step) {
    const uint8_t* block = packed + (size_t)rb * (kDqHeadBytes + (size_t)kt_count * kDqTileBytes);
    step = fp16_to_f32(*reinterpret_cast<const uint16_t*>(block + 2 * row));
    return block + kDqHeadBytes;
  }
  __device__ static void load(Half32Regs& r, const uint8_t* tile, int half, int lg, int row) {
    const BufView v(tile, kDqTileBytes);
    const uint32_t co = (uint32_t)(((4 * half + 2 * lg) * kTileRows + row) * 16);
#pragma unroll
    for (int j = 0; j < 2; ++j) r.c[j] = v.b128<true>(co + j * (kTileRows * 16));
    r.sc = v.b16((uint32_t)(kDqScodeOff + row * 8 + 4 * half + 2 * lg));
    r.zb = v.b8((uint32_t)(kDqZeroOff + row * 4 + 2 * half + lg));
  }
  __device__ static float scale(uint32_t sc, int jj, float step) {
    return (float)((sc >> (8 * jj)) & 0xffu) * step;
  }
  __device__ static uint32_t pair(const Regs& r, int jj, int d, int e, uint32_t mask_s, uint32_t magic_v) {
    return ((r.c[jj][d] >> (4 * e)) & mask_s) | magic_v;
  }
  __device__ static uint32_t zero(const Regs& r, int jj) { return (r.zb >> (4 * jj)) & 15u; }
};

// INT5 / INT6 (HB = bits - 4 high-bit planes).  Tiles of 64 rows x 256 k:
// the low 4 bits of every code exactly as version 1, then the planes (a
// (4 HB)-byte chunk per group and row at 8192 + (j*64 + r)*4*HB), fp16
// scales (row r at +16r) and one zero-point byte per group (row r at +8r).
// The plane's bit order puts a pair's high bits where (dword >> 4e) &
// 0x000F000F puts its low bits, four places lower: INT5: (plane >> (4d + e))
// & 0x00010001; INT6: (plane dword d/2 >> (8(d%2) + 2e)) & 0x00030003.
// Codes up to 63 keep 128 + q exact in bf16.
template <int HB>
struct WnRegs {
  u32x4_t c[2];        // low-nibble chunks of groups 2lg, 2lg + 1
  uint32_t hp[2][HB];  // their high planes
  uint32_t sc;         // two fp16 scales
  uint32_t zb;         // two zero-point bytes
};

template <int HB>
struct WnLayout {
  using Regs = WnRegs<HB>;
  static constexpr int kTile = 8192 + 2048 * HB + 1536;
  static constexpr int kS = 8192 + 2048 * HB, kZ = kS + 1024;
  __device__ static const uint8_t* tiles(const uint8_t* packed, int rb, int kt_count, int, float& step) {
    step = 1.0f;
    return packed + (size_t)rb * kt_count * kTile;
  }
  // Through a buffer view of the tile (`tile` wave-uniform); the planes are
  // streamed like the codes, scales and zero points as in load_half.
  __device__ static void load(Regs& r, const uint8_t* tile, int half, int lg, int row) {
    const BufView v(tile, kTile);
    const int g0 = 4 * half;
    const uint32_t rl = (uint32_t)(2 * lg * kTileRows + row);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      r.c[j] = v.b128<true>((uint32_t)((g0 + j) * (kTileRows * 16)) + rl * 16u);
      if constexpr (HB == 1) {
        r.hp[j][0] = v.b32<true>((uint32_t)(8192 + (g0 + j) * (kTileRows * 4)) + rl * 4u);
      } else {
        const u32x2_t h = v.b64<true>((uint32_t)(8192 + (g0 + j) * (kTileRows * 8)) + rl * 8u);
        r.hp[j][0] = h.x;
        r.hp[j][1] = h.y;
      }
    }
    r.sc = v.b32((uint32_t)(kS + row * 16 + 8 * half + 4 * lg));
    r.zb = v.b16((uint32_t)(kZ + row * 8 + 4 * half + 2 * lg));
  }
  __device__ static float scale(uint32_t sc, int jj, float) {
    return fp16_to_f32((sc >> (16 * jj)) & 0xffffu);
  }
  __device__ static uint32_t high(const Regs& r, int jj, int d, int e) {
    if constexpr (HB == 1)
      return (r.hp[jj][0] >> (4 * d + e)) & 0x00010001u;
    else
      return (r.hp[jj][d >> 1] >> (8 * (d & 1) + 2 * e)) & 0x00030003u;
  }
  __device__ static uint32_t pair(const Regs& r, int jj, int d, int e, uint32_t mask_s, uint32_t magic_v) {
    return ((r.c[jj][d] >> (4 * e)) & mask_s) | magic_v | (high(r, jj, d, e) << 4);
  }
  __device__ static uint32_t zero(const Regs& r, int jj) { return (r.zb >> (8 * jj)) & 0xffu; }
};

// Split-K partition of `tiles` 256-k units into `split` contiguous ranges;
// the first (tiles % split) ranges take one extra unit.
__device__ __forceinline__ void split_range(int tiles, int split, int s, int& t0, int& t1) {
  const int base = tiles / split, rem = tiles % split;
  t0 = s * base + (s < rem ? s : rem);
  t1 = t0 + base + (s < rem ? 1 : 0);
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v),
                                                               CTRL, 0xf, 0xf, true));
}

}  // namespace qg
