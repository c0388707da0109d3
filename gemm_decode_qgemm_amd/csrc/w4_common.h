// w4_common.h -- pieces shared by the kernels that read the packed INT4
// group-32 weight (layout v1, include/qgemm.h): the per-lane half-tile load,
// the split-K partition and a DPP move helper.  Internal header.
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

template <bool NT>
__device__ __forceinline__ void load_half(HalfRegs& r, const uint8_t* tile, int half, int lane) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r.c[j] = load_stream<NT>(
        reinterpret_cast<const u32x4_t*>(tile + ((4 * half + j) * kTileRows + lane) * 16));
  // Scales and zero points of the two half tiles share 128-byte lines, and
  // the other half is read by another wave of the same workgroup moments
  // later: these loads keep the default (temporal) policy so that wave hits
  // in L2 instead of fetching the line from HBM again.
  r.sc = load_stream<false>(reinterpret_cast<const u32x2_t*>(tile + kScaleOff + lane * 16 + 8 * half));
  r.zw = load_stream<false>(reinterpret_cast<const uint16_t*>(tile + kZeroOff + lane * 4 + 2 * half));
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

template <bool NT>
__device__ __forceinline__ void load_half32(Half32Regs& r, const uint8_t* tile, int half, int lg,
                                            int row) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
    r.c[j] = load_stream<NT>(
        reinterpret_cast<const u32x4_t*>(tile + ((4 * half + 2 * lg + j) * kTileRows + row) * 16));
  // Temporal, as in load_half: the other half tile's metadata shares these lines.
  r.sc = load_stream<false>(reinterpret_cast<const uint32_t*>(tile + kScaleOff + row * 16 + 8 * half + 4 * lg));
  r.zb = load_stream<false>(tile + kZeroOff + row * 4 + 2 * half + lg);
}

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
