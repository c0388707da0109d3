// dispatch.h -- host-side dispatch rules of the C ABI (include/qgemm.h):
// the split-K table for split_k = 0 and the GEMV workgroup shape, measured
// on MI355X.  Internal header of the host-side launch code.
#pragma once

#include <stdint.h>

#include "qgemm.h"
#include "qg_common.h"

namespace qg {

// Split-K default, measured on MI355X at the decode layer shapes.
//  * M <= 4 (GEMV, 32-row workgroups): one split whenever the grid has at
//    least half a workgroup per CU (N >= 4096): a second split costs a second
//    launch and the partials' traffic, which the extra parallelism does not
//    repay at these shapes (6656 x 4096: 5.1 us at 1 against 7.1 at 2 for
//    M = 1, 5.4 against 7.4 for M = 4; 8448 x 6656, M = 4: 10.7 against
//    11.1); below that, the smallest split giving a workgroup per CU, at
//    most 4 (2048 x 8192, M = 4: 6.7 us at 4 against 7.4 at 1; 256 x 6656:
//    5.3 us at 4, 5.9 at 8).
//  * M > 4 (matrix-core kernels): the smallest split with 64-row blocks x
//    split >= 120 for the register form, at most 8 (6656 x 19968, M = 16:
//    24.7 us at 2 against 40.3 at 1; 8448 x 6656: 15.7 us at 1 against 17.7
//    at 2), >= 300 for the LDS-staged form (17..64 rows), whose workgroups
//    hold more LDS and need more of them in flight (8448 x 6656, M = 32: 19.6
//    us at 4 against 26.5 at 1; M = 64: 32.4 at 4 against 37.6 at 1).
// Both are capped by K / 256 (one tile per split).
inline int32_t default_split(int64_t m, int64_t n, int64_t k) {
  const int64_t kt = k / QG_TILE_K;
  int32_t s = 1;
  if (m <= 4) {
    const int64_t n32 = (n + 31) / 32;
    if (n32 >= kCUs / 2) return 1;
    while (s < 4 && 2 * s <= kt && n32 * s < kCUs) s *= 2;
    return s;
  }
  const int64_t rbs = (n + QG_TILE_ROWS - 1) / QG_TILE_ROWS;
  const int64_t want = qg::mfma_lds_form(m) ? 300 : 120;
  while (s < 8 && 2 * s <= kt && rbs * s < want) s *= 2;
  return s;
}

// Workgroup shape of the M <= 4 GEMVs: 32 rows and 16 waves, except with one
// split where the 32-row grid spills a few workgroups into a second round
// over the CUs while the 64-row grid fits in one (N = 8448: 264 against 132
// workgroups; M = 1: 9.1 us against 10.2).  The M = 2..4 matrix-instruction
// GEMV places two 32-row workgroups per CU, so once most CUs hold two its
// 32-row form wins again (measured, us, 64 / 32 rows: 8448 x 6656 M = 4
// 10.07 / 10.65, 10240 x 5120 M = 2 8.66 / 8.90, 12288 x 4096 M = 4 8.09 /
// 7.95, 16384 x 6656 M = 4 12.33 / 11.86): there 64 rows up to 160 blocks.
// The W4A8 M = 2..4 GEMV follows the same rule (8448 x 6656 M = 4: per row
// 12.3 / 14.4, per group of 32 11.35 / 12.9).
struct GemvShape {
  int rows, waves;
};
inline GemvShape gemv_shape(int64_t m, int64_t n, int32_t split) {
  const int64_t n32 = (n + 31) / 32, n64 = (n + 63) / 64;
  if (split == 1 && n32 > kCUs && n64 <= (m == 1 ? kCUs : kCUs * 5 / 8)) return {64, 16};
  return {32, 16};
}

// INT5 / INT6 on the matrix cores (M > 4) carry more work per weight than
// INT4, and more splits pay (measured on the INT6 layers of the 30B export,
// buckets 16 and 64: 5376 x 21504 best at 8, 4096 x 5376 and 6656 x 19968 at
// 4, 1024 x 6656 at 8): the smallest split with 64-row blocks x split >= 400,
// at most 8, and one step back when that leaves under 4 tiles of 256 k per
// workgroup while the grid still has a workgroup per CU.  M <= 4 keeps the
// INT4 rule (5376 x 21504 M = 1: 21.3 us at 1 against 19.9 at 4).
inline int32_t default_split_intn(int64_t m, int64_t n, int64_t k) {
  if (m <= 4) return default_split(m, n, k);
  const int64_t kt = k / QG_TILE_K;
  const int64_t rbs = (n + QG_TILE_ROWS - 1) / QG_TILE_ROWS;
  int32_t s = 1;
  while (s < 8 && 2 * s <= kt && rbs * s < 400) s *= 2;
  if (s > 1 && kt < 4 * s && rbs * (s / 2) >= kCUs) s /= 2;
  return s;
}

// W4A8 with one activation scale per group of 32, M > 4: the matrix-core
// kernels also load each group's activation scales and multiply them in, and
// above 32 rows more splits pay than for W4A16 (measured, µs, best split
// marked *: 39936 x 6656 M = 64: 126.5 at 1, 113.2* at 2; 8448 x 6656 M = 64:
// 42.9 at 4, 41.0* at 8, M = 48: 40.6 / 38.7*; 6656 x 4096 M = 64: 22.8* at
// 4, 27.8 at 8; the one loss, 6656 x 19968 M = 64: 67.8 at 4, 69.0 at 8):
// the smallest split with 64-row blocks x split >= 1200, at most 8, with at
// least 3 tiles of 256 k per split.  Up to 32 rows the W4A16 rule.
inline int32_t default_split_g32(int64_t m, int64_t n, int64_t k) {
  if (m <= 32) return default_split(m, n, k);
  const int64_t kt = k / QG_TILE_K;
  const int64_t rbs = (n + QG_TILE_ROWS - 1) / QG_TILE_ROWS;
  int32_t s = 1;
  while (s < 8 && kt >= 3 * (2 * s) && rbs * s < 1200) s *= 2;
  return s;
}

enum class SplitRule { kW4, kIntN, kW4A8G32 };

inline int32_t resolve_split(int64_t m, int64_t n, int64_t k, int32_t split_k, int32_t* out,
                             SplitRule rule = SplitRule::kW4) {
  if (split_k == 0) {
    *out = rule == SplitRule::kIntN     ? default_split_intn(m, n, k)
           : rule == SplitRule::kW4A8G32 ? default_split_g32(m, n, k)
                                         : default_split(m, n, k);
    return QG_OK;
  }
  if (split_k != 1 && split_k != 2 && split_k != 4 && split_k != 8) return QG_E_SPLIT;
  if (split_k > k / QG_TILE_K) return QG_E_SPLIT;
  *out = split_k;
  return QG_OK;
}

}  // namespace qg
