// qg_common.h -- device helpers and layout constants shared by the HIP
// kernels of the quantized GEMV library (gfx950, wave64).  Internal header:
// the public contract is include/qgemm.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemm.h"

namespace qg {

// Packed INT4 layout, version 1 (see include/qgemm.h): tiles of 64 rows x
// 256 k, codes | fp16 scales | 4-bit zero points, 9472 bytes.
constexpr int kTileRows = 64;
constexpr int64_t kCUs = 256;   // compute units of an MI355X
constexpr int kTileK = 256;
constexpr int kGroupsPerTile = 8;
constexpr int kScaleOff = 8192;
constexpr int kZeroOff = 9216;
constexpr int kTileBytes = 9472;
// Version 2 (scale codes): a row block is a 128-byte head of the 64 rows'
// fp16 scale steps, then tiles of codes | uint8 scale codes | zero points.
constexpr int kDqHeadBytes = 128;
constexpr int kDqScodeOff = 8192;
constexpr int kDqZeroOff = 8704;
constexpr int kDqTileBytes = 8960;

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// binary32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float fp16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// sum = a.lo*b.lo + a.hi*b.hi + c on bf16 pairs (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// (a & mask) | c in one v_and_or_b32.  gfx9 VOP3 encodings take no 32-bit
// literal, so the mask rides in an SGPR and the constant in a VGPR; left to
// itself the compiler splits this into and + or with two literals.
__device__ __forceinline__ uint32_t and_or_sv(uint32_t a, uint32_t mask_s, uint32_t c_v) {
  uint32_t d;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "s"(mask_s), "v"(c_v));
  return d;
}

// Two 4-bit codes as the bf16 pair (128 + q_lo, 128 + q_hi): 0x4300 is 128.0
// in bf16 and its 7-bit fraction has unit spacing, so OR-ing a nibble into the
// low bits adds it exactly.  `w >> 4i` masked with 0x000F000F selects the
// codes of k = 8d+2i (low half) and 8d+2i+1 (high half) of a packed dword.
// `mask_s` must hold 0x000F000F and `magic_v` 0x43004300.  The result comes
// from inline asm, whose VALU write the compiler cannot see: it may feed VALU
// and DPP instructions (which the asm blocks pad with wait states themselves)
// but not an MFMA source operand directly.
__device__ __forceinline__ uint32_t nibble_pair_bf16(uint32_t w, int i, uint32_t mask_s,
                                                     uint32_t magic_v) {
  return and_or_sv(i == 0 ? w : (w >> (4 * i)), mask_s, magic_v);
}

// Streaming load; NT sets the non-temporal cache policy (the weight is read
// once per call and should not displace x or the L2-resident partials).
template <bool NT, typename T>
__device__ __forceinline__ T load_stream(const T* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

// Which matrix-core kernel runs M = 5..64 (host side): the register form up
// to 16 rows, the LDS-staged form above (measured on MI355X over five layer
// shapes and every split: 39936 x 6656, 32 rows 52.7 us against 57.4, 64 rows
// 91.9 against 115.5; 8448 x 6656, 64 rows 32.4 against 39.9).
inline bool mfma_lds_form(int64_t m) { return m > 16; }

__device__ __forceinline__ int wave_id_uniform() {
  return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
}

}  // namespace qg
