// gemv_w4a16_mx4.hip -- decode GEMV for the packed INT4 group-32 weight,
// M = 2..4, on the 4x4x4 sixteen-block bf16 matrix instruction.
//
// Same product as gemv_w4a16.hip: y[m, n] = sum_k x[m, k] (q[n,k] - zp[n,g])
// s[n,g], the "dequant + F.linear" reference of executorch
// test_int4_quantized_gemm.py (module docstring, `_dequant_matmul`), with no
// dequantized weight ever written (gpt-fast issue #114).
//
// Why a matrix instruction for a GEMV: with one v_dot2c per weight pair and
// activation row, M = 4 spends four times the M = 1 VALU work per weight and
// stops being bound by HBM (39936 x 6656: 35.5 us at M = 4 against 23.8 at
// M = 1 on MI355X).  v_mfma_f32_4x4x4_16b_bf16 computes sixteen independent
// 4x4x4 products: block b takes A from lanes 4b..4b+3 (row i in lane 4b+i,
// four k in its register pair), B from the same lanes (column j in lane
// 4b+j) and writes D[i][j] to element i of lane 4b+j (layout measured on
// MI355X).  With A = x (row i = activation row m) and B = the weight (column
// j = the lane's own weight row), every lane keeps the codes it loaded, needs
// no transpose, and ends with y[0..3] of its row in its four result
// registers.  The matrix work per weight is the same for M = 2, 3 and 4.
//
// Mapping: the 32-row workgroups of gemv_w4a16.hip (lane l holds row l & 31
// and groups 2(l >> 5), 2(l >> 5) + 1 of each half tile), so both kernels
// share the work split and the code-load pattern.  Per half tile and wave:
//  * the M x 128 activations are read once, coalesced (16 bytes per lane),
//    and written to a wave-private LDS slot; loading the A operands straight
//    from memory (16 lanes asking for each address) was twice as slow;
//  * the same lanes form the group sums X_g of x (v_dot2c with (1, 1), a
//    quad DPP reduction) and leave them in LDS next to x;
//  * per group, 8 A-operand reads from LDS and 8 matrix instructions with
//    B = (128 + q) as exact bf16 pairs (the nibble trick of nibble_pair_bf16)
//    give D[m] = sum x (128 + q); then acc[m] += s (D[m] - (128 + zp) X_g[m]).
// A rows at or above M repeat row M - 1: their results land in result
// registers that are never read, so no masking is needed.
// With one split and a little over one 32-row workgroup per CU (N = 8448:
// 264, leaving a few CUs with two and the rest with one), the kernel takes
// whole 64-row blocks instead (132 workgroups): lane = row, each lane
// loads both group pairs of its row and takes the half tile's 4 groups in
// turn, and with one workgroup per CU it keeps the next half tile's loads in
// flight in a second register set (the rule is in dispatch.h).
#include "qg_common.h"
#include "dispatch.h"
#include "w4_common.h"

namespace qg {

typedef short s16x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_4x4x4(u32x2_t a, u32x2_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}

// Two codes as the bf16 pair (128 + q(8d+2e), 128 + q(8d+2e+1)) in plain C:
// the matrix instruction reads it, and an inline-asm VALU write ahead of a
// matrix-instruction read hides the dependency from the compiler's hazard
// tracking.  mask_s = 0x000F000F (an SGPR), magic_v = 0x43004300 (a VGPR).
__device__ __forceinline__ uint32_t code_pair(uint32_t w, int e, uint32_t mask_s, uint32_t magic_v) {
  return ((w >> (4 * e)) & mask_s) | magic_v;
}

// x rows in a wave's LDS slot: 288 bytes apart, groups 2-3 of a half tile 16
// bytes after groups 0-1.  An A-operand read (fixed group and k-step) touches
// at most 8 distinct 16-byte chunks, (row i, group pair) at 288 i + 144 pair
// bytes; these sit at distinct 16-byte positions modulo 128 and modulo 256
// bytes, i.e. on disjoint banks.
constexpr int kMx4RowBytes = 288;
constexpr int kMx4PairBytes = 144;

// 8 waves per SIMD (two 16-wave workgroups per CU) keep enough weight loads
// in flight; the kernel fits the 64 VGPRs that allows without spilling.
// R64: one 64-row block per workgroup, one workgroup per CU, so 128 VGPRs and
// two register sets in turn (the next half tile's loads in flight while the
// current one is computed).
template <int M, int WAVES, class L, bool R64 = false>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(R64 ? 4 : 8))) void w4a16_gemv_mx4_kernel(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ packed, int n, int k,
    void* __restrict__ y, int y_f32, float* __restrict__ partial, int split) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[WAVES][M * kMx4RowBytes];
  __shared__ __attribute__((aligned(16))) float xsum[WAVES][4][4];   // [group][m]
  __shared__ float red[WAVES * M * 64];
  const int lane = threadIdx.x & 63;
  const int lg = R64 ? 0 : lane >> 5;              // group pair of this lane (R64: both, in turn)
  const int xrow = (lane & 3) < M ? (lane & 3) : M - 1;   // A row of this lane
  const int wave = wave_id_uniform();
  const int rb = R64 ? blockIdx.x : blockIdx.x >> 1;       // 64-row block
  const int row = R64 ? lane : 32 * (blockIdx.x & 1) + (lane & 31);
  const int kt_count = k >> 8;
  int t0, t1;
  split_range(kt_count, split, blockIdx.y, t0, t1);
  float step;
  const uint8_t* tiles = L::tiles(packed, rb, kt_count, row, step);
  // Staging: lane l < 16 M copies k = 8 (l % 16) .. + 8 of x row l / 16.
  const bool stager = lane < 16 * M;
  const int sm = stager ? lane >> 4 : 0, sc = lane & 15;
  const uint16_t* xsrc = x + (size_t)sm * k + 8 * sc;
  uint8_t* const slot = xs[wave];
  const int swr = sm * kMx4RowBytes + 16 * sc + (sc >= 8 ? 16 : 0);
  const int srd = xrow * kMx4RowBytes + lg * kMx4PairBytes;
  const uint32_t mask_s = __builtin_amdgcn_readfirstlane(0x000F000Fu);
  uint32_t magic_v = 0x43004300u;
  asm volatile("" : "+v"(magic_v));
  uint32_t ones_v = 0x3f803f80u;   // bf16 (1, 1), kept out of literal operands
  asm volatile("" : "+v"(ones_v));

  float acc[M];
#pragma unroll
  for (int m = 0; m < M; ++m) acc[m] = 0.0f;

  constexpr int NP = R64 ? 2 : 1;   // group pairs per lane
  using Regs = typename L::Regs;
  auto load = [&](Regs (&r)[NP], u32x4_t& xv, int hs) {   // tile hs/2, half hs%2
#pragma unroll
    for (int p = 0; p < NP; ++p) L::load(r[p], tiles + (size_t)(hs >> 1) * L::kTile, hs & 1, lg + p, row);
    xv = u32x4_t{0u, 0u, 0u, 0u};
    if (stager) xv = *reinterpret_cast<const u32x4_t*>(xsrc + (size_t)hs * 128);
  };
  auto compute = [&](const Regs (&r)[NP], const u32x4_t& xv) {
    // Group sums of x: 8 k per stager lane, then the 4 lanes of a group.
    float xp = dot2_bf16(xv.x, ones_v, 0.0f);
    xp = dot2_bf16(xv.y, ones_v, xp);
    xp = dot2_bf16(xv.z, ones_v, xp);
    xp = dot2_bf16(xv.w, ones_v, xp);
    xp += dpp_mov<0xB1>(xp);   // quad_perm [1,0,3,2]
    xp += dpp_mov<0x4E>(xp);   // quad_perm [2,3,0,1]
    // The slot is private to the wave and a wave's LDS operations complete in
    // order, so the previous unit's reads are done before this write and the
    // reads below see it; the fences only keep the compiler from moving LDS
    // accesses across.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    if (stager) {
      *reinterpret_cast<u32x4_t*>(slot + swr) = xv;
      if ((sc & 3) == 0) xsum[wave][sc >> 2][sm] = xp;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // One group at a time: 8 A reads, x[xrow][32 (2 pr + jj) + 8 q .. + 8]
    // for group pair pr = lg + p (two k-steps each), 8 chained products, the
    // group's epilogue.
#pragma unroll
    for (int p = 0; p < NP; ++p)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      u32x4_t xa[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        xa[q] = *reinterpret_cast<const u32x4_t*>(slot + srd + p * kMx4PairBytes + 64 * jj + 16 * q);
      f32x4_t d = {0.0f, 0.0f, 0.0f, 0.0f};
      // k-step t covers k = 4t..4t+3 of the group: code dword t/2, pairs
      // 2(t%2) and 2(t%2)+1; x dwords 2t, 2t+1.
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const u32x2_t b = {L::pair(r[p], jj, t >> 1, 2 * (t & 1), mask_s, magic_v),
                           L::pair(r[p], jj, t >> 1, 2 * (t & 1) + 1, mask_s, magic_v)};
        const u32x4_t xq = xa[t >> 1];
        const u32x2_t a = (t & 1) ? u32x2_t{xq.z, xq.w} : u32x2_t{xq.x, xq.y};
        d = mfma_4x4x4(a, b, d);
      }
      const float s = L::scale(r[p].sc, jj, step);
      const f32x4_t xg = *reinterpret_cast<const f32x4_t*>(&xsum[wave][2 * (lg + p) + jj][0]);
      const float zb = (float)(L::zero(r[p], jj) | 0x80u);   // 128 + zp (zp <= 63)
#pragma unroll
      for (int m = 0; m < M; ++m) acc[m] = __builtin_fmaf(s, __builtin_fmaf(-zb, xg[m], d[m]), acc[m]);
    }
  };

  if constexpr (!R64) {
    for (int hs = 2 * t0 + wave; hs < 2 * t1; hs += WAVES) {
      Regs r[NP];
      u32x4_t xv;
      load(r, xv, hs);
      compute(r, xv);
    }
  } else {
    // One workgroup per CU: two register sets used in turn, the next half
    // tile's loads in flight while the current one is computed (scheduling
    // barriers keep the compiler from sinking the loads).
    const int h_end = 2 * t1;
    int hs = 2 * t0 + wave;
    if (hs < h_end) {                                    // uniform
      Regs ra[NP], rb_[NP];
      u32x4_t xa, xb;
      load(ra, xa, hs);
      __builtin_amdgcn_sched_barrier(0);
      while (true) {
        if (hs + WAVES >= h_end) { compute(ra, xa); break; }
        load(rb_, xb, hs + WAVES);
        __builtin_amdgcn_sched_barrier(0);
        compute(ra, xa);
        hs += WAVES;
        if (hs + WAVES >= h_end) { compute(rb_, xb); break; }
        load(ra, xa, hs + WAVES);
        __builtin_amdgcn_sched_barrier(0);
        compute(rb_, xb);
        hs += WAVES;
      }
    }
  }

  // Sum over waves and (32-row form) over the two lane halves of a row, in a
  // fixed order.
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
      if (partial != nullptr)
        partial[((size_t)blockIdx.y * M + m) * n + col] = v;
      else if (y_f32)
        static_cast<float*>(y)[(size_t)m * n + col] = v;
      else
        static_cast<uint16_t*>(y)[(size_t)m * n + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

template <int M, int WAVES, class L>
static hipError_t launch_mx4_t(const void* x, const void* packed, int n, int k, void* y, int y_f32,
                               float* partial, int split, hipStream_t stream) {
  const int rbs = (n + kTileRows - 1) / kTileRows;
  if (gemv_shape(M, n, split).rows == 64)
    hipLaunchKernelGGL((w4a16_gemv_mx4_kernel<M, WAVES, L, true>), dim3(rbs, split), dim3(WAVES * 64), 0,
                       stream, static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(packed),
                       n, k, y, y_f32, partial, split);
  else
    hipLaunchKernelGGL((w4a16_gemv_mx4_kernel<M, WAVES, L>), dim3(2 * rbs, split), dim3(WAVES * 64), 0,
                       stream, static_cast<const uint16_t*>(x), static_cast<const uint8_t*>(packed),
                       n, k, y, y_f32, partial, split);
  return hipGetLastError();
}

hipError_t launch_w4a16_gemv_mx4(int m, const void* x, const void* packed, int n, int k, void* y,
                                 int y_f32, float* partial, int split, int waves,
                                 hipStream_t stream) {
#define QG_MX4_CASE(MM, WW) \
  if (m == MM && waves == WW) return launch_mx4_t<MM, WW, W4Layout<false>>(x, packed, n, k, y, y_f32, partial, split, stream);
#define QG_MX4_M(MM) QG_MX4_CASE(MM, 16)
  QG_MX4_M(2) QG_MX4_M(3) QG_MX4_M(4)
#undef QG_MX4_M
#undef QG_MX4_CASE
  return hipErrorInvalidValue;
}

// M = 2..4 on the scale-code layout (version 2).
hipError_t launch_w4a16_gemv_mx4_dq(int m, const void* x, const void* packed, int n, int k, void* y,
                                    int y_f32, float* partial, int split, hipStream_t stream) {
  switch (m) {
    case 2: return launch_mx4_t<2, 16, W4Layout<true>>(x, packed, n, k, y, y_f32, partial, split, stream);
    case 3: return launch_mx4_t<3, 16, W4Layout<true>>(x, packed, n, k, y, y_f32, partial, split, stream);
    case 4: return launch_mx4_t<4, 16, W4Layout<true>>(x, packed, n, k, y, y_f32, partial, split, stream);
    default: return hipErrorInvalidValue;
  }
}

// M = 2..4 on the INT5 / INT6 layout.
template <int HB>
static hipError_t launch_mx4_wn(int m, const void* x, const void* packed, int n, int k, void* y, int y_f32,
                                float* partial, int split, hipStream_t stream) {
  switch (m) {
    case 2: return launch_mx4_t<2, 16, WnLayout<HB>>(x, packed, n, k, y, y_f32, partial, split, stream);
    case 3: return launch_mx4_t<3, 16, WnLayout<HB>>(x, packed, n, k, y, y_f32, partial, split, stream);
    case 4: return launch_mx4_t<4, 16, WnLayout<HB>>(x, packed, n, k, y, y_f32, partial, split, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_wn_a16_gemv_mx4(int bits, int m, const void* x, const void* packed, int n, int k, void* y,
                                  int y_f32, float* partial, int split, hipStream_t stream) {
  if (bits == 5) return launch_mx4_wn<1>(m, x, packed, n, k, y, y_f32, partial, split, stream);
  if (bits == 6) return launch_mx4_wn<2>(m, x, packed, n, k, y, y_f32, partial, split, stream);
  return hipErrorInvalidValue;
}

}  // namespace qg
