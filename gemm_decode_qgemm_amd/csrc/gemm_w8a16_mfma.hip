// gemm_w8a16_mfma.hip -- int8 weight-only linear layer for M = 5..64 rows on
// the matrix cores: y[m, n] = (sum_k x[m,k] W[n,k]) * s[n].
//
// gpt-fast issue #114 ("Question about the generated code of
// WeightOnlyInt8Linear"): the layer is F.linear(x, W.to(bf16)) * scales on
// the caller's row-major int8 [N, K] weight; the thread closes by asking how
// to fuse it for batch sizes above 1.  Here, as in the decode GEMV, the int8
// -> float convert stays in registers and W is read once; with 5..64
// activation rows each weight feeds enough products for the matrix cores.
//
// Arithmetic, v_mfma_f32_16x16x32_bf16 on exact operands:
//   B = w + 128 in 0..255 (a byte XORed with 0x80, converted exactly to bf16),
//   D = x . B accumulated over the whole K range in the matrix unit,
//   X = x . ones (the activation row sums, one more product per m-tile),
//   y = s * (D - 128 X),
// so every product is exact and the sums are fp32 (integer activations with
// sum |x| * 255 below 2^24 give the exact integer result).  The scale is per
// output row, so nothing is applied per group and the accumulators stay in
// the matrix unit from the first k to the last.
//
// Two forms on the same arithmetic; launch_w8a16_mfma picks one per call.
// The LDS-staged form (layers of at least 16384 rows, and above 32 rows on
// any layer) is described with its kernel below.
//
// Register form (gfx950, wave64): a workgroup owns NT n-tiles of 16 weight rows
// and all M rows (MT m-tiles of 16); its KW waves take the BK-k blocks of
// K round robin.  In a block, lane (i, a) = (lane % 16, lane / 16) loads BK/4
// contiguous weight bytes of row 16 t + i (k = BK b + (BK/4) a .. + BK/4) and
// the same k of x row 16 mt + i; step j of BK/32 uses k = BK b + (BK/4) a +
// 8 j .. + 8 in lane group a, the same for A and B, so the steps cover the
// block's k once.  The next block's weights and activations are loaded while
// the current one computes.
// The KW partial sums meet in LDS and are added in wave order.
#include "qg_common.h"

namespace qg {

constexpr int kW8KW = 8;    // waves per workgroup, along K

// 8 int8 weights (two dwords, k ascending) as the bf16 pairs (w + 128) of a
// B operand: each byte XORed with 0x80 is w + 128, converted exactly to fp32
// (v_cvt_f32_ubyte*), whose upper half is the exact bf16; v_perm_b32 joins two
// upper halves.  Plain C: the results feed a matrix instruction directly.
__device__ __forceinline__ bf16x8_t w8_operand(uint32_t d0, uint32_t d1, uint32_t sel_hi) {
  const uint32_t u[2] = {d0 ^ 0x80808080u, d1 ^ 0x80808080u};
  uint32_t b[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const uint32_t v = u[h >> 1] >> (16 * (h & 1));
    const float lo = (float)(v & 0xffu);
    const float hi = (float)((v >> 8) & 0xffu);
    b[h] = __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), sel_hi);
  }
  return __builtin_bit_cast(bf16x8_t, u32x4_t{b[0], b[1], b[2], b[3]});
}

// One block of BK k: a lane's weight bytes (BK / 4 contiguous k of each of
// the 2 rows 16 t + i it owns) and activations (the same k of its MT rows).
template <int MT, int NT, int BK, bool PX>
struct W8Blk {
  u32x4_t w[NT][BK / 64];                        // 16 bytes = 16 k each
  u32x4_t xa[PX ? MT : 1][PX ? BK / 32 : 1];     // 8 bf16 = 8 k each (PX: loaded ahead)
};

// PX: the activations are loaded a block ahead with the weights (registers
// permitting); otherwise at the start of their block.
template <int MT, int NT, int BK, bool PX>
__global__ __launch_bounds__(kW8KW * 64) void w8a16_mfma_kernel(
    const uint16_t* __restrict__ x, int m, const int8_t* __restrict__ w,
    const uint16_t* __restrict__ scale, int n, int k, void* __restrict__ y, int y_f32) {
  constexpr int NACC = NT * MT + MT;            // per wave: the products, then X
  constexpr int KL = BK / 4;                       // k per lane group and block
  __shared__ f32x4_t red[kW8KW][NACC][64];
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, a = lane >> 4;
  const int wave = wave_id_uniform();
  const int row0 = blockIdx.x * (16 * NT);
  const int nblk = k / BK;
  const uint32_t sel_hi = __builtin_amdgcn_readfirstlane(0x07060302u);   // upper halves of (S1, S0)
  uint32_t one2 = 0x3f803f80u;           // bf16 pair (1, 1), kept in a VGPR
  asm volatile("" : "+v"(one2));
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{one2, one2, one2, one2});

  // Rows past n or m read the last row instead (a valid address); their
  // results are never stored.
  const int8_t* wr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wr[t] = w + (size_t)min(row0 + 16 * t + i, n - 1) * k + KL * a;
  const uint16_t* xr[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) xr[mt] = x + (size_t)min(16 * mt + i, m - 1) * k + KL * a;

  f32x4_t acc[NT][MT], xs[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    xs[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t][mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }

  auto load = [&](W8Blk<MT, NT, BK, PX>& u, int b) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int q = 0; q < BK / 64; ++q)
        u.w[t][q] = load_stream<true>(reinterpret_cast<const u32x4_t*>(wr[t] + (size_t)b * BK) + q);
    if constexpr (PX) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < BK / 32; ++j)
          u.xa[mt][j] = *reinterpret_cast<const u32x4_t*>(xr[mt] + (size_t)b * BK + 8 * j);
    }
  };
  // step j: k = BK b + KL a + 8 j .. + 8 in lane group a, for A and B alike
  auto compute = [&](const W8Blk<MT, NT, BK, PX>& u, int b) {
    u32x4_t xl[PX ? 1 : MT][PX ? 1 : BK / 32];
    if constexpr (!PX) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < BK / 32; ++j)
          xl[mt][j] = *reinterpret_cast<const u32x4_t*>(xr[mt] + (size_t)b * BK + 8 * j);
    }
    auto xa = [&](int mt, int j) { return __builtin_bit_cast(bf16x8_t, PX ? u.xa[mt][j] : xl[mt][j]); };
#pragma unroll
    for (int j = 0; j < BK / 32; ++j) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4_t& q = u.w[t][j >> 1];
        const bf16x8_t bv = (j & 1) ? w8_operand(q.z, q.w, sel_hi) : w8_operand(q.x, q.y, sel_hi);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa(mt, j), bv, acc[t][mt], 0, 0, 0);
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        xs[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa(mt, j), ones, xs[mt], 0, 0, 0);
    }
  };

  // Two register sets used in turn: the next block's weights and activations
  // are loaded before the current block computes (uniform loop conditions).
  int b = wave;
  if (b < nblk) {
    W8Blk<MT, NT, BK, PX> ua, ub;
    load(ua, b);
    while (true) {
      if (b + kW8KW >= nblk) { compute(ua, b); break; }
      load(ub, b + kW8KW);
      compute(ua, b);
      b += kW8KW;
      if (b + kW8KW >= nblk) { compute(ub, b); break; }
      load(ua, b + kW8KW);
      compute(ub, b);
      b += kW8KW;
    }
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int t = 0; t < NT; ++t) red[wave][t * MT + mt][lane] = acc[t][mt];
    red[wave][NT * MT + mt][lane] = xs[mt];
  }
  __syncthreads();
  // One thread per (n-tile, m-tile, lane): the wave partials in wave order.
  for (int q = threadIdx.x; q < NT * MT * 64; q += kW8KW * 64) {
    const int l = q & 63, tm = q >> 6;             // tm = t * MT + mt
    const int t = tm / MT, mt = tm % MT;
    f32x4_t d = red[0][tm][l], xsum = red[0][NT * MT + mt][l];
    for (int ww = 1; ww < kW8KW; ++ww) {
      const f32x4_t r = red[ww][tm][l], rx = red[ww][NT * MT + mt][l];
      d = f32x4_t{d[0] + r[0], d[1] + r[1], d[2] + r[2], d[3] + r[3]};
      xsum = f32x4_t{xsum[0] + rx[0], xsum[1] + rx[1], xsum[2] + rx[2], xsum[3] + rx[3]};
    }
    // lane l of n-tile t holds rows 16 mt + 4 (l / 16) + e of column 16 t + l % 16
    const int col = row0 + 16 * t + (l & 15);
    if (col >= n) continue;
    const float s = bf16_to_f32(scale[col]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * mt + 4 * (l >> 4) + e;
      if (row >= m) continue;
      const float v = (d[e] - 128.0f * xsum[e]) * s;
      if (y_f32)
        static_cast<float*>(y)[(size_t)row * n + col] = v;
      else
        static_cast<uint16_t*>(y)[(size_t)row * n + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

// Wait until at most N vector-memory loads of this wave are outstanding
// (s_waitcnt fields: vmcnt bits 3:0, expcnt 6:4 and lgkmcnt 11:8 left at
// their maxima).  The builtin, not inline asm: the compiler's own wait
// insertion then knows which loads have landed.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// A barrier that leaves vector-memory loads in flight: this wave's LDS reads
// are complete first (lgkmcnt 0; vmcnt 63 and expcnt 7 mean no wait), so no
// other wave's copy into the buffer they read can overtake them.
__device__ __forceinline__ void barrier_keep_loads() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
}

// ---------------------------------------------------------------------------
// LDS-staged form: a workgroup of 4 waves owns NT n-tiles (16 NT weight rows)
// and all M rows, and streams x through LDS one 256-k tile at a time (copied
// by global_load_lds_dwordx4, no VGPRs), shared by its waves.  Wave w takes
// n-tile w % NT and slice w / NT of each tile's 8 k-steps (4 / NT waves per
// n-tile), so each int8 weight is converted once for all MT m-tiles.
// In a tile, lane (i, a) holds the 16-byte chunks q of its weight row at
// k = 64 q + 16 a .. + 16; step (q, h) uses k = 64 q + 16 a + 8 h .. + 8 in
// lane group a, for A and B alike, so the 8 steps cover the tile once.  The
// activation row sums X take one product per m-tile per step, spread over
// the 4 waves (each does a quarter of the steps).  At the end the waves'
// partial sums meet in LDS (reusing the activation buffers) and are added
// in wave order: y = s * (D - 128 X).
// LDS layout of a staged tile: 16-byte piece c of x row r (k = 8c .. 8c+8)
// at piece index 32 r + (c ^ (r & 15)): the 16 lanes of a lane group read 16
// distinct bank quads.
template <int MT, int NT>
__global__ __launch_bounds__(256) void w8a16_mfma2_kernel(
    const uint16_t* __restrict__ x, int m, const int8_t* __restrict__ w,
    const uint16_t* __restrict__ scale, int n, int k, void* __restrict__ y, int y_f32) {
  constexpr int TK = 256;                        // k per tile
  constexpr int KS = 4 / NT;                     // waves per n-tile
  constexpr int QW = TK / 64 / KS;               // 64-k chunks per wave and tile
  constexpr int PR = TK / 8;                     // 16-byte pieces per staged x row
  constexpr int MR = 16 * MT;                    // staged x rows
  static_assert(QW * KS * 64 == TK, "a tile's chunks must split evenly over the waves of an n-tile");
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][MR * PR * 16];
  static_assert(2 * 4 * MT * 64 * 16 <= 2 * MR * PR * 16, "reduction must fit the x buffers");
  const int lane = threadIdx.x & 63;
  const int i = lane & 15, a = lane >> 4;
  const int wv = wave_id_uniform();
  const int t = wv % NT, ks = wv / NT;
  const int row0 = blockIdx.x * (16 * NT);
  const int kt_count = k / TK;
  const uint32_t sel_hi = __builtin_amdgcn_readfirstlane(0x07060302u);
  uint32_t one2 = 0x3f803f80u;           // bf16 pair (1, 1), kept in a VGPR
  asm volatile("" : "+v"(one2));
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, u32x4_t{one2, one2, one2, one2});
  // a row past n reads row n - 1 instead (a valid address; never stored)
  const u32x4_t* wr = reinterpret_cast<const u32x4_t*>(
      w + (size_t)min(row0 + 16 * t + i, n - 1) * k + 64 * QW * ks + 16 * a);

  auto stage = [&](int kt, int buf) {
    static_assert(MR * PR % 256 == 0, "every wave issues the same number of copies");
#pragma unroll
    for (int j = 0; j < MR * PR / 256; ++j) {
      const int u = wv + 4 * j;
      const int r = u * (64 / PR) + lane / PR;
      const int c = (lane % PR) ^ (r & 15);
      const int src = r < m ? r : m - 1;        // rows past m repeat row m - 1
      __builtin_amdgcn_global_load_lds(x + (size_t)src * k + (size_t)kt * TK + 8 * c,
                                       (__attribute__((address_space(3))) void*)(xs[buf] + 1024 * u),
                                       16, 0, 0);
    }
  };
  auto load_w = [&](u32x4_t (&wq)[QW], int kt) {
#pragma unroll
    for (int q = 0; q < QW; ++q) wq[q] = load_stream<true>(wr + (size_t)kt * (TK / 16) + 4 * q);
  };

  f32x4_t acc[MT], xsum[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    acc[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    xsum[mt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  // this wave's row-sum steps: h == t % 2 (NT >= 2), and q % 2 == t / 2 (NT = 4)
  auto x_step = [&](int qq, int h) {
    if constexpr (NT == 1) return true;
    else if constexpr (NT == 2) return h == t;
    else return h == (t & 1) && (qq & 1) == (t >> 1);
  };
  // `issue` runs after the first k-step (see the tile loop below).
  auto compute = [&](const u32x4_t (&wq)[QW], int buf, auto&& issue) {
    const uint8_t* xb = xs[buf];
#pragma unroll
    for (int qq = 0; qq < QW; ++qq) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int c = 8 * (QW * ks + qq) + 2 * a + h;
        bf16x8_t av[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int r = 16 * mt + i;
          av[mt] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(
                                                    xb + 16 * (PR * r + (c ^ (r & 15)))));
        }
        const bf16x8_t bv = h ? w8_operand(wq[qq].z, wq[qq].w, sel_hi) : w8_operand(wq[qq].x, wq[qq].y, sel_hi);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], bv, acc[mt], 0, 0, 0);
        if (x_step(qq, h)) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            xsum[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[mt], ones, xsum[mt], 0, 0, 0);
        }
        if (qq == 0 && h == 0) issue();
      }
    }
  };

  // Weights two tiles ahead, activations one.  Loads complete in issue order,
  // so before the barrier that hands over x tile kt + 1 a wave waits until
  // only its weight loads of tile kt + 2 are outstanding.  The barrier is a
  // bare s_barrier after this wave's LDS reads: a fenced one would wait for
  // those loads too.  Three register sets take turns (the loop is unrolled
  // three times), so no register holding a load in flight is ever copied.
  // A tile's loads are issued after its first k-step: the compiler's own
  // waits at the loop head (it cannot prove the weights there have landed)
  // then cost nothing.
  // One tile; returns whether another follows (the loop leaves exactly on
  // the path that skips the wait, so no path into the next step carries a
  // load the wait did not cover).
  auto step = [&](int kt, const u32x4_t (&wc)[QW], u32x4_t (&wl)[QW]) {
    const bool more = kt + 1 < kt_count;         // uniform
    const bool more2 = kt + 2 < kt_count;
    compute(wc, kt & 1, [&]() {
      if (more) stage(kt + 1, (kt + 1) & 1);
      if (more2) load_w(wl, kt + 2);
    });
    if (!more) return false;
    if (more2)
      wait_vm<QW>();
    else
      wait_vm<0>();
    barrier_keep_loads();
    return true;
  };
  {
    u32x4_t wa[QW], wb[QW], wc[QW];
    stage(0, 0);
    load_w(wa, 0);
    if (kt_count > 1) {
      load_w(wb, 1);
      wait_vm<QW>();
    } else {
      wait_vm<0>();
    }
    barrier_keep_loads();
    for (int kt = 0;; kt += 3) {
      if (!step(kt, wa, wc)) break;
      if (!step(kt + 1, wb, wa)) break;
      if (!step(kt + 2, wc, wb)) break;
    }
  }

  // partial sums of every wave: D at [wave][mt][lane], X after all of them
  __syncthreads();
  f32x4_t* red = reinterpret_cast<f32x4_t*>(&xs[0][0]);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    red[(wv * MT + mt) * 64 + lane] = acc[mt];
    red[((4 + wv) * MT + mt) * 64 + lane] = xsum[mt];
  }
  __syncthreads();
  // one thread per (n-tile, m-tile, lane); partials added in wave order
  for (int q = threadIdx.x; q < NT * MT * 64; q += 256) {
    const int l = q & 63, tm = q >> 6;
    const int tt = tm / MT, mt = tm % MT;
    f32x4_t d = red[(tt * MT + mt) * 64 + l];
#pragma unroll
    for (int kk = 1; kk < KS; ++kk) {
      const f32x4_t r = red[((tt + NT * kk) * MT + mt) * 64 + l];
      d = f32x4_t{d[0] + r[0], d[1] + r[1], d[2] + r[2], d[3] + r[3]};
    }
    f32x4_t xv = red[(4 * MT + mt) * 64 + l];
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) {
      const f32x4_t r = red[((4 + ww) * MT + mt) * 64 + l];
      xv = f32x4_t{xv[0] + r[0], xv[1] + r[1], xv[2] + r[2], xv[3] + r[3]};
    }
    // lane l of n-tile tt holds rows 16 mt + 4 (l / 16) + e of column 16 tt + l % 16
    const int col = row0 + 16 * tt + (l & 15);
    if (col >= n) continue;
    const float s = bf16_to_f32(scale[col]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 16 * mt + 4 * (l >> 4) + e;
      if (row >= m) continue;
      const float v = (d[e] - 128.0f * xv[e]) * s;
      if (y_f32)
        static_cast<float*>(y)[(size_t)row * n + col] = v;
      else
        static_cast<uint16_t*>(y)[(size_t)row * n + col] = (uint16_t)f32_to_bf16_rne(v);
    }
  }
}

template <int MT, int NT>
static hipError_t launch_w8_mfma2_t(const void* x, int m, const int8_t* w, const void* scale, int n, int k,
                                    void* y, int y_f32, hipStream_t stream) {
  hipLaunchKernelGGL((w8a16_mfma2_kernel<MT, NT>), dim3((n + 16 * NT - 1) / (16 * NT)), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), m, w, static_cast<const uint16_t*>(scale), n, k, y, y_f32);
  return hipGetLastError();
}

template <int MT, int NT, int BK, bool PX>
static hipError_t launch_w8_mfma_t(const void* x, int m, const int8_t* w, const void* scale, int n, int k,
                                   void* y, int y_f32, hipStream_t stream) {
  hipLaunchKernelGGL((w8a16_mfma_kernel<MT, NT, BK, PX>), dim3((n + 16 * NT - 1) / (16 * NT)), dim3(kW8KW * 64), 0,
                     stream, static_cast<const uint16_t*>(x), m, w, static_cast<const uint16_t*>(scale), n, k, y,
                     y_f32);
  return hipGetLastError();
}

template <int NT>
static hipError_t launch_w8_mfma2_m(int m, const void* x, const int8_t* w, const void* scale, int n, int k,
                                    void* y, int y_f32, hipStream_t stream) {
  switch ((m + 15) / 16) {
    case 1: return launch_w8_mfma2_t<1, NT>(x, m, w, scale, n, k, y, y_f32, stream);
    case 2: return launch_w8_mfma2_t<2, NT>(x, m, w, scale, n, k, y, y_f32, stream);
    case 3: return launch_w8_mfma2_t<3, NT>(x, m, w, scale, n, k, y, y_f32, stream);
    case 4: return launch_w8_mfma2_t<4, NT>(x, m, w, scale, n, k, y, y_f32, stream);
    default: return hipErrorInvalidValue;
  }
}

// 5..64 rows.  The LDS-staged form on layers of at least 16384 rows and
// above 32 rows everywhere, with 4 n-tiles per workgroup from 16384 rows, 2
// above 4096, 1 below; otherwise the register form.  Measured on MI355X (us,
// LDS form against the register form): 64 rows, 39936 x 6656 101.3 against
// 210.7, 32768 x 8192 83.0 against 198.8, 6656 x 19968 84.7 against 129.5,
// 8192 x 8192 37.7 against 52.6, 4096 x 4096 18.0 against 26.8; 48 rows,
// 8448 x 6656 38.6 against 64.6; 32 rows, 28672 x 8192 62.9 against 106.1,
// but 8192 x 8192 29.7 against 29.1 and 6656 x 19968 67.9 against 66.6;
// 16 rows, 8192 x 8192 26.3 against 21.6.
hipError_t launch_w8a16_mfma(int m, const void* x, const int8_t* w, const void* scale, int n, int k, void* y,
                             int y_f32, hipStream_t stream) {
  if (n >= 16384) return launch_w8_mfma2_m<4>(m, x, w, scale, n, k, y, y_f32, stream);
  if (m > 32) {
    if (n > 4096) return launch_w8_mfma2_m<2>(m, x, w, scale, n, k, y, y_f32, stream);
    return launch_w8_mfma2_m<1>(m, x, w, scale, n, k, y, y_f32, stream);
  }
  // Register form, 5..32 rows: MT = ceil(m / 16) m-tiles, rows past m
  // masked, 128-k blocks, two n-tiles (32 weight rows) per workgroup.
  // Loading the activations a block ahead pays at 17..32 rows only (8192 x
  // 8192: 28.8 us against 33.3 at 32 rows, but 30.7 against 25.0 at 16;
  // 256-k blocks at 16 rows: 30.7).
  if (m <= 16) return launch_w8_mfma_t<1, 2, 128, false>(x, m, w, scale, n, k, y, y_f32, stream);
  return launch_w8_mfma_t<2, 2, 128, true>(x, m, w, scale, n, k, y, y_f32, stream);
}

}  // namespace qg
