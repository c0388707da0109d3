// api.hip -- the C ABI declared in include/qgemm.h: argument checks on the
// host, then kernel launches on the caller's stream.
//
// Rules follow executorch test_int4_quantized_gemm.py,
// Int4QuantizedGemmLegalityTest (every rule checked before anything is
// launched; "K must be a multiple of 256"; "static M must be within" the
// supported buckets, the largest being 64) and
// Int4QuantizedGemmRulesTest.test_split_k_needs_one_k_tile_per_split
// (a split is legal iff split <= K / 256).  The library never allocates and
// never synchronizes.
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "dispatch.h"
#include "qg_common.h"
#include "qgemm.h"

namespace qg {
hipError_t launch_quantize_int4_g32(const void* w, int64_t n, int64_t k, void* packed,
                                    uint32_t* status, hipStream_t stream);
hipError_t launch_quantize_int4_g32_dq(const void* w, int64_t n, int64_t k, void* packed,
                                       uint32_t* status, hipStream_t stream);
hipError_t launch_w4a16_gemv32_dq(int m, const void* x, const void* packed, int n, int k, void* y,
                                  int y_f32, float* partial, int split, hipStream_t stream);
hipError_t launch_w4a16_gemv_dq(int m, const void* x, const void* packed, int n, int k, void* y,
                                int y_f32, float* partial, int split, hipStream_t stream);
hipError_t launch_w4a16_gemv_mx4_dq(int m, const void* x, const void* packed, int n, int k, void* y,
                                    int y_f32, float* partial, int split, hipStream_t stream);
hipError_t launch_quantize_intn_g32(const void* w, int64_t n, int64_t k, int bits, void* packed,
                                    uint32_t* status, hipStream_t stream);
hipError_t launch_wn_a16_gemv32(int bits, const void* x, const void* packed, int n, int k, void* y,
                                int y_f32, float* partial, int split, hipStream_t stream);
hipError_t launch_wn_a16_gemv_mx4(int bits, int m, const void* x, const void* packed, int n, int k, void* y,
                                  int y_f32, float* partial, int split, hipStream_t stream);
hipError_t launch_wn_a16_mfma(int bits, int m, const void* x, const void* packed, int n, int k, void* y,
                              int y_f32, float* partial, int split, hipStream_t stream);
hipError_t launch_w4a16_mfma_dq(int m, const void* x, const void* packed, int n, int k, void* y, int y_f32,
                                float* partial, int split, hipStream_t stream,
                                const float* row_scale = nullptr);
hipError_t launch_w4a8_actquant_g32_bf16(int m, const void* x, int k, void* xq, float* sxg,
                                         hipStream_t stream);
hipError_t launch_w4a8g_mfma(bool dq, int m, const void* xq, const float* act_scale, const void* packed, int n,
                             int k, void* y, int y_f32, float* partial, int split, hipStream_t stream);
hipError_t launch_w4a8_actquant_bf16(int m, const void* x, int k, void* xq, float* sx,
                                     hipStream_t stream);
hipError_t launch_w4a8_rowscale_reduce(const float* partial, int split, int m, int n, const float* sx,
                                       void* y, int y_f32, hipStream_t stream);
hipError_t launch_w4a8_dq(int m, bool group_scales, const void* x, const void* packed, int n, int k,
                          void* y, int y_f32, float* partial, int split, hipStream_t stream);
hipError_t launch_quantize_int8_rowwise(const void* w, int64_t n, int64_t k, int8_t* q,
                                        void* scales, uint32_t* status, hipStream_t stream);
hipError_t launch_w4a16_gemv(int m, const void* x, const void* packed, int n, int k, void* y,
                             int y_f32, float* partial, int split, int waves, hipStream_t stream);
hipError_t launch_w4a16_gemv32(int m, const void* x, const void* packed, int n, int k, void* y,
                               int y_f32, float* partial, int split, int waves, hipStream_t stream);
hipError_t launch_w4a16_gemv_mx4(int m, const void* x, const void* packed, int n, int k, void* y,
                                 int y_f32, float* partial, int split, int waves,
                                 hipStream_t stream);
hipError_t launch_splitk_reduce(const float* partial, int split, int64_t mn, void* y, int y_f32,
                                hipStream_t stream);
int w8a16_chunks_per_wave(int k);
hipError_t launch_w4a16_mfma(int m, const void* x, const void* packed, int n, int k, void* y,
                             int y_f32, float* partial, int split, hipStream_t stream,
                             const float* row_scale = nullptr);
hipError_t launch_w4a8_gemv(int m, const void* x, const void* packed, int n, int k, void* y,
                            int y_f32, float* partial, int split, int rows, int waves,
                            hipStream_t stream);
hipError_t launch_w4a8_gemv_lds(int m, bool group_scales, const void* x, const void* packed, int n,
                                int k, void* y, int y_f32, float* partial, int split,
                                hipStream_t stream);
hipError_t launch_w4a8_gemv_mx4(int m, bool group_scales, const void* x, const void* packed, int n,
                                int k, void* y, int y_f32, float* partial, int split,
                                hipStream_t stream);
hipError_t launch_w8a16_gemv(int m, const void* x, const int8_t* w, const void* scale, int n,
                             int k, void* y, int y_f32, hipStream_t stream);
hipError_t launch_w8a16_mfma(int m, const void* x, const int8_t* w, const void* scale, int n, int k, void* y,
                             int y_f32, hipStream_t stream);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int blocks,
                              hipStream_t stream);
}  // namespace qg

namespace {

using qg::default_split;
using qg::default_split_intn;
using qg::gemv_shape;
using qg::GemvShape;
using qg::resolve_split;

constexpr int64_t kMaxDim = (int64_t)1 << 30;   // n, k fit the kernels' int32 indexing

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int32_t check_nk(int64_t n, int64_t k) {
  if (n < 1 || k < 1 || n > kMaxDim || k > kMaxDim) return QG_E_SHAPE;
  if (k % QG_TILE_K != 0) return QG_E_K_MULTIPLE;
  return QG_OK;
}

int32_t check_mnk(int64_t m, int64_t n, int64_t k) {
  if (m < 1) return QG_E_SHAPE;
  int32_t st = check_nk(n, k);
  if (st != QG_OK) return st;
  if (m > QG_MAX_M) return QG_E_M_RANGE;
  return QG_OK;
}

int32_t hip_status(hipError_t e) { return e == hipSuccess ? QG_OK : QG_E_HIP; }

// Workspace of W4A8 at m > 4: xq as bf16 [m, k]; then the activation
// scales: per row, fp32 [m] (256 bytes), per group of 32, fp32 [k/32][64]
// (8 k bytes); then the fp32 partial sums [split, m, n], split >= 1.
int64_t w4a8_scales_bytes(int64_t k) { return k * 8 > 256 ? k * 8 : 256; }
int64_t w4a8_mfma_ws(int64_t m, int64_t n, int64_t k, int32_t split) {
  return m * k * 2 + w4a8_scales_bytes(k) + (int64_t)split * m * n * 4;
}

}  // namespace

extern "C" {

const char* qg_status_string(int32_t s) {
  switch (s) {
    case QG_OK: return "ok";
    case QG_E_NULL: return "a required pointer is NULL";
    case QG_E_SHAPE: return "m, n and k must be >= 1 (and fit the kernels' limits)";
    case QG_E_K_MULTIPLE: return "K must be a multiple of 256";
    case QG_E_M_RANGE: return "M must be within the supported buckets (1..64)";
    case QG_E_SPLIT: return "split_k must be 0, 1, 2, 4 or 8 and at most K/256 (one K tile per split)";
    case QG_E_BUFFER: return "a buffer (packed weight or workspace) is too small";
    case QG_E_ALIGN: return "data pointers must be 16-byte aligned";
    case QG_E_DTYPE: return "y_dtype must be QG_BF16 or QG_F32";
    case QG_E_HIP: return "a HIP launch failed";
    case QG_E_BITS: return "bits must be 5 or 6";
    case QG_E_SCRATCH:
      return "the split needs more partial-sum space than the library's static scratch holds "
             "(split * m * n * 4 > QG_SCRATCH_BYTES); pass a smaller split_k or use qgemm_w4a16";
    default: return "unknown qgemm status";
  }
}

int64_t qg_int4_packed_bytes(int64_t n, int64_t k) {
  int32_t st = check_nk(n, k);
  if (st != QG_OK) return st;
  return ((n + QG_TILE_ROWS - 1) / QG_TILE_ROWS) * (k / QG_TILE_K) * (int64_t)QG_TILE_BYTES;
}

int64_t qg_int4_dq_packed_bytes(int64_t n, int64_t k) {
  int32_t st = check_nk(n, k);
  if (st != QG_OK) return st;
  return ((n + QG_TILE_ROWS - 1) / QG_TILE_ROWS) *
         (QG_DQ_HEAD_BYTES + (k / QG_TILE_K) * (int64_t)QG_DQ_TILE_BYTES);
}

int64_t qg_intn_packed_bytes(int64_t n, int64_t k, int32_t bits) {
  int32_t st = check_nk(n, k);
  if (st != QG_OK) return st;
  if (bits != 5 && bits != 6) return QG_E_BITS;
  return ((n + QG_TILE_ROWS - 1) / QG_TILE_ROWS) * (k / QG_TILE_K) *
         (int64_t)(8192 + 2048 * (bits - 4) + 1536);
}

int32_t qg_default_split_k(int64_t m, int64_t n, int64_t k) {
  int32_t st = check_mnk(m, n, k);
  if (st != QG_OK) return st;
  return default_split(m, n, k);
}

int64_t qg_workspace_bytes(int64_t m, int64_t n, int64_t k, int32_t split_k) {
  int32_t st = check_mnk(m, n, k);
  if (st != QG_OK) return st;
  int32_t split;
  st = resolve_split(m, n, k, split_k, &split);
  if (st != QG_OK) return st;
  if (split_k != 0) {
    const int64_t bytes = split > 1 ? (int64_t)split * m * n * 4 : 0;
    if (m <= 4) return bytes;
    const int64_t w8 = w4a8_mfma_ws(m, n, k, split);   // W4A8 at m > 4
    return w8 > bytes ? w8 : bytes;
  }
  // split_k = 0: enough for the default of every entry point, W4A8 at M > 4
  // included (quantized x, its scales and the partials at that default)
  int64_t units = split > 1 ? (int64_t)split * m : 0;
  const int32_t si = default_split_intn(m, n, k);
  if (si > 1 && (int64_t)si * m > units) units = (int64_t)si * m;
  const int64_t bytes = units * n * 4;
  if (m <= 4) return bytes;
  int64_t w8 = w4a8_mfma_ws(m, n, k, split);
  const int64_t w8g = w4a8_mfma_ws(m, n, k, qg::default_split_g32(m, n, k));   // per group of 32
  if (w8g > w8) w8 = w8g;
  return w8 > bytes ? w8 : bytes;
}

int32_t qg_default_split_k_g32(int64_t m, int64_t n, int64_t k) {
  int32_t st = check_mnk(m, n, k);
  if (st != QG_OK) return st;
  return qg::default_split_g32(m, n, k);
}

int32_t qg_default_split_k_intn(int64_t m, int64_t n, int64_t k) {
  int32_t st = check_mnk(m, n, k);
  if (st != QG_OK) return st;
  return default_split_intn(m, n, k);
}

int32_t quantize_int4_g32(const void* w_bf16, int64_t n, int64_t k, void* packed,
                          int64_t packed_bytes, uint32_t* status_dev, void* stream) {
  if (!w_bf16 || !packed) return QG_E_NULL;
  int32_t st = check_nk(n, k);
  if (st != QG_OK) return st;
  if (packed_bytes < qg_int4_packed_bytes(n, k)) return QG_E_BUFFER;
  if (!aligned16(w_bf16) || !aligned16(packed) || ((uintptr_t)status_dev & 3u)) return QG_E_ALIGN;
  return hip_status(qg::launch_quantize_int4_g32(w_bf16, n, k, packed, status_dev,
                                                 static_cast<hipStream_t>(stream)));
}

int32_t quantize_int4_g32_dq(const void* w_bf16, int64_t n, int64_t k, void* packed,
                             int64_t packed_bytes, uint32_t* status_dev, void* stream) {
  if (!w_bf16 || !packed) return QG_E_NULL;
  int32_t st = check_nk(n, k);
  if (st != QG_OK) return st;
  if (packed_bytes < qg_int4_dq_packed_bytes(n, k)) return QG_E_BUFFER;
  if (!aligned16(w_bf16) || !aligned16(packed) || ((uintptr_t)status_dev & 3u)) return QG_E_ALIGN;
  return hip_status(qg::launch_quantize_int4_g32_dq(w_bf16, n, k, packed, status_dev,
                                                    static_cast<hipStream_t>(stream)));
}

int32_t quantize_intn_g32(const void* w_bf16, int64_t n, int64_t k, int32_t bits, void* packed,
                          int64_t packed_bytes, uint32_t* status_dev, void* stream) {
  if (!w_bf16 || !packed) return QG_E_NULL;
  int32_t st = check_nk(n, k);
  if (st != QG_OK) return st;
  if (bits != 5 && bits != 6) return QG_E_BITS;
  if (packed_bytes < qg_intn_packed_bytes(n, k, bits)) return QG_E_BUFFER;
  if (!aligned16(w_bf16) || !aligned16(packed) || ((uintptr_t)status_dev & 3u)) return QG_E_ALIGN;
  return hip_status(qg::launch_quantize_intn_g32(w_bf16, n, k, bits, packed, status_dev,
                                                 static_cast<hipStream_t>(stream)));
}

int32_t quantize_int8_rowwise(const void* w_bf16, int64_t n, int64_t k, int8_t* q,
                              void* scale_bf16, uint32_t* status_dev, void* stream) {
  if (!w_bf16 || !q || !scale_bf16) return QG_E_NULL;
  int32_t st = check_nk(n, k);
  if (st != QG_OK) return st;
  if (n > 0x7fffffff) return QG_E_SHAPE;
  if (!aligned16(w_bf16) || !aligned16(q) || !aligned16(scale_bf16) || ((uintptr_t)status_dev & 3u))
    return QG_E_ALIGN;
  return hip_status(qg::launch_quantize_int8_rowwise(w_bf16, n, k, q, scale_bf16, status_dev,
                                                     static_cast<hipStream_t>(stream)));
}

}  // extern "C"

namespace {

// Checks of qgemm_w4a16 that do not involve the workspace; sets the split.
int32_t w4a16_check(const void* x_bf16, int64_t m, int64_t k, const void* packed,
                    int64_t packed_bytes, int64_t n, const void* y, int32_t y_dtype,
                    int32_t split_k, int32_t* split) {
  if (!x_bf16 || !packed || !y) return QG_E_NULL;
  int32_t st = check_mnk(m, n, k);
  if (st != QG_OK) return st;
  if (y_dtype != QG_BF16 && y_dtype != QG_F32) return QG_E_DTYPE;
  st = resolve_split(m, n, k, split_k, split);
  if (st != QG_OK) return st;
  if (packed_bytes < qg_int4_packed_bytes(n, k)) return QG_E_BUFFER;
  if (!aligned16(x_bf16) || !aligned16(packed) || !aligned16(y)) return QG_E_ALIGN;
  return QG_OK;
}

// The launches of qgemm_w4a16 once every argument is checked; `partial` holds
// split * m * n fp32 partial sums when split > 1 (every element the reduce
// pass reads is written by the first pass of the same call).
int32_t w4a16_launch(const void* x_bf16, int64_t m, int64_t k, const void* packed, int64_t n,
                     void* y, int32_t y_dtype, int32_t split, float* partial, hipStream_t s) {
  int32_t st;
  if (m > 4) {
    // 5..64 rows: matrix-core kernel (rows padded to 16 and masked).
    st = hip_status(qg::launch_w4a16_mfma((int)m, x_bf16, packed, (int)n, (int)k, y,
                                          y_dtype == QG_F32, partial, split, s));
  } else {
    // M = 1: v_dot2c GEMV; M = 2..4: the same 32-row mapping on the 4x4x4
    // matrix instruction, whose cost does not grow with M.
    const GemvShape g = gemv_shape(m, n, split);
    if (m >= 2)
      st = hip_status(qg::launch_w4a16_gemv_mx4((int)m, x_bf16, packed, (int)n, (int)k, y,
                                                y_dtype == QG_F32, partial, split, g.waves, s));
    else if (g.rows == 32)
      st = hip_status(qg::launch_w4a16_gemv32((int)m, x_bf16, packed, (int)n, (int)k, y,
                                              y_dtype == QG_F32, partial, split, g.waves, s));
    else
      st = hip_status(qg::launch_w4a16_gemv((int)m, x_bf16, packed, (int)n, (int)k, y,
                                            y_dtype == QG_F32, partial, split, g.waves, s));
  }
  if (st != QG_OK || split == 1) return st;
  return hip_status(qg::launch_splitk_reduce(partial, split, m * n, y, y_dtype == QG_F32, s));
}

// The library's own device scratch for qgemm_w4a16_noalloc: one array per
// device (each GPU the library runs on holds its copy until the process
// ends).  Host code never uses the name `scratch` as an address (on the host
// it is a stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device with that device current, and is
// kept in scratch_addr.
static __device__ __align__(256) unsigned char scratch[QG_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_addr[kMaxDevices];
std::mutex scratch_mutex;

// Device address of the scratch array on the device `stream` belongs to (the
// current device for the default stream).
int32_t scratch_on(hipStream_t stream, void** out) {
  int dev = -1;
  if (stream ? hipStreamGetDevice(stream, &dev) != hipSuccess : hipGetDevice(&dev) != hipSuccess)
    return QG_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return QG_E_HIP;
  void* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (p) {
    *out = p;
    return QG_OK;
  }
  std::lock_guard<std::mutex> lock(scratch_mutex);
  p = scratch_addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return QG_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return QG_E_HIP;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return QG_E_HIP;
    if (e != hipSuccess || !p) return QG_E_HIP;
    scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return QG_OK;
}

}  // namespace

extern "C" {

int32_t qgemm_w4a16(const void* x_bf16, int64_t m, int64_t k, const void* packed,
                    int64_t packed_bytes, int64_t n, void* y, int32_t y_dtype, int32_t split_k,
                    void* ws, int64_t ws_bytes, void* stream) {
  int32_t split;
  int32_t st = w4a16_check(x_bf16, m, k, packed, packed_bytes, n, y, y_dtype, split_k, &split);
  if (st != QG_OK) return st;
  const int64_t need_ws = split > 1 ? (int64_t)split * m * n * 4 : 0;
  if (need_ws > 0 && (!ws || ws_bytes < need_ws)) return ws ? QG_E_BUFFER : QG_E_NULL;
  if (ws && !aligned16(ws)) return QG_E_ALIGN;
  return w4a16_launch(x_bf16, m, k, packed, n, y, y_dtype, split,
                      split > 1 ? static_cast<float*>(ws) : nullptr, static_cast<hipStream_t>(stream));
}

int32_t qgemm_w4a16_noalloc(const void* x_bf16, int64_t m, int64_t k, const void* packed,
                            int64_t packed_bytes, int64_t n, void* y, int32_t y_dtype,
                            int32_t split_k, void* stream) {
  int32_t split;
  int32_t st = w4a16_check(x_bf16, m, k, packed, packed_bytes, n, y, y_dtype, split_k, &split);
  if (st != QG_OK) return st;
  const int64_t need = split > 1 ? (int64_t)split * m * n * 4 : 0;
  if (need > QG_SCRATCH_BYTES) return QG_E_SCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* partial = nullptr;
  if (need > 0) {
    st = scratch_on(s, &partial);
    if (st != QG_OK) return st;
  }
  return w4a16_launch(x_bf16, m, k, packed, n, y, y_dtype, split, static_cast<float*>(partial), s);
}

int32_t qgemm_w4a16_dq(const void* x_bf16, int64_t m, int64_t k, const void* packed,
                       int64_t packed_bytes, int64_t n, void* y, int32_t y_dtype, int32_t split_k,
                       void* ws, int64_t ws_bytes, void* stream) {
  if (!x_bf16 || !packed || !y) return QG_E_NULL;
  int32_t st = check_mnk(m, n, k);
  if (st != QG_OK) return st;
  if (y_dtype != QG_BF16 && y_dtype != QG_F32) return QG_E_DTYPE;
  int32_t split;
  st = resolve_split(m, n, k, split_k, &split);
  if (st != QG_OK) return st;
  if (packed_bytes < qg_int4_dq_packed_bytes(n, k)) return QG_E_BUFFER;
  const int64_t need_ws = split > 1 ? (int64_t)split * m * n * 4 : 0;
  if (need_ws > 0 && (!ws || ws_bytes < need_ws)) return ws ? QG_E_BUFFER : QG_E_NULL;
  if (!aligned16(x_bf16) || !aligned16(packed) || !aligned16(y) || (ws && !aligned16(ws)))
    return QG_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* partial = split > 1 ? static_cast<float*>(ws) : nullptr;
  // the kernels of qgemm_w4a16 reading the scale-code layout: M = 1 the
  // v_dot2c GEMV (32- or 64-row workgroups by the same rule), M = 2..4 the
  // 4x4x4 matrix instruction, M = 5..64 the matrix cores
  if (m > 4)
    st = hip_status(qg::launch_w4a16_mfma_dq((int)m, x_bf16, packed, (int)n, (int)k, y, y_dtype == QG_F32,
                                             partial, split, s));
  else if (m >= 2)
    st = hip_status(qg::launch_w4a16_gemv_mx4_dq((int)m, x_bf16, packed, (int)n, (int)k, y,
                                                 y_dtype == QG_F32, partial, split, s));
  else if (gemv_shape(m, n, split).rows == 64)
    st = hip_status(qg::launch_w4a16_gemv_dq((int)m, x_bf16, packed, (int)n, (int)k, y,
                                             y_dtype == QG_F32, partial, split, s));
  else
    st = hip_status(qg::launch_w4a16_gemv32_dq((int)m, x_bf16, packed, (int)n, (int)k, y,
                                               y_dtype == QG_F32, partial, split, s));
  if (st != QG_OK || split == 1) return st;
  return hip_status(qg::launch_splitk_reduce(partial, split, m * n, y, y_dtype == QG_F32, s));
}

int32_t qgemm_wn_a16(const void* x_bf16, int64_t m, int64_t k, int32_t bits, const void* packed,
                     int64_t packed_bytes, int64_t n, void* y, int32_t y_dtype, int32_t split_k,
                     void* ws, int64_t ws_bytes, void* stream) {
  if (!x_bf16 || !packed || !y) return QG_E_NULL;
  int32_t st = check_mnk(m, n, k);
  if (st != QG_OK) return st;
  if (bits != 5 && bits != 6) return QG_E_BITS;
  if (y_dtype != QG_BF16 && y_dtype != QG_F32) return QG_E_DTYPE;
  int32_t split;
  st = resolve_split(m, n, k, split_k, &split, qg::SplitRule::kIntN);
  if (st != QG_OK) return st;
  if (packed_bytes < qg_intn_packed_bytes(n, k, bits)) return QG_E_BUFFER;
  const int64_t need_ws = split > 1 ? (int64_t)split * m * n * 4 : 0;
  if (need_ws > 0 && (!ws || ws_bytes < need_ws)) return ws ? QG_E_BUFFER : QG_E_NULL;
  if (!aligned16(x_bf16) || !aligned16(packed) || !aligned16(y) || (ws && !aligned16(ws)))
    return QG_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* partial = split > 1 ? static_cast<float*>(ws) : nullptr;
  // as for INT4: M = 1 the v_dot2c GEMV, M = 2..4 the 4x4x4 matrix-instruction
  // GEMV, M = 5..64 the matrix-core kernels
  if (m > 4)
    st = hip_status(qg::launch_wn_a16_mfma(bits, (int)m, x_bf16, packed, (int)n, (int)k, y,
                                           y_dtype == QG_F32, partial, split, s));
  else if (m >= 2)
    st = hip_status(qg::launch_wn_a16_gemv_mx4(bits, (int)m, x_bf16, packed, (int)n, (int)k, y,
                                               y_dtype == QG_F32, partial, split, s));
  else
    st = hip_status(qg::launch_wn_a16_gemv32(bits, x_bf16, packed, (int)n, (int)k, y, y_dtype == QG_F32,
                                             partial, split, s));
  if (st != QG_OK || split == 1) return st;
  return hip_status(qg::launch_splitk_reduce(partial, split, m * n, y, y_dtype == QG_F32, s));
}

int32_t qgemm_w8a16(const void* x_bf16, int64_t m, int64_t k, const int8_t* w,
                    const void* scale_bf16, int64_t n, void* y, int32_t y_dtype, void* stream) {
  if (!x_bf16 || !w || !scale_bf16 || !y) return QG_E_NULL;
  int32_t st = check_mnk(m, n, k);
  if (st != QG_OK) return st;
  if (y_dtype != QG_BF16 && y_dtype != QG_F32) return QG_E_DTYPE;
  // the M <= 4 GEMV holds a lane's x in registers: K up to 65536
  if (m <= 4 && qg::w8a16_chunks_per_wave((int)k) < 0) return QG_E_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(w) || !aligned16(y) || ((uintptr_t)scale_bf16 & 1u))
    return QG_E_ALIGN;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m > 4)   // 5..64 rows: the matrix cores
    return hip_status(qg::launch_w8a16_mfma((int)m, x_bf16, w, scale_bf16, (int)n, (int)k, y,
                                            y_dtype == QG_F32, s));
  return hip_status(qg::launch_w8a16_gemv((int)m, x_bf16, w, scale_bf16, (int)n, (int)k, y,
                                          y_dtype == QG_F32, s));
}

// One launch sequence of the M <= 4 W4A8 kernels (plus the split-K pass).
static int32_t w4a8_rows(const void* x_bf16, int64_t m, int64_t k, const void* packed, int64_t n,
                         void* y, int32_t y_dtype, int32_t split, float* partial, hipStream_t s,
                         bool group_scales, bool dq) {
  int32_t st;
  if (dq) {
    // the scale-code layout: the 32-row kernels of the branches below
    st = hip_status(qg::launch_w4a8_dq((int)m, group_scales, x_bf16, packed, (int)n, (int)k, y,
                                       y_dtype == QG_F32, partial, split, s));
  } else if (m > 1) {
    // M = 2..4: group dots on the 4x4x4 int8 matrix instruction
    st = hip_status(qg::launch_w4a8_gemv_mx4((int)m, group_scales, x_bf16, packed, (int)n, (int)k,
                                             y, y_dtype == QG_F32, partial, split, s));
  } else if (group_scales) {
    // M = 1, one scale per group: activations quantized once per workgroup through LDS
    st = hip_status(qg::launch_w4a8_gemv_lds((int)m, group_scales, x_bf16, packed, (int)n, (int)k,
                                             y, y_dtype == QG_F32, partial, split, s));
  } else {
    const GemvShape g = gemv_shape(m, n, split);
    st = hip_status(qg::launch_w4a8_gemv((int)m, x_bf16, packed, (int)n, (int)k, y,
                                         y_dtype == QG_F32, partial, split, g.rows, g.waves, s));
  }
  if (st != QG_OK || split == 1) return st;
  return hip_status(qg::launch_splitk_reduce(partial, split, m * n, y, y_dtype == QG_F32, s));
}

static int32_t w4a8_common(const void* x_bf16, int64_t m, int64_t k, const void* packed,
                           int64_t packed_bytes, int64_t n, void* y, int32_t y_dtype, int32_t split_k,
                           void* ws, int64_t ws_bytes, void* stream, bool group_scales, bool dq = false) {
  if (!x_bf16 || !packed || !y) return QG_E_NULL;
  int32_t st = check_mnk(m, n, k);
  if (st != QG_OK) return st;
  if (y_dtype != QG_BF16 && y_dtype != QG_F32) return QG_E_DTYPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (m > 4 && !group_scales) {
    // Per-row scales at 5..64 rows: x quantized once into the workspace (xq
    // exact in bf16), the bf16 matrix-core kernel on xq, then sx per row
    // after the split-K sum.
    int32_t split;
    st = resolve_split(m, n, k, split_k, &split);
    if (st != QG_OK) return st;
    if (packed_bytes < (dq ? qg_int4_dq_packed_bytes(n, k) : qg_int4_packed_bytes(n, k))) return QG_E_BUFFER;
    if (!ws || ws_bytes < w4a8_mfma_ws(m, n, k, split)) return ws ? QG_E_BUFFER : QG_E_NULL;
    if (!aligned16(x_bf16) || !aligned16(packed) || !aligned16(y) || !aligned16(ws)) return QG_E_ALIGN;
    char* w = static_cast<char*>(ws);
    float* sx = reinterpret_cast<float*>(w + m * k * 2);
    float* partial = reinterpret_cast<float*>(w + m * k * 2 + w4a8_scales_bytes(k));
    st = hip_status(qg::launch_w4a8_actquant_bf16((int)m, x_bf16, (int)k, w, sx, s));
    if (st != QG_OK) return st;
    if (split == 1) {
      // one split: the matrix-core kernel applies sx in its own store
      return hip_status(dq ? qg::launch_w4a16_mfma_dq((int)m, w, packed, (int)n, (int)k, y, y_dtype == QG_F32,
                                                      nullptr, 1, s, sx)
                           : qg::launch_w4a16_mfma((int)m, w, packed, (int)n, (int)k, y, y_dtype == QG_F32,
                                                   nullptr, 1, s, sx));
    }
    st = hip_status(dq ? qg::launch_w4a16_mfma_dq((int)m, w, packed, (int)n, (int)k, y, y_dtype == QG_F32,
                                                  partial, split, s)
                       : qg::launch_w4a16_mfma((int)m, w, packed, (int)n, (int)k, y, y_dtype == QG_F32,
                                               partial, split, s));
    if (st != QG_OK) return st;
    return hip_status(qg::launch_w4a8_rowscale_reduce(partial, split, (int)m, (int)n, sx, y,
                                                      y_dtype == QG_F32, s));
  }
  if (m > 4) {
    // One scale per group of 32 at 5..64 rows: x quantized once into the
    // workspace (xq exact in bf16, sx group-major), then the matrix-core
    // kernel scales each group's integer dot by s * sx, one weight pass.
    int32_t split;
    st = resolve_split(m, n, k, split_k, &split, qg::SplitRule::kW4A8G32);
    if (st != QG_OK) return st;
    if (packed_bytes < (dq ? qg_int4_dq_packed_bytes(n, k) : qg_int4_packed_bytes(n, k))) return QG_E_BUFFER;
    if (!ws || ws_bytes < w4a8_mfma_ws(m, n, k, split)) return ws ? QG_E_BUFFER : QG_E_NULL;
    if (!aligned16(x_bf16) || !aligned16(packed) || !aligned16(y) || !aligned16(ws)) return QG_E_ALIGN;
    char* w = static_cast<char*>(ws);
    float* sxg = reinterpret_cast<float*>(w + m * k * 2);
    float* partial = split > 1 ? reinterpret_cast<float*>(w + m * k * 2 + w4a8_scales_bytes(k)) : nullptr;
    st = hip_status(qg::launch_w4a8_actquant_g32_bf16((int)m, x_bf16, (int)k, w, sxg, s));
    if (st != QG_OK) return st;
    st = hip_status(qg::launch_w4a8g_mfma(dq, (int)m, w, sxg, packed, (int)n, (int)k, y, y_dtype == QG_F32,
                                          partial, split, s));
    if (st != QG_OK || split == 1) return st;
    return hip_status(qg::launch_splitk_reduce(partial, split, m * n, y, y_dtype == QG_F32, s));
  }
  const int64_t rows = m;
  int32_t split;
  st = resolve_split(rows, n, k, split_k, &split);
  if (st != QG_OK) return st;
  if (packed_bytes < (dq ? qg_int4_dq_packed_bytes(n, k) : qg_int4_packed_bytes(n, k))) return QG_E_BUFFER;
  const int64_t need_ws = split > 1 ? (int64_t)split * rows * n * 4 : 0;
  if (need_ws > 0 && (!ws || ws_bytes < need_ws)) return ws ? QG_E_BUFFER : QG_E_NULL;
  if (!aligned16(x_bf16) || !aligned16(packed) || !aligned16(y) || (ws && !aligned16(ws)))
    return QG_E_ALIGN;
  float* partial = split > 1 ? static_cast<float*>(ws) : nullptr;
  return w4a8_rows(x_bf16, m, k, packed, n, y, y_dtype, split, partial, s, group_scales, dq);
}

int32_t qgemm_w4a8(const void* x_bf16, int64_t m, int64_t k, const void* packed,
                   int64_t packed_bytes, int64_t n, void* y, int32_t y_dtype, int32_t split_k,
                   void* ws, int64_t ws_bytes, void* stream) {
  return w4a8_common(x_bf16, m, k, packed, packed_bytes, n, y, y_dtype, split_k, ws, ws_bytes,
                     stream, false);
}

int32_t qgemm_w4a8_g32(const void* x_bf16, int64_t m, int64_t k, const void* packed,
                       int64_t packed_bytes, int64_t n, void* y, int32_t y_dtype, int32_t split_k,
                       void* ws, int64_t ws_bytes, void* stream) {
  return w4a8_common(x_bf16, m, k, packed, packed_bytes, n, y, y_dtype, split_k, ws, ws_bytes,
                     stream, true);
}

int32_t qgemm_w4a8_dq(const void* x_bf16, int64_t m, int64_t k, const void* packed,
                      int64_t packed_bytes, int64_t n, void* y, int32_t y_dtype, int32_t split_k,
                      void* ws, int64_t ws_bytes, void* stream) {
  return w4a8_common(x_bf16, m, k, packed, packed_bytes, n, y, y_dtype, split_k, ws, ws_bytes,
                     stream, false, true);
}

int32_t qgemm_w4a8_g32_dq(const void* x_bf16, int64_t m, int64_t k, const void* packed,
                          int64_t packed_bytes, int64_t n, void* y, int32_t y_dtype, int32_t split_k,
                          void* ws, int64_t ws_bytes, void* stream) {
  return w4a8_common(x_bf16, m, k, packed, packed_bytes, n, y, y_dtype, split_k, ws, ws_bytes,
                     stream, true, true);
}

int32_t qg_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t blocks,
                       void* stream) {
  if (!src || !sink) return QG_E_NULL;
  if (bytes < 16 || bytes % 16 != 0) return QG_E_SHAPE;
  if (blocks < 1 || blocks > 65536) return QG_E_SHAPE;
  if (!aligned16(src) || ((uintptr_t)sink & 3u)) return QG_E_ALIGN;
  return hip_status(qg::launch_stream_read(src, bytes, sink, blocks, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
