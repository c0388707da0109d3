// stream_read.hip -- the measured read ceiling that the GEMVs' bandwidth is
// compared with: a plain streaming read of a device buffer, one 16-byte
// non-temporal load per lane per step, no arithmetic but an XOR that keeps
// the loads alive.  Not part of the layer; the benchmark times it over the
// same rotating weight copies the GEMV reads.
//
// Mapping: a workgroup of 256 lanes reads 2 x 16 bytes per lane per step
// (8 KB, 64 whole 128-byte lines) and strides over the buffer by the grid's
// size; each wave leaves one XOR word in `sink`.
#include "qg_common.h"

namespace qg {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  const int tid = threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * 512;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * 512; base < n16; base += stride) {
    const int64_t i0 = base + tid, i1 = i0 + 256;
    if (i1 < n16) {
      const u32x4_t a = __builtin_nontemporal_load(src + i0);
      const u32x4_t b = __builtin_nontemporal_load(src + i1);
      acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    } else if (i0 < n16) {
      const u32x4_t a = __builtin_nontemporal_load(src + i0);
      acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off, 64);
  if ((tid & 63) == 0) sink[(int64_t)blockIdx.x * 4 + (tid >> 6)] = acc;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int blocks,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const u32x4_t*>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace qg
