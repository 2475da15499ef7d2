// Measurement aid: a plain streaming-read kernel, used to report the HBM read
// rate the device sustains next to the decode kernels' rate.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kvattn_measure.h"

namespace kvattn {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, size_t n,
                                                          uint32_t *sink) {
  constexpr int U = 8;  // 16-byte words in flight per lane
  const size_t stride = (size_t)gridDim.x * 256 * U;
  uint32_t acc = 0;
  for (size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x; i < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + (size_t)u * 256;
      v[u] = j < n ? __builtin_nontemporal_load(p + j) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x9e3779b9u) sink[blockIdx.x] = acc;
}

}  // namespace kvattn

extern "C" int kvattn_measure_stream_read(const void *buf, size_t bytes, int workgroups, uint32_t *sink,
                                          void *stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0 || workgroups <= 0)
    return KVATTN_ERR_INVALID_ARG;
  kvattn::stream_read_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream>>>(
      (const kvattn::u32x4 *)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ERR_HIP;
}
