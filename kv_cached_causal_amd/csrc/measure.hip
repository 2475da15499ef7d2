// Measurement aids: a plain streaming-read kernel, used to report the HBM read
// rate the device sustains next to the decode kernels' rate; a plain
// streaming-write kernel, whose byte count calibrates the write counters; a plain
// matrix-core loop, used to report the fp16 MFMA rate it sustains next to the
// prefill kernel's rate; and a plain exp2 loop, used to report the rate of the
// exponentials (one per score) that bound prefill at small head dims.
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

// Writes n 16-byte words, each lane storing whole words with a grid stride
// (plain coalesced stores, as the attention kernels' output and cache rows).
__global__ __launch_bounds__(256) void stream_write_kernel(u32x4 *__restrict__ p, size_t n) {
  constexpr int U = 4;
  const size_t stride = (size_t)gridDim.x * 256 * U;
  for (size_t i = (size_t)blockIdx.x * 256 * U + threadIdx.x; i < n; i += stride) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t j = i + (size_t)u * 256;
      const uint32_t w = (uint32_t)j;
      if (j < n) p[j] = u32x4{w, w ^ 0x55555555u, w + 1u, ~w};
    }
  }
}

// Each wave runs `iters` rounds of NCH independent accumulation chains of
// v_mfma_f32_16x16x32_f16 on register operands (no memory traffic in the
// loop); enough independent chains keep the matrix pipeline full.
constexpr int kMfmaChains = 8;
__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(int iters, float *sink) {
  const _Float16 x = (_Float16)(1.0f + (float)(threadIdx.x & 7) * 0.0078125f);
  half8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = x;
    b[i] = (_Float16)(0.5f) - x * (_Float16)(0.001f * (float)i);
  }
  float4_t acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = float4_t{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[c], 0, 0, 0);
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) r += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  if (r == 1234.5f) sink[blockIdx.x] = r;
}

// Each thread runs `iters` rounds of NCH independent chains x <- exp2(-x)
// (v_exp_f32 with a negated source: one instruction per exponential; the
// chains settle near 0.64, always normal numbers).  Enough chains that the
// instruction's latency is hidden: with 8 chains on 1024 workgroups the loop
// measured 13.3 T exp2/s, with 32 chains on 4096 workgroups 18.9.
constexpr int kExpChains = 32;
__global__ __launch_bounds__(256, 2) void exp_loop_kernel(int iters, float *sink) {
  float x[kExpChains];
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) x[c] = (float)(threadIdx.x & 7) * 0.125f + (float)c * 0.01f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kExpChains; ++c) x[c] = fast_exp2(-x[c]);
  }
  float r = 0.f;
#pragma unroll
  for (int c = 0; c < kExpChains; ++c) r += x[c];
  if (r == 1234.5f) sink[blockIdx.x] = r;
}

}  // namespace kvattn

extern "C" int kvattn_measure_exp2(int workgroups, int iters, float *sink, void *stream) {
  if (!sink || workgroups <= 0 || iters <= 0) return KVATTN_ERR_INVALID_ARG;
  kvattn::exp_loop_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ERR_HIP;
}

extern "C" double kvattn_measure_exp2_count(int workgroups, int iters) {
  if (workgroups <= 0 || iters <= 0) return 0.0;
  return (double)workgroups * 256 * iters * kvattn::kExpChains;
}

extern "C" int kvattn_measure_mfma_f16(int workgroups, int iters, float *sink, void *stream) {
  if (!sink || workgroups <= 0 || iters <= 0) return KVATTN_ERR_INVALID_ARG;
  kvattn::mfma_loop_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream>>>(iters, sink);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ERR_HIP;
}

extern "C" double kvattn_measure_mfma_f16_flops(int workgroups, int iters) {
  if (workgroups <= 0 || iters <= 0) return 0.0;
  return (double)workgroups * 4 /* waves */ * iters * kvattn::kMfmaChains * (16.0 * 16.0 * 32.0 * 2.0);
}

extern "C" int kvattn_measure_stream_write(void *buf, size_t bytes, int workgroups, void *stream) {
  if (!buf || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0 || workgroups <= 0)
    return KVATTN_ERR_INVALID_ARG;
  kvattn::stream_write_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream>>>(
      (kvattn::u32x4 *)buf, bytes / 16);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ERR_HIP;
}

extern "C" int kvattn_measure_stream_read(const void *buf, size_t bytes, int workgroups, uint32_t *sink,
                                          void *stream) {
  if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || ((uintptr_t)buf & 15u) != 0 || workgroups <= 0)
    return KVATTN_ERR_INVALID_ARG;
  kvattn::stream_read_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream>>>(
      (const kvattn::u32x4 *)buf, bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? KVATTN_OK : KVATTN_ERR_HIP;
}
