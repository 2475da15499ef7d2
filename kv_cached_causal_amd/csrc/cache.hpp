// The contiguous cache object behind the opaque kvattn_cache handle, shared by
// the C ABI (kvattn.hip) and the decoder that drives it (model.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

#include "kvattn.h"

struct kvattn_cache {
  int layers, batch, q_heads, kv_heads, head_dim, max_T;
  kvattn_dtype dt;
  int elem;               // bytes per element
  size_t payload_bytes;   // = kvattn_cache_bytes(...)
  size_t layer_bytes;     // K block + V block of one layer
  char *base;             // payload (device)
  bool owns_base;
  int32_t *d_len;         // [layers][batch] (device)
  std::vector<int32_t> h_len;  // host mirror
  std::vector<int> window, sink;  // per layer: sliding window (0: none), sink positions
  float *d_ws;            // decode split-K workspace (device)
  int32_t *d_cnt;         // fused decode step: [B][kStepSlots] (counter, attended count)
  float *d_pws;           // prefill split workspace (null when no prompt up to max_T splits)
  int32_t *d_pcnt;        // prefill split counters, zero between calls
  int chunk, n_splits;
  int device;
};

namespace kvattn {

inline char *cache_layer_k(const kvattn_cache *c, int layer) { return c->base + (size_t)layer * c->layer_bytes; }
inline char *cache_layer_v(const kvattn_cache *c, int layer) { return cache_layer_k(c, layer) + c->layer_bytes / 2; }

}  // namespace kvattn
