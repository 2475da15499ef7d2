// The cache objects behind the opaque kvattn_cache and kvattn_paged handles,
// shared by the C ABI (kvattn.hip), its host-side validation (validate.hpp)
// and the decoder that drives the contiguous cache (model.hip).  Plain host
// structs: device memory appears only as pointers.
#pragma once

#include <stddef.h>
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

// The block-paged cache: one pool allocation laid out
// [layer][K|V][num_blocks][Hkv][block_size][D]; one block table per slot
// (device, [slots][max_blocks], the same for every layer); lengths
// [layer][slots] on the device with a host mirror.
struct kvattn_paged {
  int layers, slots, q_heads, kv_heads, head_dim;
  int num_blocks, block_size, block_log2, max_blocks;
  kvattn_dtype dt;
  int elem;
  size_t payload_bytes, layer_bytes;
  char *base;
  bool owns_base;
  int32_t *d_len;              // [layers][slots]
  std::vector<int32_t> h_len;  // host mirror
  int32_t *d_table;            // [slots][max_blocks]
  int32_t *d_nblk;             // [slots] blocks assigned per slot (device copy of h_nblk)
  std::vector<int> h_nblk;     // table entries set per slot
  std::vector<int> window, sink;  // per layer; window 0 = none
  float *d_ws;
  int chunk, n_splits;
  int device;
};

namespace kvattn {

inline char *cache_layer_k(const kvattn_cache *c, int layer) { return c->base + (size_t)layer * c->layer_bytes; }
inline char *cache_layer_v(const kvattn_cache *c, int layer) { return cache_layer_k(c, layer) + c->layer_bytes / 2; }

}  // namespace kvattn
