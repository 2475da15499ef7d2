// Host-side validation of the C ABI's calls, and the updates of the host
// mirror of the lengths that follow a successful enqueue.
//
// Every entry point checks all of its arguments and the cache state here
// before it touches the device, so a refused call (INVALID_ARG, UNSUPPORTED,
// CAPACITY, STATE) changes neither the device lengths nor their host mirror.
// Plain C++ over the host fields of the cache objects: no HIP, so the
// checks can be exercised on a machine without a GPU, on cache objects
// built on the host.
#pragma once

#include <stdint.h>

#include <cmath>

#include "cache.hpp"
#include "kvattn.h"

namespace kvattn {

inline int elem_bytes(kvattn_dtype dt) {
  switch (dt) {
    case KVATTN_F32: return 4;
    case KVATTN_F16: return 2;
    case KVATTN_BF16: return 2;
  }
  return 0;
}

inline bool supported_dim(int d) { return d == 32 || d == 64 || d == 128; }

// the softmax scale: finite and positive (NaN fails the first test)
inline bool valid_scale(float scale) { return scale > 0.f && std::isfinite(scale); }

// ---------------------------------------------------------------- contiguous cache
inline bool valid_out_dtype(const kvattn_cache *c, kvattn_dtype o) { return o == c->dt || o == KVATTN_F32; }

inline int check_layer(const kvattn_cache *c, int layer) {
  if (!c) return KVATTN_ERR_INVALID_ARG;
  if (layer < 0 || layer >= c->layers) return KVATTN_ERR_INVALID_ARG;
  return KVATTN_OK;
}

inline const int32_t *host_lengths(const kvattn_cache *c, int layer) { return &c->h_len[(size_t)layer * c->batch]; }

// set_lengths: layer >= 0 or -1 (all); each length in [0, max_T]
inline int validate_set_lengths(const kvattn_cache *c, int layer, const int32_t *host_lens) {
  if (!c || !host_lens) return KVATTN_ERR_INVALID_ARG;
  if (layer != -1 && (layer < 0 || layer >= c->layers)) return KVATTN_ERR_INVALID_ARG;
  for (int b = 0; b < c->batch; ++b)
    if (host_lens[b] < 0 || host_lens[b] > c->max_T) return KVATTN_ERR_CAPACITY;
  return KVATTN_OK;
}

inline int validate_set_window(const kvattn_cache *c, int layer, int window, int sink) {
  if (!c) return KVATTN_ERR_INVALID_ARG;
  if (layer != -1 && (layer < 0 || layer >= c->layers)) return KVATTN_ERR_INVALID_ARG;
  if (window < 0 || sink < 0) return KVATTN_ERR_INVALID_ARG;
  return KVATTN_OK;
}

// prefill: every length of the layer 0, 1 <= T <= max_T
inline int validate_prefill(const kvattn_cache *c, int layer, const void *q, const void *k, const void *v,
                            const void *o, int T, float scale, kvattn_dtype o_dtype) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  if (!q || !k || !v || !o) return KVATTN_ERR_INVALID_ARG;
  if (T <= 0 || !valid_scale(scale)) return KVATTN_ERR_INVALID_ARG;
  if (!valid_out_dtype(c, o_dtype)) return KVATTN_ERR_UNSUPPORTED;
  if (T > c->max_T) return KVATTN_ERR_CAPACITY;
  const int32_t *hl = host_lengths(c, layer);
  for (int b = 0; b < c->batch; ++b)
    if (hl[b] != 0) return KVATTN_ERR_STATE;
  return KVATTN_OK;
}

// extend: len[b] + T <= max_T for every sequence
inline int validate_extend(const kvattn_cache *c, int layer, const void *q, const void *k, const void *v,
                           const void *o, int T, float scale, kvattn_dtype o_dtype) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  if (!q || !k || !v || !o) return KVATTN_ERR_INVALID_ARG;
  if (T <= 0 || !valid_scale(scale)) return KVATTN_ERR_INVALID_ARG;
  if (!valid_out_dtype(c, o_dtype)) return KVATTN_ERR_UNSUPPORTED;
  const int32_t *hl = host_lengths(c, layer);
  for (int b = 0; b < c->batch; ++b)
    if (hl[b] > c->max_T - T) return KVATTN_ERR_CAPACITY;
  return KVATTN_OK;
}

// append: every sequence below max_T
inline int validate_append(const kvattn_cache *c, int layer, const void *k_new, const void *v_new) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  if (!k_new || !v_new) return KVATTN_ERR_INVALID_ARG;
  const int32_t *hl = host_lengths(c, layer);
  for (int b = 0; b < c->batch; ++b)
    if (hl[b] >= c->max_T) return KVATTN_ERR_CAPACITY;
  return KVATTN_OK;
}

// decode: every sequence holds at least one position
inline int validate_decode(const kvattn_cache *c, int layer, const void *q, const void *o, float scale,
                           kvattn_dtype o_dtype) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  if (!q || !o) return KVATTN_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return KVATTN_ERR_INVALID_ARG;
  if (!valid_out_dtype(c, o_dtype)) return KVATTN_ERR_UNSUPPORTED;
  const int32_t *hl = host_lengths(c, layer);
  for (int b = 0; b < c->batch; ++b)
    if (hl[b] <= 0) return KVATTN_ERR_STATE;
  return KVATTN_OK;
}

// the fused step: the append's capacity check; a length of 0 is allowed (the
// query then sees its own row only)
inline int validate_append_decode(const kvattn_cache *c, int layer, const void *k_new, const void *v_new,
                                  const void *q, const void *o, float scale, kvattn_dtype o_dtype) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  if (!k_new || !v_new || !q || !o) return KVATTN_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return KVATTN_ERR_INVALID_ARG;
  if (!valid_out_dtype(c, o_dtype)) return KVATTN_ERR_UNSUPPORTED;
  const int32_t *hl = host_lengths(c, layer);
  for (int b = 0; b < c->batch; ++b)
    if (hl[b] >= c->max_T) return KVATTN_ERR_CAPACITY;
  return KVATTN_OK;
}

// mirror updates, after the work is enqueued
inline void mirror_set(kvattn_cache *c, int layer, int32_t value) {
  for (int b = 0; b < c->batch; ++b) c->h_len[(size_t)layer * c->batch + b] = value;
}
inline void mirror_add(kvattn_cache *c, int layer, int32_t delta) {
  for (int b = 0; b < c->batch; ++b) c->h_len[(size_t)layer * c->batch + b] += delta;
}
inline void mirror_copy(kvattn_cache *c, int layer, const int32_t *host_lens) {
  const int first = layer < 0 ? 0 : layer;
  const int count = layer < 0 ? c->layers : 1;
  for (int l = first; l < first + count; ++l)
    for (int b = 0; b < c->batch; ++b) c->h_len[(size_t)l * c->batch + b] = host_lens[b];
}

// ---------------------------------------------------------------- paged cache
inline int paged_check_layer(const kvattn_paged *p, int layer) {
  if (!p || layer < 0 || layer >= p->layers) return KVATTN_ERR_INVALID_ARG;
  return KVATTN_OK;
}

inline int paged_capacity(const kvattn_paged *p, int slot) { return p->h_nblk[slot] * p->block_size; }

inline const int32_t *paged_host_lengths(const kvattn_paged *p, int layer) {
  return &p->h_len[(size_t)layer * p->slots];
}

// set_blocks: ids inside the pool, at most max_blocks, and no layer's length
// of the slot past the new blocks
inline int validate_paged_set_blocks(const kvattn_paged *p, int slot, const int32_t *ids, int n_blocks) {
  if (!p || slot < 0 || slot >= p->slots || n_blocks < 0 || n_blocks > p->max_blocks) return KVATTN_ERR_INVALID_ARG;
  if (n_blocks > 0 && !ids) return KVATTN_ERR_INVALID_ARG;
  for (int i = 0; i < n_blocks; ++i)
    if (ids[i] < 0 || ids[i] >= p->num_blocks) return KVATTN_ERR_INVALID_ARG;
  for (int l = 0; l < p->layers; ++l)
    if (p->h_len[(size_t)l * p->slots + slot] > n_blocks * p->block_size) return KVATTN_ERR_CAPACITY;
  return KVATTN_OK;
}

inline int validate_paged_set_lengths(const kvattn_paged *p, int layer, const int32_t *host_lens) {
  if (!p || !host_lens) return KVATTN_ERR_INVALID_ARG;
  if (layer != -1 && (layer < 0 || layer >= p->layers)) return KVATTN_ERR_INVALID_ARG;
  for (int s = 0; s < p->slots; ++s)
    if (host_lens[s] < 0 || host_lens[s] > paged_capacity(p, s)) return KVATTN_ERR_CAPACITY;
  return KVATTN_OK;
}

inline int validate_paged_prefill(const kvattn_paged *p, int layer, const void *q, const void *k, const void *v,
                                  const void *o, int T, float scale, kvattn_dtype o_dtype) {
  int rc = paged_check_layer(p, layer);
  if (rc) return rc;
  if (!q || !k || !v || !o) return KVATTN_ERR_INVALID_ARG;
  if (T <= 0 || !valid_scale(scale)) return KVATTN_ERR_INVALID_ARG;
  if (o_dtype != p->dt && o_dtype != KVATTN_F32) return KVATTN_ERR_UNSUPPORTED;
  const int32_t *hl = paged_host_lengths(p, layer);
  for (int s = 0; s < p->slots; ++s)
    if (hl[s] != 0) return KVATTN_ERR_STATE;
  for (int s = 0; s < p->slots; ++s)
    if (T > paged_capacity(p, s)) return KVATTN_ERR_CAPACITY;
  return KVATTN_OK;
}

inline int validate_paged_append(const kvattn_paged *p, int layer, const void *k_new, const void *v_new) {
  int rc = paged_check_layer(p, layer);
  if (rc) return rc;
  if (!k_new || !v_new) return KVATTN_ERR_INVALID_ARG;
  const int32_t *hl = paged_host_lengths(p, layer);
  for (int s = 0; s < p->slots; ++s)
    if (hl[s] >= paged_capacity(p, s)) return KVATTN_ERR_CAPACITY;
  return KVATTN_OK;
}

inline int validate_paged_extend(const kvattn_paged *p, int layer, const void *q, const void *k, const void *v,
                                 const void *o, int T, float scale, kvattn_dtype o_dtype) {
  int rc = paged_check_layer(p, layer);
  if (rc) return rc;
  if (!q || !k || !v || !o) return KVATTN_ERR_INVALID_ARG;
  if (T <= 0 || !valid_scale(scale)) return KVATTN_ERR_INVALID_ARG;
  if (o_dtype != p->dt && o_dtype != KVATTN_F32) return KVATTN_ERR_UNSUPPORTED;
  const int32_t *hl = paged_host_lengths(p, layer);
  for (int s = 0; s < p->slots; ++s)
    if (hl[s] > paged_capacity(p, s) - T) return KVATTN_ERR_CAPACITY;
  return KVATTN_OK;
}

inline int validate_paged_decode(const kvattn_paged *p, int layer, const void *q, const void *o, float scale,
                                 kvattn_dtype o_dtype) {
  int rc = paged_check_layer(p, layer);
  if (rc) return rc;
  if (!q || !o) return KVATTN_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return KVATTN_ERR_INVALID_ARG;
  if (o_dtype != p->dt && o_dtype != KVATTN_F32) return KVATTN_ERR_UNSUPPORTED;
  const int32_t *hl = paged_host_lengths(p, layer);
  for (int s = 0; s < p->slots; ++s)
    if (hl[s] <= 0) return KVATTN_ERR_STATE;
  return KVATTN_OK;
}

inline void paged_mirror_set(kvattn_paged *p, int layer, int32_t value) {
  for (int s = 0; s < p->slots; ++s) p->h_len[(size_t)layer * p->slots + s] = value;
}
inline void paged_mirror_add(kvattn_paged *p, int layer, int32_t delta) {
  for (int s = 0; s < p->slots; ++s) p->h_len[(size_t)layer * p->slots + s] += delta;
}

}  // namespace kvattn
