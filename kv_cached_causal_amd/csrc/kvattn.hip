// The C ABI of libkvattn: cache object, host-side validation, launches.
//
// The cache is one device allocation laid out [layer][K|V][B][Hkv][max_T][D],
// sized by the inference chapter's capacity formula (section 9.3), plus a
// lengths array [layer][B] (int32, device) with a host mirror, and a split-K
// workspace for decode.  Every entry point validates all of its arguments on
// the host before it enqueues anything, so a failed call never mutates the
// cache or its mirror.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "cache.hpp"
#include "common.hpp"
#include "kvattn.h"
#include "kvattn_measure.h"
#include "validate.hpp"

using namespace kvattn;


namespace {

thread_local char g_last_error[256] = "";

int hip_fail(hipError_t e, const char *where) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", where, hipGetErrorString(e));
  return KVATTN_ERR_HIP;
}

int check_device(const kvattn_cache *c) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != c->device) {
    std::snprintf(g_last_error, sizeof g_last_error,
                  "cache lives on device %d but device %d is current", c->device, dev);
    return KVATTN_ERR_STATE;
  }
  return KVATTN_OK;
}

char *layer_k(const kvattn_cache *c, int layer) { return c->base + (size_t)layer * c->layer_bytes; }
char *layer_v(const kvattn_cache *c, int layer) {
  return layer_k(c, layer) + c->layer_bytes / 2;
}

}  // namespace

// Split-K workspace of kvattn_decode_noalloc: a fixed device array, so that
// call allocates nothing.  Each device that loads the library holds its own
// copy until the process ends.  In host code `scratch` is only a stand-in
// for the device array: its device address comes from hipGetSymbolAddress,
// looked up once per device (with that device current) and kept below.
static __device__ __align__(256) float scratch[KVATTN_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

std::mutex g_scratch_mu;
std::vector<float *> g_scratch_ptr;  // per device ordinal; null until looked up

// device address of `scratch` on the current device, or null on error
float *scratch_on_current_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = (float *)p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

size_t kvattn_cache_bytes(int layers, int batch, int kv_heads, int head_dim, int max_T,
                          kvattn_dtype dt) {
  const int e = elem_bytes(dt);
  if (layers <= 0 || batch <= 0 || kv_heads <= 0 || head_dim <= 0 || max_T <= 0 || e == 0) return 0;
  return (size_t)2 * layers * kv_heads * head_dim * (size_t)max_T * e * batch;
}

int kvattn_cache_alloc(kvattn_cache **out, int layers, int batch, int q_heads, int kv_heads,
                       int head_dim, int max_T, kvattn_dtype dt, void *device_buf,
                       size_t device_buf_bytes) {
  if (!out) return KVATTN_ERR_INVALID_ARG;
  *out = nullptr;
  if (layers <= 0 || batch <= 0 || q_heads <= 0 || kv_heads <= 0 || head_dim <= 0 || max_T <= 0)
    return KVATTN_ERR_INVALID_ARG;
  if (elem_bytes(dt) == 0 || !supported_dim(head_dim) || q_heads % kv_heads != 0)
    return KVATTN_ERR_UNSUPPORTED;
  const size_t bytes = kvattn_cache_bytes(layers, batch, kv_heads, head_dim, max_T, dt);
  if (device_buf) {
    if (device_buf_bytes < bytes) return KVATTN_ERR_OOM;
    if (((uintptr_t)device_buf & 255u) != 0) return KVATTN_ERR_INVALID_ARG;
  }

  kvattn_cache *c = new (std::nothrow) kvattn_cache();
  if (!c) return KVATTN_ERR_OOM;
  c->layers = layers;
  c->batch = batch;
  c->q_heads = q_heads;
  c->kv_heads = kv_heads;
  c->head_dim = head_dim;
  c->max_T = max_T;
  c->dt = dt;
  c->elem = elem_bytes(dt);
  c->payload_bytes = bytes;
  c->layer_bytes = bytes / layers;
  c->chunk = decode_chunk(head_dim, q_heads / kv_heads, max_T);
  c->n_splits = (max_T + c->chunk - 1) / c->chunk;
  c->h_len.assign((size_t)layers * batch, 0);
  c->window.assign(layers, 0);
  c->sink.assign(layers, 0);

  hipError_t e = hipGetDevice(&c->device);
  if (e != hipSuccess) {
    delete c;
    return hip_fail(e, "hipGetDevice");
  }
  if (device_buf) {
    c->base = (char *)device_buf;
    c->owns_base = false;
  } else {
    e = hipMalloc((void **)&c->base, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      delete c;
      std::snprintf(g_last_error, sizeof g_last_error, "hipMalloc(%zu): %s", bytes,
                    hipGetErrorString(e));
      return KVATTN_ERR_OOM;
    }
    c->owns_base = true;
  }
  const size_t len_bytes = sizeof(int32_t) * (size_t)layers * batch;
  // split-K workspace for decode and for the short extends run on the decode
  // kernels (up to kMaxVerifyTokens query positions per head)
  const size_t ws_bytes = sizeof(float) * (size_t)batch * q_heads * kMaxVerifyTokens * c->n_splits * (head_dim + 2);
  const size_t cnt_bytes = sizeof(int32_t) * step_counter_ints(batch, q_heads);
  // prefill split of heavy query tiles: partials and counters for the
  // largest split any prompt up to max_T takes
  const int split_max = prefill_uses_split(dt, head_dim) ? prefill_split_tiles_max(max_T, q_heads) : 0;
  const size_t pws_bytes = sizeof(float) * (size_t)split_max * batch * q_heads * 2 * prefill_split_half_floats(head_dim);
  const size_t pcnt_bytes = sizeof(int32_t) * (size_t)split_max * batch * q_heads;
  e = hipMalloc((void **)&c->d_len, len_bytes);
  if (e == hipSuccess) e = hipMalloc((void **)&c->d_ws, ws_bytes);
  if (e == hipSuccess) e = hipMalloc((void **)&c->d_cnt, cnt_bytes);
  if (e == hipSuccess && split_max) e = hipMalloc((void **)&c->d_pws, pws_bytes);
  if (e == hipSuccess && split_max) e = hipMalloc((void **)&c->d_pcnt, pcnt_bytes);
  if (e == hipSuccess) e = hipMemset(c->d_len, 0, len_bytes);
  if (e == hipSuccess) e = hipMemset(c->d_cnt, 0, cnt_bytes);
  if (e == hipSuccess && split_max) e = hipMemset(c->d_pcnt, 0, pcnt_bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    int rc = hip_fail(e, "cache side buffers");
    (void)hipGetLastError();
    if (c->d_len) (void)hipFree(c->d_len);
    if (c->d_ws) (void)hipFree(c->d_ws);
    if (c->d_cnt) (void)hipFree(c->d_cnt);
    if (c->d_pws) (void)hipFree(c->d_pws);
    if (c->d_pcnt) (void)hipFree(c->d_pcnt);
    if (c->owns_base) (void)hipFree(c->base);
    delete c;
    return e == hipErrorOutOfMemory ? KVATTN_ERR_OOM : rc;
  }
  *out = c;
  return KVATTN_OK;
}

int kvattn_cache_free(kvattn_cache *c) {
  if (!c) return KVATTN_ERR_INVALID_ARG;
  hipError_t e = hipDeviceSynchronize();
  hipError_t e1 = hipFree(c->d_len);
  hipError_t e2 = hipFree(c->d_ws);
  hipError_t e4 = hipFree(c->d_cnt);
  hipError_t e5 = c->d_pws ? hipFree(c->d_pws) : hipSuccess;
  hipError_t e6 = c->d_pcnt ? hipFree(c->d_pcnt) : hipSuccess;
  hipError_t e3 = c->owns_base ? hipFree(c->base) : hipSuccess;
  delete c;
  if (e != hipSuccess) return hip_fail(e, "kvattn_cache_free sync");
  if (e1 != hipSuccess) return hip_fail(e1, "hipFree(lengths)");
  if (e2 != hipSuccess) return hip_fail(e2, "hipFree(workspace)");
  if (e4 != hipSuccess) return hip_fail(e4, "hipFree(split counters)");
  if (e5 != hipSuccess) return hip_fail(e5, "hipFree(prefill split workspace)");
  if (e6 != hipSuccess) return hip_fail(e6, "hipFree(prefill split counters)");
  if (e3 != hipSuccess) return hip_fail(e3, "hipFree(payload)");
  return KVATTN_OK;
}

int kvattn_cache_kv_ptr(const kvattn_cache *c, int layer, void **k, void **v) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  if (!k || !v) return KVATTN_ERR_INVALID_ARG;
  *k = layer_k(c, layer);
  *v = layer_v(c, layer);
  return KVATTN_OK;
}

int kvattn_cache_set_lengths(kvattn_cache *c, int layer, const int32_t *host_lens, void *stream) {
  int rc = validate_set_lengths(c, layer, host_lens);
  if (rc) return rc;
  rc = check_device(c);
  if (rc) return rc;
  const int first = layer < 0 ? 0 : layer;
  const int count = layer < 0 ? c->layers : 1;
  hipError_t e = launch_set_lengths(c->d_len + (size_t)first * c->batch, count, c->batch, host_lens,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "set_lengths launch");
  mirror_copy(c, layer, host_lens);
  return KVATTN_OK;
}

int kvattn_cache_set_window(kvattn_cache *c, int layer, int window, int sink) {
  int rc = validate_set_window(c, layer, window, sink);
  if (rc) return rc;
  const int first = layer < 0 ? 0 : layer;
  const int count = layer < 0 ? c->layers : 1;
  for (int l = first; l < first + count; ++l) {
    c->window[l] = window;
    c->sink[l] = window > 0 ? sink : 0;
  }
  return KVATTN_OK;
}

int kvattn_cache_get_window(const kvattn_cache *c, int layer, int *window, int *sink) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  if (!window || !sink) return KVATTN_ERR_INVALID_ARG;
  *window = c->window[layer];
  *sink = c->sink[layer];
  return KVATTN_OK;
}

int kvattn_cache_get_lengths(const kvattn_cache *c, int layer, int32_t *host_lens) {
  int rc = check_layer(c, layer);
  if (rc) return rc;
  if (!host_lens) return KVATTN_ERR_INVALID_ARG;
  std::memcpy(host_lens, &c->h_len[(size_t)layer * c->batch], sizeof(int32_t) * c->batch);
  return KVATTN_OK;
}

}  // extern "C"

namespace {

int prefill_impl(kvattn_cache *c, int layer, const void *q, const void *k, const void *v, void *o, int T,
                 float scale, kvattn_dtype o_dtype, void *stream, uint64_t *clock_sample) {
  int rc = validate_prefill(c, layer, q, k, v, o, T, scale, o_dtype);
  if (rc) return rc;
  rc = check_device(c);
  if (rc) return rc;

  PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.cache_k = layer_k(c, layer);
  a.cache_v = layer_v(c, layer);
  a.len = c->d_len + (size_t)layer * c->batch;
  a.offsets = nullptr;
  a.batch = c->batch;
  a.q_heads = c->q_heads;
  a.kv_heads = c->kv_heads;
  a.head_dim = c->head_dim;
  a.T = T;
  a.max_T = c->max_T;
  a.kv_rows = T;
  a.write_cache = 1;
  a.window = c->window[layer];
  a.sink = c->sink[layer];
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dt = c->dt;
  a.o_dt = o_dtype;
  a.clock_sample = clock_sample;
  a.split_ws = c->d_pws;
  a.split_cnt = c->d_pcnt;
  hipError_t e = launch_prefill(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  mirror_set(c, layer, T);
  return KVATTN_OK;
}

}  // namespace

extern "C" {

int kvattn_prefill(kvattn_cache *c, int layer, const void *q, const void *k, const void *v,
                   void *o, int T, float scale, kvattn_dtype o_dtype, void *stream) {
  return prefill_impl(c, layer, q, k, v, o, T, scale, o_dtype, stream, nullptr);
}

int kvattn_measure_prefill_clock(kvattn_cache *c, int layer, const void *q, const void *k, const void *v,
                                 void *o, int T, float scale, kvattn_dtype o_dtype, uint64_t *sample,
                                 void *stream) {
  if (!sample) return KVATTN_ERR_INVALID_ARG;
  return prefill_impl(c, layer, q, k, v, o, T, scale, o_dtype, stream, sample);
}

int kvattn_extend(kvattn_cache *c, int layer, const void *q, const void *k, const void *v, void *o,
                  int T, float scale, kvattn_dtype o_dtype, void *stream) {
  int rc = validate_extend(c, layer, q, k, v, o, T, scale, o_dtype);
  if (rc) return rc;
  rc = check_device(c);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  int32_t *len = c->d_len + (size_t)layer * c->batch;

  // 1. the new K/V rows go to cache rows [len[b], len[b] + T)
  ExtendCopyArgs cp;
  cp.k_layer = layer_k(c, layer);
  cp.v_layer = layer_v(c, layer);
  cp.k_new = (const char *)k;
  cp.v_new = (const char *)v;
  cp.len = len;
  cp.batch = c->batch;
  cp.kv_heads = c->kv_heads;
  cp.max_T = c->max_T;
  cp.row_bytes = c->head_dim * c->elem;
  cp.T = T;
  hipError_t e = launch_extend_copy(cp, st);
  if (e != hipSuccess) return hip_fail(e, "extend copy launch");

  const int G = c->q_heads / c->kv_heads;
  if (T == 1 || verify_on_decode(G, T, c->window[layer])) {
    // short extend (one decode step, or a multi-token verification): the
    // decode kernels with T query positions per head, token t at position
    // len[b] + t (the lengths do not include the new rows yet), then the
    // lengths are committed
    DecodeArgs d;
    d.k_layer = layer_k(c, layer);
    d.v_layer = layer_v(c, layer);
    d.q = q;
    d.o = o;
    d.ws = c->d_ws;
    d.len = len;
    d.batch = c->batch;
    d.q_heads = c->q_heads;
    d.kv_heads = c->kv_heads;
    d.head_dim = c->head_dim;
    d.max_T = c->max_T;
    d.chunk = c->chunk;
    d.n_splits = c->n_splits;
    d.window = c->window[layer];
    d.sink = c->sink[layer];
    d.scale_log2 = scale * 1.4426950408889634f;
    d.dt = c->dt;
    d.o_dt = o_dtype;
    d.table = nullptr;
    d.block_log2 = 0;
    d.max_blocks = 0;
    d.tokens = T;
    d.len_pending = 1;
    e = launch_decode(d, st);
    if (e != hipSuccess) return hip_fail(e, "extend (decode form) launch");
    e = launch_add_lengths(len, c->batch, T, c->max_T, nullptr, 0, st);
    if (e != hipSuccess) return hip_fail(e, "extend length update launch");
    mirror_add(c, layer, T);
    return KVATTN_OK;
  }

  // 2. attention of the T new queries over cache rows [0, len[b] + T)
  PrefillArgs a;
  a.q = q;
  a.k = layer_k(c, layer);
  a.v = layer_v(c, layer);
  a.o = o;
  a.cache_k = layer_k(c, layer);
  a.cache_v = layer_v(c, layer);
  a.len = len;
  a.offsets = len;
  a.batch = c->batch;
  a.q_heads = c->q_heads;
  a.kv_heads = c->kv_heads;
  a.head_dim = c->head_dim;
  a.T = T;
  a.max_T = c->max_T;
  a.kv_rows = c->max_T;
  a.write_cache = 0;
  a.window = c->window[layer];
  a.sink = c->sink[layer];
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dt = c->dt;
  a.o_dt = o_dtype;
  e = launch_extend_attention(a, st);
  if (e != hipSuccess) return hip_fail(e, "extend attention launch");

  // 3. commit: len[b] += T
  e = launch_add_lengths(len, c->batch, T, c->max_T, nullptr, 0, st);
  if (e != hipSuccess) return hip_fail(e, "extend length update launch");
  mirror_add(c, layer, T);
  return KVATTN_OK;
}

int kvattn_append(kvattn_cache *c, int layer, const void *k_new, const void *v_new, void *stream) {
  int rc = validate_append(c, layer, k_new, v_new);
  if (rc) return rc;
  rc = check_device(c);
  if (rc) return rc;
  AppendArgs a;
  a.k_layer = layer_k(c, layer);
  a.v_layer = layer_v(c, layer);
  a.k_new = (const char *)k_new;
  a.v_new = (const char *)v_new;
  a.len = c->d_len + (size_t)layer * c->batch;
  a.batch = c->batch;
  a.kv_heads = c->kv_heads;
  a.max_T = c->max_T;
  a.row_bytes = c->head_dim * c->elem;
  a.table = nullptr;
  a.block_log2 = 0;
  a.max_blocks = 0;
  hipError_t e = launch_append(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  mirror_add(c, layer, 1);
  return KVATTN_OK;
}

}  // extern "C"

namespace {

DecodeArgs cache_decode_args(kvattn_cache *c, int layer, const void *q, void *o, float scale, kvattn_dtype o_dtype) {
  DecodeArgs a;
  a.k_layer = layer_k(c, layer);
  a.v_layer = layer_v(c, layer);
  a.q = q;
  a.o = o;
  a.ws = c->d_ws;
  a.len = c->d_len + (size_t)layer * c->batch;
  a.batch = c->batch;
  a.q_heads = c->q_heads;
  a.kv_heads = c->kv_heads;
  a.head_dim = c->head_dim;
  a.max_T = c->max_T;
  a.chunk = c->chunk;
  a.n_splits = c->n_splits;
  a.window = c->window[layer];
  a.sink = c->sink[layer];
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dt = c->dt;
  a.o_dt = o_dtype;
  a.table = nullptr;
  a.block_log2 = 0;
  a.max_blocks = 0;
  return a;
}

}  // namespace

extern "C" {

int kvattn_append_decode(kvattn_cache *c, int layer, const void *k_new, const void *v_new, const void *q, void *o,
                         float scale, kvattn_dtype o_dtype, void *stream) {
  int rc = validate_append_decode(c, layer, k_new, v_new, q, o, scale, o_dtype);
  if (rc) return rc;
  rc = check_device(c);
  if (rc) return rc;
  DecodeArgs a = cache_decode_args(c, layer, q, o, scale, o_dtype);
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache_rw = layer_k(c, layer);
  a.v_cache_rw = layer_v(c, layer);
  a.len_rw = c->d_len + (size_t)layer * c->batch;
  a.counters = c->d_cnt;
  hipError_t e = launch_decode_step(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode step launch");
  mirror_add(c, layer, 1);
  return KVATTN_OK;
}

int kvattn_decode(kvattn_cache *c, int layer, const void *q, void *o, float scale,
                  kvattn_dtype o_dtype, void *stream) {
  int rc = validate_decode(c, layer, q, o, scale, o_dtype);
  if (rc) return rc;
  rc = check_device(c);
  if (rc) return rc;
  DecodeArgs a = cache_decode_args(c, layer, q, o, scale, o_dtype);
  hipError_t e = launch_decode(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return KVATTN_OK;
}

int kvattn_decode_noalloc(const void *k_cache, const void *v_cache, const int32_t *lengths, int batch,
                          int q_heads, int kv_heads, int head_dim, int max_T, kvattn_dtype dt, const void *q,
                          void *o, float scale, kvattn_dtype o_dtype, void *stream) {
  if (!k_cache || !v_cache || !lengths || !q || !o) return KVATTN_ERR_INVALID_ARG;
  if (batch <= 0 || q_heads <= 0 || kv_heads <= 0 || head_dim <= 0 || max_T <= 0) return KVATTN_ERR_INVALID_ARG;
  if (!valid_scale(scale)) return KVATTN_ERR_INVALID_ARG;
  if (elem_bytes(dt) == 0 || !supported_dim(head_dim) || q_heads % kv_heads != 0) return KVATTN_ERR_UNSUPPORTED;
  if (o_dtype != dt && o_dtype != KVATTN_F32) return KVATTN_ERR_UNSUPPORTED;
  // split-K partials (m, l, u[D]) of every (sequence, query head, split);
  // the split count depends on the capacity only, not on the lengths
  const int chunk = decode_chunk(head_dim, q_heads / kv_heads, max_T);
  const int n_splits = (max_T + chunk - 1) / chunk;
  const size_t need = sizeof(float) * (size_t)batch * q_heads * n_splits * (head_dim + 2);
  if (need > (size_t)KVATTN_NOALLOC_SCRATCH_BYTES) {
    std::snprintf(g_last_error, sizeof g_last_error,
                  "kvattn_decode_noalloc: this shape needs %zu bytes of split-K scratch, the fixed array holds %zu",
                  need, (size_t)KVATTN_NOALLOC_SCRATCH_BYTES);
    return KVATTN_ERR_CAPACITY;
  }
  float *ws = scratch_on_current_device();
  if (!ws) return KVATTN_ERR_HIP;
  DecodeArgs a;
  a.k_layer = k_cache;
  a.v_layer = v_cache;
  a.q = q;
  a.o = o;
  a.ws = ws;
  a.len = lengths;
  a.batch = batch;
  a.q_heads = q_heads;
  a.kv_heads = kv_heads;
  a.head_dim = head_dim;
  a.max_T = max_T;
  a.chunk = chunk;
  a.n_splits = n_splits;
  a.window = 0;
  a.sink = 0;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dt = dt;
  a.o_dt = o_dtype;
  a.table = nullptr;
  a.block_log2 = 0;
  a.max_blocks = 0;
  hipError_t e = launch_decode(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode (no-alloc) launch");
  return KVATTN_OK;
}

// ---------------------------------------------------------------- paged cache
// Inference chapter, section 9.6: the cache managed in fixed-size blocks
// instead of one max-length region per sequence; llm-perf-lab README: vLLM
// style paging with prefix sharing.  One pool allocation laid out
// [layer][K|V][num_blocks][Hkv][block_size][D]; one block table per slot
// (device, [slots][max_blocks], the same for every layer); lengths
// [layer][slots] on the device with a host mirror.

}  // extern "C"


namespace {

int paged_check_device(const kvattn_paged *p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != p->device) {
    std::snprintf(g_last_error, sizeof g_last_error,
                  "paged cache lives on device %d but device %d is current", p->device, dev);
    return KVATTN_ERR_STATE;
  }
  return KVATTN_OK;
}

char *paged_k(const kvattn_paged *p, int layer) { return p->base + (size_t)layer * p->layer_bytes; }
char *paged_v(const kvattn_paged *p, int layer) { return paged_k(p, layer) + p->layer_bytes / 2; }

}  // namespace

extern "C" {

size_t kvattn_paged_bytes(int layers, int num_blocks, int block_size, int kv_heads, int head_dim,
                          kvattn_dtype dt) {
  const int e = elem_bytes(dt);
  if (layers <= 0 || num_blocks <= 0 || block_size <= 0 || kv_heads <= 0 || head_dim <= 0 || e == 0) return 0;
  return (size_t)2 * layers * num_blocks * (size_t)block_size * kv_heads * head_dim * e;
}

int kvattn_paged_alloc(kvattn_paged **out, int layers, int slots, int max_blocks, int num_blocks,
                       int block_size, int q_heads, int kv_heads, int head_dim, kvattn_dtype dt,
                       void *device_buf, size_t device_buf_bytes) {
  if (!out) return KVATTN_ERR_INVALID_ARG;
  *out = nullptr;
  if (layers <= 0 || slots <= 0 || max_blocks <= 0 || num_blocks <= 0 || block_size <= 0 || q_heads <= 0 ||
      kv_heads <= 0 || head_dim <= 0)
    return KVATTN_ERR_INVALID_ARG;
  if (elem_bytes(dt) == 0 || !supported_dim(head_dim) || q_heads % kv_heads != 0)
    return KVATTN_ERR_UNSUPPORTED;
  if (block_size < 16 || block_size > 4096 || (block_size & (block_size - 1)) != 0)
    return KVATTN_ERR_UNSUPPORTED;
  if ((long long)max_blocks * block_size > (1LL << 30)) return KVATTN_ERR_UNSUPPORTED;
  const int capacity = max_blocks * block_size;
  const int chunk = decode_chunk(head_dim, q_heads / kv_heads, capacity);
  if (paged_tab_entries(chunk, block_size, false) > kPagedTab) return KVATTN_ERR_UNSUPPORTED;
  const size_t bytes = kvattn_paged_bytes(layers, num_blocks, block_size, kv_heads, head_dim, dt);
  if (device_buf) {
    if (device_buf_bytes < bytes) return KVATTN_ERR_OOM;
    if (((uintptr_t)device_buf & 255u) != 0) return KVATTN_ERR_INVALID_ARG;
  }
  kvattn_paged *p = new (std::nothrow) kvattn_paged();
  if (!p) return KVATTN_ERR_OOM;
  p->layers = layers;
  p->slots = slots;
  p->q_heads = q_heads;
  p->kv_heads = kv_heads;
  p->head_dim = head_dim;
  p->num_blocks = num_blocks;
  p->block_size = block_size;
  p->block_log2 = __builtin_ctz((unsigned)block_size);
  p->max_blocks = max_blocks;
  p->dt = dt;
  p->elem = elem_bytes(dt);
  p->payload_bytes = bytes;
  p->layer_bytes = bytes / layers;
  p->chunk = chunk;
  p->n_splits = (capacity + chunk - 1) / chunk;
  p->h_len.assign((size_t)layers * slots, 0);
  p->h_nblk.assign(slots, 0);
  p->window.assign(layers, 0);
  p->sink.assign(layers, 0);
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipGetDevice");
  }
  if (device_buf) {
    p->base = (char *)device_buf;
    p->owns_base = false;
  } else {
    e = hipMalloc((void **)&p->base, bytes);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      delete p;
      std::snprintf(g_last_error, sizeof g_last_error, "hipMalloc(%zu): %s", bytes, hipGetErrorString(e));
      return KVATTN_ERR_OOM;
    }
    p->owns_base = true;
  }
  const size_t len_bytes = sizeof(int32_t) * (size_t)layers * slots;
  const size_t tab_bytes = sizeof(int32_t) * (size_t)slots * max_blocks;
  const size_t ws_bytes = sizeof(float) * (size_t)slots * q_heads * kMaxVerifyTokens * p->n_splits * (head_dim + 2);
  const size_t nblk_bytes = sizeof(int32_t) * (size_t)slots;
  e = hipMalloc((void **)&p->d_len, len_bytes);
  if (e == hipSuccess) e = hipMalloc((void **)&p->d_table, tab_bytes);
  if (e == hipSuccess) e = hipMalloc((void **)&p->d_nblk, nblk_bytes);
  if (e == hipSuccess) e = hipMalloc((void **)&p->d_ws, ws_bytes);
  if (e == hipSuccess) e = hipMemset(p->d_len, 0, len_bytes);
  if (e == hipSuccess) e = hipMemset(p->d_table, 0, tab_bytes);
  if (e == hipSuccess) e = hipMemset(p->d_nblk, 0, nblk_bytes);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    int rc = hip_fail(e, "paged cache side buffers");
    (void)hipGetLastError();
    if (p->d_len) (void)hipFree(p->d_len);
    if (p->d_table) (void)hipFree(p->d_table);
    if (p->d_nblk) (void)hipFree(p->d_nblk);
    if (p->d_ws) (void)hipFree(p->d_ws);
    if (p->owns_base) (void)hipFree(p->base);
    delete p;
    return e == hipErrorOutOfMemory ? KVATTN_ERR_OOM : rc;
  }
  *out = p;
  return KVATTN_OK;
}

int kvattn_paged_free(kvattn_paged *p) {
  if (!p) return KVATTN_ERR_INVALID_ARG;
  hipError_t e = hipDeviceSynchronize();
  hipError_t e1 = hipFree(p->d_len);
  hipError_t e2 = hipFree(p->d_table);
  hipError_t e5 = hipFree(p->d_nblk);
  hipError_t e3 = hipFree(p->d_ws);
  hipError_t e4 = p->owns_base ? hipFree(p->base) : hipSuccess;
  delete p;
  if (e != hipSuccess) return hip_fail(e, "kvattn_paged_free sync");
  if (e1 != hipSuccess) return hip_fail(e1, "hipFree(lengths)");
  if (e2 != hipSuccess) return hip_fail(e2, "hipFree(block tables)");
  if (e5 != hipSuccess) return hip_fail(e5, "hipFree(block counts)");
  if (e3 != hipSuccess) return hip_fail(e3, "hipFree(workspace)");
  if (e4 != hipSuccess) return hip_fail(e4, "hipFree(pool)");
  return KVATTN_OK;
}

int kvattn_paged_kv_ptr(const kvattn_paged *p, int layer, void **k, void **v) {
  int rc = paged_check_layer(p, layer);
  if (rc) return rc;
  if (!k || !v) return KVATTN_ERR_INVALID_ARG;
  *k = paged_k(p, layer);
  *v = paged_v(p, layer);
  return KVATTN_OK;
}

int kvattn_paged_set_blocks(kvattn_paged *p, int slot, const int32_t *host_block_ids, int n_blocks,
                            void *stream) {
  int rc = validate_paged_set_blocks(p, slot, host_block_ids, n_blocks);
  if (rc) return rc;
  rc = paged_check_device(p);
  if (rc) return rc;
  if (n_blocks > 0) {
    hipError_t e = launch_set_lengths(p->d_table + (size_t)slot * p->max_blocks, 1, n_blocks, host_block_ids,
                                      (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "block table upload");
  }
  // the device copy of the slot's block count bounds every write at a
  // device-held position (appends and extends replayed from a graph)
  const int32_t nb = n_blocks;
  hipError_t e = launch_set_lengths(p->d_nblk + slot, 1, 1, &nb, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "block count upload");
  p->h_nblk[slot] = n_blocks;
  return KVATTN_OK;
}

int kvattn_paged_set_lengths(kvattn_paged *p, int layer, const int32_t *host_lens, void *stream) {
  int rc = validate_paged_set_lengths(p, layer, host_lens);
  if (rc) return rc;
  rc = paged_check_device(p);
  if (rc) return rc;
  const int first = layer < 0 ? 0 : layer;
  const int count = layer < 0 ? p->layers : 1;
  hipError_t e = launch_set_lengths(p->d_len + (size_t)first * p->slots, count, p->slots, host_lens,
                                    (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "set_lengths launch");
  for (int l = first; l < first + count; ++l)
    std::memcpy(&p->h_len[(size_t)l * p->slots], host_lens, sizeof(int32_t) * p->slots);
  return KVATTN_OK;
}

int kvattn_paged_get_lengths(const kvattn_paged *p, int layer, int32_t *host_lens) {
  int rc = paged_check_layer(p, layer);
  if (rc) return rc;
  if (!host_lens) return KVATTN_ERR_INVALID_ARG;
  std::memcpy(host_lens, &p->h_len[(size_t)layer * p->slots], sizeof(int32_t) * p->slots);
  return KVATTN_OK;
}

int kvattn_paged_set_window(kvattn_paged *p, int layer, int window, int sink) {
  if (!p) return KVATTN_ERR_INVALID_ARG;
  if (layer != -1 && (layer < 0 || layer >= p->layers)) return KVATTN_ERR_INVALID_ARG;
  if (window < 0 || sink < 0) return KVATTN_ERR_INVALID_ARG;
  // a windowed decode split may stage the table entries of two runs
  if (window > 0 && paged_tab_entries(p->chunk, p->block_size, true) > kPagedTab) return KVATTN_ERR_UNSUPPORTED;
  const int first = layer < 0 ? 0 : layer;
  const int count = layer < 0 ? p->layers : 1;
  for (int l = first; l < first + count; ++l) {
    p->window[l] = window;
    p->sink[l] = window > 0 ? sink : 0;
  }
  return KVATTN_OK;
}

int kvattn_paged_get_window(const kvattn_paged *p, int layer, int *window, int *sink) {
  int rc = paged_check_layer(p, layer);
  if (rc) return rc;
  if (!window || !sink) return KVATTN_ERR_INVALID_ARG;
  *window = p->window[layer];
  *sink = p->sink[layer];
  return KVATTN_OK;
}

int kvattn_paged_prefill(kvattn_paged *p, int layer, const void *q, const void *k, const void *v, void *o,
                         int T, float scale, kvattn_dtype o_dtype, void *stream) {
  int rc = validate_paged_prefill(p, layer, q, k, v, o, T, scale, o_dtype);
  if (rc) return rc;
  rc = paged_check_device(p);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  int32_t *len = p->d_len + (size_t)layer * p->slots;

  // 1. causal attention over the prompt (the prefill kernels, cache copy off)
  PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.cache_k = paged_k(p, layer);
  a.cache_v = paged_v(p, layer);
  a.len = len;
  a.offsets = nullptr;
  a.batch = p->slots;
  a.q_heads = p->q_heads;
  a.kv_heads = p->kv_heads;
  a.head_dim = p->head_dim;
  a.T = T;
  a.max_T = T;
  a.kv_rows = T;
  a.write_cache = 0;
  a.window = p->window[layer];
  a.sink = p->sink[layer];
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dt = p->dt;
  a.o_dt = o_dtype;
  hipError_t e = launch_prefill(a, st);
  if (e != hipSuccess) return hip_fail(e, "paged prefill attention launch");

  // 2. the prompt rows to their blocks; len = T
  PagedWriteArgs w;
  w.k_pool = paged_k(p, layer);
  w.v_pool = paged_v(p, layer);
  w.k_new = (const char *)k;
  w.v_new = (const char *)v;
  w.len = len;
  w.table = p->d_table;
  w.batch = p->slots;
  w.kv_heads = p->kv_heads;
  w.T = T;
  w.row_bytes = p->head_dim * p->elem;
  w.block_log2 = p->block_log2;
  w.max_blocks = p->max_blocks;
  w.slot_blocks = p->d_nblk;
  e = launch_paged_write(w, st);
  if (e != hipSuccess) return hip_fail(e, "paged prefill write launch");
  paged_mirror_set(p, layer, T);
  return KVATTN_OK;
}

int kvattn_paged_append(kvattn_paged *p, int layer, const void *k_new, const void *v_new, void *stream) {
  int rc = validate_paged_append(p, layer, k_new, v_new);
  if (rc) return rc;
  rc = paged_check_device(p);
  if (rc) return rc;
  AppendArgs a;
  a.k_layer = paged_k(p, layer);
  a.v_layer = paged_v(p, layer);
  a.k_new = (const char *)k_new;
  a.v_new = (const char *)v_new;
  a.len = p->d_len + (size_t)layer * p->slots;
  a.batch = p->slots;
  a.kv_heads = p->kv_heads;
  a.max_T = 0;
  a.row_bytes = p->head_dim * p->elem;
  a.table = p->d_table;
  a.block_log2 = p->block_log2;
  a.max_blocks = p->max_blocks;
  a.slot_blocks = p->d_nblk;
  hipError_t e = launch_append(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "paged append launch");
  paged_mirror_add(p, layer, 1);
  return KVATTN_OK;
}

int kvattn_paged_extend(kvattn_paged *p, int layer, const void *q, const void *k, const void *v, void *o, int T,
                        float scale, kvattn_dtype o_dtype, void *stream) {
  int rc = validate_paged_extend(p, layer, q, k, v, o, T, scale, o_dtype);
  if (rc) return rc;
  rc = paged_check_device(p);
  if (rc) return rc;
  hipStream_t st = (hipStream_t)stream;
  int32_t *len = p->d_len + (size_t)layer * p->slots;

  // 1. the new K/V rows go to positions [len[b], len[b] + T) of their blocks
  ExtendCopyArgs cp;
  cp.k_layer = paged_k(p, layer);
  cp.v_layer = paged_v(p, layer);
  cp.k_new = (const char *)k;
  cp.v_new = (const char *)v;
  cp.len = len;
  cp.batch = p->slots;
  cp.kv_heads = p->kv_heads;
  cp.max_T = 0;
  cp.row_bytes = p->head_dim * p->elem;
  cp.T = T;
  cp.table = p->d_table;
  cp.block_log2 = p->block_log2;
  cp.max_blocks = p->max_blocks;
  cp.slot_blocks = p->d_nblk;
  hipError_t e = launch_extend_copy(cp, st);
  if (e != hipSuccess) return hip_fail(e, "paged extend copy launch");

  const int G = p->q_heads / p->kv_heads;
  if (T == 1 || verify_on_decode(G, T, p->window[layer])) {
    // short extend on the decode kernels, as for the contiguous cache
    DecodeArgs d;
    d.k_layer = paged_k(p, layer);
    d.v_layer = paged_v(p, layer);
    d.q = q;
    d.o = o;
    d.ws = p->d_ws;
    d.len = len;
    d.batch = p->slots;
    d.q_heads = p->q_heads;
    d.kv_heads = p->kv_heads;
    d.head_dim = p->head_dim;
    d.max_T = p->max_blocks * p->block_size;
    d.chunk = p->chunk;
    d.n_splits = p->n_splits;
    d.window = p->window[layer];
    d.sink = p->sink[layer];
    d.scale_log2 = scale * 1.4426950408889634f;
    d.dt = p->dt;
    d.o_dt = o_dtype;
    d.table = p->d_table;
    d.block_log2 = p->block_log2;
    d.max_blocks = p->max_blocks;
    d.tokens = T;
    d.len_pending = 1;
    d.slot_blocks = p->d_nblk;
    e = launch_decode(d, st);
    if (e != hipSuccess) return hip_fail(e, "paged extend (decode form) launch");
    e = launch_add_lengths(len, p->slots, T, 0, p->d_nblk, p->block_log2, st);
    if (e != hipSuccess) return hip_fail(e, "paged extend length update launch");
    paged_mirror_add(p, layer, T);
    return KVATTN_OK;
  }

  // 2. attention of the T new queries over positions [0, len[b] + T), rows
  //    found through the block table
  PrefillArgs a;
  a.q = q;
  a.k = paged_k(p, layer);
  a.v = paged_v(p, layer);
  a.o = o;
  a.cache_k = paged_k(p, layer);
  a.cache_v = paged_v(p, layer);
  a.len = len;
  a.offsets = len;
  a.batch = p->slots;
  a.q_heads = p->q_heads;
  a.kv_heads = p->kv_heads;
  a.head_dim = p->head_dim;
  a.T = T;
  a.max_T = 0;
  a.kv_rows = 0;
  a.write_cache = 0;
  a.window = p->window[layer];
  a.sink = p->sink[layer];
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dt = p->dt;
  a.o_dt = o_dtype;
  a.table = p->d_table;
  a.block_log2 = p->block_log2;
  a.max_blocks = p->max_blocks;
  a.slot_blocks = p->d_nblk;
  e = launch_extend_attention(a, st);
  if (e != hipSuccess) return hip_fail(e, "paged extend attention launch");

  // 3. commit: len[b] += T
  e = launch_add_lengths(len, p->slots, T, 0, p->d_nblk, p->block_log2, st);
  if (e != hipSuccess) return hip_fail(e, "paged extend length update launch");
  paged_mirror_add(p, layer, T);
  return KVATTN_OK;
}

int kvattn_paged_decode(kvattn_paged *p, int layer, const void *q, void *o, float scale, kvattn_dtype o_dtype,
                        void *stream) {
  int rc = validate_paged_decode(p, layer, q, o, scale, o_dtype);
  if (rc) return rc;
  rc = paged_check_device(p);
  if (rc) return rc;
  DecodeArgs a;
  a.k_layer = paged_k(p, layer);
  a.v_layer = paged_v(p, layer);
  a.q = q;
  a.o = o;
  a.ws = p->d_ws;
  a.len = p->d_len + (size_t)layer * p->slots;
  a.batch = p->slots;
  a.q_heads = p->q_heads;
  a.kv_heads = p->kv_heads;
  a.head_dim = p->head_dim;
  a.max_T = p->max_blocks * p->block_size;
  a.chunk = p->chunk;
  a.n_splits = p->n_splits;
  a.window = p->window[layer];
  a.sink = p->sink[layer];
  a.scale_log2 = scale * 1.4426950408889634f;
  a.dt = p->dt;
  a.o_dt = o_dtype;
  a.table = p->d_table;
  a.block_log2 = p->block_log2;
  a.max_blocks = p->max_blocks;
  a.slot_blocks = p->d_nblk;
  hipError_t e = launch_decode(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "paged decode launch");
  return KVATTN_OK;
}

const char *kvattn_status_string(int status) {
  switch (status) {
    case KVATTN_OK: return "ok";
    case KVATTN_ERR_INVALID_ARG: return "invalid argument";
    case KVATTN_ERR_UNSUPPORTED: return "unsupported dtype, head_dim or head layout";
    case KVATTN_ERR_CAPACITY: return "cache capacity exceeded";
    case KVATTN_ERR_STATE: return "cache state does not allow this call";
    case KVATTN_ERR_OOM: return "device memory allocation failed";
    case KVATTN_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *kvattn_last_error(void) { return g_last_error; }

}  // extern "C"
