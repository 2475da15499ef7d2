// Host-side validation of libkvattn's entry points, on cache objects built on
// the host (no device memory, no GPU needed): every refused call returns its
// status (INVALID_ARG, UNSUPPORTED, CAPACITY, STATE) and leaves the lengths'
// host mirror as it was; a call whose arguments pass but that cannot reach a
// device (none, or not the cache's) returns HIP or STATE, enqueues nothing
// and changes nothing either.  Built and run by tests/test_host_validation.py.
#include <cmath>
#include <cstdio>
#include <vector>

#include "cache.hpp"
#include "kvattn.h"

static int g_fail = 0;
static int g_checks = 0;
#define EXPECT(cond)                                                     \
  do {                                                                   \
    ++g_checks;                                                          \
    if (!(cond)) {                                                       \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);        \
      ++g_fail;                                                          \
    }                                                                    \
  } while (0)

// any pointer the checks only test for null; never dereferenced
static void *const P = reinterpret_cast<void *>(0x1000);

static kvattn_cache host_cache(int layers, int batch, int max_T, kvattn_dtype dt) {
  kvattn_cache c{};
  c.layers = layers;
  c.batch = batch;
  c.q_heads = 4;
  c.kv_heads = 2;
  c.head_dim = 64;
  c.max_T = max_T;
  c.dt = dt;
  c.h_len.assign((size_t)layers * batch, 0);
  c.window.assign(layers, 0);
  c.sink.assign(layers, 0);
  c.device = -1;  // no device has this ordinal: a call that passes validation stops there
  return c;
}

static kvattn_paged host_paged(int layers, int slots, int max_blocks, int num_blocks, int block_size) {
  kvattn_paged p{};
  p.layers = layers;
  p.slots = slots;
  p.q_heads = 4;
  p.kv_heads = 2;
  p.head_dim = 64;
  p.num_blocks = num_blocks;
  p.block_size = block_size;
  p.max_blocks = max_blocks;
  p.dt = KVATTN_F16;
  p.h_len.assign((size_t)layers * slots, 0);
  p.h_nblk.assign(slots, 0);
  p.window.assign(layers, 0);
  p.sink.assign(layers, 0);
  p.device = -1;
  return p;
}

static bool no_device(int rc) { return rc == KVATTN_ERR_HIP || rc == KVATTN_ERR_STATE; }

static void contiguous() {
  kvattn_cache c = host_cache(2, 3, 100, KVATTN_F16);
  const float s = 0.125f;
  // prefill (lengths all 0 so far)
  std::vector<int32_t> before = c.h_len;
  EXPECT(kvattn_prefill(&c, -1, P, P, P, P, 10, s, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_prefill(&c, 2, P, P, P, P, 10, s, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_prefill(&c, 0, nullptr, P, P, P, 10, s, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_prefill(&c, 0, P, P, P, P, 0, s, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_prefill(&c, 0, P, P, P, P, 10, 0.f, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_prefill(&c, 0, P, P, P, P, 10, NAN, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_prefill(&c, 0, P, P, P, P, 10, INFINITY, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_prefill(&c, 0, P, P, P, P, 10, s, KVATTN_BF16, nullptr) == KVATTN_ERR_UNSUPPORTED);
  EXPECT(kvattn_prefill(&c, 0, P, P, P, P, 101, s, KVATTN_F16, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(no_device(kvattn_prefill(&c, 0, P, P, P, P, 100, s, KVATTN_F32, nullptr)));
  EXPECT(c.h_len == before);
  // state: layer 0 holds [5, 0, 99], layer 1 holds [100, 100, 100]
  c.h_len = {5, 0, 99, 100, 100, 100};
  before = c.h_len;
  EXPECT(kvattn_prefill(&c, 0, P, P, P, P, 10, s, KVATTN_F16, nullptr) == KVATTN_ERR_STATE);
  // append: layer 1 is full
  EXPECT(kvattn_append(&c, 0, nullptr, P, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_append(&c, 1, P, P, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(no_device(kvattn_append(&c, 0, P, P, nullptr)));
  // the fused step: capacity as append; a length of 0 is allowed
  EXPECT(kvattn_append_decode(&c, 1, P, P, P, P, s, KVATTN_F16, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(kvattn_append_decode(&c, 0, P, P, nullptr, P, s, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_append_decode(&c, 0, P, P, P, P, -s, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_append_decode(&c, 0, P, P, P, P, s, KVATTN_BF16, nullptr) == KVATTN_ERR_UNSUPPORTED);
  EXPECT(no_device(kvattn_append_decode(&c, 0, P, P, P, P, s, KVATTN_F32, nullptr)));
  // extend: len + T must fit (99 + 2 > 100)
  EXPECT(kvattn_extend(&c, 0, P, P, P, P, 2, s, KVATTN_F16, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(kvattn_extend(&c, 0, P, P, P, P, 0, s, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_extend(&c, 1, P, P, P, P, 1, s, KVATTN_F16, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(no_device(kvattn_extend(&c, 0, P, P, P, P, 1, s, KVATTN_F16, nullptr)));
  // decode: sequence 1 of layer 0 is empty
  EXPECT(kvattn_decode(&c, 0, P, P, s, KVATTN_F16, nullptr) == KVATTN_ERR_STATE);
  EXPECT(kvattn_decode(&c, 1, P, nullptr, s, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(no_device(kvattn_decode(&c, 1, P, P, s, KVATTN_F16, nullptr)));
  // set_lengths: each in [0, max_T]
  const int32_t neg[3] = {1, -1, 1}, big[3] = {1, 101, 1}, ok[3] = {1, 2, 3};
  EXPECT(kvattn_cache_set_lengths(&c, 0, neg, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(kvattn_cache_set_lengths(&c, -1, big, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(kvattn_cache_set_lengths(&c, 2, ok, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_cache_set_lengths(&c, 0, nullptr, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(no_device(kvattn_cache_set_lengths(&c, -1, ok, nullptr)));
  EXPECT(c.h_len == before);
  int32_t got[3] = {0, 0, 0};
  EXPECT(kvattn_cache_get_lengths(&c, 0, got) == KVATTN_OK && got[0] == 5 && got[1] == 0 && got[2] == 99);
  // windows are host state only: a valid call succeeds, a refused one changes nothing
  EXPECT(kvattn_cache_set_window(&c, 0, -1, 0) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_cache_set_window(&c, 5, 8, 0) == KVATTN_ERR_INVALID_ARG);
  EXPECT(c.window[0] == 0 && c.window[1] == 0);
  EXPECT(kvattn_cache_set_window(&c, -1, 16, 4) == KVATTN_OK);
  int w = 0, sk = 0;
  EXPECT(kvattn_cache_get_window(&c, 1, &w, &sk) == KVATTN_OK && w == 16 && sk == 4);
  EXPECT(kvattn_cache_set_window(&c, 1, 0, 4) == KVATTN_OK);
  EXPECT(kvattn_cache_get_window(&c, 1, &w, &sk) == KVATTN_OK && w == 0 && sk == 0);
}

static void paged() {
  kvattn_paged p = host_paged(2, 2, 4, 6, 16);
  const float s = 0.125f;
  p.h_nblk = {1, 3};  // capacities 16 and 48 positions
  p.h_len = {16, 10, 0, 0};
  const std::vector<int32_t> before = p.h_len;
  const std::vector<int> nblk = p.h_nblk;
  const int32_t ids_bad[2] = {0, 6}, ids_one[1] = {0};
  EXPECT(kvattn_paged_set_blocks(&p, 0, ids_bad, 2, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_paged_set_blocks(&p, 2, ids_one, 1, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(kvattn_paged_set_blocks(&p, 0, ids_one, 5, nullptr) == KVATTN_ERR_INVALID_ARG);
  // slot 1 holds 10 positions in layer 0: zero blocks cannot hold them
  EXPECT(kvattn_paged_set_blocks(&p, 1, nullptr, 0, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(no_device(kvattn_paged_set_blocks(&p, 1, ids_one, 1, nullptr)));
  const int32_t lens_big[2] = {17, 0}, lens_ok[2] = {3, 4};
  EXPECT(kvattn_paged_set_lengths(&p, 0, lens_big, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(no_device(kvattn_paged_set_lengths(&p, -1, lens_ok, nullptr)));
  EXPECT(kvattn_paged_prefill(&p, 0, P, P, P, P, 4, s, KVATTN_F16, nullptr) == KVATTN_ERR_STATE);
  EXPECT(kvattn_paged_prefill(&p, 1, P, P, P, P, 17, s, KVATTN_F16, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(kvattn_paged_prefill(&p, 1, P, P, P, P, 4, s, KVATTN_BF16, nullptr) == KVATTN_ERR_UNSUPPORTED);
  EXPECT(no_device(kvattn_paged_prefill(&p, 1, P, P, P, P, 16, s, KVATTN_F16, nullptr)));
  EXPECT(kvattn_paged_append(&p, 0, P, P, nullptr) == KVATTN_ERR_CAPACITY);  // slot 0 full
  EXPECT(no_device(kvattn_paged_append(&p, 1, P, P, nullptr)));
  EXPECT(kvattn_paged_extend(&p, 0, P, P, P, P, 1, s, KVATTN_F16, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(kvattn_paged_extend(&p, 1, P, P, P, P, 17, s, KVATTN_F16, nullptr) == KVATTN_ERR_CAPACITY);
  EXPECT(no_device(kvattn_paged_extend(&p, 1, P, P, P, P, 16, s, KVATTN_F16, nullptr)));
  EXPECT(kvattn_paged_decode(&p, 1, P, P, s, KVATTN_F16, nullptr) == KVATTN_ERR_STATE);
  EXPECT(kvattn_paged_decode(&p, 0, P, P, NAN, KVATTN_F16, nullptr) == KVATTN_ERR_INVALID_ARG);
  EXPECT(no_device(kvattn_paged_decode(&p, 0, P, P, s, KVATTN_F32, nullptr)));
  EXPECT(p.h_len == before);
  EXPECT(p.h_nblk == nblk);
}

int main() {
  contiguous();
  paged();
  std::printf("%d checks, %d failed\n", g_checks, g_fail);
  return g_fail == 0 ? 0 : 1;
}
