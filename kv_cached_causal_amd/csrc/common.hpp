// Internal helpers shared by the libkvattn kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvattn.h"

namespace kvattn {

typedef _Float16 half_t;
typedef __bf16 bf16_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf168_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
// 16 raw bytes as a native vector: plain loads/stores that stay in registers
// (HIP's uint4 struct is copied with memcpy, which can force it into scratch)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- launch args
struct AppendArgs {
  char *k_layer;        // layer's K block (B, Hkv, max_T, D)
  char *v_layer;        // layer's V block
  const char *k_new;    // (B, Hkv, 1, D)
  const char *v_new;
  int32_t *len;         // layer's lengths [B]
  int batch, kv_heads, max_T, row_bytes;
  // paged cache: k_layer/v_layer are the layer's block pools (num_blocks, Hkv,
  // 2^block_log2, D) and row p of sequence b lives in block table[b *
  // max_blocks + (p >> block_log2)]; null for the contiguous cache
  const int32_t *table;
  int block_log2, max_blocks;
  const int32_t *slot_blocks = nullptr;  // paged: blocks assigned to each sequence [B] (device)
};

struct DecodeArgs {
  const void *k_layer;  // (B, Hkv, max_T, D)
  const void *v_layer;
  const void *q;        // (B, H, tokens, D)
  void *o;              // (B, H, tokens, D) in o_dtype
  float *ws;            // (B, H * tokens, n_splits, D + 2) fp32: m (log2 domain), l, u[D]
  const int32_t *len;   // layer's lengths [B] (after the tokens' own rows were added)
  int batch, q_heads, kv_heads, head_dim, max_T, chunk, n_splits;
  int window, sink;     // sliding window (0: none) and attention-sink positions
  float scale_log2;     // scale * log2(e)
  kvattn_dtype dt, o_dt;
  // paged cache (as in AppendArgs); null table for the contiguous cache
  const int32_t *table;
  int block_log2, max_blocks;
  // query positions per sequence: 1 for decode; T for the short extend
  // (multi-token verification), whose token t sits at position len - T + t
  // and sees the keys up to it (no window)
  int tokens = 1;
  // extends on the decode kernels: the lengths do not include the `tokens`
  // new rows yet (they are advanced afterwards), so L = len[b] + tokens, and
  // a sequence for which that passes its capacity is skipped
  int len_pending = 0;
  const int32_t *slot_blocks = nullptr;  // paged: blocks assigned to each sequence [B] (device)
  // the fused decode step (append + decode, contiguous cache): the new rows
  // (B, Hkv, 1, D), writable views of the layer's K/V blocks and lengths, and
  // step_counter_ints(B, H) ints: per sequence kStepSlots (a counter that is
  // zero between calls, and the attended count recorded for the merge
  // kernel), then per (sequence, unit of query heads) a merge counter, zero
  // between calls
  const void *k_new = nullptr, *v_new = nullptr;
  void *k_cache_rw = nullptr, *v_cache_rw = nullptr;
  int32_t *len_rw = nullptr;
  int32_t *counters = nullptr;
};

// ints per sequence of the fused decode step's device record (counter, count)
constexpr int kStepSlots = 2;
inline size_t step_counter_ints(int batch, int q_heads) { return (size_t)batch * (kStepSlots + q_heads); }
// fused decode steps over several splits whose grid has at most this many
// workgroups (a fraction of one round on 256 CUs) merge the splits inside the
// decode kernel: at that size a second launch costs more than it saves
constexpr size_t kInKernelMergeMaxWorkgroups = 256;

// Prompts whose per-sequence grid (query tiles x heads) fills between half
// a round and one round of the pipelined prefill kernel (128 to 256
// workgroups, one per CU) split their heavier half of query tiles in two
// (see PrefillArgs): the heaviest tile then no longer sets the time of the
// round.  A function of T and H only, so that a sequence's result does not
// depend on the batch it is in.  Measured on MI355X: 16 heads of D = 32 at
// T = 4096 (256 tiles) 62.5 -> 50.5 us; a batch of 4 sequences of 12 heads
// of D = 64 at T = 2048 (96 tiles each, 1.5 rounds together) 57 -> 68 us
// when split, so grids under half a round stay whole.
constexpr int kMaxPrefillQt = 64;                       // query tiles of 256 rows
constexpr int kMaxPrefillItems = kMaxPrefillQt * 3 / 2;
inline int prefill_split_tiles(int T, int q_heads) {
  const int n_qt = (T + 255) / 256;
  if (n_qt < 8 || n_qt > kMaxPrefillQt || n_qt * q_heads < 128 || n_qt * q_heads > 256) return 0;
  return n_qt / 2;
}
// floats of one half's partial state (8 waves x 64 lanes x (m, l and the
// lane's D / 2 accumulator elements))
constexpr size_t prefill_split_half_floats(int head_dim) { return (size_t)8 * 64 * (2 + head_dim / 2); }
// the most query tiles split for any prompt of up to max_T positions (the
// split workspace and counters are sized for it)
inline int prefill_split_tiles_max(int max_T, int q_heads) {
  int best = 0;
  const int top = max_T < kMaxPrefillQt * 256 ? max_T : kMaxPrefillQt * 256;
  for (int T = 256; T < top + 256; T += 256) {
    const int n = prefill_split_tiles(T < top ? T : top, q_heads);
    best = n > best ? n : best;
  }
  return best;
}

// the longest extend served by the decode kernels (its workspace is sized
// for this many query positions per head)
constexpr int kMaxVerifyTokens = 8;
// An extend of T positions over a cache with G query heads per KV head runs
// on the decode kernels when one workgroup can hold all G * T query rows of a
// KV head (the instantiated row counts 2, 3, 4, 8) and no window is set.
inline bool verify_on_decode(int G, int T, int window) {
  const int r = G * T;
  return T >= 2 && T <= kMaxVerifyTokens && window == 0 && (r == 2 || r == 3 || r == 4 || r == 8);
}

// Positions sequence b may hold: the capacity of the contiguous cache, or
// for a paged cache the blocks assigned to the sequence.  The entry points
// check every write against their host copy of the lengths; the kernels that
// write at device-held positions (append, extend) check again against this,
// because a replayed HIP graph advances only the device lengths.
__device__ inline int seq_capacity(const int32_t *slot_blocks, int b, int block_log2, int max_T) {
  return slot_blocks ? (slot_blocks[b] << block_log2) : max_T;
}

// Row index (in rows of D elements) of position `pos` of KV head g of
// sequence b in a paged pool [num_blocks][Hkv][2^block_log2][D].
__device__ inline size_t paged_row(const int32_t *table, int b, int max_blocks, int block_log2, int kv_heads,
                                   int g, int pos) {
  const int blk = table[(size_t)b * max_blocks + (pos >> block_log2)];
  return (((size_t)blk * kv_heads + g) << block_log2) + (pos & ((1 << block_log2) - 1));
}

// table entries a paged decode split stages in LDS: a run of `chunk` positions
// spans at most chunk / block_size + 2 blocks (+1 when unaligned), and under a
// window a split may hold two runs (sink rows, then window rows)
constexpr int kPagedTab = 512;
inline int paged_tab_entries(int chunk, int block_size, bool window) {
  return (window ? 2 : 1) * (chunk / block_size + 2);
}

// The keys a decode query at position L - 1 sees, as one run of visible
// indices 0 .. count - 1: the first `sink` positions, then the last `window`
// ones (all L positions without a window).  Visible index i is cache row
// i + (i >= first ? gap : 0).
struct VisibleKeys {
  int count, first, gap;
};
__host__ __device__ inline VisibleKeys visible_keys(int L, int window, int sink) {
  if (window <= 0 || window + sink >= L) return VisibleKeys{L, L, 0};
  const int s = sink < L ? sink : L;
  const int lo = (L - window) > s ? (L - window) : s;
  return VisibleKeys{s + (L - lo), s, lo - s};
}

struct PrefillArgs {
  const void *q;        // (B, H, T, D): the T query positions of each sequence
  const void *k;        // (B, Hkv, kv_rows, D): keys 0 .. off_b + T - 1 of sequence b
  const void *v;
  void *o;              // (B, H, T, D) in o_dtype
  void *cache_k;        // layer's K block (B, Hkv, max_T, D)
  void *cache_v;
  int32_t *len;         // layer's lengths [B]
  const int32_t *offsets;  // [B] absolute position of query 0 (device), or null for 0
  int batch, q_heads, kv_heads, head_dim, T, max_T;
  int kv_rows;          // rows per (sequence, KV head) in k/v: T for a prompt, max_T for the cache
  int write_cache;      // prefill: copy k/v rows [0, T) to the cache and set len = T
  int window, sink;     // sliding window (0: none) and attention-sink positions
  float scale_log2;
  kvattn_dtype dt, o_dt;
  // paged cache (extend): k/v are the layer's block pools (num_blocks, Hkv,
  // 2^block_log2, D) and key j of sequence b sits in block
  // table[b * max_blocks + (j >> block_log2)]; null for the layouts above
  const int32_t *table = nullptr;
  int block_log2 = 0, max_blocks = 0;
  const int32_t *slot_blocks = nullptr;  // paged: blocks assigned to each sequence [B] (device)
  // measurement aid: when set, workgroup 0 of the pipelined kernel records
  // the shader-clock and real-time counters at its start and its end
  uint64_t *clock_sample = nullptr;
  // split query tiles (pipelined kernel, prompts): the n_split heaviest query
  // tiles run as two workgroups each, over the first and the second half of
  // their key tiles, and the second to finish merges the two partial
  // results.  Workgroup i takes item i / (B * H) of the table (query tile,
  // part: 0 whole, 1 first half, 2 second half), heaviest items first.
  int n_split = 0, n_items = 0;
  uint8_t item_qt[kMaxPrefillItems], item_part[kMaxPrefillItems];
  float *split_ws = nullptr;     // [n_split][B * H][2 halves][prefill_split_half_floats(D)]
  int32_t *split_cnt = nullptr;  // [n_split][B * H], zero between calls
};

struct ExtendCopyArgs {
  char *k_layer;        // layer's K block (B, Hkv, max_T, D), or the block pools with a table
  char *v_layer;
  const char *k_new;    // (B, Hkv, T, D)
  const char *v_new;
  const int32_t *len;   // layer's lengths [B] (not modified)
  int batch, kv_heads, max_T, row_bytes, T;
  const int32_t *table = nullptr;  // paged: [B][max_blocks] block ids
  int block_log2 = 0, max_blocks = 0;
  const int32_t *slot_blocks = nullptr;  // paged: blocks assigned to each sequence [B] (device)
};

// Prefill rows [0, T) of each (sequence, KV head) copied into a paged
// cache's blocks (bit copies); len[b] = T.
struct PagedWriteArgs {
  char *k_pool;         // layer's K blocks (num_blocks, Hkv, 2^block_log2, D)
  char *v_pool;
  const char *k_new;    // (B, Hkv, T, D)
  const char *v_new;
  int32_t *len;         // layer's lengths [B]
  const int32_t *table; // [B][max_blocks]
  int batch, kv_heads, T, row_bytes, block_log2, max_blocks;
  const int32_t *slot_blocks;  // blocks assigned to each sequence [B] (device)
};

hipError_t launch_append(const AppendArgs &a, hipStream_t s);
hipError_t launch_paged_write(const PagedWriteArgs &a, hipStream_t s);
hipError_t launch_set_lengths(int32_t *dst, int layers, int batch, const int32_t *host_lens,
                              hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_step(const DecodeArgs &a, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s);
// whether prompts of this dtype and head dim run on the pipelined kernel,
// which can split heavy query tiles (and needs the split workspace)
bool prefill_uses_split(kvattn_dtype dt, int head_dim);
hipError_t launch_extend_attention(const PrefillArgs &a, hipStream_t s);
hipError_t launch_extend_copy(const ExtendCopyArgs &a, hipStream_t s);
hipError_t launch_add_lengths(int32_t *len, int batch, int T, int max_T, const int32_t *slot_blocks,
                              int block_log2, hipStream_t s);

// decode splits per (sequence, KV head) are capped, which bounds the
// workspace and the merge's rounds of loads
constexpr int kMaxSplits = 64;

// decode split size in keys: a function of the head dim, the query-group size
// and the capacity, never of the batch (so each sequence's result is
// independent of the others).  384 keys (96 KB of K and of V at D = 128)
// rather than a power of two: with 256- or 512-key splits the concurrently
// streaming workgroups sit at aligned offsets and the ragged batch-32 decode
// ran at 4.9 TB/s instead of 6.3 TB/s on MI355X (measured over split sizes
// 256..576).  Groups of >= 4 query heads per KV head run best with fewer,
// longer streams: 2048-key splits with 8-wave workgroups (GQA 32/8, batch
// 16 at 4096 keys, one decode step of 32 layers: 1.552 ms against 1.573 ms
// for 1024-key splits of 4 waves; 768, 1088, 1366 and 4096 keys, 4 or 8
// waves, measured slower, and so was starting each split's stream at a
// rotated offset).  At D = 32 a 768-key split is two batches of the
// workgroup's loads, and contexts up to 6144 keys take at most eight splits
// (one round of the merge's loads): the 8-layer, 16-head step at 4096-4224
// keys took 61.8 us against 67.7 us with 512-key splits (nine splits), 68.0
// with 1024 (three batches) and 71.5 with 1536.
inline int decode_chunk(int head_dim, int group, int max_T) {
  int c = head_dim <= 32 ? 768 : (group >= 4 ? 2048 : 384);
  while ((max_T + c - 1) / c > kMaxSplits) c *= 2;
  return c;
}

// ---------------------------------------------------------------- device side
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t word4(const uint4 &x, int i) {
  return i == 0 ? x.x : i == 1 ? x.y : i == 2 ? x.z : x.w;
}

}  // namespace kvattn
