/*
 * kvattn.h -- C ABI of libkvattn: exact causal softmax attention over a
 * preallocated per-layer KV cache, for AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For batch entry b, query head h and a query at absolute
 * position i, over keys j = 0..i (the diagonal included):
 *     s_ij = scale * <q[b,h,i,:], k[b,g,j,:]>,   g = h / (H / Hkv)
 *     o[b,h,i,:] = sum_j softmax_j(s_i.) * v[b,g,j,:]
 * This is the attention of the roadmap page's project 11 (cached self
 * attention: scores q k^T / sqrt(D), softmax over keys, times V, past K/V
 * concatenated on the time axis of a (B, H, T, D) layout) with the causal
 * mask a decoder-only model needs, and the MQA/GQA head sharing of project 12.
 * The inference chapter (section 9.3) fixes the two phases: prefill
 * processes the prompt and builds each layer's K/V cache; decode appends one
 * position and reads the whole cache.  Only K and V are cached.  Section 9.7:
 * the tiled (flash-style) computation is the same attention up to ordinary
 * floating-point rounding, and never writes the T x T matrix to memory.
 *
 * Layouts (all row-major and contiguous, element type = the cache dtype):
 *   q, o in prefill      (B, H, T, D)
 *   k, v in prefill      (B, Hkv, T, D)
 *   q, o in decode       (B, H, 1, D)
 *   k_new, v_new         (B, Hkv, 1, D)
 *   cache, per layer     K then V, each (B, Hkv, max_T, D), inside one device
 *                        allocation laid out [layer][K|V][B][Hkv][max_T][D]
 *   lengths              int32 [layer][B] on the device, mirrored on the host
 * Pointers named q, k, v, o, k_new, v_new, device_buf are DEVICE pointers;
 * host_lens is a HOST pointer.  `stream` is a hipStream_t (NULL = the null
 * stream).
 *
 * Supported: dtype F32, F16, BF16; head_dim D in {32, 64, 128}; H % Hkv == 0.
 * Arithmetic: scores, softmax statistics and output accumulation in fp32; for
 * F16/BF16 the two products run on the matrix cores with fp32 accumulation.
 *
 * Ownership.  The caller owns q/k/v/o/k_new/v_new and the stream.  The library
 * owns the cache object, its length arrays and its split-K workspace; it owns
 * the cache payload too unless the caller passes `device_buf`, which must then
 * stay alive until kvattn_cache_free.  A cache object is not thread-safe, and
 * all work on one cache must be issued on one stream (the split-K workspace is
 * shared by every layer of the cache).
 *
 * Errors.  0 on success, a negative kvattn_status otherwise.  Every argument is
 * validated on the host before anything is enqueued, so a failed call leaves
 * the cache and its lengths unchanged.  All calls only enqueue work on
 * `stream`; none synchronises except kvattn_cache_free.  A kernel fault shows
 * up as KVATTN_ERR_HIP on a later call.
 */
#ifndef KVATTN_H
#define KVATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KVATTN_F32 = 0, KVATTN_F16 = 1, KVATTN_BF16 = 2 } kvattn_dtype;

typedef enum {
  KVATTN_OK = 0,
  KVATTN_ERR_INVALID_ARG = -1, /* null pointer, negative size, bad layer index  */
  KVATTN_ERR_UNSUPPORTED = -2, /* dtype, head_dim not in {32,64,128}, H % Hkv   */
  KVATTN_ERR_CAPACITY = -3,    /* append on a full sequence; prefill T > max_T  */
  KVATTN_ERR_STATE = -4,       /* prefill on a non-empty layer; decode at len 0 */
  KVATTN_ERR_OOM = -5,         /* device allocation failed / buffer too small   */
  KVATTN_ERR_HIP = -6          /* a HIP runtime call or kernel launch failed    */
} kvattn_status;

typedef struct kvattn_cache kvattn_cache; /* opaque, library-owned */

/* Cache payload bytes by the inference chapter's capacity formula (section
 * 9.3): 2 * layers * kv_heads * head_dim * max_T * bytes(dt) * batch.  The 2
 * counts K and V; lengths and workspace are not included.  Pure host function;
 * returns 0 for a non-positive argument or an unknown dtype. */
size_t kvattn_cache_bytes(int layers, int batch, int kv_heads, int head_dim, int max_T,
                          kvattn_dtype dt);

/* Create a cache of `layers` layers for `batch` sequences of up to `max_T`
 * positions (the preallocated cache with O(1) append of the llm-perf-lab
 * README's kv_cache module).  q_heads is H (needed to size the decode
 * workspace); kv_heads is Hkv.  If device_buf is NULL the library allocates
 * the payload; otherwise device_buf (>= kvattn_cache_bytes bytes, 256-byte
 * aligned) is adopted.  All lengths start at 0 (on the device and the host).
 * Needs a current HIP device; synchronises that device once. */
int kvattn_cache_alloc(kvattn_cache **out, int layers, int batch, int q_heads, int kv_heads,
                       int head_dim, int max_T, kvattn_dtype dt, void *device_buf,
                       size_t device_buf_bytes);

/* Synchronise the device, release what the library allocated and the object. */
int kvattn_cache_free(kvattn_cache *c);

/* Device addresses of layer `layer`'s K and V blocks, each (B, Hkv, max_T, D). */
int kvattn_cache_kv_ptr(const kvattn_cache *c, int layer, void **k, void **v);

/* Set the valid lengths of one layer (layer >= 0) or of every layer (-1) to
 * host_lens[0..B-1], each in [0, max_T].  Truncation and rollback to an
 * accepted prefix (the README's speculative loop rolls the cache back);
 * rows at or past a length are never read.  Enqueued on `stream`; host_lens
 * is copied before the call returns. */
int kvattn_cache_set_lengths(kvattn_cache *c, int layer, const int32_t *host_lens, void *stream);

/* Copy the host mirror of one layer's lengths into host_lens[0..B-1].  The
 * mirror is updated at enqueue time, so it already includes enqueued work. */
int kvattn_cache_get_lengths(const kvattn_cache *c, int layer, int32_t *host_lens);

/* Sliding-window and attention-sink masks of one layer (layer >= 0) or of
 * every layer (-1), the long-context variants of the roadmap page (project 13:
 * attend only a recent window; keep the first few positions).  With window W
 * > 0 and sink S >= 0, the query at position i sees key j iff j <= i and
 * (i - j < W or j < S); window 0 (the default) is the plain causal mask and
 * resets the sink to 0.  Later prefill, extend and decode calls on the layer
 * use the mask; decode then reads only the min(len, S) sink rows and the last
 * W rows of each sequence.  INVALID_ARG for a negative W or S or a bad layer.
 * Host-only: enqueues nothing. */
int kvattn_cache_set_window(kvattn_cache *c, int layer, int window, int sink);

/* The window and sink set for one layer (0, 0 when none). */
int kvattn_cache_get_window(const kvattn_cache *c, int layer, int *window, int *sink);

/* Prefill of one layer (inference chapter 9.1/9.3): causal attention of the T
 * prompt queries over the T prompt keys, o = attn(q, k, v), and a bit-exact
 * copy of k, v into cache rows [0, T); the layer's lengths become T.
 * q (B,H,T,D), k/v (B,Hkv,T,D) in the cache dtype; o (B,H,T,D) in o_dtype,
 * which is the cache dtype or F32.  Requires every length of the layer to be
 * 0 (else STATE) and 1 <= T <= max_T (else CAPACITY / INVALID_ARG).  scale is
 * normally 1/sqrt(D).  No T x T buffer is ever allocated or written. */
int kvattn_prefill(kvattn_cache *c, int layer, const void *q, const void *k, const void *v,
                   void *o, int T, float scale, kvattn_dtype o_dtype, void *stream);

/* Append one position per sequence (inference chapter 9.3: decode appends one
 * position to the cache): k_new/v_new (B,Hkv,1,D) are copied bit-exactly to
 * row len[b] of sequence b, then len[b] += 1.  CAPACITY if any len[b] ==
 * max_T.  That check runs on the host, at enqueue time, against the
 * library's host copy of the lengths; the kernel reads len[b] from device
 * memory, so a call captured in a HIP graph appends at the current length on
 * every replay, and a replay at len[b] == max_T leaves that sequence's cache
 * and length unchanged (no error is reported from the device). */
int kvattn_append(kvattn_cache *c, int layer, const void *k_new, const void *v_new, void *stream);

/* Extend one layer by T positions per sequence after its cached prefix: the
 * chunked prefill of a long prompt (the README's chunked attention equals the
 * one-shot form for any chunk size) and the multi-token verification step of
 * its speculative decoding loop (draft tokens checked in one pass; rejected
 * ones are rolled back with kvattn_cache_set_lengths).  k/v (B,Hkv,T,D) are
 * copied bit-exactly to cache rows [len[b], len[b] + T); query t of sequence b
 * (q (B,H,T,D)) sits at position len[b] + t and attends cache rows
 * 0 .. len[b] + t (the causal mask aligned to the bottom right); o (B,H,T,D)
 * in o_dtype (cache dtype or F32); then len[b] += T.  Lengths may differ
 * between sequences and may be 0 (then this is a prefill).  CAPACITY if any
 * len[b] + T > max_T; T >= 1.  Three kernels are enqueued on `stream` (copy,
 * attention, length update). */
int kvattn_extend(kvattn_cache *c, int layer, const void *q, const void *k, const void *v, void *o,
                  int T, float scale, kvattn_dtype o_dtype, void *stream);

/* Decode of one layer (inference chapter, section 9.3: decode appends one
 * position and reads the whole cache; section 9.1: that read of the cached
 * history makes decode memory-bandwidth bound; roadmap page, project 11: the
 * new query attends the past keys concatenated with its own, and project 12:
 * query heads that share a KV head read it once): query q[b,h] (B,H,1,D) sits
 * at position len[b]-1 and attends all len[b] cached keys of its KV head (the
 * causal mask aligned to the bottom right); o (B,H,1,D) in o_dtype (cache
 * dtype or F32).  Lengths are
 * read from device memory, so the call needs no host synchronisation after an
 * append.  STATE if any len[b] == 0.  Long contexts are split across
 * workgroups and merged by log-sum-exp; the split depends only on len[b],
 * never on the batch, so each sequence's output is independent of the
 * others. */
int kvattn_decode(kvattn_cache *c, int layer, const void *q, void *o, float scale,
                  kvattn_dtype o_dtype, void *stream);

/* One decode step of one layer in one launch: kvattn_append followed by
 * kvattn_decode (inference chapter, section 9.3: decode appends the new
 * token's K and V to the cache and attends the whole cache).  k_new/v_new
 * (B,Hkv,1,D) are copied bit-exactly to row len[b] of sequence b; query
 * q[b,h] (B,H,1,D) at position len[b] attends cache rows 0 .. len[b] (the new
 * row included, within the layer's window and sink if set); o (B,H,1,D) in
 * o_dtype (cache dtype or F32); then len[b] += 1.  The result equals that of
 * the two calls.  The new row is taken from k_new/v_new for the attention and
 * stored into the cache by the same kernel.  The splits of each sequence are
 * merged by log-sum-exp: inside the launch when its grid has at most 256
 * workgroups (the last of a sequence's workgroups then advances its length),
 * else by a second kernel on the same stream, which also advances the
 * lengths; both give the same bits.  The call needs no host synchronisation
 * and may be captured in a HIP graph.  CAPACITY if any len[b] == max_T
 * (checked on the host against its copy of the lengths); on a replayed graph
 * a sequence found full on the device is left unchanged, cache, length and
 * output rows alike.  Lengths may be 0 (the query then sees only its own
 * row).  Calls on one cache must be ordered on one stream (the split
 * counters and workspace are shared by its layers). */
int kvattn_append_decode(kvattn_cache *c, int layer, const void *k_new, const void *v_new, const void *q, void *o,
                         float scale, kvattn_dtype o_dtype, void *stream);

/* Bytes of the fixed device array that holds kvattn_decode_noalloc's split-K
 * partials (one copy per device, kept until the process ends). */
#define KVATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/* Decode that allocates nothing, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  It computes what kvattn_decode computes, with the same
 * kernels, over a caller-owned contiguous cache: k_cache and v_cache are
 * device arrays (batch, kv_heads, max_T, head_dim) in `dt`, lengths a device
 * int32 array [batch] (query q[b,h] (B,H,1,D) sits at position lengths[b]-1
 * and attends cache rows 0 .. lengths[b]-1), o (B,H,1,D) in o_dtype (dt or
 * F32).  No window, no block table.  The split-K partials go to a fixed
 * device array of KVATTN_NOALLOC_SCRATCH_BYTES inside the library instead of
 * a cache object's workspace; a shape needs
 * 4 * batch * q_heads * ceil(max_T / split) * (head_dim + 2) bytes of it
 * (split = the decode split size, 384-2048 keys by head dim and group size,
 * doubled while max_T / split > 64), and CAPACITY is returned, with the
 * sizes in kvattn_last_error, when that exceeds the array.  The array is
 * shared by every call on a device and keeps the last call's contents:
 * calls that overlap on one device (concurrent streams) race on it.  Every
 * partial is written before it is read within a call, so nothing needs
 * clearing between calls.  Lengths are read on the device only: each must be
 * in [1, max_T]; a larger one is read as max_T and a sequence with a length
 * <= 0 gets no output written.  The first call on a device looks up the
 * array's device address (no allocation).  INVALID_ARG / UNSUPPORTED as for
 * kvattn_decode; nothing is enqueued on error. */
int kvattn_decode_noalloc(const void *k_cache, const void *v_cache, const int32_t *lengths, int batch,
                          int q_heads, int kv_heads, int head_dim, int max_T, kvattn_dtype dt, const void *q,
                          void *o, float scale, kvattn_dtype o_dtype, void *stream);

/* ---------------------------------------------------------------- paged cache
 * The cache managed in fixed-size blocks instead of one max-length region per
 * sequence (inference chapter, section 9.6, Continuous Batching and Paged KV;
 * the llm-perf-lab README's vLLM-style paging with prefix sharing).  A pool of
 * num_blocks blocks per layer, laid out [layer][K|V][num_blocks][Hkv]
 * [block_size][D]; each of `slots` sequences has a block table (the same for
 * every layer): its position p lives in block table[p / block_size], row
 * p % block_size.  Tables may share blocks (prefix sharing); rows of a shared
 * block must be the same for every slot that writes them.  Calls cover every
 * slot, like the contiguous cache (slots = batch); lengths are per (layer,
 * slot) with a host mirror; a slot holds at most n_blocks * block_size
 * positions.  Sliding window and sink masks as for the contiguous cache
 * (kvattn_paged_set_window). */
typedef struct kvattn_paged kvattn_paged; /* opaque, library-owned */

/* Pool bytes: 2 * layers * num_blocks * block_size * kv_heads * head_dim *
 * bytes(dt) (the capacity formula with T = num_blocks * block_size, batch 1);
 * 0 for a non-positive argument or an unknown dtype.  Pure host function. */
size_t kvattn_paged_bytes(int layers, int num_blocks, int block_size, int kv_heads, int head_dim,
                          kvattn_dtype dt);

/* Create a paged cache: `slots` sequences of up to max_blocks blocks each,
 * from a pool of num_blocks blocks of block_size positions (a power of two in
 * [16, 4096], else UNSUPPORTED).  device_buf as for kvattn_cache_alloc.  All
 * tables are empty and all lengths 0.  Synchronises the device once. */
int kvattn_paged_alloc(kvattn_paged **out, int layers, int slots, int max_blocks, int num_blocks,
                       int block_size, int q_heads, int kv_heads, int head_dim, kvattn_dtype dt,
                       void *device_buf, size_t device_buf_bytes);

/* Synchronise the device, release what the library allocated and the object. */
int kvattn_paged_free(kvattn_paged *p);

/* Device addresses of layer `layer`'s K and V pools, each (num_blocks, Hkv,
 * block_size, D). */
int kvattn_paged_kv_ptr(const kvattn_paged *p, int layer, void **k, void **v);

/* Set the block table of one slot to host_block_ids[0..n_blocks-1] (pool
 * indices; n_blocks <= max_blocks).  INVALID_ARG for an index outside the
 * pool; CAPACITY if a layer's length of the slot exceeds n_blocks *
 * block_size.  Enqueued on `stream` (the ids are copied before the call
 * returns); later calls must be on the same stream or ordered after it. */
int kvattn_paged_set_blocks(kvattn_paged *p, int slot, const int32_t *host_block_ids, int n_blocks,
                            void *stream);

/* Lengths of one layer (>= 0) or of every layer (-1), each within its slot's
 * blocks (else CAPACITY): truncation and rollback, as for the contiguous cache. */
int kvattn_paged_set_lengths(kvattn_paged *p, int layer, const int32_t *host_lens, void *stream);
int kvattn_paged_get_lengths(const kvattn_paged *p, int layer, int32_t *host_lens);

/* Window and sink of one layer (>= 0) or of every layer (-1), with the
 * meaning of kvattn_cache_set_window; later prefill, extend and decode calls
 * on the layer use them, and decode reads only the visible rows' blocks.
 * UNSUPPORTED when a windowed decode split would stage more block-table
 * entries than its on-chip table holds (2 * (split / block_size + 2) > 512;
 * only for very small blocks with very long capacities).  Host-only. */
int kvattn_paged_set_window(kvattn_paged *p, int layer, int window, int sink);
int kvattn_paged_get_window(const kvattn_paged *p, int layer, int *window, int *sink);

/* Prefill of one layer: causal attention of the T prompt queries of every
 * slot (q (slots,H,T,D), k/v (slots,Hkv,T,D), o in o_dtype) as
 * kvattn_prefill, then a bit-exact copy of k, v into each slot's blocks at
 * positions [0, T); lengths become T.  STATE unless every length is 0;
 * CAPACITY if T exceeds a slot's blocks. */
int kvattn_paged_prefill(kvattn_paged *p, int layer, const void *q, const void *k, const void *v,
                         void *o, int T, float scale, kvattn_dtype o_dtype, void *stream);

/* Append one position per slot (k_new/v_new (slots,Hkv,1,D)) at its length,
 * in the block that holds that position; len += 1.  CAPACITY if a slot's
 * blocks are full (checked on the host at enqueue time; on the device a
 * position past the slot's block-table row is dropped, as in kvattn_append,
 * but one past its assigned blocks is not detected there). */
int kvattn_paged_append(kvattn_paged *p, int layer, const void *k_new, const void *v_new, void *stream);

/* Extend over the paged cache: as kvattn_extend (chunked prefill, multi-token
 * verification), with the new rows written to positions [len, len + T) of
 * each slot's blocks and the attention reading every key through the slot's
 * block table; len += T.  CAPACITY if len + T exceeds a slot's blocks. */
int kvattn_paged_extend(kvattn_paged *p, int layer, const void *q, const void *k, const void *v, void *o,
                        int T, float scale, kvattn_dtype o_dtype, void *stream);

/* Decode over the paged cache: as kvattn_decode, each slot's query attending
 * its len positions (or its window and sink), read through its block table. */
int kvattn_paged_decode(kvattn_paged *p, int layer, const void *q, void *o, float scale,
                        kvattn_dtype o_dtype, void *stream);

/* Static description of a status code. */
const char *kvattn_status_string(int status);

/* Text of the last HIP error this thread's calls saw ("" if none). */
const char *kvattn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_H */
