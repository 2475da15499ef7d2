// Append one K/V position per sequence, and set lengths.
//
// Inference chapter, section 9.3: during decode the new token's K and V are
// appended to each layer's cache; the llm-perf-lab README's cache module
// preallocates storage so that this append is O(1).  The copy moves raw bits
// (16-byte integer loads and stores), never converting through float, so the
// cache holds exactly the caller's bytes.
#include "common.hpp"

namespace kvattn {

// One workgroup per sequence b: copies the Hkv rows of k_new/v_new to row
// len[b] of the cache, then (after every thread has read len[b]) bumps it.
// The entry points check capacity against their host copy of the lengths at
// enqueue time; a replayed graph of appends advances only the device lengths,
// so the kernel also keeps every write inside the cache: a sequence at
// max_T positions (paged: at the end of the blocks assigned to it) is left
// as it is, its length unchanged.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int b = blockIdx.x;
  const int pos = a.len[b];
  if (pos >= seq_capacity(a.slot_blocks, b, a.block_log2, a.max_T)) return;  // workgroup-uniform
  const int vec_per_row = a.row_bytes >> 4;
  const int n_vec = a.kv_heads * vec_per_row;
  for (int i = threadIdx.x; i < n_vec; i += blockDim.x) {
    const int h = i / vec_per_row;
    const int w = i - h * vec_per_row;
    const size_t src = ((size_t)(b * a.kv_heads + h) * a.row_bytes) + (size_t)w * 16;
    size_t row;
    if (a.table) {  // paged: the block holding position pos of sequence b
      const int blk = a.table[(size_t)b * a.max_blocks + (pos >> a.block_log2)];
      row = (((size_t)blk * a.kv_heads + h) << a.block_log2) + (pos & ((1 << a.block_log2) - 1));
    } else {
      row = (size_t)(b * a.kv_heads + h) * a.max_T + pos;
    }
    const size_t dst = row * a.row_bytes + (size_t)w * 16;
    const uint4 kv = *reinterpret_cast<const uint4 *>(a.k_new + src);
    const uint4 vv = *reinterpret_cast<const uint4 *>(a.v_new + src);
    *reinterpret_cast<uint4 *>(a.k_layer + dst) = kv;
    *reinterpret_cast<uint4 *>(a.v_layer + dst) = vv;
  }
  __syncthreads();
  if (threadIdx.x == 0) a.len[b] = pos + 1;
}

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
  append_kernel<<<dim3(a.batch), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

// Extend: T rows per (sequence, KV head) copied to cache rows [len[b], len[b] + T)
// (bit copies; through the block table for a paged cache); grid (row chunks, Hkv, B).  The lengths are only read here and
// advanced by add_lengths_kernel once the attention over them has run.  A
// sequence whose T new rows would pass its capacity (only on a replayed
// graph: the entry point checks its host copy of the lengths) is left as it
// is by all three kernels of the extend: copy, attention and length update.
__global__ __launch_bounds__(256) void extend_copy_kernel(ExtendCopyArgs a) {
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  const int vec_per_row = a.row_bytes >> 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.T * vec_per_row) return;
  const int len0 = a.len[b];
  if (len0 + a.T > seq_capacity(a.slot_blocks, b, a.block_log2, a.max_T)) return;
  const int t = idx / vec_per_row;
  const int w = idx - t * vec_per_row;
  const int pos = len0 + t;
  const size_t src = ((size_t)(b * a.kv_heads + h) * a.T + t) * a.row_bytes + (size_t)w * 16;
  const size_t row = a.table ? paged_row(a.table, b, a.max_blocks, a.block_log2, a.kv_heads, h, pos)
                             : (size_t)(b * a.kv_heads + h) * a.max_T + pos;
  const size_t dst = row * a.row_bytes + (size_t)w * 16;
  *reinterpret_cast<uint4 *>(a.k_layer + dst) = *reinterpret_cast<const uint4 *>(a.k_new + src);
  *reinterpret_cast<uint4 *>(a.v_layer + dst) = *reinterpret_cast<const uint4 *>(a.v_new + src);
}

hipError_t launch_extend_copy(const ExtendCopyArgs &a, hipStream_t s) {
  const int vec_per_row = a.row_bytes >> 4;
  const unsigned chunks = (unsigned)(((size_t)a.T * vec_per_row + 255) / 256);
  extend_copy_kernel<<<dim3(chunks, a.kv_heads, a.batch), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

// Paged prefill: prompt rows [0, T) of each (sequence, KV head) to their
// blocks (bit copies); grid (row chunks, Hkv, B).  len[b] = T.
__global__ __launch_bounds__(256) void paged_write_kernel(PagedWriteArgs a) {
  const int b = blockIdx.z;
  const int h = blockIdx.y;
  // a prompt longer than the sequence's blocks (blocks reassigned after a
  // graph was captured) is not written
  if (a.T > (a.slot_blocks[b] << a.block_log2)) return;
  if (blockIdx.x == 0 && h == 0 && threadIdx.x == 0) a.len[b] = a.T;
  const int vec_per_row = a.row_bytes >> 4;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.T * vec_per_row) return;
  const int t = idx / vec_per_row;
  const int w = idx - t * vec_per_row;
  const int blk = a.table[(size_t)b * a.max_blocks + (t >> a.block_log2)];
  const size_t row = (((size_t)blk * a.kv_heads + h) << a.block_log2) + (t & ((1 << a.block_log2) - 1));
  const size_t src = ((size_t)(b * a.kv_heads + h) * a.T + t) * a.row_bytes + (size_t)w * 16;
  const size_t dst = row * a.row_bytes + (size_t)w * 16;
  *reinterpret_cast<uint4 *>(a.k_pool + dst) = *reinterpret_cast<const uint4 *>(a.k_new + src);
  *reinterpret_cast<uint4 *>(a.v_pool + dst) = *reinterpret_cast<const uint4 *>(a.v_new + src);
}

hipError_t launch_paged_write(const PagedWriteArgs &a, hipStream_t s) {
  const int vec_per_row = a.row_bytes >> 4;
  const unsigned chunks = (unsigned)(((size_t)a.T * vec_per_row + 255) / 256);
  paged_write_kernel<<<dim3(chunks, a.kv_heads, a.batch), dim3(256), 0, s>>>(a);
  return hipGetLastError();
}

__global__ void add_lengths_kernel(int32_t *len, int batch, int T, int max_T, const int32_t *slot_blocks,
                                   int block_log2) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch && len[b] + T <= seq_capacity(slot_blocks, b, block_log2, max_T)) len[b] += T;
}

hipError_t launch_add_lengths(int32_t *len, int batch, int T, int max_T, const int32_t *slot_blocks,
                              int block_log2, hipStream_t s) {
  add_lengths_kernel<<<dim3((batch + 255) / 256), dim3(256), 0, s>>>(len, batch, T, max_T, slot_blocks,
                                                                     block_log2);
  return hipGetLastError();
}

// Lengths travel by value in the kernel arguments, so the caller's host array
// need not outlive the call and no host-to-device copy is enqueued.
constexpr int kLenChunk = 256;
struct LenChunk {
  int32_t v[kLenChunk];
};

__global__ void set_lengths_kernel(int32_t *dst, int batch, int offset, int n, LenChunk c) {
  const int i = threadIdx.x;
  if (i < n) dst[(size_t)blockIdx.x * batch + offset + i] = c.v[i];
}

hipError_t launch_set_lengths(int32_t *dst, int layers, int batch, const int32_t *host_lens,
                              hipStream_t s) {
  for (int off = 0; off < batch; off += kLenChunk) {
    LenChunk c;
    const int n = batch - off < kLenChunk ? batch - off : kLenChunk;
    for (int i = 0; i < n; ++i) c.v[i] = host_lens[off + i];
    set_lengths_kernel<<<dim3(layers), dim3(kLenChunk), 0, s>>>(dst, batch, off, n, c);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace kvattn
