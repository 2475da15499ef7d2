// Decode: one query per (sequence, query head) over that sequence's whole
// cache prefix [0, len[b]).
//
// Inference chapter, section 9.1: decode re-reads the cached history every
// step and is limited by memory bandwidth, so this path is a streaming kernel
// on the vector ALUs (no matrix cores): K and V rows are read once per KV head
// with 16-byte loads, the G query heads that share a KV head (roadmap page,
// project 12, MQA/GQA) are served by the same workgroup, and long contexts
// are split across workgroups.  Each split keeps the online-softmax state
// (m, l, u) -- the chunked-attention recurrence of the README -- and a small
// second kernel merges the splits of each (sequence, KV head) by log-sum-exp.
// Merging in the last-arriving workgroup instead was measured twice: with a
// device-scope fence per workgroup (which on this multi-XCD part writes back
// and invalidates the whole L2) ten times slower; with the partials written
// and read by device-scope stores and loads and one atomic counter per unit
// (no L2 flush) about 1 % slower on the ragged batch-32 decode and 2.5 % on
// the 4-token verification, and level on the GQA batch-16 decode, whose
// workgroups all finish together so that the merge is exposed either way.  Scores carry log2(e) inside the scale so that every
// exponential is a single exp2.
#include "common.hpp"

namespace kvattn {

struct TagF32 {
  static constexpr int EPL = 4;  // elements per 16-byte load
  static constexpr int bytes = 4;
};
struct TagF16 {
  static constexpr int EPL = 8;
  static constexpr int bytes = 2;
};
struct TagBF16 {
  static constexpr int EPL = 8;
  static constexpr int bytes = 2;
};

// <q, k> over one 16-byte slice, fp32 accumulation
__device__ __forceinline__ float dot16(TagF32, const uint4 &q, const uint4 &k) {
  float d = __uint_as_float(q.x) * __uint_as_float(k.x);
  d = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), d);
  d = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), d);
  d = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), d);
  return d;
}
__device__ __forceinline__ float dot16(TagF16, const uint4 &q, const uint4 &k) {
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, word4(q, i)),
                               __builtin_bit_cast(half2_t, word4(k, i)), d, false);
  return d;
}
__device__ __forceinline__ float dot16(TagBF16, const uint4 &q, const uint4 &k) {
  float d = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162_t, word4(q, i)),
                                        __builtin_bit_cast(bf162_t, word4(k, i)), d, false);
  return d;
}

// element e of a 16-byte slice, widened to fp32
__device__ __forceinline__ float elem(TagF32, const uint4 &x, int e) {
  return __uint_as_float(word4(x, e));
}
__device__ __forceinline__ float elem(TagF16, const uint4 &x, int e) {
  return (float)__builtin_bit_cast(half2_t, word4(x, e >> 1))[e & 1];
}
__device__ __forceinline__ float elem(TagBF16, const uint4 &x, int e) {
  const uint32_t w = word4(x, e >> 1);
  return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
}

// DPP lane permutations inside a row of 16 lanes
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_XOR1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141; // lane i <- lane 7-i within 8
constexpr int DPP_MIRROR = 0x140;      // lane i <- lane 15-i within 16

// sum over the LPR consecutive lanes that share one key row; every one of
// those lanes ends with the full sum
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  if constexpr (LPR >= 2) x += dpp<DPP_XOR1>(x);
  if constexpr (LPR >= 4) x += dpp<DPP_XOR2>(x);
  if constexpr (LPR >= 8) x += dpp<DPP_HALF_MIRROR>(x);
  if constexpr (LPR >= 16) x += dpp<DPP_MIRROR>(x);
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

__device__ __forceinline__ void store_out(void *o, size_t idx, float x, kvattn_dtype dt) {
  if (dt == KVATTN_F32)
    ((float *)o)[idx] = x;
  else if (dt == KVATTN_F16)
    ((half_t *)o)[idx] = (half_t)x;
  else
    ((bf16_t *)o)[idx] = (bf16_t)x;
}

// Keys attended by sequence b's last query position (decode and the extends
// run on the decode kernels), from its device length len_in: a length past
// the capacity is read as the capacity, so no row outside the sequence's
// region is ever touched (a length <= 0 leaves every split empty and the
// sequence's output unwritten).  With len_pending the lengths do not include
// the extend's `tokens` new rows yet; an extend that would pass the
// sequence's capacity (only on a replayed graph) gives -1: skipped.
__device__ inline int attended_keys(const DecodeArgs &a, int b, int len_in) {
  const int cap = seq_capacity(a.slot_blocks, b, a.block_log2, a.max_T);
  if (a.len_pending) return len_in + a.tokens <= cap ? len_in + a.tokens : -1;
  return min(len_in, cap);
}

// Log-sum-exp merge of the ns non-empty splits of one unit (sequence b, GT
// query rows from h0): THREADS threads each own whole output elements.  Per
// element the splits are folded in rounds of eight (their m, l and u loaded
// together: one dependent round trip per round), in split order, so the
// result does not depend on which workgroup runs it.  COHERENT: the partials
// were written in the same launch by workgroups on other XCDs and are read
// with device-scope loads.
template <int D, int GT, int THREADS, bool COHERENT>
__device__ void merge_unit(const DecodeArgs &a, int b, int h0, int ns) {
  constexpr int SB = 8;  // splits per round of loads
  const int RS = a.q_heads * a.tokens;
  const float *ws_unit = a.ws + (size_t)(b * RS + h0) * a.n_splits * (D + 2);
  auto ld = [](const float *p) -> float {
    if constexpr (COHERENT)
      return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      return *p;
  };
  // E elements per thread per pass, their loads issued together
  constexpr int E = GT * D >= THREADS ? GT * D / THREADS : 1;
  for (int t0 = 0; t0 < GT * D; t0 += E * THREADS) {
    float M[E], num[E], den[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
      M[e] = -INFINITY;
      num[e] = 0.f;
      den[e] = 0.f;
    }
    for (int s0 = 0; s0 < ns; s0 += SB) {
      float ms[E][SB], ls[E][SB], us[E][SB];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        // elements past the unit's GT * D are clamped to its last (in bounds, never stored)
        const int t = min(t0 + e * THREADS + (int)threadIdx.x, GT * D - 1);
        const int g = t / D;
        const int d = t - g * D;
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          // clamped (always in bounds) and masked below
          const float *st = ws_unit + ((size_t)g * a.n_splits + min(s0 + i, ns - 1)) * (D + 2);
          ms[e][i] = ld(st);
          ls[e][i] = ld(st + 1);
          us[e][i] = ld(st + 2 + d);
        }
      }
#pragma unroll
      for (int e = 0; e < E; ++e) {
        float mx = M[e];
#pragma unroll
        for (int i = 0; i < SB; ++i) mx = fmaxf(mx, s0 + i < ns ? ms[e][i] : -INFINITY);
        // split 0 holds at least one visible key, so mx is finite from the first round on
        const float f = fast_exp2(M[e] - mx);
        num[e] *= f;
        den[e] *= f;
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          const float w = s0 + i < ns ? fast_exp2(ms[e][i] - mx) : 0.f;
          num[e] = fmaf(w, us[e][i], num[e]);
          den[e] = fmaf(w, ls[e][i], den[e]);
        }
        M[e] = mx;
      }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int t = t0 + e * THREADS + (int)threadIdx.x;
      if (t < GT * D) {
        const int g = t / D;
        const int d = t - g * D;
        store_out(a.o, (size_t)(b * RS + h0 + g) * D + d, num[e] / den[e], a.o_dt);
      }
    }
  }
}

// grid (n_splits, Hkv * G/GT, B), 256 threads.  A workgroup owns one split of
// `chunk` keys of one KV head, for GT query heads of its group.  LPR lanes
// share one key row, each holding NV 16-byte slices of it (columns cl + v *
// LPR * EPL), so one load instruction reads RPW whole rows.
//
// VER (the short extend, `tokens` = T > 1 query positions per head): the
// query rows of a KV head are its G heads x T tokens, GT = G * T of them per
// workgroup (grid (n_splits, Hkv, B)); token t sits at position L - T + t and
// its scores past that position are masked, so each K/V byte is still read
// once for all G * T rows.
//
// FUSED (the decode step, kvattn_append_decode): the sequence's new K/V row,
// at position len[b], is read from k_new/v_new instead of the cache and
// folded in by the workgroup whose split holds it, which also stores it into
// the cache.  This kernel only reads len[b]; the advanced length is written
// after every workgroup of the sequence has read it: by the merge kernel
// (from the attended count this kernel records) when the cache has several
// splits and the grid is large, else by the last of the sequence's
// workgroups to count itself in on an atomic counter.
//
// INM (with FUSED, for grids too small to fill the device, where a second
// launch costs more than it saves): the splits are merged in this kernel by
// the last of a unit's workgroups to finish, with the merge kernel's
// arithmetic (merge_unit), so the result is the same bits either way.
template <class Tag, int D, int GT, int U, int NV, int NW, bool PAGED, bool VER = false, bool FUSED = false,
          bool INM = false>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeArgs a) {
  static_assert(!INM || (FUSED && !PAGED && !VER), "in-kernel merge: fused decode step only");
  constexpr int EPL = Tag::EPL;
  constexpr int LPR = D / (EPL * NV);  // lanes that share one key row
  constexpr int RPW = 64 / LPR;        // key rows per wave per load instruction
  constexpr int VSTRIDE = LPR * EPL;   // columns between a lane's slices
  constexpr int ESZ = Tag::bytes;
  constexpr int ROWS_PER_STEP = NW * RPW;  // key rows covered by one load across the NW waves
  static_assert(LPR >= 1 && LPR <= 32 && LPR * EPL * NV == D, "row split");

  const int b = blockIdx.z;
  const int split = blockIdx.x;
  const int TK = VER ? a.tokens : 1;       // query positions per head
  const int RS = a.q_heads * TK;            // query rows per sequence: (head, token)
  const int RK = (a.q_heads / a.kv_heads) * TK;  // query rows per KV head
  const int subs = RK / GT;
  const int unit = blockIdx.y;  // (kv head, sub-group of GT query rows)
  const int kvh = unit / subs;
  const int h0 = kvh * RK + (unit - kvh * subs) * GT;  // first query row
  const int tid = threadIdx.x;
  // splits run over the visible keys (all L, or the sink and window ones).
  // FUSED: one thread reads len[b] (the workgroup takes it from LDS), so
  // that once that thread has counted the workgroup in below, no thread of
  // it reads len[b] any more
  __shared__ int s_len;
  if constexpr (FUSED) {
    if (tid == 0) s_len = a.len[b];
    __syncthreads();
  }
  const int len_in = FUSED ? s_len : a.len[b];
  // FUSED: a full sequence is left as it is (cache, length, output); every
  // workgroup of the sequence reads the same len_in, so they all skip it
  const bool full = FUSED && len_in >= a.max_T;
  int32_t *const step_b = FUSED ? a.counters + (size_t)b * kStepSlots : nullptr;
  // several splits merged by the merge kernel: the attended count (or -1:
  // skipped) for it, which commits it as the new length
  if (FUSED && !INM && a.n_splits > 1 && split == 0 && blockIdx.y == 0 && tid == 0)
    step_b[1] = full ? -1 : len_in + 1;
  if (full) return;
  const int L = FUSED ? len_in + 1 : attended_keys(a, b, len_in);
  if (L < 0) return;  // an extend past the sequence's capacity: skipped
  // one split, or the in-kernel merge: every workgroup of the sequence
  // (empty splits included) counts itself in after its read of len[b]; the
  // last one advances len[b] and clears the counter
  const bool counted = FUSED && (INM || a.n_splits == 1);
  int len_ticket = 0;
  if (counted && tid == 0) len_ticket = __hip_atomic_fetch_add(step_b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  auto finish_len = [&]() {
    if (counted && tid == 0 && len_ticket == (int)(gridDim.x * gridDim.y) - 1) {
      __hip_atomic_store(step_b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.len_rw[b] = len_in + 1;
    }
  };
  const VisibleKeys vk = visible_keys(L, a.window, a.sink);
  const int kb = split * a.chunk;  // first visible index of this split
  if (kb >= vk.count) {  // empty split (never with FUSED and a single split)
    finish_len();
    return;
  }
  const int rows = min(a.chunk, vk.count - kb);
  const int n_valid = (vk.count + a.chunk - 1) / a.chunk;
  // FUSED: the split holding the last visible key holds the new row, which
  // is not streamed from the cache
  const bool holds_new = FUSED && kb + rows == vk.count;
  const int srows = rows - (holds_new ? 1 : 0);  // rows streamed from the cache

  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int rg = lane / LPR;
  const int cl = (lane % LPR) * EPL;

  // contiguous: this split's first row; paged: the pool (rows are found
  // through the block table, whose entries for this split sit in LDS)
  const size_t base = PAGED ? (size_t)cl : ((size_t)(b * a.kv_heads + kvh) * a.max_T + kb) * D + cl;
  const char *Kb = (const char *)a.k_layer + base * ESZ;
  const char *Vb = (const char *)a.v_layer + base * ESZ;
  // rows of this split at or past `jump` lie after the gap between sink and window
  const int jump = vk.first - kb;
  const int gap = vk.gap;
  __shared__ int32_t s_tab[PAGED ? kPagedTab : 1];
  // paged: the table entries of this split's rows, staged in LDS.  Rows
  // before `jump` (sink run) sit at position kb + r, the others (window run)
  // at kb + r + gap; entry (pos >> block_log2) + shift_a (resp. shift_b).
  int shift_a = 0, shift_b = 0;
  if constexpr (PAGED) {
    const int n_sink = max(0, min(rows, jump));  // rows of the sink run
    const int blk_a = kb >> a.block_log2;
    const int n_a = n_sink > 0 ? ((kb + n_sink - 1) >> a.block_log2) - blk_a + 1 : 0;
    const int pos_b = kb + n_sink + gap;
    const int blk_b = pos_b >> a.block_log2;
    const int n_b = n_sink < rows ? ((kb + rows - 1 + gap) >> a.block_log2) - blk_b + 1 : 0;
    const int32_t *tab = a.table + (size_t)b * a.max_blocks;
    for (int i = tid; i < n_a + n_b; i += NW * 64) s_tab[i] = i < n_a ? tab[blk_a + i] : tab[blk_b + i - n_a];
    shift_a = -blk_a;
    shift_b = n_a - blk_b;
    __syncthreads();
  }

  uint4 qv[GT][NV];
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int v = 0; v < NV; ++v)
      qv[g][v] = *(const uint4 *)((const char *)a.q +
                                  ((size_t)(b * RS + h0 + g) * D + cl + v * VSTRIDE) * ESZ);
  // VER: the last key row (relative to this split) that query row g sees
  int last_rel[VER ? GT : 1];
  if constexpr (VER) {
#pragma unroll
    for (int g = 0; g < GT; ++g) last_rel[g] = vk.count - TK + (h0 + g) % TK - kb;
  }

  // m: the row's reference point (log2 units), raised only when a score
  // exceeds it by more than kLazyMax, so P = exp2(s - m) <= 2^kLazyMax and the
  // rescale of (l, acc) is rare.  -inf until the first visible key.
  constexpr float kLazyMax = 8.f;
  float m[GT], l[GT], acc[GT][NV * EPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < NV * EPL; ++e) acc[g][e] = 0.f;
  }

  const int steps = (srows + ROWS_PER_STEP - 1) / ROWS_PER_STEP;
  const int nb = (steps + U - 1) / U;
  const float c = a.scale_log2;

  uint4 k0[U][NV], v0[U][NV], k1[U][NV], v1[U][NV];
  // Rows past the split's end are clamped to its last row (always valid: the
  // split is non-empty; with FUSED a split holding only the new row clamps
  // to that row's cache slot, inside the sequence's region and never used)
  // and their scores masked to -inf.  Keeping the loads free of branches
  // lets the compiler wait for one batch while the next is still in flight.
  const int last_row = max(srows, 1) - 1;
  auto load = [&](int ib, uint4 (&kr)[U][NV], uint4 (&vr)[U][NV]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int r = min(((ib * U + u) * NW + wave) * RPW + rg, last_row);
      size_t row;
      if constexpr (PAGED) {
        const bool in_b = r >= jump;
        const int pos = kb + r + (in_b ? gap : 0);
        const int blk = s_tab[(pos >> a.block_log2) + (in_b ? shift_b : shift_a)];
        row = (((size_t)blk * a.kv_heads + kvh) << a.block_log2) + (pos & ((1 << a.block_log2) - 1));
      } else {
        row = (size_t)(r + (r >= jump ? gap : 0));
      }
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        // streamed once: nontemporal loads (measured 5% faster than cached ones)
        const size_t off = (row * D + v * VSTRIDE) * ESZ;
        const u32x4 tk = __builtin_nontemporal_load((const u32x4 *)(Kb + off));
        const u32x4 tv = __builtin_nontemporal_load((const u32x4 *)(Vb + off));
        kr[u][v] = make_uint4(tk[0], tk[1], tk[2], tk[3]);
        vr[u][v] = make_uint4(tv[0], tv[1], tv[2], tv[3]);
      }
    }
  };
  auto compute = [&](int ib, const uint4 (&kr)[U][NV], const uint4 (&vr)[U][NV]) {
    float sc[U][GT];  // raw q.k; the scale is applied inside the exponent
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = ((ib * U + u) * NW + wave) * RPW + rg;
      const bool ok = r < srows;
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float d = dot16(Tag{}, qv[g][0], kr[u][0]);
#pragma unroll
        for (int v = 1; v < NV; ++v) d += dot16(Tag{}, qv[g][v], kr[u][v]);
        d = row_sum<LPR>(d);
        if constexpr (VER)
          sc[u][g] = ok && r <= last_rel[g] ? d : -INFINITY;
        else
          sc[u][g] = ok ? d : -INFINITY;
      }
    }
    float mx[GT];
    bool raise = false;
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      mx[g] = sc[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mx[g] = fmaxf(mx[g], sc[u][g]);
      mx[g] *= c;
      raise |= mx[g] > m[g] + kLazyMax;
    }
    if (__any(raise)) {
      asm volatile("" ::);  // rare: keep it a real branch
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float mn = fmaxf(m[g], mx[g]);
        const float al = fast_exp2(m[g] - (mn == -INFINITY ? 0.f : mn));
        l[g] *= al;
#pragma unroll
        for (int e = 0; e < NV * EPL; ++e) acc[g][e] *= al;
        m[g] = mn;
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float ms = m[g] == -INFINITY ? 0.f : m[g];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(fmaf(sc[u][g], c, -ms));
        l[g] += p;
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            acc[g][v * EPL + e] = fmaf(p, elem(Tag{}, vr[u][v], e), acc[g][v * EPL + e]);
      }
    }
  };

  // two register buffers: the loads of batch i+1 are in flight while batch i
  // computes.  The loads are issued unconditionally (a batch past the end
  // re-reads the clamped last row) so that only the compute is branched over.
  // The scheduling barriers keep the compiler from sinking the loads below
  // the compute (which it does to shorten register live ranges).
  load(0, k0, v0);
  for (int ib = 0; ib < nb; ib += 2) {
    load(ib + 1, k1, v1);
    __builtin_amdgcn_sched_barrier(0);
    compute(ib, k0, v0);
    load(ib + 2, k0, v0);
    __builtin_amdgcn_sched_barrier(0);
    if (ib + 1 < nb) compute(ib + 1, k1, v1);
  }

  if constexpr (FUSED) {
    // the new row: its score and value folded into the state of wave 0's
    // first row group (exact maximum, no lazy threshold), and written into
    // the cache by the first query sub-group of the KV head
    if (holds_new && wave == 0 && rg == 0) {
      const size_t nr = ((size_t)(b * a.kv_heads + kvh) * D + cl) * ESZ;
      uint4 kn[NV], vn[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        kn[v] = *(const uint4 *)((const char *)a.k_new + nr + (size_t)v * VSTRIDE * ESZ);
        vn[v] = *(const uint4 *)((const char *)a.v_new + nr + (size_t)v * VSTRIDE * ESZ);
      }
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        float d = dot16(Tag{}, qv[g][0], kn[0]);
#pragma unroll
        for (int v = 1; v < NV; ++v) d += dot16(Tag{}, qv[g][v], kn[v]);
        const float sn = row_sum<LPR>(d) * c;
        const float mn = fmaxf(m[g], sn);
        const float al = fast_exp2(m[g] - mn);
        const float p = fast_exp2(sn - mn);
        l[g] = fmaf(l[g], al, p);
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            acc[g][v * EPL + e] = fmaf(p, elem(Tag{}, vn[v], e), acc[g][v * EPL + e] * al);
        m[g] = mn;
      }
      if (unit == kvh * subs) {
        const size_t dst = ((size_t)(b * a.kv_heads + kvh) * a.max_T + len_in) * D + cl;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          *(uint4 *)((char *)a.k_cache_rw + (dst + (size_t)v * VSTRIDE) * ESZ) = kn[v];
          *(uint4 *)((char *)a.v_cache_rw + (dst + (size_t)v * VSTRIDE) * ESZ) = vn[v];
        }
      }
    }
  }

  // merge the row groups of this wave (lanes that hold the same columns)
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      const float mo = __shfl_xor(m[g], off);
      const float lo = __shfl_xor(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      const float a1 = fast_exp2(m[g] - ms);
      const float a2 = fast_exp2(mo - ms);
      l[g] = l[g] * a1 + lo * a2;
#pragma unroll
      for (int e = 0; e < NV * EPL; ++e) {
        const float ao = __shfl_xor(acc[g][e], off);
        acc[g][e] = acc[g][e] * a1 + ao * a2;
      }
      m[g] = mn;
    }
  }

  // merge the four waves through LDS
  __shared__ float s_m[NW][GT], s_l[NW][GT];
  __shared__ float s_acc[NW][GT][D];
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_acc[wave][g][cl + v * VSTRIDE + e] = acc[g][v * EPL + e];
      if (lane == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();

  if (n_valid == 1) {
    // the whole context fits one split: normalise and store directly
    for (int t = tid; t < GT * D; t += NW * 64) {
      const int g = t / D;
      const int d = t - g * D;
      float M = s_m[0][g];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float al = fast_exp2(s_m[w][g] - M);
        num = fmaf(al, s_acc[w][g][d], num);
        den = fmaf(al, s_l[w][g], den);
      }
      store_out(a.o, (size_t)(b * RS + h0 + g) * D + d, num / den, a.o_dt);
    }
    finish_len();
    return;
  }

  // write this split's (m, l, u) for the GT heads; decode_merge combines them
  // (INM: device-scope stores, written through to the level every XCD shares,
  // then read back by this unit's last workgroup with device-scope loads)
  auto put = [&](float *p, float x) {
    if constexpr (INM)
      __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *p = x;
  };
  for (int t = tid; t < GT * D; t += NW * 64) {
    const int g = t / D;
    const int d = t - g * D;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, s_m[w][g]);
    // VER: a token may see no key of this split (all its scores masked); it
    // then contributes (-inf, 0, 0)
    const float Ms = (VER && M == -INFINITY) ? 0.f : M;
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float al = fast_exp2(s_m[w][g] - Ms);
      num = fmaf(al, s_acc[w][g][d], num);
      den = fmaf(al, s_l[w][g], den);
    }
    float *dst = a.ws + ((size_t)(b * RS + h0 + g) * a.n_splits + split) * (D + 2);
    put(dst + 2 + d, num);
    if (d == 0) {
      put(dst, M);
      put(dst + 1, den);
    }
  }
  if constexpr (INM) {
    // count this split in; the unit's last one to finish merges all of them
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __shared__ int s_last;
    if (tid == 0) {
      int32_t *cu = a.counters + (size_t)a.batch * kStepSlots + (size_t)b * a.q_heads + unit;
      const int last = __hip_atomic_fetch_add(cu, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_valid - 1;
      if (last) __hip_atomic_store(cu, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (s_last) merge_unit<D, GT, NW * 64, true>(a, b, h0, n_valid);
    finish_len();
  }
}

// query heads per decode workgroup for G query heads per KV head: the
// largest of 8 .. 1 that divides G.  Each K/V byte is read once for G <= 8
// and G / group_tile(G) times for larger groups (the G accumulators of a
// lane would not fit its registers).
inline int group_tile(int G) {
  for (int t = 8; t > 1; --t)
    if (G % t == 0) return t;
  return 1;
}

// threads of the merge kernel: one per output element up to 256, else a
// block size that divides the GT * D outputs evenly
template <int D, int GT>
constexpr int merge_threads() {
  return GT * D <= 256 ? GT * D
                       : (GT * D % 256 == 0 ? 256 : GT * D % 128 == 0 ? 128 : GT * D % 64 == 0 ? 64 : 32);
}

// grid (Hkv * G/GT, B): log-sum-exp merge of the non-empty splits of one
// (sequence, KV head, GT query heads) unit.  Units whose context fits one split
// were finished by decode_kernel.  The kernel is bound by load latency, so
// each thread owns whole output elements and issues the loads of eight
// splits (their m, l and its u column) at once: one dependent round trip per
// eight splits, no shared memory and no barrier.
//
// STEP (the fused decode step over several splits): the attended count comes
// from the decode kernel's record instead of len[b] (-1: the sequence was
// full and is skipped), and unit 0 of each sequence commits it as the new
// length; no workgroup of this kernel reads len[b].
template <int D, int GT, bool STEP = false>
__global__ __launch_bounds__((merge_threads<D, GT>())) void decode_merge_kernel(DecodeArgs a) {
  constexpr int THREADS = merge_threads<D, GT>();
  static_assert(GT * D % THREADS == 0, "outputs split evenly");
  const int b = blockIdx.y;
  const int RK = (a.q_heads / a.kv_heads) * a.tokens;  // query rows per KV head
  const int subs = RK / GT;
  const int unit = blockIdx.x;
  const int kvh = unit / subs;
  const int h0 = kvh * RK + (unit - kvh * subs) * GT;
  const int L = STEP ? a.counters[(size_t)b * kStepSlots + 1] : attended_keys(a, b, a.len[b]);
  if (L < 0) return;
  if (STEP && unit == 0 && threadIdx.x == 0) a.len_rw[b] = L;
  const int ns = (visible_keys(L, a.window, a.sink).count + a.chunk - 1) / a.chunk;
  if (ns <= 1) return;
  merge_unit<D, GT, THREADS, false>(a, b, h0, ns);
}

template <class Tag, int D, int GT, bool PAGED, bool VER>
static hipError_t launch_gt_layout(const DecodeArgs &a, hipStream_t s) {
  // 16-byte K and V loads per lane per batch (two batches are in flight):
  // six for one to three query heads per workgroup, four for larger groups
  // (which hold GT accumulators; eight heads would not fit 256 registers
  // with six).  Measured on the GQA 32/8 batch-16 decode at 4096 keys:
  // two slices per lane (NV = 2) or six or eight loads were no faster; none
  // of the vector-ALU work is on the critical path there (removing the dot
  // products and the P.V updates left the time unchanged).  Groups of >= 4
  // query heads stream 2048-key splits with 8-wave workgroups (one per CU at
  // that shape): 1.5 % faster per step than 1024-key splits of 4 waves.
  // The short extends keep 4 waves.
  constexpr int NV = 1, NW = (!VER && GT >= 4) ? 8 : 4;
  constexpr int U = GT >= 4 ? 4 : 6;
  const int units = a.q_heads * a.tokens / GT;  // = Hkv * (G * tokens / GT)
  decode_kernel<Tag, D, GT, U, NV, NW, PAGED, VER><<<dim3(a.n_splits, units, a.batch), NW * 64, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  decode_merge_kernel<D, GT><<<dim3(units, a.batch), merge_threads<D, GT>(), 0, s>>>(a);
  return hipGetLastError();
}

// the fused decode step (contiguous cache, one query per head): one launch
// for a single-split cache, else the decode kernel and the merge kernel that
// commits the lengths
template <class Tag, int D, int GT>
static hipError_t launch_gt_step(const DecodeArgs &a, hipStream_t s) {
  constexpr int NV = 1, NW = GT >= 4 ? 8 : 4;
  constexpr int U = GT >= 4 ? 4 : 6;
  const int units = a.q_heads / GT;
  const dim3 grid(a.n_splits, units, a.batch);
  if (a.n_splits > 1 && (size_t)a.n_splits * units * a.batch <= kInKernelMergeMaxWorkgroups) {
    decode_kernel<Tag, D, GT, U, NV, NW, false, false, true, true><<<grid, NW * 64, 0, s>>>(a);
    return hipGetLastError();
  }
  decode_kernel<Tag, D, GT, U, NV, NW, false, false, true><<<grid, NW * 64, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_splits == 1) return e;
  decode_merge_kernel<D, GT, true><<<dim3(units, a.batch), merge_threads<D, GT>(), 0, s>>>(a);
  return hipGetLastError();
}

template <class Tag, int D, int GT, bool VER = false>
static hipError_t launch_gt(const DecodeArgs &a, hipStream_t s) {
  if (a.table) return launch_gt_layout<Tag, D, GT, true, VER>(a, s);
  return launch_gt_layout<Tag, D, GT, false, VER>(a, s);
}

template <class Tag, int D>
static hipError_t launch_typed(const DecodeArgs &a, hipStream_t s) {
  const int G = a.q_heads / a.kv_heads;
  if (a.tokens > 1) {
    // short extend: one workgroup per KV head and split holds all G * T rows
    switch (G * a.tokens) {
      case 8: return launch_gt<Tag, D, 8, true>(a, s);
      case 4: return launch_gt<Tag, D, 4, true>(a, s);
      case 3: return launch_gt<Tag, D, 3, true>(a, s);
      case 2: return launch_gt<Tag, D, 2, true>(a, s);
      default: return hipErrorInvalidValue;  // the host routes other shapes to the prefill kernels
    }
  }
  switch (group_tile(G)) {
    case 8: return launch_gt<Tag, D, 8>(a, s);
    case 7: return launch_gt<Tag, D, 7>(a, s);
    case 6: return launch_gt<Tag, D, 6>(a, s);
    case 5: return launch_gt<Tag, D, 5>(a, s);
    case 4: return launch_gt<Tag, D, 4>(a, s);
    case 3: return launch_gt<Tag, D, 3>(a, s);
    case 2: return launch_gt<Tag, D, 2>(a, s);
    default: return launch_gt<Tag, D, 1>(a, s);
  }
}

template <class Tag, int D>
static hipError_t launch_step_typed(const DecodeArgs &a, hipStream_t s) {
  switch (group_tile(a.q_heads / a.kv_heads)) {
    case 8: return launch_gt_step<Tag, D, 8>(a, s);
    case 7: return launch_gt_step<Tag, D, 7>(a, s);
    case 6: return launch_gt_step<Tag, D, 6>(a, s);
    case 5: return launch_gt_step<Tag, D, 5>(a, s);
    case 4: return launch_gt_step<Tag, D, 4>(a, s);
    case 3: return launch_gt_step<Tag, D, 3>(a, s);
    case 2: return launch_gt_step<Tag, D, 2>(a, s);
    default: return launch_gt_step<Tag, D, 1>(a, s);
  }
}

template <class Tag>
static hipError_t launch_step_dim(const DecodeArgs &a, hipStream_t s) {
  switch (a.head_dim) {
    case 32: return launch_step_typed<Tag, 32>(a, s);
    case 64: return launch_step_typed<Tag, 64>(a, s);
    case 128: return launch_step_typed<Tag, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

template <class Tag>
static hipError_t launch_dim(const DecodeArgs &a, hipStream_t s) {
  switch (a.head_dim) {
    case 32: return launch_typed<Tag, 32>(a, s);
    case 64: return launch_typed<Tag, 64>(a, s);
    case 128: return launch_typed<Tag, 128>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_step(const DecodeArgs &a, hipStream_t s) {
  if (a.table || a.tokens != 1 || !a.k_new || !a.v_new || !a.counters || !a.len_rw) return hipErrorInvalidValue;
  switch (a.dt) {
    case KVATTN_F32: return launch_step_dim<TagF32>(a, s);
    case KVATTN_F16: return launch_step_dim<TagF16>(a, s);
    case KVATTN_BF16: return launch_step_dim<TagBF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  switch (a.dt) {
    case KVATTN_F32: return launch_dim<TagF32>(a, s);
    case KVATTN_F16: return launch_dim<TagF16>(a, s);
    case KVATTN_BF16: return launch_dim<TagBF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvattn
