// Prefill: causal attention of a T-token prompt, with a bit-exact copy of the
// prompt's K and V into the layer's cache.
//
// Inference chapter, section 9.1: prefill is matrix-multiply shaped and
// builds the cache; section 9.7 (and the roadmap page's project 15): tiling
// with on-chip storage computes the same attention while never writing the
// T x T score matrix to device memory.  The README's chunked attention with
// the online-softmax recurrence is the algebra used here, tile by tile.
//
// gfx950 design (F16/BF16): a workgroup owns a block of query rows of one
// (b, h); each wave keeps its 32 query rows in registers as MFMA operands and
// computes, per K/V tile of BN keys staged through LDS,
//     S^T = K Q^T   (fp32 accumulate)
//     O^T += V^T P^T
// The plain kernel below (4 waves, v_mfma_f32_16x16x32) serves windows, block
// tables and bf16 at D = 32; the pipelined kernel further down (8 waves,
// v_mfma_f32_32x32x16, the next tile's scores overlapped with this tile's
// softmax) serves the other prompts and extends.
// The transposed orientation puts one query in one lane column for both
// products, so the running max / sum and the rescale of O stay per-lane; row
// statistics need two cross-lane steps per tile (one with the 32x32 shape).  V is transposed while
// it is staged to LDS so that its reduction axis (keys) is contiguous for the
// MFMA operand.  Tiles past the diagonal are never visited.  The workgroups
// that own the diagonal tile of the first query head of a KV group also
// store that K/V tile into the cache from the registers it was loaded into.
//
// F32 takes a plain vector-ALU kernel (four lanes per query row).
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.hpp"

namespace kvattn {

template <typename T>
struct Mfma;
template <>
struct Mfma<half_t> {
  typedef half8_t vec;
  static constexpr bool kSplitP = false;  // fp16 P (11-bit significand) is accurate enough
  static __device__ __forceinline__ float4_t mma(const vec &a, const vec &b, const float4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // acc + sum of the 8 elements, in fp32
  static __device__ __forceinline__ float sum8(const vec &x, float acc) {
    const half2_t one = {(half_t)1.0f, (half_t)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = __builtin_amdgcn_fdot2(half2_t{x[2 * i], x[2 * i + 1]}, one, acc, false);
    return acc;
  }
};
template <>
struct Mfma<bf16_t> {
  typedef bf168_t vec;
  // bf16 keeps 8 significand bits: P is carried as hi + lo bf16 parts (two MFMAs)
  static constexpr bool kSplitP = true;
  static __device__ __forceinline__ float4_t mma(const vec &a, const vec &b, const float4_t &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ float sum8(const vec &x, float acc) {
    const bf162_t one = {(bf16_t)1.0f, (bf16_t)1.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(bf162_t{x[2 * i], x[2 * i + 1]}, one, acc, false);
    return acc;
  }
};

__device__ __forceinline__ void store4(void *o, size_t idx, const float4_t &x, float s,
                                       kvattn_dtype dt) {
  if (dt == KVATTN_F32) {
    *(float4_t *)((float *)o + idx) = x * s;
  } else if (dt == KVATTN_F16) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 r;
    r[0] = (half_t)(x[0] * s); r[1] = (half_t)(x[1] * s);
    r[2] = (half_t)(x[2] * s); r[3] = (half_t)(x[3] * s);
    *(h4 *)((half_t *)o + idx) = r;
  } else {
    typedef __bf16 b4 __attribute__((ext_vector_type(4)));
    b4 r;
    r[0] = (bf16_t)(x[0] * s); r[1] = (bf16_t)(x[1] * s);
    r[2] = (bf16_t)(x[2] * s); r[3] = (bf16_t)(x[3] * s);
    *(b4 *)((bf16_t *)o + idx) = r;
  }
}

template <int D, int BN>
struct PrefillLds {
  static constexpr int KSTR = D + 8;   // K row stride (elements): conflict-free 16-B reads
  // V^T row stride (elements): 34 dwords for BN = 64, so the 16 lanes of a
  // quarter-wave reading 8 bytes each from consecutive rows hit distinct bank pairs
  static constexpr int VSTR = BN + 4;
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr size_t BYTES = 2 * BUF * 2;  // two buffers of 2-byte elements
};

// The running maximum of a row is only raised when a tile's maximum exceeds
// it by more than 2^kLazyMax (in exp2 units), so most tiles skip the rescale
// of O; P then stays below 2^kLazyMax, well inside fp16/bf16 range, and the
// result is the same attention (softmax is invariant to the reference point).
constexpr float kLazyMax = 8.0f;

// 1-D grid over (q-tile, b, h), heaviest (last) query tiles first.  With NW = 4
// every thread stages both K and V; with NW = 8 waves 0-3 stage K and waves 4-7
// stage V.
template <typename T, int D, int QW, int BN, int NW, bool PAGED = false>
__global__ __launch_bounds__(NW * 64, NW == 4 ? 2 : 1) void prefill_mfma_kernel(PrefillArgs a) {
  typedef typename Mfma<T>::vec vec8;
  typedef PrefillLds<D, BN> LDS;
  constexpr int BM = NW * QW;
  constexpr int NT = QW / 16;  // query sub-tiles per wave
  constexpr int KT = BN / 16;  // key sub-tiles per tile
  constexpr int KS = D / 32;   // MFMA k-steps over D
  constexpr int DT = D / 16;   // output sub-tiles over D
  constexpr int PS = BN / 32;  // MFMA k-steps over keys
  constexpr int KCH = BN * D / 8 / 256;       // 16-B K chunks per staging thread
  constexpr int VPAIRS = (BN / 4) * (D / 8);  // (4-key group, 8-column slice) pairs
  constexpr bool SPLIT_STAGE = NW == 8;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  static_assert(KCH >= 1 && BN * D / 8 == KCH * 256, "K tile must split evenly over 256 threads");
  static_assert(VPAIRS <= 256 && VPAIRS % 64 == 0, "V tile must cover whole waves");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  T *smem = reinterpret_cast<T *>(smem_raw);

  const int Tn = a.T;
  const int H = a.q_heads;
  const int G = H / a.kv_heads;
  const int n_qt = (Tn + BM - 1) / BM;
  const int BH = a.batch * H;
  const int qt = n_qt - 1 - (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int b = bh / H;
  const int h = bh - b * H;
  const int g = h / G;
  const bool writer = (h - g * G) == 0;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l16 = lane & 15;
  const int lg = lane >> 4;
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * QW;
  // staging roles
  const int stid = SPLIT_STAGE ? (tid & 255) : tid;
  const bool stage_k = SPLIT_STAGE ? (tid < 256) : true;
  const bool stage_v = (SPLIT_STAGE ? (tid >= 256) : true) && stid < VPAIRS;

  const T *qb = (const T *)a.q + (size_t)bh * Tn * D;
  // query row i sits at absolute position off + i and sees keys 0 .. off + i
  const int off = a.offsets ? a.offsets[b] : 0;
  // an extend past the sequence's capacity (only on a replayed graph) is
  // left to the copy and length kernels to skip; no output row is written
  if (a.offsets && off + Tn > seq_capacity(a.slot_blocks, b, a.block_log2, a.max_T)) return;
  const int last_key = off + Tn - 1;
  // paged (extend over a paged cache): k/v are the block pools and a key's
  // row is found through the sequence's block table
  const T *kb = (const T *)a.k + (PAGED ? 0 : (size_t)(b * a.kv_heads + g) * a.kv_rows * D);
  const T *vb = (const T *)a.v + (PAGED ? 0 : (size_t)(b * a.kv_heads + g) * a.kv_rows * D);
  auto row_of = [&](int key) -> size_t {
    if constexpr (PAGED) return paged_row(a.table, b, a.max_blocks, a.block_log2, a.kv_heads, g, key);
    return (size_t)key;
  };
  T *ckb = (T *)a.cache_k + (size_t)(b * a.kv_heads + g) * a.max_T * D;
  T *cvb = (T *)a.cache_v + (size_t)(b * a.kv_heads + g) * a.max_T * D;

  if (a.write_cache && qt == 0 && h == 0 && tid == 0) a.len[b] = Tn;

  // query fragments (B operand of S^T = K Q^T): lane holds 8 columns of one row
  vec8 qf[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = min(qw0 + nt * 16 + l16, Tn - 1);  // rows past T are never stored
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[nt][ks] = *(const vec8 *)(qb + (size_t)row * D + ks * 32 + lg * 8);
  }

  float4_t oacc[DT][NT];
  float mrow[NT], lrow[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    mrow[nt] = -INFINITY;
    lrow[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
  }

  const int kv_end = off + min(q0 + BM, Tn);
  const int n_tiles = (kv_end + BN - 1) / BN;
  // With a sliding window W the workgroup visits the tiles holding the S sink
  // keys, then the tiles from the one holding its first row's oldest visible
  // key; the tiles in between are never read.  Without a window: all tiles.
  const int W = a.window, S = a.sink;
  int sink_tiles = 0, win_tile0 = 0;
  if (W > 0) {
    sink_tiles = min((S + BN - 1) / BN, n_tiles);
    win_tile0 = max(sink_tiles, max(0, off + q0 - W + 1) / BN);
  }
  const int n_iter = sink_tiles + (n_tiles - win_tile0);
  auto tile_of = [&](int it) { return it < sink_tiles ? it : it - sink_tiles + win_tile0; };

  u32x4 kreg[KCH];
  u32x4 vreg[4];
  const int v_kg = stid % (BN / 4);
  const int v_ds = stid / (BN / 4);

  // Global loads of one K/V tile into registers.  Keys past T are clamped to
  // the last key (always in bounds) and masked in the scores, so the loads
  // carry no per-lane branches.
  auto load_tile = [&](int j) {
    const int k0 = j * BN;
    if (stage_k) {
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int idx = c * 256 + stid;
        const int key = min(k0 + idx / (D / 8), last_key);
        kreg[c] = *(const u32x4 *)(kb + row_of(key) * D + (idx % (D / 8)) * 8);
      }
    }
    if (stage_v) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = min(k0 + 4 * v_kg + r, last_key);
        vreg[r] = *(const u32x4 *)(vb + row_of(key) * D + v_ds * 8);
      }
    }
  };

  // Registers -> LDS (V transposed); the rows of this workgroup's own query
  // range also go to the cache (bit copies), by the first query head of
  // each KV group.
  auto store_tile = [&](int j, int buf) {
    const int k0 = j * BN;
    T *Ks = smem + buf * LDS::BUF;
    T *Vt = Ks + LDS::K_ELEMS;
    const bool to_cache = a.write_cache && writer && k0 + BN > q0;  // workgroup-uniform
    if (stage_k) {
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int idx = c * 256 + stid;
        *(u32x4 *)(Ks + (idx / (D / 8)) * LDS::KSTR + (idx % (D / 8)) * 8) = kreg[c];
      }
      if (to_cache) {
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
          const int idx = c * 256 + stid;
          const int key = k0 + idx / (D / 8);
          if (key >= q0 && key < Tn) *(u32x4 *)(ckb + (size_t)key * D + (idx % (D / 8)) * 8) = kreg[c];
        }
      }
    }
    if (stage_v) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t r0 = vreg[0][w], r1 = vreg[1][w];
        const uint32_t r2 = vreg[2][w], r3 = vreg[3][w];
        u32x2 out;
        if (e & 1) {
          out[0] = (r0 >> 16) | (r1 & 0xffff0000u);
          out[1] = (r2 >> 16) | (r3 & 0xffff0000u);
        } else {
          out[0] = (r0 & 0xffffu) | (r1 << 16);
          out[1] = (r2 & 0xffffu) | (r3 << 16);
        }
        *(u32x2 *)(Vt + (v_ds * 8 + e) * LDS::VSTR + 4 * v_kg) = out;
      }
      if (to_cache) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = k0 + 4 * v_kg + r;
          if (key >= q0 && key < Tn) *(u32x4 *)(cvb + (size_t)key * D + v_ds * 8) = vreg[r];
        }
      }
    }
  };

  load_tile(tile_of(0));
  store_tile(tile_of(0), 0);
  __syncthreads();

  const float c = a.scale_log2;
  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_iter) load_tile(tile_of(it + 1));
    // keep the next tile's loads ahead of this tile's math
    __builtin_amdgcn_sched_barrier(0);

    const int k0 = tile_of(it) * BN;
    // wave-uniform: skip a tile no row of the wave sees (past the diagonal, or
    // wholly older than every row's window and not a sink tile)
    const bool seen = k0 <= off + qw0 + QW - 1 && !(W > 0 && k0 >= S && k0 + BN - 1 <= off + qw0 - W);
    if (seen) {
      const T *Ks = smem + buf * LDS::BUF;
      const T *Vt = Ks + LDS::K_ELEMS;
      float4_t s[KT][NT];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) s[kt][nt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
          const vec8 ka = *(const vec8 *)(Ks + (kt * 16 + l16) * LDS::KSTR + ks * 32 + lg * 8);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) s[kt][nt] = Mfma<T>::mma(ka, qf[nt][ks], s[kt][nt]);
        }
      }
      // mask (diagonal tiles, and tiles at the lower edge of a window): lane
      // holds S^T[key = k0 + 16kt + 4lg + i][query = qw0 + 16nt + l16]
      const bool diag = k0 + BN - 1 > off + qw0;
      const bool edge = W > 0 && k0 + BN > S && k0 <= off + qw0 + QW - 1 - W;
      if (diag || edge) {
        asm volatile("" ::);  // rare tiles only: keep it a real branch
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = k0 + kt * 16 + lg * 4 + i;
              const int qr = off + qw0 + nt * 16 + l16;
              if (key > qr || (W > 0 && key <= qr - W && key >= S)) s[kt][nt][i] = -INFINITY;
            }
      }
      // online softmax per query column
      vec8 pb[PS][NT];
      vec8 pl[Mfma<T>::kSplitP ? PS : 1][NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        float mx = s[0][nt][0];
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kt][nt][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mx2 = mx * c;
        // m stays -inf while a row has seen no visible key (possible under a
        // window); the -inf guards keep such rows at p = 0 instead of NaN
        if (__any(mx2 > mrow[nt] + kLazyMax)) {
          asm volatile("" ::);  // rare: keep it a real branch
          const float mn = fmaxf(mrow[nt], mx2);
          const float al = fast_exp2(mrow[nt] - (mn == -INFINITY ? 0.f : mn));
          mrow[nt] = mn;
          lrow[nt] *= al;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) oacc[dt][nt] *= al;
        }
        const float mn = mrow[nt] == -INFINITY ? 0.f : mrow[nt];
        float ls = 0.f;
        if constexpr (Mfma<T>::kSplitP) {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float p = fast_exp2(fmaf(s[kt][nt][i], c, -mn));
              const T hi = (T)p;
              ls += p;
              pb[kt >> 1][nt][(kt & 1) * 4 + i] = hi;
              pl[kt >> 1][nt][(kt & 1) * 4 + i] = (T)(p - (float)hi);
            }
          }
        } else {
#pragma unroll
          for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              pb[kt >> 1][nt][(kt & 1) * 4 + i] = (T)fast_exp2(fmaf(s[kt][nt][i], c, -mn));
          }
          // the row sum is taken over the same rounded P that enters the MFMA
#pragma unroll
          for (int ps = 0; ps < PS; ++ps) ls = Mfma<T>::sum8(pb[ps][nt], ls);
        }
        lrow[nt] += ls;
      }
      // O^T += V^T P^T ; A operand: V^T[d][keys of this lane's k-slots]
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const T *vrow = Vt + (dt * 16 + l16) * LDS::VSTR + ps * 32 + lg * 4;
          const u32x2 lo = *(const u32x2 *)vrow;
          const u32x2 hi = *(const u32x2 *)(vrow + 16);
          const u32x4 raw = {lo[0], lo[1], hi[0], hi[1]};
          const vec8 va = __builtin_bit_cast(vec8, raw);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            oacc[dt][nt] = Mfma<T>::mma(va, pb[ps][nt], oacc[dt][nt]);
            if constexpr (Mfma<T>::kSplitP) oacc[dt][nt] = Mfma<T>::mma(va, pl[ps][nt], oacc[dt][nt]);
          }
        }
      }
    }

    if (it + 1 < n_iter) store_tile(tile_of(it + 1), buf ^ 1);
    __syncthreads();
  }

  // normalise and store: lane holds O^T[d = 16dt + 4lg + i][query = qw0 + 16nt + l16]
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float lt = lrow[nt] + __shfl_xor(lrow[nt], 16);
    lt += __shfl_xor(lt, 32);
    const float inv = 1.0f / lt;
    const int qr = qw0 + nt * 16 + l16;
    if (qr < Tn) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        store4(a.o, ((size_t)bh * Tn + qr) * D + dt * 16 + lg * 4, oacc[dt][nt], inv, a.o_dt);
    }
  }
}

// ---------------------------------------------------------------- pipelined kernel
// Software-pipelined variant: while the vector ALUs turn the scores of
// tile j into P (max, exp2, rounding, row sums), the matrix cores already
// compute the scores of tile j+1; then P_j V_j runs.  K and V live in separate
// two-deep LDS rings: iteration j reads K_{j+1} and V_j and stages K_{j+2} and
// V_{j+1}, so a single barrier per tile suffices.  The rare branches (lazy
// rescale of O, the causal mask of a wave's diagonal tiles) sit between the
// overlapped blocks.
//
// Both products run on v_mfma_f32_32x32x16_{f16,bf16} (bf16 carries P as hi +
// lo parts, two P V MFMAs), whose 32 output columns are a
// wave's 32 query rows: S^T = K Q^T (two 32-key blocks per 64-key tile, eight
// k-steps over D = 128) and O^T += V^T P^T (four 32-wide d-blocks, four
// 16-key k-steps).  A lane then holds one query column (lanes l and l ^ 32 the
// same one), so the row maximum and sum take one permlane32 swap, and a lane's
// scores of k-step ps are already its P^T operand of that step: the MFMA's
// k-index 8 hh + i stands for key 16 ps + 8 (i / 4) + 4 hh + i % 4, and the
// V^T operand is read with the same key order (two 8-byte LDS reads).  Half
// as many matrix instructions as with the 16x16x32 shape, and per-lane row
// statistics for one query instead of two.
template <int D, int BN>
struct PipeLds {
  static constexpr int KSTR = D + 8;   // K row stride (elements)
  static constexpr int VSTR = BN + 4;  // V^T row stride (elements)
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr size_t STAGE_BYTES = (size_t)(2 * K_ELEMS + 2 * V_ELEMS) * 2;
  // the output rows of the 8 waves (32 each, 16-byte padded) staged at the end
  static constexpr size_t out_bytes(int esz) { return (size_t)8 * 32 * (D * esz + 16); }
  static constexpr size_t bytes(int out_esz) {
    return STAGE_BYTES > out_bytes(out_esz) ? STAGE_BYTES : out_bytes(out_esz);
  }
  static constexpr size_t MAX_BYTES = bytes(4);
};

typedef float float16v_t __attribute__((ext_vector_type(16)));
__device__ __forceinline__ float16v_t mma32(const half8_t &a, const half8_t &b, const float16v_t &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float16v_t mma32(const bf168_t &a, const bf168_t &b, const float16v_t &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// x combined over lanes l and l ^ 32 (the two lanes holding one query column)
template <bool MAX>
__device__ __forceinline__ float across_h(float x) {
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return MAX ? fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1])) : __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Output of one wave of the pipelined kernel: its O^T accumulators (lane l
// holds query l % 32, head dims 32 db + 8 g + 4 (l / 32) + i), scaled by
// `inv` and rounded to OT, are written row-major into the wave's own region
// of the (idle) LDS, with a 16-byte pad per row, then read back so that each
// store instruction writes whole rows of D elements: 16-byte pieces of 32
// different rows had each been written as a separate partial line.
template <typename OT, int D>
__device__ __forceinline__ void store_rows_via_lds(unsigned char *smem, int wave, int lane,
                                                   const float16v_t (&oacc)[D / 32], float inv, OT *o,
                                                   size_t row0, int valid) {
  constexpr int DB = D / 32;
  constexpr int VPC = 16 / (int)sizeof(OT);  // elements per 16-byte chunk
  constexpr int STR = D + VPC;               // row stride (elements)
  constexpr int CPR = D / VPC;               // chunks per row
  constexpr int RPI = 64 / CPR;              // rows per store instruction
  static_assert(RPI >= 1 && 64 % CPR == 0, "a row must fit one wave's chunks");
  OT *buf = reinterpret_cast<OT *>(smem) + (size_t)wave * 32 * STR;
  const int l32 = lane & 31, hh = lane >> 5;
  typedef OT ot4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      ot4 x;
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (OT)(oacc[db][4 * g4 + i] * inv);
      *(ot4 *)(buf + l32 * STR + db * 32 + 8 * g4 + 4 * hh) = x;
    }
  __syncthreads();
#pragma unroll
  for (int r0 = 0; r0 < 32; r0 += RPI) {
    const int r = r0 + lane / CPR;
    const int c = lane % CPR;
    if (r < valid) *(u32x4 *)(o + (row0 + r) * D + c * VPC) = *(const u32x4 *)(buf + r * STR + c * VPC);
  }
}

// SPLIT: the grid runs the item table of a prompt whose heavier query tiles
// are split (a separate instance, so that other prompts keep the registers
// of the plain schedule).
template <typename T, int D, int BN, bool SPLIT = false>
__global__ __launch_bounds__(512, 1) void prefill_pipe_kernel(PrefillArgs a) {
  typedef typename Mfma<T>::vec vec8;
  constexpr bool SPL = Mfma<T>::kSplitP;
  typedef PipeLds<D, BN> LDS;
  constexpr int NW = 8, QW = 32;
  constexpr int BM = NW * QW;
  constexpr int KB = BN / 32;    // key blocks of 32 per tile
  constexpr int KS = D / 16;     // score k-steps over D
  constexpr int DB = D / 32;     // output d-blocks
  constexpr int PS = BN / 16;    // P V k-steps over keys
  constexpr int KCH = BN * D / 8 / 256;
  constexpr int VPAIRS = (BN / 4) * (D / 8);
  static_assert(KCH >= 1 && KCH <= 4 && BN * D / 8 == KCH * 256, "K tile: 1-4 chunks per staging thread");
  static_assert(VPAIRS <= 256 && VPAIRS % 64 == 0, "V tile must cover whole waves");

  extern __shared__ __align__(16) unsigned char smem_raw[];
  T *const Kbuf = reinterpret_cast<T *>(smem_raw);
  T *const Vbuf = Kbuf + 2 * LDS::K_ELEMS;

  const int Tn = a.T;
  const int H = a.q_heads;
  const int G = H / a.kv_heads;
  const int n_qt = (Tn + BM - 1) / BM;
  const int BH = a.batch * H;
  // heaviest query tiles of all heads first (from the item table when heavy
  // tiles are split).  (Giving each XCD all query tiles of one head at a
  // time, so that they share its L2, measured 3.5 % slower at T = 8192, 32
  // heads.)
  const int item = (int)(blockIdx.x / BH);
  const int qt = SPLIT ? (int)a.item_qt[item] : n_qt - 1 - item;
  const int part = SPLIT ? (int)a.item_part[item] : 0;
  const int bh = blockIdx.x % BH;
  const int b = bh / H;
  const int h = bh - b * H;
  const int g = h / G;
  const bool writer = (h - g * G) == 0;

  uint64_t clk0 = 0, rt0 = 0;
  if (a.clock_sample && blockIdx.x == 0 && threadIdx.x == 0) {
    clk0 = __builtin_amdgcn_s_memtime();
    rt0 = __builtin_amdgcn_s_memrealtime();
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * QW;
  const int off = a.offsets ? a.offsets[b] : 0;
  // an extend past the sequence's capacity (only on a replayed graph) is
  // left to the copy and length kernels to skip; no output row is written
  if (a.offsets && off + Tn > seq_capacity(a.slot_blocks, b, a.block_log2, a.max_T)) return;
  const int dlo = (off + qw0) / BN;
  const int dhi = (off + qw0 + QW - 1) / BN;
  const int stid = tid & 255;
  const bool stage_k = tid < 256;

  const T *qb = (const T *)a.q + (size_t)bh * Tn * D;
  const T *kb = (const T *)a.k + (size_t)(b * a.kv_heads + g) * a.kv_rows * D;
  const T *vb = (const T *)a.v + (size_t)(b * a.kv_heads + g) * a.kv_rows * D;
  T *ckb = (T *)a.cache_k + (size_t)(b * a.kv_heads + g) * a.max_T * D;
  T *cvb = (T *)a.cache_v + (size_t)(b * a.kv_heads + g) * a.max_T * D;
  const bool writer_c = writer && a.write_cache;
  if (a.write_cache && qt == 0 && h == 0 && tid == 0) a.len[b] = Tn;

  // Q^T fragments (B operand): lane holds Q[qw0 + l32][16 ks + 8 hh .. + 7]
  vec8 qf[KS];
  {
    const int row = min(qw0 + l32, Tn - 1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const vec8 *)(qb + (size_t)row * D + ks * 16 + hh * 8);
  }
  float16v_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[db][j] = 0.f;
  float mrow = -INFINITY, lrow = 0.f;

  const int kv_end = off + min(q0 + BM, Tn);
  const int n_tiles = (kv_end + BN - 1) / BN;
  // key tiles [t0, t1) of this workgroup: all, or one half of a split tile
  // (the first half lies below every query row of the tile, so only the
  // second holds diagonal tiles)
  const int t0 = part == 2 ? n_tiles / 2 : 0;
  const int t1 = part == 1 ? n_tiles / 2 : n_tiles;

  u32x4 sreg[4];
  const int v_kg = stid % (BN / 4);
  const int v_ds = stid / (BN / 4);
  const int slab_bytes = (off + Tn) * D * (int)sizeof(T);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void *)kb, (short)0, slab_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void *)vb, (short)0, slab_bytes, 0x00020000);
  const int k_voff = ((stid / (D / 8)) * D + (stid % (D / 8)) * 8) * (int)sizeof(T);
  const int v_voff = ((4 * v_kg) * D + v_ds * 8) * (int)sizeof(T);
  auto load_k = [&](int t) {
    if (stage_k) {
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int soff = (t * BN + c * (256 / (D / 8))) * D * (int)sizeof(T);
        sreg[c] = __builtin_amdgcn_raw_buffer_load_b128(krs, k_voff, soff, 0);
      }
    }
  };
  // waves 4-7 stage V, (4-key group, 8-column slice) pairs of the tile
  const bool stage_v = !stage_k && stid < VPAIRS;
  auto load_v = [&](int t) {
    if (stage_v) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        sreg[r] = __builtin_amdgcn_raw_buffer_load_b128(vrs, v_voff + r * D * (int)sizeof(T), t * BN * D * (int)sizeof(T), 0);
    }
  };
  auto store_k = [&](int t, int slot) {
    if (stage_k) {
      T *Ks = Kbuf + slot * LDS::K_ELEMS;
#pragma unroll
      for (int c = 0; c < KCH; ++c) {
        const int idx = c * 256 + stid;
        *(u32x4 *)(Ks + (idx / (D / 8)) * LDS::KSTR + (idx % (D / 8)) * 8) = sreg[c];
      }
      if (writer_c && t * BN + BN > q0) {
#pragma unroll
        for (int c = 0; c < KCH; ++c) {
          const int idx = c * 256 + stid;
          const int key = t * BN + idx / (D / 8);
          if (key >= q0 && key < Tn) *(u32x4 *)(ckb + (size_t)key * D + (idx % (D / 8)) * 8) = sreg[c];
        }
      }
    }
  };
  auto store_v = [&](int t, int slot) {
    if (stage_v) {
      T *Vt = Vbuf + slot * LDS::V_ELEMS;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t r0 = sreg[0][w], r1 = sreg[1][w];
        const uint32_t r2 = sreg[2][w], r3 = sreg[3][w];
        u32x2 out;
        if (e & 1) {
          out[0] = (r0 >> 16) | (r1 & 0xffff0000u);
          out[1] = (r2 >> 16) | (r3 & 0xffff0000u);
        } else {
          out[0] = (r0 & 0xffffu) | (r1 << 16);
          out[1] = (r2 & 0xffffu) | (r3 << 16);
        }
        *(u32x2 *)(Vt + (v_ds * 8 + e) * LDS::VSTR + 4 * v_kg) = out;
      }
      if (writer_c && t * BN + BN > q0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = t * BN + 4 * v_kg + r;
          if (key >= q0 && key < Tn) *(u32x4 *)(cvb + (size_t)key * D + v_ds * 8) = sreg[r];
        }
      }
    }
  };

  // S^T (keys x queries) = K_t Q^T: lane holds S^T[key = 32 kb + 8 (j / 4) + 4 hh + j % 4][query = qw0 + l32]
  auto scores = [&](int slot, float16v_t (&s)[KB]) {
    const T *Ks = Kbuf + slot * LDS::K_ELEMS;
#pragma unroll
    for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[k2][j] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int k2 = 0; k2 < KB; ++k2) {
        const vec8 ka = *(const vec8 *)(Ks + (k2 * 32 + l32) * LDS::KSTR + ks * 16 + hh * 8);
        s[k2] = mma32(ka, qf[ks], s[k2]);
      }
    }
  };
  auto mask = [&](int t, float16v_t (&s)[KB]) {
#pragma unroll
    for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (t * BN + k2 * 32 + 8 * (j / 4) + 4 * hh + (j % 4) > off + qw0 + l32) s[k2][j] = -INFINITY;
  };
  const float c = a.scale_log2;
  auto stats = [&](float16v_t (&s)[KB], float &al) -> bool {
    float mx = s[0][0];
#pragma unroll
    for (int k2 = 0; k2 < KB; ++k2)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = fmaxf(mx, s[k2][j]);
    const float mx2 = across_h<true>(mx) * c;
    const bool resc = __any(mx2 > mrow + kLazyMax);
    const float mn = resc ? fmaxf(mrow, mx2) : mrow;
    al = fast_exp2(mrow - mn);
    mrow = mn;
    return resc;
  };
  // P for k-step ps: S elements 8 (ps % 2) .. + 7 of block ps / 2 -- the lane's
  // keys 16 ps + 8 (i / 4) + 4 hh + i % 4, matched by the V^T fragment below
  auto expo = [&](float16v_t (&s)[KB], vec8 (&pb)[PS], vec8 (&pl)[SPL ? PS : 1], float al) {
    float ls = 0.f;
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
      if constexpr (SPL) {
        // bf16 keeps 8 significand bits: P as hi + lo parts, the sum in fp32
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p = fast_exp2(fmaf(s[ps / 2][8 * (ps % 2) + i], c, -mrow));
          const T hi = (T)p;
          ls += p;
          pb[ps][i] = hi;
          pl[ps][i] = (T)(p - (float)hi);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) pb[ps][i] = (T)fast_exp2(fmaf(s[ps / 2][8 * (ps % 2) + i], c, -mrow));
        ls = Mfma<T>::sum8(pb[ps], ls);
      }
    }
    lrow = fmaf(lrow, al, ls);
  };
  // O^T += V_t^T P^T: A operand V^T[d = 32 db + l32][keys 16 ps + 4 hh + 0..3, 16 ps + 8 + 4 hh + 0..3]
  auto pv = [&](int slot, const vec8 (&pb)[PS], const vec8 (&pl)[SPL ? PS : 1]) {
    const T *Vt = Vbuf + slot * LDS::V_ELEMS;
#pragma unroll
    for (int ps = 0; ps < PS; ++ps) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const T *vrow = Vt + (db * 32 + l32) * LDS::VSTR + ps * 16 + hh * 4;
        const u32x2 lo = *(const u32x2 *)vrow;
        const u32x2 hi = *(const u32x2 *)(vrow + 8);
        const u32x4 raw = {lo[0], lo[1], hi[0], hi[1]};
        const vec8 va = __builtin_bit_cast(vec8, raw);
        oacc[db] = mma32(va, pb[ps], oacc[db]);
        if constexpr (SPL) oacc[db] = mma32(va, pl[ps], oacc[db]);
      }
    }
  };

  // LDS slot of key tile t: its parity counted from t0
  load_k(t0);
  load_v(t0);
  store_k(t0, 0);
  store_v(t0, 0);
  if (t0 + 1 < t1) {
    load_k(t0 + 1);
    store_k(t0 + 1, 1);
  }
  __syncthreads();

  float16v_t sa[KB], sb[KB];
  scores(0, sa);
  if (t0 >= dlo && t0 <= dhi) mask(t0, sa);

  auto step = [&](int j, float16v_t (&cur)[KB], float16v_t (&nxt)[KB]) {
    if (j + 2 < t1) load_k(j + 2);
    if (j + 1 < t1) load_v(j + 1);
    __builtin_amdgcn_sched_barrier(0);
    if (j <= dhi) {
      vec8 pb[PS];
      vec8 pl[SPL ? PS : 1];
      float al;
      __builtin_amdgcn_s_setprio(2);
      const bool any_resc = stats(cur, al);
      scores((j + 1 - t0) & 1, nxt);
      expo(cur, pb, pl, al);
      {
        constexpr int NMF = KB * KS;
        constexpr int VPM = (QW * BN / 64 * (SPL ? 5 : 3)) / NMF + 1;
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < NMF; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
          if (i + 4 < NMF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      if (any_resc) {
        asm volatile("" ::);
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db] *= al;
      }
      pv((j - t0) & 1, pb, pl);
      if (j + 1 >= dlo && j + 1 <= dhi) {
        int t = j + 1;
        asm volatile("" : "+v"(t));
        mask(t, nxt);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (j + 2 < t1) store_k(j + 2, (j - t0) & 1);
    if (j + 1 < t1) store_v(j + 1, (j + 1 - t0) & 1);
    __syncthreads();
  };
  for (int j = t0; j < t1; j += 2) {
    step(j, sa, sb);
    if (j + 1 < t1) step(j + 1, sb, sa);
  }

  // lane holds O^T[d = 32 db + 8 g + 4 hh + i][query = qw0 + l32]
  float lsum = across_h<false>(lrow);
  if (SPLIT && part != 0) {
    // one half of a split tile: publish this half's (m, l, O) rows, count it
    // in, and let the second half to finish merge the two.  The L2 is per
    // XCD, so the partials are written with device-scope stores (written
    // through to the level every XCD shares) and read back with device-scope
    // loads; each thread waits for its stores before the barrier after
    // which the half is counted (a device-scope atomic).
    const int si = qt - (n_qt - a.n_split);
    const size_t pair = (size_t)si * BH + bh;
    // each half's partial: per wave, NVAL values per lane (m, l, then the
    // lane's 16 DB accumulator elements), stored value-major so that a wave
    // writes (and the merging workgroup, whose lanes hold the same rows and
    // head dims, reads) 256 contiguous bytes per instruction
    constexpr int NVAL = 2 + 16 * DB;
    static_assert((size_t)NW * 64 * NVAL == prefill_split_half_floats(D), "workspace layout");
    float *mine = a.split_ws + ((pair * 2 + (part - 1)) * NW + wave) * NVAL * 64 + lane;
    const float *other = a.split_ws + ((pair * 2 + (2 - part)) * NW + wave) * NVAL * 64 + lane;
    __hip_atomic_store(mine, mrow, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(mine + 64, lsum, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k4 = 0; k4 < 16; ++k4)
        __hip_atomic_store(mine + (2 + db * 16 + k4) * 64, oacc[db][k4], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    __shared__ int s_last;
    if (tid == 0) {
      int32_t *cnt = a.split_cnt + pair;
      const int last = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1;
      if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last) return;
    // both halves hold a finite reference point (every wave visits at least
    // one key tile in each).  The two are combined in a fixed order, first
    // half then second, whichever finished last, so that the result does
    // not depend on the order the halves finished in.
    const bool first = part == 1;
    const float mo = __hip_atomic_load(other, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float lo = __hip_atomic_load(other + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float m1 = first ? mrow : mo, m2 = first ? mo : mrow;
    const float l1 = first ? lsum : lo, l2 = first ? lo : lsum;
    const float mn = fmaxf(m1, m2);
    const float a1 = fast_exp2(m1 - mn), a2 = fast_exp2(m2 - mn);
    lsum = fmaf(l1, a1, l2 * a2);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int k4 = 0; k4 < 16; ++k4) {
        const float uo = __hip_atomic_load(other + (2 + db * 16 + k4) * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float u1 = first ? oacc[db][k4] : uo, u2 = first ? uo : oacc[db][k4];
        oacc[db][k4] = fmaf(u1, a1, u2 * a2);
      }
  }
  // the loop's last barrier has freed the K/V buffers, which now stage each
  // wave's rows so that every store writes whole rows
  const float inv = 1.0f / lsum;
  const size_t orow0 = (size_t)bh * Tn + qw0;
  const int valid = Tn - qw0;
  if (a.o_dt == KVATTN_F32)
    store_rows_via_lds<float, D>(smem_raw, wave, lane, oacc, inv, (float *)a.o, orow0, valid);
  else
    store_rows_via_lds<T, D>(smem_raw, wave, lane, oacc, inv, (T *)a.o, orow0, valid);
  if (a.clock_sample && blockIdx.x == 0 && tid == 0) {
    const uint64_t clk1 = __builtin_amdgcn_s_memtime();
    const uint64_t rt1 = __builtin_amdgcn_s_memrealtime();
    a.clock_sample[0] = clk1 - clk0;
    a.clock_sample[1] = rt1 - rt0;
  }
}

// ---------------------------------------------------------------- fp32 path
// Vector-ALU kernel: one workgroup of four waves per (16-query tile, b, h).
// Four lanes per query row, each holding a contiguous quarter of the head
// dim, so a score is a quarter dot product per lane plus two in-quad DPP
// additions, and each lane accumulates its quarter of O.  Keys are staged in
// LDS in tiles of 4096 / D rows, every lane issuing its four 16-byte K and
// four V loads of a tile at once, with the next tile's loads in flight while
// the current one is folded in; each wave folds a quarter of every tile into
// its own (m, l, o) state, and the four states are merged at the end by the
// chunked-softmax rule (the prompts this kernel serves are short, so the work
// of one query tile is spread over four waves to cut its latency).
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  return x;
}
constexpr int kF32Waves = 4;
template <int D>
__global__ __launch_bounds__(64 * kF32Waves) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int NWF = kF32Waves, RPW = 16, LPQ = 4, DL = D / LPQ;
  constexpr int BNF = 4096 / D;       // keys per tile
  constexpr int KPW = BNF / NWF;      // keys of a tile per wave
  constexpr int C4 = D / 4;           // 16-byte chunks per row
  constexpr int NV = BNF * C4 / (64 * NWF);  // 16-byte loads per thread per tile, of K and of V
  static_assert(NV * 64 * NWF == BNF * C4, "tile chunks must cover the workgroup");
  // K/V tiles while streaming; the waves' (m, l, o) states for the final merge
  constexpr int STAGE_F = 2 * BNF * D, MERGE_F = NWF * 64 * (DL + 2);
  __shared__ float4_t lds4[(STAGE_F > MERGE_F ? STAGE_F : MERGE_F) / 4];
  float4_t(*Ks)[C4] = (float4_t(*)[C4])lds4;
  float4_t(*Vs)[C4] = (float4_t(*)[C4])(lds4 + BNF * C4);
  const int Tn = a.T;
  const int H = a.q_heads;
  const int G = H / a.kv_heads;
  const int n_qt = (Tn + RPW - 1) / RPW;
  const int BH = a.batch * H;
  const int qt = n_qt - 1 - (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int b = bh / H;
  const int h = bh - b * H;
  const int g = h / G;
  const bool writer = a.write_cache && (h - g * G) == 0;
  const int tid = (int)threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int q0 = qt * RPW;
  const int row = q0 + lane / LPQ;
  const int c0 = (lane % LPQ) * (DL / 4);  // this lane's first 16-byte chunk of the head dim

  const float *qb = (const float *)a.q + (size_t)bh * Tn * D;
  const int off = a.offsets ? a.offsets[b] : 0;  // absolute position of query row 0
  // an extend past the sequence's capacity (only on a replayed graph) is
  // left to the copy and length kernels to skip; no output row is written
  if (a.offsets && off + Tn > seq_capacity(a.slot_blocks, b, a.block_log2, a.max_T)) return;
  // with a block table, k/v are the paged pools and rows are looked up per key
  const float4_t *kb = (const float4_t *)a.k + (a.table ? 0 : (size_t)(b * a.kv_heads + g) * a.kv_rows * C4);
  const float4_t *vb = (const float4_t *)a.v + (a.table ? 0 : (size_t)(b * a.kv_heads + g) * a.kv_rows * C4);
  float4_t *ckb = (float4_t *)a.cache_k + (size_t)(b * a.kv_heads + g) * a.max_T * C4;
  float4_t *cvb = (float4_t *)a.cache_v + (size_t)(b * a.kv_heads + g) * a.max_T * C4;
  if (a.write_cache && qt == 0 && h == 0 && tid == 0) a.len[b] = Tn;

  float qr[DL], o[DL];
#pragma unroll
  for (int i = 0; i < DL; ++i) {
    qr[i] = row < Tn ? qb[(size_t)row * D + 4 * c0 + i] : 0.f;
    o[i] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float c = a.scale_log2;
  const int n_keys = off + Tn;
  const int kv_end = off + min(q0 + RPW, Tn);
  const int W = a.window, S = a.sink;
  const int pos = off + row;
  // the first tile at or after k that some row of the workgroup sees: tiles
  // older than every row's window and past the sink are never read
  const int lim = off + q0 - W;
  auto live = [&](int k) {
    return (W > 0 && k >= S && k + BNF - 1 <= lim) ? ((lim + 1) / BNF) * BNF : k;
  };
  // chunk ch = tid + 64 NWF n of a tile: key row ch / C4, 16-byte column ch % C4
  float4_t kr[NV], vr[NV];
  auto load = [&](int k0) {
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int ch = tid + 64 * NWF * n;
      const int key = min(k0 + ch / C4, n_keys - 1);  // in range; rows past the end are zeroed below
      const size_t rk = a.table ? paged_row(a.table, b, a.max_blocks, a.block_log2, a.kv_heads, g, key)
                                : (size_t)key;
      kr[n] = kb[rk * C4 + ch % C4];
      vr[n] = vb[rk * C4 + ch % C4];
    }
  };
  int k0 = live(0);
  if (k0 < kv_end) load(k0);
  while (k0 < kv_end) {
    __syncthreads();  // the previous tile's LDS reads are done
#pragma unroll
    for (int n = 0; n < NV; ++n) {
      const int ch = tid + 64 * NWF * n;
      const int key = k0 + ch / C4;
      const bool in = key < n_keys;
      const float4_t z = {0.f, 0.f, 0.f, 0.f};
      Ks[ch / C4][ch % C4] = in ? kr[n] : z;
      Vs[ch / C4][ch % C4] = in ? vr[n] : z;
      // this workgroup's own prompt rows go to the cache: a bit copy of what was loaded
      if (writer && in && key >= q0 && key < q0 + RPW) {
        ckb[(size_t)key * C4 + ch % C4] = kr[n];
        cvb[(size_t)key * C4 + ch % C4] = vr[n];
      }
    }
    const int k1 = live(k0 + BNF);
    if (k1 < kv_end) load(k1);  // in flight while this tile is folded in
    __syncthreads();
    const int kw = k0 + wave * KPW;  // this wave's keys: [kw, kw + KPW)
    if (kw <= off + q0 + RPW - 1) {  // wave-uniform: some row of the tile sees a key of the quarter
      float s[KPW];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < KPW; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int i4 = 0; i4 < DL / 4; ++i4) {
          const float4_t kx = Ks[wave * KPW + j][c0 + i4];
          acc = fmaf(qr[4 * i4], kx[0], acc);
          acc = fmaf(qr[4 * i4 + 1], kx[1], acc);
          acc = fmaf(qr[4 * i4 + 2], kx[2], acc);
          acc = fmaf(qr[4 * i4 + 3], kx[3], acc);
        }
        acc = quad_sum(acc);
        const int key = kw + j;
        const bool vis = key <= pos && (W == 0 || pos - key < W || key < S);
        s[j] = vis ? acc * c : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float mn = fmaxf(m, mx);
      const float ms = mn == -INFINITY ? 0.f : mn;  // no visible key yet: p = 0, not NaN
      const float al = fast_exp2(m - ms);
      l *= al;
#pragma unroll
      for (int i = 0; i < DL; ++i) o[i] *= al;
#pragma unroll
      for (int j = 0; j < KPW; ++j) {
        const float p = fast_exp2(s[j] - ms);
        l += p;
#pragma unroll
        for (int i4 = 0; i4 < DL / 4; ++i4) {
          const float4_t vx = Vs[wave * KPW + j][c0 + i4];
          o[4 * i4] = fmaf(p, vx[0], o[4 * i4]);
          o[4 * i4 + 1] = fmaf(p, vx[1], o[4 * i4 + 1]);
          o[4 * i4 + 2] = fmaf(p, vx[2], o[4 * i4 + 2]);
          o[4 * i4 + 3] = fmaf(p, vx[3], o[4 * i4 + 3]);
        }
      }
      m = mn;
    }
    k0 = k1;
  }
  // merge the waves' states: m = max_w m_w, l = sum_w l_w 2^(m_w - m), o likewise
  __syncthreads();  // the last tile's LDS reads are done
  float *mf = (float *)lds4;  // [NWF][64] m, then [NWF][64] l, then [NWF][DL][64] o
  float *lf = mf + NWF * 64;
  float *of = lf + NWF * 64;
  if (wave > 0) {
    mf[wave * 64 + lane] = m;
    lf[wave * 64 + lane] = l;
#pragma unroll
    for (int i = 0; i < DL; ++i) of[(wave * DL + i) * 64 + lane] = o[i];
  }
  __syncthreads();
  if (wave == 0 && row < Tn) {
    float mw[NWF];
    mw[0] = m;
    float mt = m;
#pragma unroll
    for (int w = 1; w < NWF; ++w) {
      mw[w] = mf[w * 64 + lane];
      mt = fmaxf(mt, mw[w]);
    }
    // every row sees at least its own key, so mt is finite
    float sc[NWF];
#pragma unroll
    for (int w = 0; w < NWF; ++w) sc[w] = fast_exp2(mw[w] - mt);
    float lt = l * sc[0];
#pragma unroll
    for (int w = 1; w < NWF; ++w) lt = fmaf(lf[w * 64 + lane], sc[w], lt);
    const float inv = 1.0f / lt;
    float *ob = (float *)a.o + ((size_t)bh * Tn + row) * D + 4 * c0;
#pragma unroll
    for (int i = 0; i < DL; ++i) {
      float acc = o[i] * sc[0];
#pragma unroll
      for (int w = 1; w < NWF; ++w) acc = fmaf(of[(w * DL + i) * 64 + lane], sc[w], acc);
      ob[i] = acc * inv;
    }
  }
}

// Tile configurations, chosen by measurement on MI355X: the pipelined kernel
// (8 waves of 32 query rows, 32x32x16 MFMA) for f16 at every head dim and for
// bf16 at D = 64 and 128, with 64-key tiles at D = 64 and 128 and 128-key
// tiles at D = 32 (against the plain kernel: B = 4, 12 heads, T = 2048,
// D = 64: 65 against 76 us in f16, 78 against 90 us in bf16; T = 8192,
// 16 heads, D = 32: 155 against 165 us; T = 8192, 32 heads, D = 128 in
// bf16: 815 against 878 us).  bf16 at D = 32, whose two-part P would spill
// heavily with 128-key tiles, takes the plain kernel (4 waves of 32 rows).
template <typename T, int D>
struct PrefillConfig {
  static constexpr bool kPipe = std::is_same<T, half_t>::value || D != 32;
  static constexpr int NW = kPipe ? 8 : 4;
  static constexpr int QW = 32;
  static constexpr int BN = D == 32 ? 128 : 64;
};

// Launch with `lds` bytes of dynamic LDS.  The kernel's maximum dynamic LDS
// attribute (`lds_max`, or `lds` when 0) is set once per device (bit d of
// `attr_done`; always for device ids past 63).
template <typename KernelT>
static hipError_t launch_with_lds(KernelT kern, dim3 grid, int threads, size_t lds, hipStream_t s,
                                  std::atomic<uint64_t> &attr_done, const PrefillArgs &a, size_t lds_max = 0) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(lds_max ? lds_max : lds));
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  kern<<<grid, threads, lds, s>>>(a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_extend_mfma(const PrefillArgs &a, hipStream_t s);

// The pipelined kernel's items for a prompt whose heavier query tiles are
// split (prefill_split_tiles): every query tile whole, except the n_split
// heaviest, each as its first and second half of key tiles; ordered by
// their key-tile counts, largest first (ties: later query tile first).
// Returns the item count (0: no split).
static int plan_split(PrefillArgs &a, int BM, int BN) {
  a.n_items = 0;
  a.n_split = 0;
  if (!a.split_ws || !a.split_cnt || a.offsets || a.window > 0) return 0;
  const int ns = prefill_split_tiles(a.T, a.q_heads);
  if (ns == 0) return 0;
  const int n_qt = (a.T + BM - 1) / BM;
  int size[kMaxPrefillItems], n = 0;
  for (int qt = n_qt - 1; qt >= 0; --qt) {
    const int nt = (min((qt + 1) * BM, a.T) + BN - 1) / BN;
    if (qt >= n_qt - ns) {
      a.item_qt[n] = (uint8_t)qt, a.item_part[n] = 2, size[n++] = nt - nt / 2;
      a.item_qt[n] = (uint8_t)qt, a.item_part[n] = 1, size[n++] = nt / 2;
    } else {
      a.item_qt[n] = (uint8_t)qt, a.item_part[n] = 0, size[n++] = nt;
    }
  }
  // insertion sort, stable: equal sizes keep the later query tile first
  for (int i = 1; i < n; ++i)
    for (int j = i; j > 0 && size[j] > size[j - 1]; --j) {
      std::swap(size[j], size[j - 1]);
      std::swap(a.item_qt[j], a.item_qt[j - 1]);
      std::swap(a.item_part[j], a.item_part[j - 1]);
    }
  a.n_split = ns;
  a.n_items = n;
  return n;
}

template <typename T, int D>
static hipError_t launch_mfma(const PrefillArgs &a_in, hipStream_t s) {
  typedef PrefillConfig<T, D> C;
  constexpr int BM = C::NW * C::QW;
  const int n_qt = (a_in.T + BM - 1) / BM;
  const dim3 grid((unsigned)n_qt * a_in.batch * a_in.q_heads);
  static std::atomic<uint64_t> attr_done{0};
  if constexpr (C::kPipe) {
    // the plain kernel takes the window mask, and prompts whose K/V slab does
    // not fit the 32-bit range of the pipelined kernel's buffer loads
    if (a_in.window > 0 || (size_t)a_in.T * D * sizeof(T) >= ((size_t)1 << 31)) return launch_extend_mfma<T, D>(a_in, s);
    PrefillArgs a = a_in;
    const int items = plan_split(a, BM, C::BN);
    if (items) {
      static std::atomic<uint64_t> attr_split{0};
      return launch_with_lds(prefill_pipe_kernel<T, D, C::BN, true>, dim3((unsigned)items * a.batch * a.q_heads),
                             C::NW * 64, PipeLds<D, C::BN>::bytes(a.o_dt == KVATTN_F32 ? 4 : 2), s, attr_split, a,
                             PipeLds<D, C::BN>::MAX_BYTES);
    }
    return launch_with_lds(prefill_pipe_kernel<T, D, C::BN>, grid, C::NW * 64,
                           PipeLds<D, C::BN>::bytes(a.o_dt == KVATTN_F32 ? 4 : 2), s, attr_done, a,
                           PipeLds<D, C::BN>::MAX_BYTES);
  } else {
    return launch_with_lds(prefill_mfma_kernel<T, D, C::QW, C::BN, C::NW>, grid, C::NW * 64,
                           PrefillLds<D, C::BN>::BYTES, s, attr_done, a_in);
  }
}

bool prefill_uses_split(kvattn_dtype dt, int head_dim) {
  return dt == KVATTN_F16 || (dt == KVATTN_BF16 && head_dim != 32);
}

template <int D>
static hipError_t launch_f32(const PrefillArgs &a, hipStream_t s) {
  const int n_qt = (a.T + 15) / 16;  // 16 query rows per workgroup
  prefill_f32_kernel<D><<<dim3((unsigned)n_qt * a.batch * a.q_heads), 64 * kF32Waves, 0, s>>>(a);
  return hipGetLastError();
}

// Extend (queries after a cached prefix, K/V read from the cache): the
// pipelined kernel where the prompt uses it (16-bit types; no window, no block
// table), else the plain kernel for every 16-bit type and head dim, the vector
// kernel for fp32.
template <typename T, int D>
static hipError_t launch_extend_mfma(const PrefillArgs &a, hipStream_t s) {
  typedef PrefillConfig<T, D> C;
  if constexpr (C::kPipe) {
    // the pipelined kernel over the contiguous cache (no window; the key slab
    // of one sequence and KV head within its buffer loads' 32-bit range)
    if (!a.table && a.window == 0 && (size_t)a.kv_rows * D * sizeof(T) < ((size_t)1 << 31)) {
      constexpr int PBM = C::NW * C::QW;
      const dim3 pgrid((unsigned)((a.T + PBM - 1) / PBM) * a.batch * a.q_heads);
      static std::atomic<uint64_t> attr_pipe{0};
      return launch_with_lds(prefill_pipe_kernel<T, D, C::BN>, pgrid, C::NW * 64,
                             PipeLds<D, C::BN>::bytes(a.o_dt == KVATTN_F32 ? 4 : 2), s, attr_pipe, a,
                             PipeLds<D, C::BN>::MAX_BYTES);
    }
  }
  constexpr int NW = 4, QW = 32, BN = D == 32 ? 128 : 64, BM = NW * QW;
  const int n_qt = (a.T + BM - 1) / BM;
  const dim3 grid((unsigned)n_qt * a.batch * a.q_heads);
  if (a.table) {
    static std::atomic<uint64_t> attr_paged{0};
    return launch_with_lds(prefill_mfma_kernel<T, D, QW, BN, NW, true>, grid, NW * 64, PrefillLds<D, BN>::BYTES, s,
                           attr_paged, a);
  }
  static std::atomic<uint64_t> attr_done{0};
  return launch_with_lds(prefill_mfma_kernel<T, D, QW, BN, NW>, grid, NW * 64, PrefillLds<D, BN>::BYTES, s,
                         attr_done, a);
}

hipError_t launch_extend_attention(const PrefillArgs &a, hipStream_t s) {
  if (a.dt == KVATTN_F32) {
    switch (a.head_dim) {
      case 32: return launch_f32<32>(a, s);
      case 64: return launch_f32<64>(a, s);
      case 128: return launch_f32<128>(a, s);
    }
  } else if (a.dt == KVATTN_F16) {
    switch (a.head_dim) {
      case 32: return launch_extend_mfma<half_t, 32>(a, s);
      case 64: return launch_extend_mfma<half_t, 64>(a, s);
      case 128: return launch_extend_mfma<half_t, 128>(a, s);
    }
  } else if (a.dt == KVATTN_BF16) {
    switch (a.head_dim) {
      case 32: return launch_extend_mfma<bf16_t, 32>(a, s);
      case 64: return launch_extend_mfma<bf16_t, 64>(a, s);
      case 128: return launch_extend_mfma<bf16_t, 128>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs &a, hipStream_t s) {
  if (a.dt == KVATTN_F32) {
    switch (a.head_dim) {
      case 32: return launch_f32<32>(a, s);
      case 64: return launch_f32<64>(a, s);
      case 128: return launch_f32<128>(a, s);
    }
  } else if (a.dt == KVATTN_F16) {
    switch (a.head_dim) {
      case 32: return launch_mfma<half_t, 32>(a, s);
      case 64: return launch_mfma<half_t, 64>(a, s);
      case 128: return launch_mfma<half_t, 128>(a, s);
    }
  } else if (a.dt == KVATTN_BF16) {
    switch (a.head_dim) {
      case 32: return launch_mfma<bf16_t, 32>(a, s);
      case 64: return launch_mfma<bf16_t, 64>(a, s);
      case 128: return launch_mfma<bf16_t, 128>(a, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace kvattn
