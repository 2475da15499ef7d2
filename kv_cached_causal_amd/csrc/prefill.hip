// Prefill: causal attention of a T-token prompt, with a bit-exact copy of the
// prompt's K and V into the layer's cache.
//
// Inference chapter, section 9.1: prefill is matrix-multiply shaped and
// builds the cache; section 9.7 (and the roadmap page's project 15): tiling
// with on-chip storage computes the same attention while never writing the
// T x T score matrix to device memory.  The README's chunked attention with
// the online-softmax recurrence is the algebra used here, tile by tile.
//
// gfx950 design (F16/BF16): a workgroup is 4 wave64s and owns BM = 4*QW query
// rows of one (b, h).  Each wave keeps its QW query rows in registers as MFMA
// operands and computes, per K/V tile of BN keys staged through LDS,
//     S^T = K Q^T   (v_mfma_f32_16x16x32_{f16,bf16}, fp32 accumulate)
//     O^T += V^T P^T
// The transposed orientation puts one query in one lane column for both
// products, so the running max / sum and the rescale of O stay per-lane; row
// statistics need only two cross-lane steps per tile.  V is transposed while
// it is staged to LDS so that its reduction axis (keys) is contiguous for the
// MFMA operand.  Tiles past the diagonal are never visited.  The workgroups
// that own the diagonal tile of the first query head of a KV group also
// store that K/V tile into the cache from the registers it was loaded into.
//
// F32 takes a plain vector-ALU kernel (one lane per query row).
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
  static constexpr int VSTR = BN + 8;  // V^T row stride (elements)
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr size_t BYTES = 2 * BUF * 2;  // two buffers of 2-byte elements
};

// 1-D grid over (q-tile, b, h), heaviest (last) query tiles first.
template <typename T, int D, int QW, int BN>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(PrefillArgs a) {
  typedef typename Mfma<T>::vec vec8;
  typedef PrefillLds<D, BN> LDS;
  constexpr int BM = 4 * QW;
  constexpr int NT = QW / 16;  // query sub-tiles per wave
  constexpr int KT = BN / 16;  // key sub-tiles per tile
  constexpr int KS = D / 32;   // MFMA k-steps over D
  constexpr int DT = D / 16;   // output sub-tiles over D
  constexpr int PS = BN / 32;  // MFMA k-steps over keys
  constexpr int KCH = BN * D / 8 / 256;  // 16-B K chunks per thread
  constexpr int VPAIRS = (BN / 4) * (D / 8);  // (4-key group, 8-column slice) pairs
  static_assert(KCH >= 1 && BN * D / 8 == KCH * 256, "K tile must split evenly");
  static_assert(VPAIRS <= 256, "V tile too large");

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

  const T *qb = (const T *)a.q + (size_t)bh * Tn * D;
  const T *kb = (const T *)a.k + (size_t)(b * a.kv_heads + g) * Tn * D;
  const T *vb = (const T *)a.v + (size_t)(b * a.kv_heads + g) * Tn * D;
  T *ckb = (T *)a.cache_k + (size_t)(b * a.kv_heads + g) * a.max_T * D;
  T *cvb = (T *)a.cache_v + (size_t)(b * a.kv_heads + g) * a.max_T * D;

  if (qt == 0 && h == 0 && tid == 0) a.len[b] = Tn;

  // query fragments (B operand of S^T = K Q^T): lane holds 8 columns of one row
  vec8 qf[NT][KS];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = qw0 + nt * 16 + l16;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (row < Tn)
        qf[nt][ks] = *(const vec8 *)(qb + (size_t)row * D + ks * 32 + lg * 8);
      else
        qf[nt][ks] = vec8{};
    }
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

  const int kv_end = min(q0 + BM, Tn);
  const int n_tiles = (kv_end + BN - 1) / BN;

  uint4 kreg[KCH];
  uint4 vreg[4];
  const int v_kg = tid % (BN / 4);
  const int v_ds = tid / (BN / 4);

  auto load_tile = [&](int j) {
    const int k0 = j * BN;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = c * 256 + tid;
      const int row = idx / (D / 8);
      const int col = (idx % (D / 8)) * 8;
      const int key = k0 + row;
      if (key < Tn) {
        kreg[c] = *(const uint4 *)(kb + (size_t)key * D + col);
        if (writer && key >= q0) *(uint4 *)(ckb + (size_t)key * D + col) = kreg[c];
      } else {
        kreg[c] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < VPAIRS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * v_kg + r;
        if (key < Tn) {
          vreg[r] = *(const uint4 *)(vb + (size_t)key * D + v_ds * 8);
          if (writer && key >= q0) *(uint4 *)(cvb + (size_t)key * D + v_ds * 8) = vreg[r];
        } else {
          vreg[r] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    T *Ks = smem + buf * LDS::BUF;
    T *Vt = Ks + LDS::K_ELEMS;
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      const int idx = c * 256 + tid;
      const int row = idx / (D / 8);
      const int col = (idx % (D / 8)) * 8;
      *(uint4 *)(Ks + row * LDS::KSTR + col) = kreg[c];
    }
    if (tid < VPAIRS) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        const uint32_t r0 = word4(vreg[0], w), r1 = word4(vreg[1], w);
        const uint32_t r2 = word4(vreg[2], w), r3 = word4(vreg[3], w);
        uint2 out;
        if (e & 1) {
          out.x = (r0 >> 16) | (r1 & 0xffff0000u);
          out.y = (r2 >> 16) | (r3 & 0xffff0000u);
        } else {
          out.x = (r0 & 0xffffu) | (r1 << 16);
          out.y = (r2 & 0xffffu) | (r3 << 16);
        }
        *(uint2 *)(Vt + (v_ds * 8 + e) * LDS::VSTR + 4 * v_kg) = out;
      }
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  const float c = a.scale_log2;
  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) load_tile(j + 1);

    const int k0 = j * BN;
    if (k0 <= qw0 + QW - 1) {  // wave-uniform: this tile has keys some row of the wave sees
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
      // causal mask: lane holds S^T[key = k0 + 16kt + 4lg + i][query = qw0 + 16nt + l16]
      if (k0 + BN - 1 > qw0) {
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = k0 + kt * 16 + lg * 4 + i;
              const int qr = qw0 + nt * 16 + l16;
              if (key > qr) s[kt][nt][i] = -INFINITY;
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
        // tile 0 holds key 0, visible to every row, so m is finite from then on
        const float mn = fmaxf(mrow[nt], mx * c);
        const float al = fast_exp2(mrow[nt] - mn);
        mrow[nt] = mn;
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
        lrow[nt] = fmaf(lrow[nt], al, ls);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt][nt] *= al;
      }
      // O^T += V^T P^T ; A operand: V^T[d][keys of this lane's k-slots]
#pragma unroll
      for (int ps = 0; ps < PS; ++ps) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const T *vrow = Vt + (dt * 16 + l16) * LDS::VSTR + ps * 32 + lg * 4;
          const uint2 lo = *(const uint2 *)vrow;
          const uint2 hi = *(const uint2 *)(vrow + 16);
          const uint4 raw = make_uint4(lo.x, lo.y, hi.x, hi.y);
          const vec8 va = __builtin_bit_cast(vec8, raw);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            oacc[dt][nt] = Mfma<T>::mma(va, pb[ps][nt], oacc[dt][nt]);
            if constexpr (Mfma<T>::kSplitP) oacc[dt][nt] = Mfma<T>::mma(va, pl[ps][nt], oacc[dt][nt]);
          }
        }
      }
    }

    if (j + 1 < n_tiles) store_tile(buf ^ 1);
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

// ---------------------------------------------------------------- fp32 path
// One wave per (64-query tile, b, h); lane = query row; keys staged in LDS in
// tiles of 32, each tile folded into the row's (m, l, o) state.
template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int BMF = 64, BNF = 32;
  __shared__ float Ks[BNF][D];
  __shared__ float Vs[BNF][D];
  const int Tn = a.T;
  const int H = a.q_heads;
  const int G = H / a.kv_heads;
  const int n_qt = (Tn + BMF - 1) / BMF;
  const int BH = a.batch * H;
  const int qt = n_qt - 1 - (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int b = bh / H;
  const int h = bh - b * H;
  const int g = h / G;
  const bool writer = (h - g * G) == 0;
  const int q0 = qt * BMF;
  const int row = q0 + threadIdx.x;

  const float *qb = (const float *)a.q + (size_t)bh * Tn * D;
  const float *kb = (const float *)a.k + (size_t)(b * a.kv_heads + g) * Tn * D;
  const float *vb = (const float *)a.v + (size_t)(b * a.kv_heads + g) * Tn * D;
  float *ckb = (float *)a.cache_k + (size_t)(b * a.kv_heads + g) * a.max_T * D;
  float *cvb = (float *)a.cache_v + (size_t)(b * a.kv_heads + g) * a.max_T * D;
  if (qt == 0 && h == 0 && threadIdx.x == 0) a.len[b] = Tn;

  float qr[D], o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qr[d] = row < Tn ? qb[(size_t)row * D + d] : 0.f;
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const float c = a.scale_log2;
  const int kv_end = min(q0 + BMF, Tn);
  for (int k0 = 0; k0 < kv_end; k0 += BNF) {
    __syncthreads();
    for (int i = threadIdx.x; i < BNF * D; i += 64) {
      const int r = i / D, d = i - r * D;
      const int key = k0 + r;
      float kx = 0.f, vx = 0.f;
      if (key < Tn) {
        kx = kb[(size_t)key * D + d];
        vx = vb[(size_t)key * D + d];
        if (writer && key >= q0) {
          // bit copy: reinterpret, never round
          ((uint32_t *)ckb)[(size_t)key * D + d] = __float_as_uint(kx);
          ((uint32_t *)cvb)[(size_t)key * D + d] = __float_as_uint(vx);
        }
      }
      Ks[r][d] = kx;
      Vs[r][d] = vx;
    }
    __syncthreads();
    float s[BNF];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) acc = fmaf(qr[d], Ks[j][d], acc);
      s[j] = (k0 + j <= row) ? acc * c : -INFINITY;
      mx = fmaxf(mx, s[j]);
    }
    const float mn = fmaxf(m, mx);
    const float al = fast_exp2(m - mn);
    l *= al;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] *= al;
#pragma unroll
    for (int j = 0; j < BNF; ++j) {
      const float p = fast_exp2(s[j] - mn);
      l += p;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] = fmaf(p, Vs[j][d], o[d]);
    }
    m = mn;
  }
  if (row < Tn) {
    const float inv = 1.0f / l;
    float *ob = (float *)a.o + ((size_t)bh * Tn + row) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) ob[d] = o[d] * inv;
  }
}

template <typename T, int D>
static hipError_t launch_mfma(const PrefillArgs &a, hipStream_t s) {
  constexpr int QW = 32, BN = 64, BM = 4 * QW;
  const size_t lds = PrefillLds<D, BN>::BYTES;
  static bool attr_done = false;
  if (!attr_done) {
    hipError_t e = hipFuncSetAttribute((const void *)prefill_mfma_kernel<T, D, QW, BN>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_done = true;
  }
  const int n_qt = (a.T + BM - 1) / BM;
  const dim3 grid((unsigned)n_qt * a.batch * a.q_heads);
  prefill_mfma_kernel<T, D, QW, BN><<<grid, 256, lds, s>>>(a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(const PrefillArgs &a, hipStream_t s) {
  const int n_qt = (a.T + 63) / 64;
  prefill_f32_kernel<D><<<dim3((unsigned)n_qt * a.batch * a.q_heads), 64, 0, s>>>(a);
  return hipGetLastError();
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
