// Decode: one query per (sequence, query head) over that sequence's whole
// cache prefix [0, len[b]).
//
// Inference chapter, section 9.1: decode re-reads the cached history every
// step and is limited by memory bandwidth, so this path is a streaming kernel
// on the vector ALUs (no matrix cores): K and V rows are read once per KV head
// with 16-byte loads, the G query heads that share a KV head (roadmap page,
// project 12, MQA/GQA) are served by the same workgroup, and long contexts
// are split across workgroups.  Each split keeps the online-softmax state
// (m, l, u) -- the chunked-attention recurrence of the README -- and a second
// kernel merges the splits by log-sum-exp.  Scores carry log2(e) inside the
// scale so that every exponential is a single exp2.
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

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = LPR / 2; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// grid (n_splits, Hkv * G/GT, B), 256 threads.  Workgroup = one split of
// `chunk` keys of one KV head, for GT query heads of its group.
template <class Tag, int D, int GT>
__global__ __launch_bounds__(256) void decode_partial_kernel(DecodeArgs a) {
  constexpr int EPL = Tag::EPL;
  constexpr int LPR = D / EPL;   // lanes that share one key row
  constexpr int RPW = 64 / LPR;  // key rows per wave per load
  constexpr int U = 8;           // loads in flight per lane and tensor
  constexpr int ESZ = Tag::bytes;

  const int b = blockIdx.z;
  const int split = blockIdx.x;
  const int G = a.q_heads / a.kv_heads;
  const int subs = G / GT;
  const int kvh = blockIdx.y / subs;
  const int h0 = kvh * G + (blockIdx.y - kvh * subs) * GT;
  const int L = a.len[b];
  const int kb = split * a.chunk;
  if (kb >= L) return;  // empty split: the merge only reads splits below L
  const int rows = min(a.chunk, L - kb);

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int rg = lane / LPR;
  const int cl = (lane % LPR) * EPL;

  const size_t head_off = (size_t)(b * a.kv_heads + kvh) * a.max_T * D;
  const char *Kb = (const char *)a.k_layer + (head_off + (size_t)kb * D + cl) * ESZ;
  const char *Vb = (const char *)a.v_layer + (head_off + (size_t)kb * D + cl) * ESZ;

  uint4 qv[GT];
#pragma unroll
  for (int g = 0; g < GT; ++g)
    qv[g] = *(const uint4 *)((const char *)a.q + ((size_t)(b * a.q_heads + h0 + g) * D + cl) * ESZ);

  float m[GT], l[GT], acc[GT][EPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    m[g] = -INFINITY;
    l[g] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;
  }

  const int steps = (rows + 4 * RPW - 1) / (4 * RPW);
  for (int s0 = 0; s0 < steps; s0 += U) {
    uint4 kr[U], vr[U];
    bool ok[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int r = ((s0 + u) * 4 + wave) * RPW + rg;
      ok[u] = r < rows;
      if (ok[u]) {
        kr[u] = *(const uint4 *)(Kb + (size_t)r * D * ESZ);
        vr[u] = *(const uint4 *)(Vb + (size_t)r * D * ESZ);
      } else {
        kr[u] = make_uint4(0, 0, 0, 0);
        vr[u] = make_uint4(0, 0, 0, 0);
      }
    }
    float sc[U][GT];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const float d = row_sum<LPR>(dot16(Tag{}, qv[g], kr[u]));
        sc[u][g] = ok[u] ? d * a.scale_log2 : -INFINITY;
      }
#pragma unroll
    for (int g = 0; g < GT; ++g) {
      float mx = sc[0][g];
#pragma unroll
      for (int u = 1; u < U; ++u) mx = fmaxf(mx, sc[u][g]);
      const float mn = fmaxf(m[g], mx);
      const float ms = (mn == -INFINITY) ? 0.f : mn;
      const float al = fast_exp2(m[g] - ms);
      l[g] *= al;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[g][e] *= al;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float p = fast_exp2(sc[u][g] - ms);
        l[g] += p;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(p, elem(Tag{}, vr[u], e), acc[g][e]);
      }
      m[g] = mn;
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
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[g][e], off);
        acc[g][e] = acc[g][e] * a1 + ao * a2;
      }
      m[g] = mn;
    }
  }

  // merge the four waves through LDS and write this split's (m, l, u)
  __shared__ float s_m[4][GT], s_l[4][GT];
  __shared__ float s_acc[4][GT][D];
  if (lane < LPR) {
#pragma unroll
    for (int g = 0; g < GT; ++g) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][g][cl + e] = acc[g][e];
      if (lane == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < GT * D; t += 256) {
    const int g = t / D;
    const int d = t - g * D;
    const float M = fmaxf(fmaxf(s_m[0][g], s_m[1][g]), fmaxf(s_m[2][g], s_m[3][g]));
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float al = fast_exp2(s_m[w][g] - M);
      num = fmaf(al, s_acc[w][g][d], num);
      den = fmaf(al, s_l[w][g], den);
    }
    float *dst = a.ws + ((size_t)(b * a.q_heads + h0 + g) * a.n_splits + split) * (D + 2);
    dst[2 + d] = num;
    if (d == 0) {
      dst[0] = M;
      dst[1] = den;
    }
  }
}

__device__ __forceinline__ void store_out(void *o, size_t idx, float x, kvattn_dtype dt) {
  if (dt == KVATTN_F32)
    ((float *)o)[idx] = x;
  else if (dt == KVATTN_F16)
    ((half_t *)o)[idx] = (half_t)x;
  else
    ((bf16_t *)o)[idx] = (bf16_t)x;
}

// grid (H, B), D threads: log-sum-exp merge of the non-empty splits.
template <int D>
__global__ __launch_bounds__(128) void decode_merge_kernel(DecodeArgs a) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int L = a.len[b];
  const int ns = (L + a.chunk - 1) / a.chunk;
  const float *w = a.ws + (size_t)(b * a.q_heads + h) * a.n_splits * (D + 2);
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, w[(size_t)s * (D + 2)]);
  const int d = threadIdx.x;
  if (d >= D) return;
  float num = 0.f, den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const float *ws = w + (size_t)s * (D + 2);
    const float al = fast_exp2(ws[0] - M);
    den = fmaf(al, ws[1], den);
    num = fmaf(al, ws[2 + d], num);
  }
  store_out(a.o, (size_t)(b * a.q_heads + h) * D + d, num / den, a.o_dt);
}

template <class Tag, int D>
static hipError_t launch_typed(const DecodeArgs &a, hipStream_t s) {
  const int G = a.q_heads / a.kv_heads;
  const int GT = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 3 == 0) ? 3 : (G % 2 == 0) ? 2 : 1;
  const dim3 grid(a.n_splits, a.kv_heads * (G / GT), a.batch);
  switch (GT) {
    case 8: decode_partial_kernel<Tag, D, 8><<<grid, 256, 0, s>>>(a); break;
    case 4: decode_partial_kernel<Tag, D, 4><<<grid, 256, 0, s>>>(a); break;
    case 3: decode_partial_kernel<Tag, D, 3><<<grid, 256, 0, s>>>(a); break;
    case 2: decode_partial_kernel<Tag, D, 2><<<grid, 256, 0, s>>>(a); break;
    default: decode_partial_kernel<Tag, D, 1><<<grid, 256, 0, s>>>(a); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  decode_merge_kernel<D><<<dim3(a.q_heads, a.batch), dim3(D < 64 ? 64 : D), 0, s>>>(a);
  return hipGetLastError();
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

hipError_t launch_decode(const DecodeArgs &a, hipStream_t s) {
  switch (a.dt) {
    case KVATTN_F32: return launch_dim<TagF32>(a, s);
    case KVATTN_F16: return launch_dim<TagF16>(a, s);
    case KVATTN_BF16: return launch_dim<TagBF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvattn
