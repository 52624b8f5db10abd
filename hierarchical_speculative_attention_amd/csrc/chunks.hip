// Chunk-mean keys and query-to-chunk scores: the retrieval side of Force 2
// in the TriForce blog ("1. The Three Forces of TriForce": the target picks
// the most critical KV blocks by key-query similarity).  A block is
// summarised by the mean of its keys; the score of a block is the dot product
// of that mean with the draft query (summed over the query heads sharing the
// KV head).  Both kernels stream HBM once with 16-byte nontemporal loads: 16
// lanes cover one 256-byte row of 128 16-bit values.
#include "tf_internal.h"

namespace tfk {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void widen8(int dtype, u32x4 x, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned w = x[i];
    if (dtype == TF_DTYPE_BF16) {
      f[2 * i] = __uint_as_float(w << 16);
      f[2 * i + 1] = __uint_as_float(w & 0xFFFF0000u);
    } else {
      f[2 * i] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
      f[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
    }
  }
}

__device__ __forceinline__ unsigned pack2(int dtype, float lo, float hi) {
  unsigned short a, b;
  if (dtype == TF_DTYPE_BF16) {
    a = __builtin_bit_cast(unsigned short, (__bf16)lo);
    b = __builtin_bit_cast(unsigned short, (__bf16)hi);
  } else {
    a = __builtin_bit_cast(unsigned short, (_Float16)lo);
    b = __builtin_bit_cast(unsigned short, (_Float16)hi);
  }
  return (unsigned)a | ((unsigned)b << 16);
}

// ---------------------------------------------------------------------------
// a1: grid (ceil(max_chunks / 16), H, B); 16 lanes per chunk, 8 dims per lane.
// ---------------------------------------------------------------------------
template <int IN_DT>
__global__ __launch_bounds__(256) void chunk_keys_kernel(
    const uint16_t* __restrict__ K, const int64_t* __restrict__ kbase, const int32_t* __restrict__ kcap,
    const int32_t* __restrict__ klen, int32_t max_len, int32_t cs, const int32_t* __restrict__ chunk_begin,
    int32_t max_chunks, void* __restrict__ ck, const int64_t* __restrict__ cbase,
    const int32_t* __restrict__ ccap, int32_t out_dtype) {
  const int b = blockIdx.z, g = blockIdx.y;
  const int cap = kcap[b];
  const int n = min(max(klen[b], 0), min(cap, max_len));
  const int C = (n + cs - 1) / cs;
  const long cb = chunk_begin ? max(chunk_begin[b], 0) : 0;
  const long c_end = min((long)C, cb + max_chunks);
  const long cl = cb + (long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int part = threadIdx.x & 15;
  if (cl >= c_end || cl >= ccap[b]) return;
  const int c = (int)cl;
  const int lo = c * cs, hi = min(n, lo + cs);
  const uint16_t* src = K + kbase[b] + ((size_t)g * cap + lo) * kHeadDim + 8 * part;
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // rows in batches of 8 loads issued together (row index clamped into the
  // chunk, surplus rows not added), summed in row order
  const int rows = hi - lo;
  for (int t0 = 0; t0 < rows; t0 += 8) {
    u32x4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      x[u] = __builtin_nontemporal_load((const u32x4*)(src + (size_t)min(t0 + u, rows - 1) * kHeadDim));
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (t0 + u < rows) {
        float f[8];
        widen8(IN_DT, x[u], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) s[j] += f[j];
      }
    }
  }
  const float cnt = (float)(hi - lo);
#pragma unroll
  for (int j = 0; j < 8; ++j) s[j] = s[j] / cnt;
  const size_t orow = (size_t)cbase[b] + ((size_t)g * ccap[b] + c) * kHeadDim + 8 * part;
  if (out_dtype == TF_DTYPE_FP32) {
    float* dst = (float*)ck + orow;
    *(f32x4*)dst = f32x4{s[0], s[1], s[2], s[3]};
    *(f32x4*)(dst + 4) = f32x4{s[4], s[5], s[6], s[7]};
  } else {
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack2(out_dtype, s[2 * i], s[2 * i + 1]);
    *(u32x4*)((uint16_t*)ck + orow) = o;
  }
}

hipError_t launch_chunk_keys(const uint16_t* K, const tf_kv_desc& kv, int32_t cs,
                             const int32_t* chunk_begin, int32_t max_chunks,
                             void* ck, const tf_kv_desc& ckd, hipStream_t stream) {
  const dim3 grid((max_chunks + 15) / 16, kv.H, kv.B), block(256);
  if (kv.dtype == TF_DTYPE_BF16)
    hipLaunchKernelGGL(chunk_keys_kernel<TF_DTYPE_BF16>, grid, block, 0, stream, K, kv.seq_base, kv.seq_cap,
                       kv.seq_len, kv.max_len, cs, chunk_begin, max_chunks, ck, ckd.seq_base, ckd.seq_cap, ckd.dtype);
  else
    hipLaunchKernelGGL(chunk_keys_kernel<TF_DTYPE_FP16>, grid, block, 0, stream, K, kv.seq_base, kv.seq_cap,
                       kv.seq_len, kv.max_len, cs, chunk_begin, max_chunks, ck, ckd.seq_base, ckd.seq_cap, ckd.dtype);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a2: grid (ceil(c_max / (16 * kCPL)), H, B), 256 threads.  Each wave scores
// 4 * kCPL consecutive chunks; its load instruction i covers chunks
// 4 i .. 4 i + 3 of its range, 1 KB of contiguous memory (16 lanes per
// 256-byte key).  The 16 partial dot products of a key are reduced across
// its 16 lanes.
// ---------------------------------------------------------------------------
constexpr int kCPL = 4;  // keys per lane group (loads in flight together); 8 and 16 measured slower

template <int CK_DT>
__global__ __launch_bounds__(256) void score_kernel(
    const uint16_t* __restrict__ q, int32_t q_dtype, int32_t Hq, int32_t H, const void* __restrict__ ck,
    const int64_t* __restrict__ cbase, const int32_t* __restrict__ ccap, const int32_t* __restrict__ clen,
    int32_t c_max_len, float* __restrict__ scores, int32_t c_max) {
  const int b = blockIdx.z, g = blockIdx.y;
  const int G = Hq / H;
  const int part = threadIdx.x & 15;        // 16-byte piece of a 256-byte key
  const int grp = (threadIdx.x >> 4) & 3;   // key of the wave instruction
  const int w = threadIdx.x >> 6;
  const int cap = ccap[b];
  const int C = min(max(clen[b], 0), min(cap, c_max_len));
  // Group query: the sum of the G query heads' vectors (8 dims of it per lane).
  float qs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int h = 0; h < G; ++h) {
    float f[8];
    widen8(q_dtype, *(const u32x4*)(q + ((size_t)b * Hq + (size_t)g * G + h) * kHeadDim + 8 * part), f);
#pragma unroll
    for (int j = 0; j < 8; ++j) qs[j] += f[j];
  }
  const int c_wave = (blockIdx.x * 4 + w) * (4 * kCPL);  // first chunk of this wave
  float dot[kCPL];
  if (CK_DT == TF_DTYPE_FP32) {
#pragma unroll
    for (int i = 0; i < kCPL; ++i) {
      const int c = c_wave + 4 * i + grp;
      float acc = 0.f;
      if (c < C) {
        const float* row = (const float*)ck + (size_t)cbase[b] + ((size_t)g * cap + c) * kHeadDim + 8 * part;
        const f32x4 x0 = __builtin_nontemporal_load((const f32x4*)row);
        const f32x4 x1 = __builtin_nontemporal_load((const f32x4*)(row + 4));
        acc = qs[0] * x0[0] + qs[1] * x0[1] + qs[2] * x0[2] + qs[3] * x0[3];
        acc = fmaf(qs[4], x1[0], fmaf(qs[5], x1[1], fmaf(qs[6], x1[2], fmaf(qs[7], x1[3], acc))));
      }
      dot[i] = acc;
    }
  } else {
    u32x4 x[kCPL];
    // (a wave wholly past C -- padding of a shorter sequence -- loads nothing)
    const bool any = c_wave < C;
#pragma unroll
    for (int i = 0; i < kCPL; ++i) {
      x[i] = u32x4{0u, 0u, 0u, 0u};
      if (any) {  // chunks past C read chunk C - 1 (in bounds) and are masked below
        const int c = min(c_wave + 4 * i + grp, C - 1);
        x[i] = __builtin_nontemporal_load(
            (const u32x4*)((const uint16_t*)ck + (size_t)cbase[b] + ((size_t)g * cap + c) * kHeadDim + 8 * part));
      }
    }
#pragma unroll
    for (int i = 0; i < kCPL; ++i) {
      float f[8];
      widen8(CK_DT, x[i], f);
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = fmaf(qs[j], f[j], acc);
      dot[i] = (c_wave + 4 * i + grp < C) ? acc : 0.f;
    }
  }
#pragma unroll
  for (int i = 0; i < kCPL; ++i) {
    float v = dot[i];
    v += __shfl_xor(v, 8, 16);
    v += __shfl_xor(v, 4, 16);
    v += __shfl_xor(v, 2, 16);
    v += __shfl_xor(v, 1, 16);
    dot[i] = v;
  }
  // lane `part` of key group `grp` writes chunk c_wave + 4 part + grp
  if (part < kCPL) {
    float v = dot[0];
#pragma unroll
    for (int i = 1; i < kCPL; ++i)
      if (part == i) v = dot[i];
    const int c = c_wave + 4 * part + grp;
    if (c < c_max) scores[((size_t)b * H + g) * c_max + c] = (c < C) ? v : -__builtin_huge_valf();
  }
}

hipError_t launch_scores(const uint16_t* q, int32_t q_dtype, int32_t Hq, const void* ck,
                         const tf_kv_desc& ckd, float* scores, int32_t c_max, hipStream_t stream) {
  const dim3 grid((c_max + 16 * kCPL - 1) / (16 * kCPL), ckd.H, ckd.B), block(256);  // 4 waves x 4 keys x kCPL
  switch (ckd.dtype) {
    case TF_DTYPE_BF16:
      hipLaunchKernelGGL(score_kernel<TF_DTYPE_BF16>, grid, block, 0, stream, q, q_dtype, Hq, ckd.H, ck,
                         ckd.seq_base, ckd.seq_cap, ckd.seq_len, ckd.max_len, scores, c_max);
      break;
    case TF_DTYPE_FP16:
      hipLaunchKernelGGL(score_kernel<TF_DTYPE_FP16>, grid, block, 0, stream, q, q_dtype, Hq, ckd.H, ck,
                         ckd.seq_base, ckd.seq_cap, ckd.seq_len, ckd.max_len, scores, c_max);
      break;
    default:
      hipLaunchKernelGGL(score_kernel<TF_DTYPE_FP32>, grid, block, 0, stream, q, q_dtype, Hq, ckd.H, ck,
                         ckd.seq_base, ckd.seq_cap, ckd.seq_len, ckd.max_len, scores, c_max);
      break;
  }
  return hipGetLastError();
}

}  // namespace tfk
