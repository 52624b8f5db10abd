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

// Sum over each row of 16 lanes, every lane ending with its row's total:
// rotations of the row by 8, 4, 2 and 1 lanes (DPP row_ror operands, in
// registers; lane shuffles compile to LDS permutes).  At each step a lane's
// rotation partner holds the same value as its xor partner would, so the
// result is the same bits as the xor butterfly.
__device__ __forceinline__ float row16_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false));  // row_ror:8
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false));  // row_ror:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false));  // row_ror:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false));  // row_ror:1
  return x;
}

// ---------------------------------------------------------------------------
// a2, 16-bit chunk keys: workgroups of four waves; wave j of the grid scores
// blocks j, j + (waves in the grid), ... of 16 consecutive chunks (4 KB of
// keys) of its row, two blocks in flight.  Load instruction i of a block
// covers chunks 4 i .. 4 i + 3 of it, 1 KB of contiguous memory (16 lanes per
// 256-byte key); the 16 partial dot products of a key are reduced across its
// 16 lanes.  Keys are read through a buffer descriptor whose size is the
// row's C keys: a load past it returns zeros without touching memory, so
// every wave issues the same loads whatever C is, its waits stay exact, and a
// block of padding costs only its -inf stores.  The grid is capped at
// kScoreWgs workgroups: one block per wave for 32 rows of 16384 chunks or 8
// rows of 32768, several for a batch (a grid of one workgroup per 64 chunks of
// the longest row would be mostly padding for the shorter sequences and
// bound by the dispatch of its workgroups).
// ---------------------------------------------------------------------------
constexpr int kScoreWaves = 4;
constexpr int kScoreLoads = 4;                 // 16-byte loads per lane per block
constexpr int kScoreBlock = 4 * kScoreLoads;   // chunks per block
constexpr int kScoreWgs = 8192;

template <int CK_DT>
__global__ __launch_bounds__(kScoreWaves * 64) void score_kernel(
    const uint16_t* __restrict__ q, int32_t q_dtype, int32_t Hq, int32_t H, const uint16_t* __restrict__ ck,
    const int64_t* __restrict__ cbase, const int32_t* __restrict__ ccap, const int32_t* __restrict__ clen,
    int32_t c_max_len, float* __restrict__ scores, int32_t c_max) {
  const int b = blockIdx.z, g = blockIdx.y;
  const int G = Hq / H;
  const int part = threadIdx.x & 15;        // 16-byte piece of a 256-byte key
  const int grp = (threadIdx.x >> 4) & 3;   // key of the load instruction
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
  const uint16_t* keys = ck + (size_t)cbase[b] + (size_t)g * cap * kHeadDim;
  // raw buffer (stride 0, size in bytes); 0x00020000 is the descriptor's last
  // word on this target: 32-bit data format, no swizzle, no index
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)keys, (short)0, C * (int)(kHeadDim * sizeof(uint16_t)), 0x00020000);
  float* out = scores + ((size_t)b * H + g) * c_max;
  const int nblk = (c_max + kScoreBlock - 1) / kScoreBlock;
  const int stride = gridDim.x * kScoreWaves;
  const unsigned lane_off = (unsigned)grp * 256u + 16u * part;
  auto fetch = [&](int blk, u32x4 (&x)[kScoreLoads]) {
#pragma unroll
    for (int i = 0; i < kScoreLoads; ++i)  // (cache policy 2: nontemporal)
      x[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (unsigned)blk * (kScoreLoads * 1024u) + i * 1024u + lane_off,
                                                   0, 2);
  };
  auto score = [&](int blk, const u32x4 (&x)[kScoreLoads]) {
    float dot[kScoreLoads];
#pragma unroll
    for (int i = 0; i < kScoreLoads; ++i) {
      float f[8];
      widen8(CK_DT, x[i], f);
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) acc = fmaf(qs[j], f[j], acc);
      acc = row16_sum(acc);
      dot[i] = acc;
    }
    // lane `part` of key group `grp` writes chunk blk * kScoreBlock + 4 part + grp
    if (part < kScoreLoads) {
      float v = dot[0];
#pragma unroll
      for (int i = 1; i < kScoreLoads; ++i)
        if (part == i) v = dot[i];
      const int c = blk * kScoreBlock + 4 * part + grp;
      if (c < c_max) out[c] = (c < C) ? v : -__builtin_huge_valf();
    }
  };
  // The pipelined loop covers the blocks holding keys only; the blocks wholly
  // past C get their -inf in a second loop with no loads, so a short row's
  // padding does not wait on loads that return zero. The second batch is
  // fetched only when it exists (a wave with one block measured 0.4-1 us
  // slower per launch otherwise); the prefetch at the end of each step stays
  // unconditional (past the row it reads zeros that are never used, and
  // guarding it cost 9 registers and a wave per SIMD).
  const int nkey = min(nblk, (C + kScoreBlock - 1) / kScoreBlock);
  int blk = blockIdx.x * kScoreWaves + w;
  {
    u32x4 xa[kScoreLoads], xb[kScoreLoads];
    fetch(blk, xa);
    if (blk + stride < nkey) fetch(blk + stride, xb);
    while (true) {
      if (blk >= nkey) break;
      score(blk, xa);
      fetch(blk + 2 * stride, xa);
      blk += stride;
      if (blk >= nkey) break;
      score(blk, xb);
      fetch(blk + 2 * stride, xb);
      blk += stride;
    }
  }
  // (blk is now the wave's first block at or past nkey)
  if (part < kScoreLoads)
    for (; blk < nblk; blk += stride) {
      const int c = blk * kScoreBlock + 4 * part + grp;
      if (c < c_max) out[c] = -__builtin_huge_valf();
    }
}

// a2, fp32 chunk keys: grid (ceil(c_max / 64), H, B), 256 threads; each wave
// scores 16 consecutive chunks, 4 per lane group.
__global__ __launch_bounds__(256) void score_kernel_f32(
    const uint16_t* __restrict__ q, int32_t q_dtype, int32_t Hq, int32_t H, const float* __restrict__ ck,
    const int64_t* __restrict__ cbase, const int32_t* __restrict__ ccap, const int32_t* __restrict__ clen,
    int32_t c_max_len, float* __restrict__ scores, int32_t c_max) {
  const int b = blockIdx.z, g = blockIdx.y;
  const int G = Hq / H;
  const int part = threadIdx.x & 15;
  const int grp = (threadIdx.x >> 4) & 3;
  const int w = threadIdx.x >> 6;
  const int cap = ccap[b];
  const int C = min(max(clen[b], 0), min(cap, c_max_len));
  float qs[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int h = 0; h < G; ++h) {
    float f[8];
    widen8(q_dtype, *(const u32x4*)(q + ((size_t)b * Hq + (size_t)g * G + h) * kHeadDim + 8 * part), f);
#pragma unroll
    for (int j = 0; j < 8; ++j) qs[j] += f[j];
  }
  const int c_wave = (blockIdx.x * 4 + w) * 16;
  float dot[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = c_wave + 4 * i + grp;
    float acc = 0.f;
    if (c < C) {
      const float* row = ck + (size_t)cbase[b] + ((size_t)g * cap + c) * kHeadDim + 8 * part;
      const f32x4 x0 = __builtin_nontemporal_load((const f32x4*)row);
      const f32x4 x1 = __builtin_nontemporal_load((const f32x4*)(row + 4));
      acc = qs[0] * x0[0] + qs[1] * x0[1] + qs[2] * x0[2] + qs[3] * x0[3];
      acc = fmaf(qs[4], x1[0], fmaf(qs[5], x1[1], fmaf(qs[6], x1[2], fmaf(qs[7], x1[3], acc))));
    }
    acc = row16_sum(acc);
    dot[i] = acc;
  }
  if (part < 4) {
    float v = dot[0];
#pragma unroll
    for (int i = 1; i < 4; ++i)
      if (part == i) v = dot[i];
    const int c = c_wave + 4 * part + grp;
    if (c < c_max) scores[((size_t)b * H + g) * c_max + c] = (c < C) ? v : -__builtin_huge_valf();
  }
}

hipError_t launch_scores(const uint16_t* q, int32_t q_dtype, int32_t Hq, const void* ck,
                         const tf_kv_desc& ckd, float* scores, int32_t c_max, hipStream_t stream) {
  if (ckd.dtype == TF_DTYPE_FP32) {
    const dim3 grid((c_max + 63) / 64, ckd.H, ckd.B), block(256);
    hipLaunchKernelGGL(score_kernel_f32, grid, block, 0, stream, q, q_dtype, Hq, ckd.H, (const float*)ck,
                       ckd.seq_base, ckd.seq_cap, ckd.seq_len, ckd.max_len, scores, c_max);
    return hipGetLastError();
  }
  const long heads = (long)ckd.H * ckd.B;
  const int nblk = (c_max + kScoreBlock - 1) / kScoreBlock;
  const int nx = (int)min(max(1L, (long)kScoreWgs / heads), (long)(nblk + kScoreWaves - 1) / kScoreWaves);
  const dim3 grid(nx, ckd.H, ckd.B), block(kScoreWaves * 64);
  if (ckd.dtype == TF_DTYPE_BF16)
    hipLaunchKernelGGL(score_kernel<TF_DTYPE_BF16>, grid, block, 0, stream, q, q_dtype, Hq, ckd.H,
                       (const uint16_t*)ck, ckd.seq_base, ckd.seq_cap, ckd.seq_len, ckd.max_len, scores, c_max);
  else
    hipLaunchKernelGGL(score_kernel<TF_DTYPE_FP16>, grid, block, 0, stream, q, q_dtype, Hq, ckd.H,
                       (const uint16_t*)ck, ckd.seq_base, ckd.seq_cap, ckd.seq_len, ckd.max_len, scores, c_max);
  return hipGetLastError();
}

}  // namespace tfk
