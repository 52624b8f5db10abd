// Top-k chunk selection (Force 2 of the TriForce blog, "1. The Three Forces
// of TriForce": keep the k most critical blocks under a token budget).
//
// One 1024-thread workgroup per (sequence, KV head) row.  Scores map to an
// order-preserving unsigned key (NaN -> key of -inf, -0.0 -> +0.0).  Thread t
// owns the contiguous index range [t * IPT, (t + 1) * IPT) and keeps its keys
// in registers for the whole kernel.  A most-significant-digit-first radix
// select (four 8-bit passes; one LDS histogram per wave, summed) finds the
// exact k-th largest key T and how many keys equal to T must be taken.  Two
// block-wide prefix sums in thread order then give (1) which T-valued items
// are taken (the lowest indices) and (2) each kept item's output slot, so the
// output is ascending and bit-exact for a given score array.
#include "tf_internal.h"

namespace tfk {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;

// Keys of real scores are >= 0x007FFFFF (the key of -inf), so 0 marks
// "no item".
__device__ __forceinline__ unsigned order_key(float f) {
  if (f != f) f = -__builtin_huge_valf();  // NaN ranks with -inf
  unsigned u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;            // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the 1024 threads in thread order.
__device__ __forceinline__ int block_excl_scan(int x, int* s_warp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_warp[w] = incl;
  __syncthreads();
  if (w == 0) {
    const int t = lane < kTopkWaves ? s_warp[lane] : 0;
    int ti = t;
#pragma unroll
    for (int off = 1; off < kTopkWaves; off <<= 1) {
      const int y = __shfl_up(ti, off);
      if (lane >= off) ti += y;
    }
    if (lane < kTopkWaves) s_warp[kTopkWaves + lane] = ti - t;  // exclusive wave offsets
  }
  __syncthreads();
  const int r = s_warp[kTopkWaves + w] + incl - x;
  __syncthreads();
  return r;
}

template <int IPT>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int32_t rows,
                                                             int32_t c_max, const int32_t* __restrict__ n_chunks,
                                                             int32_t k, int32_t* __restrict__ idx) {
  __shared__ int s_hist[kTopkWaves][256];
  __shared__ int s_warp[2 * kTopkWaves];
  __shared__ unsigned s_prefix;
  __shared__ int s_krem;
  const int row = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6;
  const float* src = scores + ((size_t)b * rows + row) * c_max;
  int32_t* dst = idx + ((size_t)b * rows + row) * k;
  const int C = min(max(n_chunks[b], 0), c_max);

  if (C <= k) {
    for (int j = tid; j < k; j += kTopkThreads) dst[j] = j < C ? j : -1;
    return;
  }

  const int i0 = tid * IPT;
  unsigned key[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j) key[j] = (i0 + j < C) ? order_key(src[i0 + j]) : 0u;

  unsigned prefix = 0;
  int krem = k;
#pragma unroll 1
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int j = tid; j < kTopkWaves * 256; j += kTopkThreads) (&s_hist[0][0])[j] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const unsigned kk = key[j];
      const bool match = kk != 0u && (pass == 0 || (kk >> (shift + 8)) == prefix);
      if (match) atomicAdd(&s_hist[w][(kk >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 256) {  // fold the per-wave histograms
      int t = 0;
#pragma unroll
      for (int x = 0; x < kTopkWaves; ++x) t += s_hist[x][tid];
      s_hist[0][tid] = t;
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 255-4l .. 252-4l (descending digit order)
      int c[4];
      int sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = s_hist[0][255 - 4 * tid - j];
        sum += c[j];
      }
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (tid >= off) incl += y;
      }
      int above = incl - sum;  // keys in higher digits than this lane's bins
      if (above < krem && krem <= incl) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (above < krem && krem <= above + c[j]) {
            s_prefix = (prefix << 8) | (unsigned)(255 - 4 * tid - j);
            s_krem = krem - above;
          }
          above += c[j];
        }
      }
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
  }
  const unsigned T = prefix;

  int n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    n_gt += key[j] > T;
    n_eq += key[j] == T;
  }
  const int eq_before = block_excl_scan(n_eq, s_warp);
  const int take_eq = min(max(krem - eq_before, 0), n_eq);
  const int mine = n_gt + take_eq;
  const int pos0 = block_excl_scan(mine, s_warp);
  int pos = pos0, eq_left = take_eq;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    bool keep = key[j] > T;
    if (!keep && key[j] == T && eq_left > 0) {
      keep = true;
      --eq_left;
    }
    if (keep && pos < k) dst[pos++] = i0 + j;
  }
}

// Rows longer than 65536 chunks: the same selection with each thread's keys
// re-read from memory (L2-resident after the first pass) instead of held in
// registers.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel_long(const float* __restrict__ scores, int32_t rows,
                                                                  int32_t c_max, const int32_t* __restrict__ n_chunks,
                                                                  int32_t k, int32_t* __restrict__ idx) {
  __shared__ int s_hist[kTopkWaves][256];
  __shared__ int s_warp[2 * kTopkWaves];
  __shared__ unsigned s_prefix;
  __shared__ int s_krem;
  const int row = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6;
  const float* src = scores + ((size_t)b * rows + row) * c_max;
  int32_t* dst = idx + ((size_t)b * rows + row) * k;
  const int C = min(max(n_chunks[b], 0), c_max);
  if (C <= k) {
    for (int j = tid; j < k; j += kTopkThreads) dst[j] = j < C ? j : -1;
    return;
  }
  const int ipt = (c_max + kTopkThreads - 1) / kTopkThreads;
  const int i0 = tid * ipt, i1 = min(C, i0 + ipt);
  unsigned prefix = 0;
  int krem = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int j = tid; j < kTopkWaves * 256; j += kTopkThreads) (&s_hist[0][0])[j] = 0;
    __syncthreads();
    for (int i = i0; i < i1; ++i) {
      const unsigned kk = order_key(src[i]);
      if (pass == 0 || (kk >> (shift + 8)) == prefix) atomicAdd(&s_hist[w][(kk >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 256) {
      int t = 0;
      for (int x = 0; x < kTopkWaves; ++x) t += s_hist[x][tid];
      s_hist[0][tid] = t;
    }
    __syncthreads();
    if (tid < 64) {
      int c[4];
      int sum = 0;
      for (int j = 0; j < 4; ++j) {
        c[j] = s_hist[0][255 - 4 * tid - j];
        sum += c[j];
      }
      int incl = sum;
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (tid >= off) incl += y;
      }
      int above = incl - sum;
      if (above < krem && krem <= incl) {
        for (int j = 0; j < 4; ++j) {
          if (above < krem && krem <= above + c[j]) {
            s_prefix = (prefix << 8) | (unsigned)(255 - 4 * tid - j);
            s_krem = krem - above;
          }
          above += c[j];
        }
      }
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
  }
  const unsigned T = prefix;
  int n_gt = 0, n_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const unsigned kk = order_key(src[i]);
    n_gt += kk > T;
    n_eq += kk == T;
  }
  const int eq_before = block_excl_scan(n_eq, s_warp);
  const int take_eq = min(max(krem - eq_before, 0), n_eq);
  const int mine = n_gt + take_eq;
  int pos = block_excl_scan(mine, s_warp);
  int eq_left = take_eq;
  for (int i = i0; i < i1; ++i) {
    const unsigned kk = order_key(src[i]);
    bool keep = kk > T;
    if (!keep && kk == T && eq_left > 0) {
      keep = true;
      --eq_left;
    }
    if (keep && pos < k) dst[pos++] = i;
  }
}

hipError_t launch_topk(const float* scores, int32_t B, int32_t rows, int32_t c_max,
                       const int32_t* n_chunks, int32_t k, int32_t* idx, hipStream_t stream) {
  const dim3 grid(rows, B), block(kTopkThreads);
  const int ipt = (c_max + kTopkThreads - 1) / kTopkThreads;
#define TF_TOPK_CASE(N) \
  if (ipt <= N) {       \
    hipLaunchKernelGGL(topk_kernel<N>, grid, block, 0, stream, scores, rows, c_max, n_chunks, k, idx); \
    return hipGetLastError(); \
  }
  TF_TOPK_CASE(1)
  TF_TOPK_CASE(2)
  TF_TOPK_CASE(4)
  TF_TOPK_CASE(8)
  TF_TOPK_CASE(16)
  TF_TOPK_CASE(32)
  TF_TOPK_CASE(64)
#undef TF_TOPK_CASE
  hipLaunchKernelGGL(topk_kernel_long, grid, block, 0, stream, scores, rows, c_max, n_chunks, k, idx);
  return hipGetLastError();
}

}  // namespace tfk
