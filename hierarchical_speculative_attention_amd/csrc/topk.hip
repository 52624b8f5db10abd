// Top-k chunk selection (Force 2 of the TriForce blog, "1. The Three Forces
// of TriForce": keep the k most critical blocks under a token budget).
//
// One 1024-thread workgroup per (sequence, KV head) row.  Scores map to an
// order-preserving unsigned key (NaN -> key of -inf, -0.0 -> +0.0).  A
// most-significant-digit-first radix select (four 8-bit passes, LDS
// histogram) finds the exact k-th largest key T and how many keys equal to T
// must be taken.  Thread t owns the contiguous index range
// [t * ipt, (t + 1) * ipt), so two block-wide prefix sums in thread order
// give (1) which of the T-valued items are taken (the lowest indices) and
// (2) each kept item's output slot; the output is therefore ascending and
// bit-exact for a given score array.
#include "tf_internal.h"

namespace tfk {

constexpr int kTopkThreads = 1024;

__device__ __forceinline__ unsigned order_key(float f) {
  if (f != f) f = -__builtin_huge_valf();  // NaN ranks with -inf
  unsigned u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;            // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the 1024 threads in thread order; returns the
// block total through *total.
__device__ __forceinline__ int block_excl_scan(int x, int* s_warp, int* total) {
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
    int t = lane < 16 ? s_warp[lane] : 0;
    int ti = t;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int y = __shfl_up(ti, off);
      if (lane >= off) ti += y;
    }
    if (lane < 16) s_warp[16 + lane] = ti - t;  // exclusive wave offsets
    if (lane == 15) s_warp[32] = ti;
  }
  __syncthreads();
  const int r = s_warp[16 + w] + incl - x;
  *total = s_warp[32];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int32_t rows,
                                                             int32_t c_max, const int32_t* __restrict__ n_chunks,
                                                             int32_t k, int32_t* __restrict__ idx) {
  __shared__ int s_hist[256];
  __shared__ int s_warp[48];
  __shared__ unsigned s_prefix;
  __shared__ int s_krem;
  const int row = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x;
  const float* src = scores + ((size_t)b * rows + row) * c_max;
  int32_t* dst = idx + ((size_t)b * rows + row) * k;
  const int C = min(max(n_chunks[b], 0), c_max);
  const int ipt = (C + kTopkThreads - 1) / kTopkThreads;
  const int i0 = tid * ipt, i1 = min(C, i0 + ipt);

  if (C <= k) {
    for (int j = tid; j < k; j += kTopkThreads) dst[j] = j < C ? j : -1;
    return;
  }

  unsigned prefix = 0;
  int krem = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int j = tid; j < 256; j += kTopkThreads) s_hist[j] = 0;
    __syncthreads();
    for (int i = i0; i < i1; ++i) {
      const unsigned key = order_key(src[i]);
      const bool match = pass == 0 || (key >> (shift + 8)) == prefix;
      if (match) atomicAdd(&s_hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l owns bins 255-4l .. 252-4l (descending digit order)
      int c[4];
      int sum = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        c[j] = s_hist[255 - 4 * tid - j];
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
    __syncthreads();
  }
  const unsigned T = prefix;

  int n_gt = 0, n_eq = 0;
  for (int i = i0; i < i1; ++i) {
    const unsigned key = order_key(src[i]);
    n_gt += key > T;
    n_eq += key == T;
  }
  int tot;
  const int eq_before = block_excl_scan(n_eq, s_warp, &tot);
  const int take_eq = min(max(krem - eq_before, 0), n_eq);
  const int mine = n_gt + take_eq;
  const int pos0 = block_excl_scan(mine, s_warp, &tot);
  int pos = pos0, eq_left = take_eq;
  const int pos_end = min(pos0 + mine, k);
  for (int i = i0; i < i1 && pos < pos_end; ++i) {
    const unsigned key = order_key(src[i]);
    bool keep = key > T;
    if (!keep && key == T && eq_left > 0) {
      keep = true;
      --eq_left;
    }
    if (keep) dst[pos++] = i;
  }
}

hipError_t launch_topk(const float* scores, int32_t B, int32_t rows, int32_t c_max,
                       const int32_t* n_chunks, int32_t k, int32_t* idx, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3(rows, B), dim3(kTopkThreads), 0, stream, scores, rows, c_max, n_chunks, k, idx);
  return hipGetLastError();
}

}  // namespace tfk
