// Cache maintenance around the decode step: drafted rows enter the caches
// before they are verified, and rejected ones leave them again.
//
//  * Force 3 of the TriForce blog ("1. The Three Forces of TriForce") reads
//    the complete cache, which under the verification layout used here
//    already holds the drafted rows as its last rows: append_kernel (full
//    mode) writes the new rows at positions n .. n + R - 1.
//  * Force 1 keeps the initial sinks plus a rolling window of the most recent
//    tokens: append_kernel (ring mode) writes logical position p to slot p
//    (p < n_sink) or n_sink + (p - n_sink) mod (cap - n_sink), and refuses a
//    ring with fewer than window + reserve slots after the sinks, so that a
//    rollback of up to `reserve` rows never exposes a slot a newer row took.
//  * "2. Dual Rejection Sampling" discards the drafts after the first
//    rejection: commit_kernel moves each length by +add, then back by the
//    gamma - n_accepted rejected drafts.
//
// The lengths live on the device (the descriptors' seq_len arrays), so a whole
// decode loop can run without a host round trip.  Each kernel is a handful of
// 16-byte copies per (sequence, head): latency, not bandwidth.
#include "tf_internal.h"

namespace tfk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int append_status(int n, int cap, int R, int mode, int n_sink, int window, int reserve) {
  if (n < 0) return TF_APPEND_BAD_LENGTH;
  if (mode == TF_APPEND_FULL) return (long)n + R > (long)cap ? TF_APPEND_NO_ROOM : TF_APPEND_OK;
  return (long)cap - n_sink < (long)window + reserve ? TF_APPEND_RING_TOO_SMALL : TF_APPEND_OK;
}

// Grid (H, B), 256 threads: head h of sequence b copies its R new rows
// (16 bytes per thread and step) into K and V.
__global__ __launch_bounds__(256) void append_kernel(const uint16_t* __restrict__ Knew,
                                                     const uint16_t* __restrict__ Vnew, int32_t R,
                                                     uint16_t* __restrict__ K, uint16_t* __restrict__ V,
                                                     const int64_t* __restrict__ seq_base,
                                                     const int32_t* __restrict__ seq_cap,
                                                     const int32_t* __restrict__ seq_len, int32_t H, int32_t mode,
                                                     int32_t n_sink, int32_t window, int32_t reserve,
                                                     int32_t* __restrict__ status) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int n = seq_len[b], cap = seq_cap[b];
  const int64_t base = seq_base[b];
  const int st = append_status(n, cap, R, mode, n_sink, window, reserve);
  if (status && h == 0 && tid == 0) status[b] = st;
  if (st != TF_APPEND_OK) return;
  const size_t src0 = ((size_t)b * H + h) * (size_t)R * kHeadDim;
  const size_t dst0 = (size_t)base + (size_t)h * (size_t)cap * kHeadDim;
  for (int e = tid; e < R * 16; e += 256) {
    const int r = e >> 4, seg = e & 15;
    const long p = (long)n + r;  // logical position of the row
    long row;
    if (mode == TF_APPEND_FULL || p < n_sink) {
      row = p;  // full mode: p < cap by the status check
    } else {
      row = n_sink + (p - n_sink) % (cap - n_sink);  // cap - n_sink >= window + reserve >= R >= 1
    }
    const size_t s = src0 + (size_t)r * kHeadDim + 8 * seg;
    const size_t d = dst0 + (size_t)row * kHeadDim + 8 * seg;
    *(u32x4*)(K + d) = *(const u32x4*)(Knew + s);
    *(u32x4*)(V + d) = *(const u32x4*)(Vnew + s);
  }
}

// One workgroup: seq_len[b] = max(0, seq_len[b] + add - drop_b) with
// drop_b = gamma - clamp(n_accepted[b], 0, gamma) (0 without n_accepted).
__global__ __launch_bounds__(256) void commit_kernel(int32_t* __restrict__ seq_len, int32_t B, int32_t add,
                                                     int32_t gamma, const int32_t* __restrict__ n_accepted) {
  for (int b = threadIdx.x; b < B; b += 256) {
    long drop = 0;
    if (n_accepted) drop = gamma - min(max(n_accepted[b], 0), gamma);
    const long v = (long)seq_len[b] + add - drop;
    seq_len[b] = (int32_t)(v < 0 ? 0 : (v > 0x7fffffffL ? 0x7fffffffL : v));
  }
}

hipError_t launch_append(const uint16_t* Knew, const uint16_t* Vnew, int32_t R, uint16_t* K, uint16_t* V,
                         const tf_kv_desc& kv, int32_t mode, int32_t n_sink, int32_t window, int32_t reserve,
                         int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(append_kernel, dim3(kv.H, kv.B), dim3(256), 0, stream, Knew, Vnew, R, K, V, kv.seq_base,
                     kv.seq_cap, kv.seq_len, kv.H, mode, n_sink, window, reserve, status);
  return hipGetLastError();
}

hipError_t launch_commit(int32_t* seq_len, int32_t B, int32_t add, int32_t gamma, const int32_t* n_accepted,
                         hipStream_t stream) {
  hipLaunchKernelGGL(commit_kernel, dim3(1), dim3(256), 0, stream, seq_len, B, add, gamma, n_accepted);
  return hipGetLastError();
}

}  // namespace tfk
