// Measurement aid for the benchmark (not part of the decode path or its C
// ABI): a kernel that only reads, with the access shape of the verification
// pass -- every workgroup streams one contiguous range of K and one of V,
// each wave instruction covering 1 KB of consecutive memory with 16-byte
// nontemporal loads, several loads per tensor in flight per wave -- so that
// the benchmark can time, on the same buffers, how fast HBM serves
// verification's bytes when nothing else is done with them.  The loaded words
// are folded into one value per workgroup and stored, so no load is dead.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kInFlight = 4;  // 16-byte loads per tensor in flight per lane

__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ K, const u32x4* __restrict__ V,
                                                       size_t n16, size_t per_wg, unsigned* __restrict__ sink) {
  const size_t lo = (size_t)blockIdx.x * per_wg;
  const size_t hi = lo + per_wg < n16 ? lo + per_wg : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // one pass covers kThreads * kInFlight consecutive 16-byte words of each tensor
  const size_t step = (size_t)kThreads * kInFlight;
  for (size_t base = lo + threadIdx.x; base < hi; base += step) {
    u32x4 a[kInFlight], b[kInFlight];
#pragma unroll
    for (int i = 0; i < kInFlight; ++i) {
      const size_t j = base + (size_t)i * kThreads;
      const size_t jj = j < hi ? j : lo;  // past the range: re-read the range's first word (in bounds)
      a[i] = __builtin_nontemporal_load(K + jj);
      b[i] = __builtin_nontemporal_load(V + jj);
    }
#pragma unroll
    for (int i = 0; i < kInFlight; ++i) acc ^= a[i] ^ b[i];
  }
  unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x ^= __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) sink[blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6)] = x;
}

}  // namespace

// Reads bytes_each bytes of K and of V (both 16-byte aligned, bytes_each a
// multiple of 16) with `grid` workgroups; sink holds grid * 4 words.
// Returns a hipError_t code.
extern "C" __attribute__((visibility("default"))) int tfb_read_kv(const void* K, const void* V, size_t bytes_each,
                                                                  int grid, unsigned* sink, hipStream_t stream) {
  if (!K || !V || !sink || grid < 1 || bytes_each % 16 != 0 || ((uintptr_t)K | (uintptr_t)V) % 16 != 0)
    return (int)hipErrorInvalidValue;
  const size_t n16 = bytes_each / 16;
  const size_t per_wg = (n16 + grid - 1) / grid;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(kThreads), 0, stream, (const u32x4*)K, (const u32x4*)V, n16,
                     per_wg, sink);
  return (int)hipGetLastError();
}
