// Measurement aid for the benchmark (not part of the decode path or its C
// ABI): a kernel that only gathers what one sparse-attention call reads -- the
// K and V rows of every selected chunk of every (sequence, KV head) -- in one
// launch.  Like the attention kernel, each workgroup owns `tpw` consecutive
// selected-chunk rows of one (sequence, KV head), reads their chunk indices
// first (the same dependent round trip) and then has two 32-row tiles per
// wave in flight at once, each wave instruction covering 1 KB of consecutive
// memory (4 rows of 256 bytes) with 16-byte nontemporal loads.  Nothing is
// computed from the rows and nothing is merged: the words are folded into one
// value per wave and stored, so no load is dead.  Timed on the same buffers
// as the sparse call, it bounds what one launch can reach on those bytes.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kHeadDim = 128;
constexpr int kTile = 32;  // rows per wave tile

__global__ __launch_bounds__(kThreads) void gather_kernel(const uint16_t* __restrict__ K,
                                                         const uint16_t* __restrict__ V,
                                                         const int64_t* __restrict__ seq_base,
                                                         const int32_t* __restrict__ seq_cap,
                                                         const int32_t* __restrict__ seq_len,
                                                         const int32_t* __restrict__ idx, int Hkv, int k, int cs,
                                                         int tpw, unsigned* __restrict__ sink) {
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int cap = seq_cap[b];
  const int n = min(max(seq_len[b], 0), max(cap, 0));
  const int nchunks = (n + cs - 1) / cs;
  const int32_t* ix = idx + ((size_t)b * Hkv + hk) * k;
  const size_t base = (size_t)seq_base[b] + (size_t)hk * (size_t)max(cap, 0) * kHeadDim;
  const int v0 = split * tpw;
  const int v1 = min(k * cs, v0 + tpw);
  u32x4 acc = {0u, 0u, 0u, 0u};
  // tiles t and t + 4 kTile of this wave together: every chunk index first,
  // then all loads of the two tiles
  for (int t = v0 + kTile * w; t < v1; t += 8 * kTile) {
    const int nt = t + 4 * kTile < v1 ? 2 : 1;  // (wave-uniform)
    // computed for every row and dropped by selection (no branch per row, so
    // the index loads are issued together); slots clamped into the k entries
    int c[16], vv[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      vv[i] = t + (i < 8 ? 0 : 4 * kTile) + 4 * (i & 7) + (lane >> 4);
      c[i] = ix[min((unsigned)vv[i] / (unsigned)cs, (unsigned)(k - 1))];
    }
    size_t off[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const unsigned slot = (unsigned)vv[i] / (unsigned)cs;
      const int row = (int)((unsigned)c[i] * (unsigned)cs + ((unsigned)vv[i] - slot * (unsigned)cs));
      const bool ok = i < 8 * nt && vv[i] < v1 && c[i] >= 0 && c[i] < nchunks && row < n;
      // rows that hold nothing read row 0 (in bounds)
      off[i] = base + (size_t)(ok ? row : 0) * kHeadDim + 8 * (lane & 15);
    }
    u32x4 a[16], bv[16];
    if (nt == 2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) a[i] = __builtin_nontemporal_load((const u32x4*)(K + off[i]));
#pragma unroll
      for (int i = 0; i < 16; ++i) bv[i] = __builtin_nontemporal_load((const u32x4*)(V + off[i]));
#pragma unroll
      for (int i = 0; i < 16; ++i) acc ^= a[i] ^ bv[i];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) a[i] = __builtin_nontemporal_load((const u32x4*)(K + off[i]));
#pragma unroll
      for (int i = 0; i < 8; ++i) bv[i] = __builtin_nontemporal_load((const u32x4*)(V + off[i]));
#pragma unroll
      for (int i = 0; i < 8; ++i) acc ^= a[i] ^ bv[i];
    }
  }
  unsigned x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  const size_t wg = ((size_t)b * Hkv + hk) * gridDim.x + split;
  if (lane == 0) sink[wg * (kThreads / 64) + w] = x;
}

}  // namespace

// Gathers the K and V rows of the chunks idx[b][hk][0 .. k) selects (cs rows
// each, cs a multiple of 4 so that an instruction's 4 rows lie in one chunk)
// for B sequences of Hkv KV heads laid out as the library's descriptors say
// (seq_base / seq_cap / seq_len: device arrays of B entries), with workgroups
// of tpw rows (a multiple of 128).  sink holds ceil(k cs / tpw) * Hkv * B * 4
// words.  Returns a hipError_t code.
extern "C" __attribute__((visibility("default"))) int tfb_gather_kv(const void* K, const void* V,
                                                                    const int64_t* seq_base, const int32_t* seq_cap,
                                                                    const int32_t* seq_len, const int32_t* idx,
                                                                    int B, int Hkv, int k, int cs, int tpw,
                                                                    unsigned* sink, hipStream_t stream) {
  if (!K || !V || !seq_base || !seq_cap || !seq_len || !idx || !sink || B < 1 || Hkv < 1 || k < 1 || cs < 4 ||
      cs % 4 != 0 || tpw < 128 || tpw % 128 != 0 || (long)k * cs > (1L << 30) ||
      ((uintptr_t)K | (uintptr_t)V) % 16 != 0)
    return (int)hipErrorInvalidValue;
  const int splits = (int)(((long)k * cs + tpw - 1) / tpw);
  hipLaunchKernelGGL(gather_kernel, dim3(splits, Hkv, B), dim3(kThreads), 0, stream, (const uint16_t*)K,
                     (const uint16_t*)V, seq_base, seq_cap, seq_len, idx, Hkv, k, cs, tpw, sink);
  return (int)hipGetLastError();
}
