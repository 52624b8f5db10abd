// Top-k chunk selection (Force 2 of the TriForce blog, "1. The Three Forces
// of TriForce": keep the k most critical blocks under a token budget).
//
// One 1024-thread workgroup per (sequence, KV head) row.  Scores map to an
// order-preserving unsigned key (NaN -> key of -inf, -0.0 -> +0.0).  Thread t
// owns the contiguous index range [t * IPT, (t + 1) * IPT) and keeps its keys
// in registers for the whole kernel.  A most-significant-digit-first radix
// select over LDS histograms finds the exact k-th largest key T and how many
// keys equal to T must be taken: the first digit is 14 bits wide (13 for
// workgroups of fewer than 16 keys per thread), the later ones 8, 8 and the
// rest; as soon as the bin holding the k-th largest key has at most 64 keys,
// those keys are copied to LDS and one wave ranks them directly instead of
// running the remaining passes.  One block-wide prefix sum in
// thread order then gives each kept item's output slot (all keys > T, then the
// lowest-index keys == T), so the output is ascending and bit-exact for a
// given score array.
//
// Costs that shaped it (measured on the chip, 32 rows of 16384 chunks,
// k = 512; kernel time 12.1 -> 10.8 us with four changes, then 10.5 us per
// call with the 14-bit first digit and 9.7 us with the DPP scans):
//  * the score loads are issued unconditionally (index clamped into the row)
//    and all at once, with the chunk count, before anything waits for them;
//    the first histogram is cleared meanwhile and the only barrier before the
//    first pass follows, so each thread counts as soon as its keys arrive;
//  * real score rows crowd a few top-byte bins and same-address LDS atomics
//    within one instruction serialise.  The first digit (sign, exponent and
//    five mantissa bits) spreads the keys over 16384 bins, one histogram
//    copy (64 KB), its bin picked by all sixteen waves; the k-th key's bin
//    then holds a few dozen keys of a real score row, so the one-wave rank
//    follows the first pass directly.  Measured per launch (32 rows of
//    16384 / GQA: 8 rows in 8 slices + merge / 256 ragged rows): 11 bits in 4
//    copies 11.9 / 14.5 / 12.6 us; 14 bits 11.4 / 15.2 / 12.0 (slices of
//    four keys per thread do not repay clearing and scanning 64 KB); 13 bits
//    11.6 / 13.8 / 12.2; 15 bits 13.0 (128 KB).  Hence 14 bits at 16 or more
//    keys per thread, 13 below.  The later 8-bit digits keep kSub copies
//    indexed by lane % kSub, one bin of different copies in different banks
//    (8 copies beat 4, 16, 32);
//  * a bin of at most 64 keys is ranked by one wave after copying its keys
//    to LDS (broadcast LDS reads, all sixteen issued before any comparison)
//    in place of the remaining passes; ranking a bin of up to 256 keys with
//    the whole block instead of an 8-bit pass measured slower;
//  * wave prefix sums (the bin picks, the output slots) run on DPP row
//    shifts and row broadcasts: lane shuffles compiled to six dependent LDS
//    permutes per scan.  With the rank's reads issued together: 11.4 ->
//    10.55 us per launch at 32 rows of 16384, 13.7 -> 12.3 us for the GQA
//    slices + merge.  The small bin is copied with one returning LDS atomic
//    per key in it: a copy through a per-thread match mask, one wave scan and
//    one atomic per wave measured 0.1-0.2 us slower (every wave then waits
//    for an atomic; here only those holding one of the few keys do);
//  * histograms are double-buffered (the next pass's copy is cleared while
//    this one fills), so a pass needs two barriers; the output prefix sum
//    needs one; both output counts share it.
//
// Few long rows (at most 16 rows of more than 16384 chunks) would leave the
// chip idle while one workgroup per row loads 32-64 keys per thread (at 32768
// chunks: 4.8 us loading, 4.6 us in pass 0, ~2.2 us per later pass).  They are
// selected in two launches instead: the same selection over 8 slices of each
// row, each writing its k best as (key, chunk index) candidates in chunk
// order, then over the row's 8 k candidates (8 rows of 32768 chunks, k = 512:
// 22.0 -> 14.1 us per call; 4 or 16 slices: 15.3 and 15.0 us).
#include "tf_internal.h"

namespace tfk {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
constexpr int kSub = 8;            // histogram copies, one per lane % kSub
constexpr int kHistStride = 257;   // words between copies (different LDS banks for one bin)
constexpr int kHistWords = kSub * kHistStride;
// Width of the first digit: 14 bits (sign, exponent, five mantissa bits) for
// workgroups of 16 or more keys per thread, 13 below.  Later digits: 8, 8 and
// the remaining 2 or 3 bits.
template <int IPT>
constexpr int wide_bits() { return IPT >= 16 ? 14 : 13; }
template <int W>
struct Wide {
  static_assert(W >= 12 && W <= 15, "first digit of 12-15 bits");
  static constexpr int kBins = 1 << W;
  static constexpr int kPerLane = kBins / kTopkThreads;  // bins per thread in the pick (4-32)
  static constexpr int kShift = W - 10;                   // log2(kPerLane)
  // LDS word of a bin.  At 16 or more bins per lane, four pad words follow
  // every kPerLane bins, so the pick's 16-byte reads (lane stride kPerLane + 4
  // words) fall in distinct banks (without: four-way conflicts); 32 rows of
  // 16384: 10.58 -> 10.42 us.  At 8 bins per lane the conflict is two-way and
  // the larger clear costs more (GQA slices 12.4 -> 12.7 us), so no pad.
  static constexpr int kPad = kPerLane >= 16 ? 4 : 0;
  static constexpr int kWords = kBins + kPad * kTopkThreads;
  __device__ static __forceinline__ int word(unsigned bin) { return (int)(bin + (bin >> kShift) * kPad); }
};
// lowest bit of the digit of pass p (0 .. 3)
template <int W>
__device__ __forceinline__ constexpr int digit_shift(int p) { return p == 0 ? 32 - W : p == 3 ? 0 : 32 - W - 8 * p; }

// Keys of real scores are >= 0x007FFFFF (the key of -inf), so 0 marks
// "no item".
__device__ __forceinline__ unsigned order_key(float f) {
  if (f != f) f = -__builtin_huge_valf();  // NaN ranks with -inf
  unsigned u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;            // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave (modulo 2^32), every lane
// active: shifts by 1, 2, 4 and 8 lanes within each row of 16, then row 15's
// and row 31's lane broadcast into the rows after them (DPP row_shr and
// row_bcast operands; a lane without a source adds 0).  The values stay in
// registers: lane shuffles compile to six dependent LDS permutes instead.
__device__ __forceinline__ unsigned wave_incl_scan(unsigned x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return (unsigned)v;
}

// Exclusive prefix sum over the 1024 threads in thread order (modulo 2^32).
// One barrier: each wave publishes its total, then every wave reads all
// sixteen totals (broadcast reads) and adds those of the waves before it.
// s_warp is written once per call, so a second call needs its own array.
__device__ __forceinline__ unsigned block_excl_scan(unsigned x, unsigned* s_warp) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const unsigned incl = wave_incl_scan(x);
  if (lane == 63) s_warp[w] = incl;
  __syncthreads();
  unsigned before = 0u;
#pragma unroll
  for (int q = 0; q < kTopkWaves / 4; ++q) {
    const uint4 t = ((const uint4*)s_warp)[q];
    before += (4 * q + 0 < w ? t.x : 0u) + (4 * q + 1 < w ? t.y : 0u) + (4 * q + 2 < w ? t.z : 0u) +
              (4 * q + 3 < w ? t.w : 0u);
  }
  return before + incl - x;
}

// Chooses, in descending digit order, the bin of histogram h (kSub copies)
// that holds the krem-th largest key, and the number of keys in it; run by
// the 64 threads of wave 0.
__device__ __forceinline__ void pick_bin(const int* h, unsigned prefix, int width, int krem, unsigned* s_prefix,
                                         int* s_krem, int* s_cnt) {
  const int lane = threadIdx.x;
  // lane l owns bins 255-4l .. 252-4l
  int c[4];
  int sum = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int bin = 255 - 4 * lane - j;
    int t = 0;
#pragma unroll
    for (int x = 0; x < kSub; ++x) t += h[x * kHistStride + bin];
    c[j] = t;
    sum += t;
  }
  const int incl = (int)wave_incl_scan((unsigned)sum);
  int above = incl - sum;  // keys in higher digits than this lane's bins
  if (above < krem && krem <= incl) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (above < krem && krem <= above + c[j]) {
        *s_prefix = (prefix << width) | (unsigned)(255 - 4 * lane - j);
        *s_krem = krem - above;
        *s_cnt = c[j];
      }
      above += c[j];
    }
  }
}

// The same choice over the 2^W bins of the first digit, by all sixteen waves:
// thread t reads P = 2^W / 1024 consecutive bins with 16-byte LDS reads (wave
// 0 lane 0 the highest P; at 16 bins per lane the histogram's pad words keep
// these reads free of bank conflicts), each wave scans its lanes' sums, the
// wave totals meet in LDS, and the one lane whose bins hold the krem-th
// largest key writes the result.  Every thread of the block calls it; it ends
// with a barrier.
template <int W>
__device__ __forceinline__ void pick_wide(const int* h, int krem, unsigned* s_tot, unsigned* s_prefix, int* s_krem,
                                          int* s_cnt) {
  constexpr int P = Wide<W>::kPerLane;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // this lane's bins, ascending: lo .. lo + P - 1 (lane 0 of wave 0 holds the highest)
  const int lo = Wide<W>::kBins - P * (64 * w + lane + 1);
  const int lo_word = Wide<W>::word((unsigned)lo);  // (a lane's bins are contiguous words)
  int c[P];
#pragma unroll
  for (int i = 0; i < P; i += 4) {
    const int4 t = *(const int4*)(h + lo_word + i);
    c[i] = t.x;
    c[i + 1] = t.y;
    c[i + 2] = t.z;
    c[i + 3] = t.w;
  }
  int sum = 0;
#pragma unroll
  for (int i = 0; i < P; ++i) sum += c[i];
  const int incl = (int)wave_incl_scan((unsigned)sum);
  if (lane == 63) s_tot[w] = (unsigned)incl;
  __syncthreads();
  int above = incl - sum;  // keys in higher bins of this wave, then of the waves before it
#pragma unroll
  for (int q = 0; q < kTopkWaves / 4; ++q) {
    const uint4 t = ((const uint4*)s_tot)[q];
    above += (int)((4 * q + 0 < w ? t.x : 0u) + (4 * q + 1 < w ? t.y : 0u) + (4 * q + 2 < w ? t.z : 0u) +
                   (4 * q + 3 < w ? t.w : 0u));
  }
  if (above < krem && krem <= above + sum) {
#pragma unroll
    for (int i = P - 1; i >= 0; --i) {  // highest bin first
      if (above < krem && krem <= above + c[i]) {
        *s_prefix = (unsigned)(lo + i);
        *s_krem = krem - above;
        *s_cnt = c[i];
      }
      above += c[i];
    }
  }
  __syncthreads();
}

// The krem-th largest of the n <= kSmall keys in s_key[0, n) (s_key[n,
// kSmall) hold 0, which no key equals or falls below), and how many keys equal
// to it are still to be taken; run by wave 0.  Lane l reads all the slots
// with broadcast LDS reads and counts the keys above its own and equal to it;
// the lanes holding the krem-th largest value write the same pair.  (Ranking
// up to 256 keys with four threads each over the whole block measured slower
// than the 8-bit pass it would replace.)
constexpr int kSmall = 64;
__device__ __forceinline__ void rank_small(const unsigned* s_key, int n, int krem, unsigned* s_T, int* s_krem) {
  const int lane = threadIdx.x;
  const unsigned mine = s_key[lane];  // (slots n .. kSmall - 1 hold 0)
  // all sixteen reads are issued before any comparison (one round trip)
  uint4 o[kSmall / 4];
#pragma unroll
  for (int q = 0; q < kSmall / 4; ++q) o[q] = ((const uint4*)s_key)[q];  // one address for every lane: a broadcast
  __builtin_amdgcn_sched_barrier(0);
  int gt = 0, eq = 0;
#pragma unroll
  for (int q = 0; q < kSmall / 4; ++q) {
    gt += (int)(o[q].x > mine) + (int)(o[q].y > mine) + (int)(o[q].z > mine) + (int)(o[q].w > mine);
    eq += (int)(o[q].x == mine) + (int)(o[q].y == mine) + (int)(o[q].z == mine) + (int)(o[q].w == mine);
  }
  if (lane < n && gt < krem && krem <= gt + eq) {
    *s_T = mine;
    *s_krem = krem - gt;
  }
}

// What one workgroup selects from:
//  kRowScores  the whole row of scores -> idx (one workgroup per row);
//  kRowSlice   slice blockIdx.z (chunks [z L, (z + 1) L)) of a row of scores ->
//              the slice's k best as (key, chunk index) candidates, ascending;
//  kRowMerge   the S k candidates of a row (slices in order, so ascending
//              chunk index; key 0 = padding) -> idx.
// An item of the row's k best (key descending, index ascending) has fewer
// than k items before it in its slice too, so it is among its slice's
// candidates; the merge's ties go to the lower candidate position, which is
// the lower chunk index.
enum : int { kRowScores = 0, kRowSlice = 1, kRowMerge = 2 };

template <int IPT, int SRC>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores, int32_t rows,
                                                             int32_t c_max, const int32_t* __restrict__ n_chunks,
                                                             int32_t k, int32_t* __restrict__ idx,
                                                             uint2* __restrict__ cand, int32_t L) {
  constexpr int W = wide_bits<IPT>();
  __shared__ __attribute__((aligned(16))) int s_wide[Wide<W>::kWords];
  __shared__ int s_hist[2][kHistWords];
  __shared__ __attribute__((aligned(16))) unsigned s_warp[2 * kTopkWaves];
  __shared__ __attribute__((aligned(16))) unsigned s_tot[kTopkWaves];
  __shared__ unsigned s_prefix;
  __shared__ int s_krem, s_cnt, s_n;
  __shared__ __attribute__((aligned(16))) unsigned s_small[kSmall];
  const int row = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const size_t row_id = (size_t)b * rows + row;
  const int i0 = tid * IPT;
  if (tid == 0) s_n = 0;
  if (tid < kSmall) s_small[tid] = 0u;
  // the row's chunk count is read now, so its round trip overlaps the loads
  const int n_chunks_b = n_chunks[b];
  asm volatile("" : : "s"(n_chunks_b));

  // Items first: every load is in bounds (index clamped into the row) and
  // none waits for another or for the chunk count.
  // (32-bit byte offsets from the row base: one address register per load)
  float v[IPT];
  uint2 cv[SRC == kRowMerge ? IPT : 1];
  int lo = 0, n_load = c_max;  // slice: chunks [lo, lo + n_load) of the row
  if (SRC == kRowSlice) {
    lo = blockIdx.z * L;
    n_load = min(L, c_max - lo);
  }
  if (SRC == kRowMerge) {
    const int nc = L;  // candidates per row (S k)
    const char* cb = (const char*)(cand + row_id * nc);
    if ((IPT & 1) == 0) {
#pragma unroll
      for (int q = 0; q < IPT / 2; ++q) {
        const uint4 x = *(const uint4*)(cb + (unsigned)min(i0 / 2 + q, nc / 2 - 1) * 16u);
        cv[2 * q] = make_uint2(x.x, x.y);
        cv[2 * q + 1] = make_uint2(x.z, x.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < IPT; ++j) cv[j] = *(const uint2*)(cb + (unsigned)min(i0 + j, nc - 1) * 8u);
    }
  } else {
    const char* srcb = (const char*)(scores + row_id * c_max + lo);
    // (16-byte loads need a 16-byte aligned row start; the scores pointer
    // itself is only required to be 4-byte aligned)
    if (IPT >= 4 && (c_max & 3) == 0 && (SRC == kRowScores || (L & 3) == 0) && ((uintptr_t)scores & 15) == 0) {
      const int last4 = n_load / 4 - 1;
#pragma unroll
      for (int q = 0; q < IPT / 4; ++q) {
        const float4 x = *(const float4*)(srcb + (unsigned)min(i0 / 4 + q, last4) * 16u);
        v[4 * q + 0] = x.x;
        v[4 * q + 1] = x.y;
        v[4 * q + 2] = x.z;
        v[4 * q + 3] = x.w;
      }
    } else if (IPT <= 32) {
#pragma unroll
      for (int j = 0; j < IPT; ++j) v[j] = *(const float*)(srcb + (unsigned)min(i0 + j, n_load - 1) * 4u);
    } else {
      // (64 keys per thread: one address register per load would not fit beside
      // the values; load in groups of 16)
#pragma unroll
      for (int g = 0; g < IPT; g += 16) {
#pragma unroll
        for (int j = g; j < g + 16 && j < IPT; ++j) v[j] = *(const float*)(srcb + (unsigned)min(i0 + j, n_load - 1) * 4u);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  // The first histogram is cleared while the loads are in flight; the
  // barrier after it is the last one before the first pass, so each thread
  // starts counting as soon as its own keys arrive.
  for (int j = tid; j < Wide<W>::kWords / 4; j += kTopkThreads) ((uint4*)s_wide)[j] = make_uint4(0u, 0u, 0u, 0u);
  __syncthreads();
  const int C = min(max(n_chunks_b, 0), c_max);

  if (C <= k) {
    if (SRC != kRowSlice) {
      int32_t* dst = idx + row_id * k;
      for (int j = tid; j < k; j += kTopkThreads) dst[j] = j < C ? j : -1;
    }
    return;  // (a slice leaves the row to the merge)
  }
  // items of this workgroup that exist: the row's C chunks, the slice's part
  // of them, or the candidates (padding has key 0)
  const int n_items = SRC == kRowScores ? C : SRC == kRowSlice ? min(max(C - lo, 0), L) : L;
  unsigned key[IPT];
#pragma unroll
  for (int j = 0; j < IPT; ++j)
    key[j] = (i0 + j < n_items) ? (SRC == kRowMerge ? cv[j].x : order_key(v[j])) : 0u;

  if (SRC == kRowSlice && n_items <= k) {
    // the whole slice is its own selection: candidates in order, then padding
    uint2* out = cand + (row_id * gridDim.z + blockIdx.z) * k;  // (slice kernel only)
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      if (i0 + j < n_items) out[i0 + j] = make_uint2(key[j], (unsigned)(lo + i0 + j));
    for (int j = n_items + tid; j < k; j += kTopkThreads) out[j] = make_uint2(0u, 0xFFFFFFFFu);
    return;
  }

  unsigned prefix = 0;
  int krem = k;
  // First pass: the W-bit top digit of every key.
  {
    for (int j = tid; j < kHistWords; j += kTopkThreads) s_hist[0][j] = 0;  // the next pass's histogram
#pragma unroll
    for (int j = 0; j < IPT; ++j)
      if (key[j] != 0u) atomicAdd(&s_wide[Wide<W>::word(key[j] >> digit_shift<W>(0))], 1);
    __syncthreads();
    pick_wide<W>(s_wide, krem, s_tot, &s_prefix, &s_krem, &s_cnt);
    prefix = s_prefix;
    krem = s_krem;
  }
  // Later passes: the next 8 (last: 5) bits of the keys still in the running,
  // then the bin holding the krem-th largest.
  auto radix_pass = [&](const int pass) {
    const int shift = digit_shift<W>(pass), width = digit_shift<W>(pass - 1) - digit_shift<W>(pass);
    int* h = s_hist[(pass - 1) & 1];
    int* hn = s_hist[pass & 1];
    if (pass < 3)
      for (int j = tid; j < kHistWords; j += kTopkThreads) hn[j] = 0;  // the next pass's histogram
    const int sub = (lane & (kSub - 1)) * kHistStride;
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const unsigned kk = key[j];
      if (kk != 0u && (kk >> digit_shift<W>(pass - 1)) == prefix) atomicAdd(&h[sub + ((kk >> shift) & ((1u << width) - 1u))], 1);
    }
    __syncthreads();
    if (tid < 64) pick_bin(h, prefix, width, krem, &s_prefix, &s_krem, &s_cnt);
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
  };
  // A bin of at most kSmall keys (after the first digit, real score rows
  // leave a few dozen there): its keys are copied to LDS and ranked by one
  // wave in place of the remaining passes (each pass costs two block barriers
  // and a bin pick).
  auto finish_small = [&](const int pass) {
    const int shift = digit_shift<W>(pass);
#pragma unroll
    for (int j = 0; j < IPT; ++j) {
      const unsigned kk = key[j];
      if (kk != 0u && (kk >> shift) == prefix) s_small[atomicAdd(&s_n, 1)] = kk;
    }
    __syncthreads();
    if (tid < 64) rank_small(s_small, s_n, krem, &s_prefix, &s_krem);
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
  };
  if (s_cnt <= kSmall) {
    finish_small(0);
  } else {
    radix_pass(1);
    if (s_cnt <= kSmall) {
      finish_small(1);
    } else {
      radix_pass(2);
      if (s_cnt <= kSmall) finish_small(2); else radix_pass(3);
    }
  }
  const unsigned T = prefix;

  // Output slots: keys > T and the krem lowest-index keys == T, in index
  // order.  Both counts share one prefix sum (gt in the low 16 bits: fewer
  // than k <= 65535 keys exceed T, so it never carries into the high half).
  unsigned n_gt = 0, n_eq = 0;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    n_gt += key[j] > T;
    n_eq += key[j] == T;
  }
  const unsigned pre = block_excl_scan((n_eq << 16) | n_gt, s_warp);
  const int eq_before = (int)(pre >> 16), gt_before = (int)(pre & 0xFFFFu);
  int eq_left = min(max(krem - eq_before, 0), (int)n_eq);
  int pos = gt_before + min(eq_before, krem);
  int32_t* dst = SRC == kRowSlice ? nullptr : idx + row_id * k;
  uint2* out = SRC == kRowSlice ? cand + (row_id * gridDim.z + blockIdx.z) * k : nullptr;
#pragma unroll
  for (int j = 0; j < IPT; ++j) {
    bool keep = key[j] > T;
    if (!keep && key[j] == T && eq_left > 0) {
      keep = true;
      --eq_left;
    }
    if (keep && pos < k) {
      if (SRC == kRowScores) dst[pos] = i0 + j;
      if (SRC == kRowSlice) out[pos] = make_uint2(key[j], (unsigned)(lo + i0 + j));
      if (SRC == kRowMerge) dst[pos] = (int32_t)cv[j].y;
      ++pos;
    }
  }
}

// Rows longer than 65536 chunks: the same selection with each thread's keys
// re-read from memory (L2-resident after the first pass) instead of held in
// registers.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel_long(const float* __restrict__ scores, int32_t rows,
                                                                  int32_t c_max, const int32_t* __restrict__ n_chunks,
                                                                  int32_t k, int32_t* __restrict__ idx) {
  __shared__ int s_hist[kTopkWaves][256];
  __shared__ __attribute__((aligned(16))) unsigned s_warp[2 * kTopkWaves];
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
  const int eq_before = (int)block_excl_scan((unsigned)n_eq, s_warp);
  const int take_eq = min(max(krem - eq_before, 0), n_eq);
  const int mine = n_gt + take_eq;
  int pos = (int)block_excl_scan((unsigned)mine, s_warp + kTopkWaves);
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

TopkSplit plan_topk(int32_t B, int32_t rows, int32_t c_max, int32_t k) {
  TopkSplit p;
  p.S = 1;
  p.L = c_max;
  // Few long rows: one workgroup per row would leave the chip idle and spend
  // most of its time loading 32+ keys per thread.  Eight slices per row, each
  // cutting its chunks to k candidates at least by half.
  if ((long)B * rows <= kTopkSplitMaxRows && c_max > 16384 && c_max <= 65536) {
    const int S = kTopkSlices;
    const int L = ((c_max + S - 1) / S + 3) / 4 * 4;
    if (2L * k <= L && (long)S * k <= 16384) {
      p.S = S;
      p.L = L;
    }
  }
  return p;
}

size_t topk_workspace_bytes(int32_t B, int32_t rows, int32_t c_max, int32_t k) {
  const TopkSplit p = plan_topk(B, rows, c_max, k);
  return p.S > 1 ? (size_t)B * rows * p.S * k * sizeof(uint2) : 0;
}

hipError_t launch_topk(const float* scores, int32_t B, int32_t rows, int32_t c_max, const int32_t* n_chunks,
                       int32_t k, int32_t* idx, void* ws, hipStream_t stream) {
  const int ipt = (c_max + kTopkThreads - 1) / kTopkThreads;
  const dim3 block(kTopkThreads);
  const TopkSplit p = plan_topk(B, rows, c_max, k);
  if (p.S > 1) {
    uint2* cand = (uint2*)ws;
    const int ipt1 = (p.L + kTopkThreads - 1) / kTopkThreads;
    const int nc = p.S * k;
    const int ipt2 = (nc + kTopkThreads - 1) / kTopkThreads;
#define TF_TOPK_SLICE(N)                                                                                  \
  if (ipt1 <= N) {                                                                                        \
    hipLaunchKernelGGL((topk_kernel<N, kRowSlice>), dim3(rows, B, p.S), block, 0, stream, scores, rows, c_max, \
                       n_chunks, k, idx, cand, p.L);                                                      \
  } else
    TF_TOPK_SLICE(1) TF_TOPK_SLICE(2) TF_TOPK_SLICE(4) TF_TOPK_SLICE(8) TF_TOPK_SLICE(16) return hipErrorInvalidValue;
#undef TF_TOPK_SLICE
#define TF_TOPK_MERGE(N)                                                                                  \
  if (ipt2 <= N) {                                                                                        \
    hipLaunchKernelGGL((topk_kernel<N, kRowMerge>), dim3(rows, B), block, 0, stream, scores, rows, c_max,   \
                       n_chunks, k, idx, cand, nc);                                                       \
    return hipGetLastError();                                                                             \
  }
    TF_TOPK_MERGE(1) TF_TOPK_MERGE(2) TF_TOPK_MERGE(4) TF_TOPK_MERGE(8) TF_TOPK_MERGE(16)
#undef TF_TOPK_MERGE
    return hipErrorInvalidValue;
  }
  // Keys per thread: the smallest instantiation that holds the row.  Steps
  // of 20, 24 and 48 keep most threads busy for rows a little longer than
  // 16384 or 32768 chunks: with powers of two only, 16448 chunks (a cache of
  // 131072 + 512 rows) took 32 keys per thread on half the threads, 19.9 us
  // against 12.3 us at 20; 40000 chunks 58.1 against 37.6 us at 48.
  const dim3 grid(rows, B);
#define TF_TOPK_CASE(N) \
  if (ipt <= N) {       \
    hipLaunchKernelGGL((topk_kernel<N, kRowScores>), grid, block, 0, stream, scores, rows, c_max, n_chunks, k, idx, \
                       (uint2*)nullptr, c_max); \
    return hipGetLastError(); \
  }
  TF_TOPK_CASE(1)
  TF_TOPK_CASE(2)
  TF_TOPK_CASE(4)
  TF_TOPK_CASE(8)
  TF_TOPK_CASE(16)
  TF_TOPK_CASE(20)
  TF_TOPK_CASE(24)
  TF_TOPK_CASE(32)
  TF_TOPK_CASE(48)
  TF_TOPK_CASE(64)
#undef TF_TOPK_CASE
  hipLaunchKernelGGL(topk_kernel_long, grid, block, 0, stream, scores, rows, c_max, n_chunks, k, idx);
  return hipGetLastError();
}

}  // namespace tfk
