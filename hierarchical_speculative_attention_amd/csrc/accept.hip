// Lossless accept / reject of a chain of gamma drafted tokens, after the
// TriForce blog, section "2. Dual Rejection Sampling: Mathematical
// Losslessness": keep draft x while min(1, p(x) / q(x)) >= u; at the first
// rejection draw the next token from max(0, p - q) normalised; if every draft
// is kept, draw a bonus token from the target's next row.
//
// Everything runs in fp64 so that every decision is taken in the same
// precision as the fp64 reference.  The vocabulary is cut into slices of
// kSlice entries and the work spread over (slice, row, sequence):
//  1. accept_stats_kernel, per (slice, row, sequence): the slice's largest
//     logit (lowest index on ties) and sum of exp(x / T - slice max / T),
//     and the row's logit at its drafted token when that falls in the slice;
//  2. accept_slice_kernel (accept_slice_small_kernel for 1 .. kFastGamma
//     drafts), per (draw slice of kDraw entries, sequence): every
//     workgroup takes the chain decision itself (one thread per draft, from
//     the row statistics), then stores and sums its slice of the draw's
//     weights -- max(0, p_j - q_j) after a rejection at j, p_gamma when all
//     drafts are kept -- and of p_j (the fallback when the residual vanishes
//     through rounding);
//  3. accept_final_kernel, per sequence: the draw slice whose running sum
//     first passes u * total, then one block prefix sum over that slice's
//     stored weights for the entry (inverse CDF, strict '>').
// The draw is bound by fp64 exponentials (two per vocabulary entry): a first
// version ran it in one workgroup per sequence (70 us at V = 32000), 4096-entry
// draw slices 25 us; 1024-entry slices spread it over 32 workgroups.  The
// final kernel once recomputed its slice's weights (two row merges and two
// exponentials per entry after the slice was found); reading the stored
// weights instead took it from 10.5 to 5.3 us, and the small-chain form of
// kernel 2 (below) the call from 34.6 to 19.7 us (gamma = 6, V = 32000).
// (kFastGamma = 15 keeps 31 rows x 4 entries in registers per thread.)
#include "tf_internal.h"

namespace tfk {

constexpr int kAccThreads = 256;
constexpr int kSlice = 4096;                   // vocabulary entries per statistics slice
constexpr int kPer = kSlice / kAccThreads;     // entries per thread within a statistics slice
constexpr int kMaxSlices = 16;                 // V <= 65536
constexpr int kDraw = 1024;                    // vocabulary entries per draw slice
constexpr int kDrawPer = kDraw / kAccThreads;  // fp64 weights per thread within a draw slice

struct SliceStat {
  float mx;   // largest logit in the slice
  int amax;   // its lowest index
  double z;   // sum over the slice of exp(x / T - mx / T)
};

struct SliceSum {  // per draw slice
  double r;   // sum of the draw's weights over the slice
  double p;   // sum of p_j over the slice (fallback weights)
  int last_r; // last index with positive weight (or -1)
  int last_p;
};

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Block-wide reductions over kAccThreads threads (4 waves); fixed order.
__device__ __forceinline__ double block_sum(double x, double* s) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if (lane == 0) s[w] = x;
  __syncthreads();
  return (s[0] + s[1]) + (s[2] + s[3]);
}

__device__ __forceinline__ int block_max(int x, int* s) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
  __syncthreads();
  if (lane == 0) s[w] = x;
  __syncthreads();
  return max(max(s[0], s[1]), max(s[2], s[3]));
}

// ---------------------------------------------------------------------------
// Kernel 1: one workgroup per (slice, row, sequence), flattened into
// grid.x = slice + nslices * (row + nrows * b).  Rows 0..gamma are target
// rows, rows gamma+1 .. 2*gamma are draft rows 0..gamma-1.  The slice's
// kPer loads per thread are issued together (index clamped into the row).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAccThreads) void accept_stats_kernel(const float* __restrict__ target,
                                                                   const float* __restrict__ draft,
                                                                   const int32_t* __restrict__ tokens, int32_t gamma,
                                                                   int32_t V, float temperature, int32_t nslices,
                                                                   SliceStat* __restrict__ stats,
                                                                   float* __restrict__ xlog) {
  __shared__ float s_v[kAccThreads / 64];
  __shared__ int s_i[kAccThreads / 64];
  __shared__ double s_z[kAccThreads / 64];
  const int nrows = 2 * gamma + 1;
  const int slice = (int)(blockIdx.x % (unsigned)nslices);
  const int r = (int)((blockIdx.x / (unsigned)nslices) % (unsigned)nrows);
  const int b = (int)(blockIdx.x / ((unsigned)nslices * (unsigned)nrows));
  const float* row = (r <= gamma) ? target + ((size_t)b * (gamma + 1) + r) * V
                                  : draft + ((size_t)b * gamma + (r - gamma - 1)) * V;
  const int v0 = slice * kSlice, v1 = min(V, v0 + kSlice);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  // the drafted token this row is tested at (target rows 0 .. gamma-1, every draft row)
  const int xt = (r == gamma) ? -1 : tokens[(size_t)b * gamma + (r < gamma ? r : r - gamma - 1)];
  float x[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) x[k] = row[min(v0 + (int)threadIdx.x + kAccThreads * k, V - 1)];
  float bv = -__builtin_huge_valf();
  int bi = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int v = v0 + (int)threadIdx.x + kAccThreads * k;
    if (v < v1 && better(x[k], v, bv, bi)) {
      bv = x[k];
      bi = v;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (better(ov, oi, bv, bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    s_v[w] = bv;
    s_i[w] = bi;
  }
  __syncthreads();
  bv = s_v[0];
  bi = s_i[0];
#pragma unroll
  for (int q = 1; q < kAccThreads / 64; ++q)
    if (better(s_v[q], s_i[q], bv, bi)) {
      bv = s_v[q];
      bi = s_i[q];
    }
  double z = 0.0;
  if (temperature > 0.f) {
    const double t = (double)temperature;
    const double zm = (double)bv / t;
#pragma unroll
    for (int k = 0; k < kPer; ++k)
      if (v0 + (int)threadIdx.x + kAccThreads * k < v1) z += exp((double)x[k] / t - zm);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
    if (lane == 0) s_z[w] = z;
    __syncthreads();
    z = (s_z[0] + s_z[1]) + (s_z[2] + s_z[3]);
  }
  if (threadIdx.x == 0) {
    SliceStat st;
    st.mx = bv;
    st.amax = bi;
    st.z = z;
    stats[((size_t)b * nrows + r) * nslices + slice] = st;
  }
  // the row's logit at its drafted token, from the thread holding that entry
  if (xt >= v0 && xt < v1 && (int)threadIdx.x == (xt - v0) % kAccThreads) {
    const int kk = (xt - v0) / kAccThreads;
    float xv = x[0];
#pragma unroll
    for (int k = 1; k < kPer; ++k)
      if (k == kk) xv = x[k];
    xlog[(size_t)b * nrows + r] = xv;
  }
}

// Distribution of one row after merging its slices.
struct RowDist {
  int mode;     // 0 softmax(x / T), 1 greedy one-hot, 2 probabilities as given
  double zmax;  // max x / T
  double Z;     // sum of exp(x / T - zmax)
  double invZ;  // 1 / Z (a product per entry instead of a division)
  int amax;
};

// All of the row's slice statistics are requested at once (one memory round
// trip), then merged in slice order.
__device__ RowDist merge_row(const SliceStat* st, int nslices, float temperature, int probs) {
  RowDist d;
  d.zmax = 0.0;
  d.Z = 1.0;
  d.invZ = 1.0;
  d.amax = 0;
  if (probs) {
    d.mode = 2;
    return d;
  }
  float mx[kMaxSlices];
  int am[kMaxSlices];
  double z[kMaxSlices];
#pragma unroll
  for (int s = 0; s < kMaxSlices; ++s) {
    const SliceStat x = st[min(s, nslices - 1)];
    mx[s] = x.mx;
    am[s] = x.amax;
    z[s] = x.z;
  }
  float bv = mx[0];
  int bi = am[0];
#pragma unroll
  for (int s = 1; s < kMaxSlices; ++s)
    if (s < nslices && better(mx[s], am[s], bv, bi)) {
      bv = mx[s];
      bi = am[s];
    }
  d.amax = bi;
  if (temperature == 0.f) {
    d.mode = 1;
    return d;
  }
  d.mode = 0;
  const double t = (double)temperature;
  // z_v = x_v / T; division by T > 0 is monotone, so max z = (max x) / T.
  d.zmax = (double)bv / t;
  double Z = 0.0;
#pragma unroll
  for (int s = 0; s < kMaxSlices; ++s) {
    if (s >= nslices) break;  // (no exponentials for absent slices)
    if (z[s] > 0.0) Z += z[s] * exp((double)mx[s] / t - d.zmax);
  }
  d.Z = Z;
  d.invZ = 1.0 / Z;
  return d;
}

__device__ __forceinline__ double dist_of(const RowDist& d, float x, int v, double t) {
  if (d.mode == 2) return (double)x;
  if (d.mode == 1) return v == d.amax ? 1.0 : 0.0;
  return exp((double)x / t - d.zmax) * d.invZ;
}

// The chain decision: the first draft i that is not kept (gamma if none).
// Threads i < gamma test draft i in parallel.
__device__ int chain_decision(const float* trow0, const float* drow0, const int32_t* tok, const double* u,
                              const SliceStat* st, int gamma, int V, int nslices, float temperature, int probs,
                              int* s_j) {
  if (threadIdx.x == 0) *s_j = gamma;
  __syncthreads();
  const double t = (double)temperature;
  for (int i = threadIdx.x; i < gamma; i += kAccThreads) {
    const int x = tok[i];
    bool keep = false;
    if (x >= 0 && x < V) {  // a token outside [0, V) is never kept
      const RowDist dp = merge_row(st + (size_t)i * nslices, nslices, temperature, probs);
      const RowDist dq = merge_row(st + (size_t)(gamma + 1 + i) * nslices, nslices, temperature, probs);
      const double px = dist_of(dp, trow0[(size_t)i * V + x], x, t);
      const double qx = dist_of(dq, drow0[(size_t)i * V + x], x, t);
      if (px > 0.0) {
        const double alpha = (qx == 0.0) ? 1.0 : fmin(1.0, px / qx);
        keep = alpha >= u[i];
      }
    }
    if (!keep) atomicMin(s_j, i);
  }
  __syncthreads();
  return *s_j;
}

// ---------------------------------------------------------------------------
// Kernel 2: one workgroup per (draw slice, sequence), flattened into
// grid.x = slice + ndraw * b.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAccThreads) void accept_slice_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ tokens,
    const double* __restrict__ uniforms, int32_t gamma, int32_t V, float temperature, int32_t probs,
    const SliceStat* __restrict__ stats, int32_t nslices, int32_t ndraw, SliceSum* __restrict__ sums,
    int32_t* __restrict__ js, double* __restrict__ weights) {
  __shared__ int s_j;
  __shared__ double s_d[kAccThreads / 64];
  __shared__ int s_i[kAccThreads / 64];
  const int slice = (int)(blockIdx.x % (unsigned)ndraw);
  const int b = (int)(blockIdx.x / (unsigned)ndraw);
  const int nrows = 2 * gamma + 1;
  const SliceStat* st = stats + (size_t)b * nrows * nslices;
  const float* trow0 = target + (size_t)b * (gamma + 1) * V;
  const float* drow0 = draft + (size_t)b * gamma * V;
  const int j = chain_decision(trow0, drow0, tokens + (size_t)b * gamma, uniforms + (size_t)b * (gamma + 1), st,
                               gamma, V, nslices, temperature, probs, &s_j);
  const bool residual = j < gamma;
  const float* tr = trow0 + (size_t)j * V;
  const float* dr = drow0 + (size_t)(residual ? j : 0) * V;
  const int v0 = slice * kDraw, v1 = min(V, v0 + kDraw);
  double* wr = weights + (size_t)b * 2 * V;  // the draw's weights, then p_j's
  double* wp = wr + V;
  float xp[kDrawPer], xq[kDrawPer];
#pragma unroll
  for (int k = 0; k < kDrawPer; ++k) {
    const int v = min(v0 + (int)threadIdx.x + kAccThreads * k, V - 1);
    xp[k] = tr[v];
    xq[k] = residual ? dr[v] : 0.f;
  }
  const RowDist dp = merge_row(st + (size_t)j * nslices, nslices, temperature, probs);
  const RowDist dq = residual ? merge_row(st + (size_t)(gamma + 1 + j) * nslices, nslices, temperature, probs) : dp;
  const double t = (double)temperature;
  double sr = 0.0, sp = 0.0;
  int lr = -1, lp = -1;
#pragma unroll
  for (int k = 0; k < kDrawPer; ++k) {
    const int v = v0 + (int)threadIdx.x + kAccThreads * k;
    if (v >= v1) continue;
    const double p = dist_of(dp, xp[k], v, t);
    const double r = residual ? fmax(0.0, p - dist_of(dq, xq[k], v, t)) : p;
    wr[v] = r;
    wp[v] = p;
    sr += r;
    sp += p;
    if (r > 0.0) lr = v;
    if (p > 0.0) lp = v;
  }
  sr = block_sum(sr, s_d);
  sp = block_sum(sp, s_d);
  lr = block_max(lr, s_i);
  lp = block_max(lp, s_i);
  if (threadIdx.x == 0) {
    SliceSum o;
    o.r = sr;
    o.p = sp;
    o.last_r = lr;
    o.last_p = lp;
    sums[(size_t)b * ndraw + slice] = o;
    if (slice == 0) js[b] = j;
  }
}

// ---------------------------------------------------------------------------
// Kernel 3: one workgroup per sequence.  Wave 0 finds the draw slice whose
// running sum first passes u * total (lane s holds slice s; a prefix sum over
// the lanes); then thread t of that slice owns its kDrawPer consecutive
// entries, so a prefix sum in thread order is one in index order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kAccThreads) void accept_final_kernel(
    const double* __restrict__ uniforms, int32_t gamma, int32_t V, int32_t ndraw, const SliceSum* __restrict__ sums,
    const int32_t* __restrict__ js, const double* __restrict__ weights, int32_t* __restrict__ n_acc,
    int32_t* __restrict__ next) {
  __shared__ int s_slice, s_use_r, s_found, s_last;
  __shared__ double s_before, s_tgt;
  __shared__ double s_w[kAccThreads / 64];
  __shared__ int s_l[kAccThreads / 64];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int j = js[b];
  if (w == 0) {
    const SliceSum o = sums[(size_t)b * ndraw + min(lane, ndraw - 1)];
    const bool in = lane < ndraw;
    const double u = uniforms[(size_t)b * (gamma + 1) + gamma];
    double wr = in ? o.r : 0.0, wp = in ? o.p : 0.0;
    double ir = wr, ip = wp;  // inclusive prefix sums over the slices
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double yr = __shfl_up(ir, off), yp = __shfl_up(ip, off);
      if (lane >= off) {
        ir += yr;
        ip += yp;
      }
    }
    // the residual's total; if it vanished (rounding), draw from p_j instead
    const double tot_r = __shfl(ir, 63);
    const bool use_r = !(j < gamma && tot_r == 0.0);
    const double total = use_r ? tot_r : __shfl(ip, 63);
    const double incl = use_r ? ir : ip, ws = use_r ? wr : wp;
    const double tgt = u * total;
    const unsigned long long cross = __ballot(in && incl > tgt);
    int last = in ? (use_r ? o.last_r : o.last_p) : -1;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) last = max(last, __shfl_xor(last, off));
    const int found = cross ? (int)__builtin_ctzll(cross) : -1;
    if (lane == 0) {
      s_slice = found;
      s_use_r = use_r;
      s_tgt = tgt;
      s_last = last;
      s_found = 0x7fffffff;
    }
    if (found >= 0 && lane == found) s_before = incl - ws;
  }
  __syncthreads();
  const int slice = s_slice;
  if (slice < 0) {
    // the running sum never passes u * total (rounding): the last index with
    // positive weight
    if (threadIdx.x == 0) {
      n_acc[b] = j;
      next[b] = s_last;
    }
    return;
  }
  const double* wsrc = weights + (size_t)b * 2 * V + (s_use_r ? 0 : V);
  const int e0 = slice * kDraw + (int)threadIdx.x * kDrawPer;
  double wv[kDrawPer];
#pragma unroll
  for (int k = 0; k < kDrawPer; ++k) wv[k] = wsrc[min(e0 + k, V - 1)];
  double local = 0.0;
  int last_pos = -1;
#pragma unroll
  for (int k = 0; k < kDrawPer; ++k) {
    if (e0 + k >= V) wv[k] = 0.0;
    local += wv[k];
    if (wv[k] > 0.0) last_pos = e0 + k;
  }
  // exclusive prefix of the per-thread sums, in thread order
  double incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_w[w] = incl;
  __syncthreads();
  double off_w = 0.0;
  for (int q = 0; q < w; ++q) off_w += s_w[q];
  double run = s_before + off_w + (incl - local);
  const double tgt = s_tgt;
  int hit = -1;
#pragma unroll
  for (int k = 0; k < kDrawPer; ++k) {
    run += wv[k];
    if (hit < 0 && wv[k] > 0.0 && run > tgt) hit = e0 + k;
  }
  if (hit >= 0) atomicMin(&s_found, hit);
  const int lastp = block_max(last_pos, s_l);
  __syncthreads();
  if (threadIdx.x == 0) {
    n_acc[b] = j;
    // without a crossing inside the slice (rounding), its last positive entry
    next[b] = s_found != 0x7fffffff ? s_found : (lastp >= 0 ? lastp : s_last);
  }
}

// ---------------------------------------------------------------------------
// Kernel 2, chains of 1 .. kFastGamma drafts: the same decision and draw
// slice with the memory round trips overlapped.  Every load is issued at the
// start: this thread's kDrawPer draw entries of every candidate row (target
// rows 0 .. gamma, draft rows 0 .. gamma-1: whichever the decision picks is
// already in registers), the slice statistics of every row, the drafted
// tokens with their logits (recorded by the statistics kernel) and the
// uniforms.  The rows' distributions are merged 16 lanes per row (lane s
// takes slice s: one exponential each, then the serial sum in slice order,
// so each equals the one merge_row gives).
// ---------------------------------------------------------------------------
constexpr int kFastGamma = 15;

__global__ __launch_bounds__(kAccThreads) void accept_slice_small_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ tokens,
    const double* __restrict__ uniforms, int32_t gamma, int32_t V, float temperature, int32_t probs,
    const SliceStat* __restrict__ stats, const float* __restrict__ xlog, int32_t nslices, int32_t ndraw,
    SliceSum* __restrict__ sums, int32_t* __restrict__ js, double* __restrict__ weights) {
  __shared__ RowDist s_rd[2 * kFastGamma + 1];
  __shared__ int s_j;
  __shared__ double s_d[kAccThreads / 64];
  __shared__ int s_i[kAccThreads / 64];
  const int tid = threadIdx.x;
  const int slice = (int)(blockIdx.x % (unsigned)ndraw);
  const int b = (int)(blockIdx.x / (unsigned)ndraw);
  const int nrows = 2 * gamma + 1;
  const float* trow0 = target + (size_t)b * (gamma + 1) * V;
  const float* drow0 = draft + (size_t)b * gamma * V;
  const int v0 = slice * kDraw, v1 = min(V, v0 + kDraw);

  float cp[kFastGamma + 1][kDrawPer], cq[kFastGamma][kDrawPer];
#pragma unroll
  for (int jj = 0; jj <= kFastGamma; ++jj) {
    const float* tr = trow0 + (size_t)min(jj, gamma) * V;
#pragma unroll
    for (int k = 0; k < kDrawPer; ++k) cp[jj][k] = tr[min(v0 + tid + kAccThreads * k, V - 1)];
  }
#pragma unroll
  for (int jj = 0; jj < kFastGamma; ++jj) {
    const float* dr = drow0 + (size_t)min(jj, gamma - 1) * V;
#pragma unroll
    for (int k = 0; k < kDrawPer; ++k) cq[jj][k] = dr[min(v0 + tid + kAccThreads * k, V - 1)];
  }
  int xtok = -1;
  float lt = 0.f, ld = 0.f;
  double ui = 0.0;
  if (tid < gamma) {
    xtok = tokens[(size_t)b * gamma + tid];
    ui = uniforms[(size_t)b * (gamma + 1) + tid];
    if (!probs) {
      lt = xlog[(size_t)b * nrows + tid];
      ld = xlog[(size_t)b * nrows + gamma + 1 + tid];
    }
  }
  if (tid == 0) s_j = gamma;

  // row distributions, 16 lanes per row
  for (int r0 = 0; r0 < nrows; r0 += kAccThreads / 16) {
    const int l16 = tid & 15, r = r0 + (tid >> 4);
    const bool live = r < nrows && l16 < nslices;
    SliceStat x;
    x.mx = -__builtin_huge_valf();
    x.amax = 0x7fffffff;
    x.z = 0.0;
    if (live && !probs) x = stats[((size_t)b * nrows + r) * nslices + l16];
    float bv = x.mx;
    int bi = x.amax;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) {
      const float ov = __shfl_xor(bv, off, 16);
      const int oi = __shfl_xor(bi, off, 16);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    RowDist d;
    d.zmax = 0.0;
    d.Z = 1.0;
    d.invZ = 1.0;
    d.amax = bi;
    d.mode = probs ? 2 : (temperature == 0.f ? 1 : 0);
    if (d.mode == 0) {
      const double t = (double)temperature;
      d.zmax = (double)bv / t;
      const double e = (live && x.z > 0.0) ? x.z * exp((double)x.mx / t - d.zmax) : 0.0;
      double Z = 0.0;
#pragma unroll
      for (int q = 0; q < 16; ++q) Z += __shfl(e, q, 16);
      d.Z = Z;
      d.invZ = 1.0 / Z;
    }
    if (r < nrows && l16 == 0) s_rd[r] = d;
  }
  __syncthreads();

  // the chain decision: threads i < gamma test draft i
  const double t = (double)temperature;
  if (tid < gamma) {
    bool keep = false;
    if (xtok >= 0 && xtok < V) {  // a token outside [0, V) is never kept
      if (probs) {
        lt = trow0[(size_t)tid * V + xtok];
        ld = drow0[(size_t)tid * V + xtok];
      }
      const double px = dist_of(s_rd[tid], lt, xtok, t);
      const double qx = dist_of(s_rd[gamma + 1 + tid], ld, xtok, t);
      if (px > 0.0) {
        const double alpha = (qx == 0.0) ? 1.0 : fmin(1.0, px / qx);
        keep = alpha >= ui;
      }
    }
    if (!keep) atomicMin(&s_j, tid);
  }
  __syncthreads();
  const int j = s_j;
  const bool residual = j < gamma;
  float xp[kDrawPer], xq[kDrawPer];
#pragma unroll
  for (int k = 0; k < kDrawPer; ++k) {
    xp[k] = cp[0][k];
    xq[k] = cq[0][k];
  }
#pragma unroll
  for (int jj = 1; jj <= kFastGamma; ++jj)
    if (jj == j) {
#pragma unroll
      for (int k = 0; k < kDrawPer; ++k) xp[k] = cp[jj][k];
    }
#pragma unroll
  for (int jj = 1; jj < kFastGamma; ++jj)
    if (jj == j) {
#pragma unroll
      for (int k = 0; k < kDrawPer; ++k) xq[k] = cq[jj][k];
    }
  const RowDist dp = s_rd[j];
  const RowDist dq = residual ? s_rd[gamma + 1 + j] : dp;
  double* wr = weights + (size_t)b * 2 * V;  // the draw's weights, then p_j's
  double* wp = wr + V;
  double sr = 0.0, sp = 0.0;
  int lr = -1, lp = -1;
#pragma unroll
  for (int k = 0; k < kDrawPer; ++k) {
    const int v = v0 + tid + kAccThreads * k;
    if (v >= v1) continue;
    const double p = dist_of(dp, xp[k], v, t);
    const double r = residual ? fmax(0.0, p - dist_of(dq, xq[k], v, t)) : p;
    wr[v] = r;
    wp[v] = p;
    sr += r;
    sp += p;
    if (r > 0.0) lr = v;
    if (p > 0.0) lp = v;
  }
  sr = block_sum(sr, s_d);
  sp = block_sum(sp, s_d);
  lr = block_max(lr, s_i);
  lp = block_max(lp, s_i);
  if (tid == 0) {
    SliceSum o;
    o.r = sr;
    o.p = sp;
    o.last_r = lr;
    o.last_p = lp;
    sums[(size_t)b * ndraw + slice] = o;
    if (slice == 0) js[b] = j;
  }
}

size_t accept_ws_bytes(int32_t B, int32_t gamma, int32_t V) {
  if (B < 1 || gamma < 0 || V < 1) return 0;
  const size_t nslices = (size_t)(V + kSlice - 1) / kSlice;
  const size_t ndraw = (size_t)(V + kDraw - 1) / kDraw;
  const size_t a = ((size_t)B * (2 * gamma + 1) * nslices * sizeof(SliceStat) + 255) & ~(size_t)255;
  const size_t b = ((size_t)B * ndraw * sizeof(SliceSum) + 255) & ~(size_t)255;
  const size_t c = ((size_t)B * sizeof(int32_t) + 255) & ~(size_t)255;
  const size_t x = ((size_t)B * (2 * gamma + 1) * sizeof(float) + 255) & ~(size_t)255;
  return a + b + c + x + (size_t)B * 2 * V * sizeof(double);
}

int32_t accept_max_vocab() { return kSlice * kMaxSlices; }

hipError_t launch_accept(const float* target, const float* draft, const int32_t* tokens,
                         const double* uniforms, int32_t B, int32_t gamma, int32_t V,
                         float temperature, int32_t flags, int32_t* n_acc, int32_t* next,
                         void* ws, hipStream_t stream) {
  const int probs = (flags & TF_ACCEPT_PROBS) != 0;
  const int nslices = (V + kSlice - 1) / kSlice;
  const int ndraw = (V + kDraw - 1) / kDraw;
  char* w = (char*)ws;
  SliceStat* stats = (SliceStat*)w;
  const size_t a = ((size_t)B * (2 * gamma + 1) * nslices * sizeof(SliceStat) + 255) & ~(size_t)255;
  SliceSum* sums = (SliceSum*)(w + a);
  const size_t bsz = ((size_t)B * ndraw * sizeof(SliceSum) + 255) & ~(size_t)255;
  int32_t* js = (int32_t*)(w + a + bsz);
  const size_t csz = ((size_t)B * sizeof(int32_t) + 255) & ~(size_t)255;
  float* xlog = (float*)(w + a + bsz + csz);
  const size_t xsz = ((size_t)B * (2 * gamma + 1) * sizeof(float) + 255) & ~(size_t)255;
  double* weights = (double*)(w + a + bsz + csz + xsz);
  if (!probs) {
    const unsigned blocks = (unsigned)nslices * (unsigned)(2 * gamma + 1) * (unsigned)B;
    hipLaunchKernelGGL(accept_stats_kernel, dim3(blocks), dim3(kAccThreads), 0, stream, target, draft, tokens, gamma,
                       V, temperature, nslices, stats, xlog);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (gamma >= 1 && gamma <= kFastGamma)
    hipLaunchKernelGGL(accept_slice_small_kernel, dim3((unsigned)ndraw * (unsigned)B), dim3(kAccThreads), 0, stream,
                       target, draft, tokens, uniforms, gamma, V, temperature, probs, stats, xlog, nslices, ndraw, sums,
                       js, weights);
  else
    hipLaunchKernelGGL(accept_slice_kernel, dim3((unsigned)ndraw * (unsigned)B), dim3(kAccThreads), 0, stream,
                       target, draft, tokens, uniforms, gamma, V, temperature, probs, stats, nslices, ndraw, sums, js,
                       weights);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(accept_final_kernel, dim3(B), dim3(kAccThreads), 0, stream, uniforms, gamma, V, ndraw, sums, js,
                     weights, n_acc, next);
  return hipGetLastError();
}

}  // namespace tfk
