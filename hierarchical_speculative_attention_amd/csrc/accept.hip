// Lossless accept / reject of a chain of gamma drafted tokens, after the
// TriForce blog, section "2. Dual Rejection Sampling: Mathematical
// Losslessness": keep draft x while min(1, p(x) / q(x)) >= u; at the first
// rejection draw the next token from max(0, p - q) normalised; if every draft
// is kept, draw a bonus token from the target's next row.
//
// Everything runs in fp64 so that every decision is taken in the same
// precision as the fp64 reference.  Two kernels:
//  1. row statistics, spread over (vocabulary slice, row, sequence): the
//     largest logit of the slice (with its lowest index) and the slice's sum
//     of exp(x / T - slice max / T);
//  2. per sequence: merge the slices of the rows it needs, walk the chain,
//     then draw the next token by inverse CDF.  Each thread sums the weights
//     of its contiguous vocabulary slice; a block prefix sum in thread order
//     locates the slice whose running sum first passes u * total, and one
//     wave re-evaluates that slice (one entry per lane, prefix sum across
//     lanes) to find the entry.
#include "tf_internal.h"

namespace tfk {

constexpr int kStatThreads = 256;
constexpr int kStatSlice = 4096;       // vocabulary entries per statistics workgroup
constexpr int kDrawThreads = 1024;
constexpr int kDrawIpt = 64;           // vocabulary entries per draw thread (at most one wave)

struct SliceStat {
  float mx;   // largest logit in the slice
  int amax;   // its lowest index
  double z;   // sum over the slice of exp(x / T - mx / T)
};

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// ---------------------------------------------------------------------------
// Kernel 1: one workgroup per (slice, row, sequence), flattened into
// grid.x = slice + nslices * (row + nrows * b).  Rows 0..gamma are target
// rows, rows gamma+1 .. 2*gamma are draft rows 0..gamma-1.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kStatThreads) void accept_stats_kernel(const float* __restrict__ target,
                                                                    const float* __restrict__ draft, int32_t gamma,
                                                                    int32_t V, float temperature, int32_t nslices,
                                                                    SliceStat* __restrict__ stats) {
  __shared__ float s_v[kStatThreads / 64];
  __shared__ int s_i[kStatThreads / 64];
  __shared__ double s_z[kStatThreads / 64];
  const int nrows = 2 * gamma + 1;
  const int slice = (int)(blockIdx.x % (unsigned)nslices);
  const int r = (int)((blockIdx.x / (unsigned)nslices) % (unsigned)nrows);
  const int b = (int)(blockIdx.x / ((unsigned)nslices * (unsigned)nrows));
  const float* row = (r <= gamma) ? target + ((size_t)b * (gamma + 1) + r) * V
                                  : draft + ((size_t)b * gamma + (r - gamma - 1)) * V;
  const int v0 = slice * kStatSlice, v1 = min(V, v0 + kStatSlice);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float bv = -__builtin_huge_valf();
  int bi = 0x7fffffff;
  for (int v = v0 + threadIdx.x; v < v1; v += kStatThreads) {
    const float x = row[v];
    if (better(x, v, bv, bi)) {
      bv = x;
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
  for (int x = 1; x < kStatThreads / 64; ++x)
    if (better(s_v[x], s_i[x], bv, bi)) {
      bv = s_v[x];
      bi = s_i[x];
    }
  double z = 0.0;
  if (temperature > 0.f) {
    const double t = (double)temperature;
    const double zm = (double)bv / t;
    for (int v = v0 + threadIdx.x; v < v1; v += kStatThreads) z += exp((double)row[v] / t - zm);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
    if (lane == 0) s_z[w] = z;
    __syncthreads();
    z = 0.0;
#pragma unroll
    for (int x = 0; x < kStatThreads / 64; ++x) z += s_z[x];
  }
  if (threadIdx.x == 0) {
    SliceStat st;
    st.mx = bv;
    st.amax = bi;
    st.z = z;
    stats[((size_t)b * nrows + r) * nslices + slice] = st;
  }
}

// Distribution of one row after merging its slices.
struct RowDist {
  int mode;     // 0 softmax(x / T), 1 greedy one-hot, 2 probabilities as given
  double zmax;  // max x / T
  double Z;     // sum of exp(x / T - zmax)
  int amax;
};

__device__ RowDist merge_row(const SliceStat* st, int nslices, float temperature, int probs) {
  RowDist d;
  d.zmax = 0.0;
  d.Z = 1.0;
  d.amax = 0;
  if (probs) {
    d.mode = 2;
    return d;
  }
  float bv = st[0].mx;
  int bi = st[0].amax;
  for (int s = 1; s < nslices; ++s)
    if (better(st[s].mx, st[s].amax, bv, bi)) {
      bv = st[s].mx;
      bi = st[s].amax;
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
  for (int s = 0; s < nslices; ++s)
    if (st[s].z > 0.0) Z += st[s].z * exp((double)st[s].mx / t - d.zmax);
  d.Z = Z;
  return d;
}

__device__ __forceinline__ double dist_p(const RowDist& d, const float* row, int v, float temperature) {
  if (d.mode == 2) return (double)row[v];
  if (d.mode == 1) return v == d.amax ? 1.0 : 0.0;
  return exp((double)row[v] / (double)temperature - d.zmax) / d.Z;
}

// Prefix sums over the 1024 threads in thread order (fp64): returns the
// inclusive sum, stores the exclusive one in *excl and the block total in
// *s_total.
__device__ __forceinline__ double block_scan(double x, double* s_scan, double* s_total, double* excl) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  double ex = __shfl_up(incl, 1);
  if (lane == 0) ex = 0.0;
  if (lane == 63) s_scan[w] = incl;
  __syncthreads();
  double off_w = 0.0;
  for (int x2 = 0; x2 < w; ++x2) off_w += s_scan[x2];
  if (threadIdx.x == kDrawThreads - 1) *s_total = off_w + incl;
  __syncthreads();
  *excl = off_w + ex;
  return off_w + incl;
}

// ---------------------------------------------------------------------------
// Kernel 2: grid (B), 1024 threads.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kDrawThreads) void accept_draw_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ tokens,
    const double* __restrict__ uniforms, int32_t gamma, int32_t V, float temperature, int32_t probs,
    const SliceStat* __restrict__ stats, int32_t nslices, int32_t* __restrict__ n_acc, int32_t* __restrict__ next) {
  __shared__ double s_scan[kDrawThreads / 64];
  __shared__ double s_tot;
  __shared__ int s_j;
  __shared__ int s_found;
  __shared__ int s_last;
  const int b = blockIdx.x;
  const int nrows = 2 * gamma + 1;
  const SliceStat* st = stats + (size_t)b * nrows * nslices;
  const float* trow0 = target + (size_t)b * (gamma + 1) * V;
  const float* drow0 = draft + (size_t)b * gamma * V;
  const double* u = uniforms + (size_t)b * (gamma + 1);

  // ---- the chain: one thread, a handful of exp() calls ----------------------
  if (threadIdx.x == 0) {
    int j = gamma;
    for (int i = 0; i < gamma; ++i) {
      const int x = tokens[(size_t)b * gamma + i];
      bool keep = false;
      if (x >= 0 && x < V) {  // a token outside [0, V) is never kept
        const RowDist dp = merge_row(st + (size_t)i * nslices, nslices, temperature, probs);
        const RowDist dq = merge_row(st + (size_t)(gamma + 1 + i) * nslices, nslices, temperature, probs);
        const double px = dist_p(dp, trow0 + (size_t)i * V, x, temperature);
        const double qx = dist_p(dq, drow0 + (size_t)i * V, x, temperature);
        if (px > 0.0) {
          const double alpha = (qx == 0.0) ? 1.0 : fmin(1.0, px / qx);
          keep = alpha >= u[i];
        }
      }
      if (!keep) {
        j = i;
        break;
      }
    }
    s_j = j;
  }
  __syncthreads();
  const int j = s_j;
  bool residual = j < gamma;
  const float* tr = trow0 + (size_t)j * V;
  const float* dr = drow0 + (size_t)(residual ? j : 0) * V;
  const RowDist dp = merge_row(st + (size_t)j * nslices, nslices, temperature, probs);
  const RowDist dq = residual ? merge_row(st + (size_t)(gamma + 1 + j) * nslices, nslices, temperature, probs) : dp;

  // ---- pass 1: each thread sums the weights of its contiguous slice --------
  const int ipt = (V + kDrawThreads - 1) / kDrawThreads;  // <= 64 (host-checked)
  const int v0 = threadIdx.x * ipt, v1 = min(V, v0 + ipt);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double local = 0.0;
  int last_pos = -1;
  for (int v = v0; v < v1; ++v) {
    const double p = dist_p(dp, tr, v, temperature);
    const double r = residual ? fmax(0.0, p - dist_p(dq, dr, v, temperature)) : p;
    if (r > 0.0) last_pos = v;
    local += r;
  }
  double before;
  double total = block_scan(local, s_scan, &s_tot, &before);
  if (residual && s_tot == 0.0) {
    // max(0, p - q) vanished (only through rounding): draw from p_j instead.
    residual = false;
    local = 0.0;
    last_pos = -1;
    for (int v = v0; v < v1; ++v) {
      const double p = dist_p(dp, tr, v, temperature);
      if (p > 0.0) last_pos = v;
      local += p;
    }
    total = block_scan(local, s_scan, &s_tot, &before);
  }
  // `total` is this thread's inclusive running sum; s_tot the row's sum.
  const double tgt = u[gamma] * s_tot;
  if (threadIdx.x == 0) {
    s_found = 0x7fffffff;
    s_last = -1;
  }
  __syncthreads();
  if (total > tgt) atomicMin(&s_found, (int)threadIdx.x);  // first slice whose end passes the target
  atomicMax(&s_last, last_pos);
  __syncthreads();
  const int tstar = s_found;
  if (tstar == 0x7fffffff) {
    // the running sum never passes u * total (rounding): the last index with
    // positive weight
    if (threadIdx.x == 0) {
      n_acc[b] = j;
      next[b] = s_last;
    }
    return;
  }
  if (threadIdx.x == tstar) s_tot = before;  // running sum before slice tstar
  __syncthreads();
  // ---- pass 2: one wave re-evaluates slice tstar, one element per lane ------
  if (w == 0) {
    const int v = tstar * ipt + lane;
    double r = 0.0;
    if (lane < ipt && v < V) {
      const double p = dist_p(dp, tr, v, temperature);
      r = residual ? fmax(0.0, p - dist_p(dq, dr, v, temperature)) : p;
    }
    double run = r;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(run, off);
      if (lane >= off) run += y;
    }
    run += s_tot;
    const unsigned long long hit = __ballot(r > 0.0 && run > tgt);
    const unsigned long long pos = __ballot(r > 0.0);
    if (lane == 0) {
      n_acc[b] = j;
      // without a crossing inside the slice (rounding), its last positive entry
      next[b] = hit ? tstar * ipt + (int)__builtin_ctzll(hit)
                    : (pos ? tstar * ipt + 63 - (int)__builtin_clzll(pos) : s_last);
    }
  }
}

size_t accept_ws_bytes(int32_t B, int32_t gamma, int32_t V) {
  if (B < 1 || gamma < 0 || V < 1) return 0;
  const size_t nslices = (size_t)(V + kStatSlice - 1) / kStatSlice;
  return ((size_t)B * (2 * gamma + 1) * nslices * sizeof(SliceStat) + 255) & ~(size_t)255;
}

int32_t accept_max_vocab() { return kDrawThreads * kDrawIpt; }

hipError_t launch_accept(const float* target, const float* draft, const int32_t* tokens,
                         const double* uniforms, int32_t B, int32_t gamma, int32_t V,
                         float temperature, int32_t flags, int32_t* n_acc, int32_t* next,
                         void* ws, hipStream_t stream) {
  const int probs = (flags & TF_ACCEPT_PROBS) != 0;
  const int nslices = (V + kStatSlice - 1) / kStatSlice;
  SliceStat* stats = (SliceStat*)ws;
  if (!probs) {
    const unsigned blocks = (unsigned)nslices * (unsigned)(2 * gamma + 1) * (unsigned)B;
    hipLaunchKernelGGL(accept_stats_kernel, dim3(blocks), dim3(kStatThreads), 0, stream, target, draft, gamma, V,
                       temperature, nslices, stats);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(accept_draw_kernel, dim3(B), dim3(kDrawThreads), 0, stream, target, draft, tokens, uniforms,
                     gamma, V, temperature, probs, stats, nslices, n_acc, next);
  return hipGetLastError();
}

}  // namespace tfk
