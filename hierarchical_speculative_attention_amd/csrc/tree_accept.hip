// Accept / reject over a candidate tree (TriForce blog: Force 3 evaluates the
// candidate tree Force 2 assembles, "1. The Three Forces of TriForce", with
// the acceptance rule and residual of "2. Dual Rejection Sampling").
//
// Node 0 is the last committed token, nodes 1 .. Q-1 candidates (parent[c] in
// [0, c), anything else hangs c off node 0).  Walking down from node 0, the
// children of the current node v are tried in index order: child c with token
// x is kept when p'(x) > 0 and u_c q_v(x) <= p'(x), where p' starts as the
// target row p_v and after each rejected sibling becomes max(0, p' - q_v)
// renormalised (p_v again if that vanishes through rounding).  A kept child
// becomes v; when no child is kept, or v has none, the next token is drawn
// from p' by inverse CDF.  With one child per node this is tf_accept.
//
// Kernels, in order.  (1) tree_stats_kernel, spread over (sequence,
// 2048-entry slice, row): for every target and draft row and every slice, the
// largest logit, its lowest index and the sum of exp(x / T - that max) in
// fp64.  Merging a row's slice statistics gives its max and normaliser, so
// p_v(x) and q_v(x) at one token cost one exponential.  (2) tree_zpass_kernel,
// once for each of the first kZPasses rejections at a node: the residual's
// normaliser after j rejections, for every node with at least j children, as
// partial sums over slices (the residuals do not depend on which path the
// walk takes, only on the node and the rejections there).  (3)
// tree_accept_kernel, one 1024-thread workgroup per sequence (the walk is
// sequential: which child is kept decides the next rows): testing a child
// needs p'(x) at one token, and with the normalisers at hand no pass over the
// vocabulary either; only a node with more rejections than were precomputed
// makes passes here (p' = max(0, p' - q_v), kept in a caller workspace as
// fp64 weights times a running scale, with q_v stored beside it when a
// further sibling may need it; thread t owns entries t, t + 1024, ..., eight
// entries' loads in flight), and then also draws the next token itself (16
// contiguous segments, one per wave: segment totals give the segment where
// the CDF passes u * total, then that segment is narrowed again and scanned).
// (4) tree_draw_slice_kernel and (5) tree_draw_final_kernel otherwise draw it
// from the chain of normalisers spread over 1024-entry slices: weights and
// their sums per slice, then one prefix over the slices and a block prefix
// sum over the crossing slice.  Everything is fp64, so decisions are taken in
// the oracle's precision.  A 7-node binary tree at V = 32000: one walk kernel
// with a pass per rejection and a one-workgroup draw took 46 us (52 us per
// call with the statistics); these kernels take 35.7 us per call.
#include "tf_internal.h"

namespace tfk {

constexpr int kTreeThreads = 1024;
constexpr int kTreeWaves = kTreeThreads / 64;
constexpr int kTreeBatch = 4;                   // fp32 entries per thread per batch
constexpr int kTreeBatchD = 4;                  // fp64 entries per thread per batch
constexpr int kTreeMaxVocab = 65536;
constexpr int kTreeMaxQ = 64;
constexpr int kTreeSlice = 2048;                // vocabulary entries per statistics slice
constexpr int kStatThreads = 256;
constexpr int kStatIpt = kTreeSlice / kStatThreads;
constexpr int kZPasses = 2;                     // rejections per node whose normalisers are summed in parallel
constexpr int kTreeDraw = 1024;                 // vocabulary entries per draw slice
constexpr int kTreeDrawPer = kTreeDraw / kStatThreads;

// Statistics of one slice of one row: largest logit, its lowest index, and
// sum over the slice of exp(x / T - max / T) (0 for greedy rows).
struct SliceStat {
  double ssum;
  float bmax;
  int amax;
};
static_assert(sizeof(SliceStat) == 16, "slice statistics are 16 bytes");

// How a row turns into a distribution: softmax(x / T) (mode 0: exp(x / T -
// zmax) * invZ), greedy one-hot at the lowest index of the largest logit
// (mode 1), or probabilities as given (mode 2).
struct RowStat {
  int mode;
  double zmax;
  double invZ;
  int amax;
};

struct TreeShared {
  double d[kTreeWaves];
  float f[kTreeWaves];
  int i[kTreeWaves];
};

__device__ __forceinline__ double scaled(float x, double t, bool div) { return div ? (double)x / t : (double)x; }

// p' at one entry after j rejections at a node, from p_v and q_v there and
// the normalisers z[0 .. j-1] of the residuals: p'_0 = p; R_i = max(0,
// p'_(i-1) - q); p'_i = R_i / z[i-1] (as a product by 1 / z), or p again when
// z[i-1] vanished.  The same arithmetic as a residual stored and rescaled.
__device__ __forceinline__ double chain_value(double p, double q, const double* z, int j) {
  double pc = p;
  for (int i = 0; i < j; ++i) {
    const double r = fmax(0.0, pc - q);
    pc = z[i] > 0.0 ? r * (1.0 / z[i]) : p;
  }
  return pc;
}

// Where the walk left a sequence: the node and the rejections there whose p'
// the next token is drawn from, or done (the walk drew it itself).
struct TreeWalk {
  int done;
  int v;
  int vj;
  int pad;
};

// ---- (1) slice statistics -------------------------------------------------
__global__ __launch_bounds__(kStatThreads) void tree_stats_kernel(const float* __restrict__ target,
                                                                  const float* __restrict__ draft, int32_t Q,
                                                                  int32_t V, int32_t nslice, float temperature,
                                                                  SliceStat* __restrict__ stats) {
  __shared__ float s_f[kStatThreads / 64];
  __shared__ int s_i[kStatThreads / 64];
  __shared__ double s_d[kStatThreads / 64];
  const int b = blockIdx.x / nslice, sl = blockIdx.x % nslice, r = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* row = r < Q ? target + ((size_t)b * Q + r) * V : draft + ((size_t)b * Q + (r - Q)) * V;
  const int v0 = sl * kTreeSlice, v1 = min(V, v0 + kTreeSlice);
  float x[kStatIpt];
#pragma unroll
  for (int j = 0; j < kStatIpt; ++j) x[j] = row[min(v0 + j * kStatThreads + tid, v1 - 1)];
  float bv = -__builtin_huge_valf();
  int bi = 0x7fffffff;
#pragma unroll
  for (int j = 0; j < kStatIpt; ++j) {
    const int e = v0 + j * kStatThreads + tid;
    if (e < v1 && (x[j] > bv || (x[j] == bv && e < bi))) {
      bv = x[j];
      bi = e;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  if (lane == 0) {
    s_f[w] = bv;
    s_i[w] = bi;
  }
  __syncthreads();
  bv = s_f[0];
  bi = s_i[0];
#pragma unroll
  for (int q = 1; q < kStatThreads / 64; ++q)
    if (s_f[q] > bv || (s_f[q] == bv && s_i[q] < bi)) {
      bv = s_f[q];
      bi = s_i[q];
    }
  double local = 0.0;
  if (temperature != 0.f && bv > -__builtin_huge_valf()) {
    const double t = (double)temperature;
    const bool div = t != 1.0;
    const double m = scaled(bv, t, div);
#pragma unroll
    for (int j = 0; j < kStatIpt; ++j) {
      const int e = v0 + j * kStatThreads + tid;
      if (e < v1) local += exp(scaled(x[j], t, div) - m);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
  if (lane == 0) s_d[w] = local;
  __syncthreads();
  if (tid == 0) {
    double sum = 0.0;
#pragma unroll
    for (int q = 0; q < kStatThreads / 64; ++q) sum += s_d[q];
    SliceStat st;
    st.ssum = sum;
    st.bmax = bv;
    st.amax = bi;
    const int slot = r < Q ? r : kTreeMaxQ + (r - Q);  // draft rows from slot kTreeMaxQ on
    stats[((size_t)b * 2 * kTreeMaxQ + slot) * nslice + sl] = st;
  }
}

// ---- (2) the walk ---------------------------------------------------------
// Block reductions in a fixed order (16 wave partials summed by every thread).
__device__ __forceinline__ double tree_sum(double x, TreeShared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  __syncthreads();
  if (lane == 0) sh.d[w] = x;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int q = 0; q < kTreeWaves; ++q) s += sh.d[q];
  return s;
}

__device__ __forceinline__ int tree_max_int(int x, TreeShared& sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = max(x, __shfl_xor(x, off));
  __syncthreads();
  if (lane == 0) sh.i[w] = x;
  __syncthreads();
  int m = sh.i[0];
#pragma unroll
  for (int q = 1; q < kTreeWaves; ++q) m = max(m, sh.i[q]);
  return m;
}

// Every row's distribution from its slices, into s_rs (target row v at slot
// v, draft row v at slot kTreeMaxQ + v).  Wave w merges rows w, w + 16, ...;
// lane s holds slice s (at most 32 slices).  The largest logit's lowest index
// wins ties.
__device__ void merge_rows(const SliceStat* st, int nslice, int nt, int nd, float temperature, int probs,
                           RowStat* s_rs) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const double t = (double)temperature;
  const bool div = t != 1.0;
  for (int r = w; r < nt + nd; r += kTreeWaves) {
    const int slot = r < nt ? r : kTreeMaxQ + (r - nt);
    RowStat d;
    d.zmax = 0.0;
    d.invZ = 1.0;
    d.amax = 0;
    if (probs) {
      d.mode = 2;
    } else {
      const bool ok = lane < nslice;
      const SliceStat x = st[(size_t)slot * nslice + min(lane, nslice - 1)];
      float bv = ok ? x.bmax : -__builtin_huge_valf();
      int bi = ok ? x.amax : 0x7fffffff;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (ov > bv || (ov == bv && oi < bi)) {
          bv = ov;
          bi = oi;
        }
      }
      d.amax = bi;
      if (temperature == 0.f) {
        d.mode = 1;
      } else {
        d.mode = 0;
        d.zmax = scaled(bv, t, div);
        double z = (ok && x.bmax > -__builtin_huge_valf()) ? x.ssum * exp(scaled(x.bmax, t, div) - d.zmax) : 0.0;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
        d.invZ = 1.0 / z;
      }
    }
    if (lane == 0) s_rs[slot] = d;
  }
}

// One row's distribution from its slices, by one wave (lane s holds slice
// s): the same result as merge_rows gives that row.
__device__ RowStat merge_row_wave(const SliceStat* st, int nslice, float temperature, int probs) {
  const int lane = threadIdx.x & 63;
  const double t = (double)temperature;
  const bool div = t != 1.0;
  RowStat d;
  d.zmax = 0.0;
  d.invZ = 1.0;
  d.amax = 0;
  if (probs) {
    d.mode = 2;
    return d;
  }
  const bool ok = lane < nslice;
  const SliceStat x = st[min(lane, nslice - 1)];
  float bv = ok ? x.bmax : -__builtin_huge_valf();
  int bi = ok ? x.amax : 0x7fffffff;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  d.amax = bi;
  if (temperature == 0.f) {
    d.mode = 1;
    return d;
  }
  d.mode = 0;
  d.zmax = scaled(bv, t, div);
  double z = (ok && x.bmax > -__builtin_huge_valf()) ? x.ssum * exp(scaled(x.bmax, t, div) - d.zmax) : 0.0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) z += __shfl_xor(z, off);
  d.invZ = 1.0 / z;
  return d;
}

// Probability of one entry under a row's distribution (runtime mode).
__device__ __forceinline__ double prob_x(float x, int e, const RowStat& d, double t) {
  if (d.mode == 2) return (double)x;
  if (d.mode == 1) return e == d.amax ? 1.0 : 0.0;
  return exp(scaled(x, t, t != 1.0) - d.zmax) * d.invZ;
}

// Normaliser of node v's residual after j rejections, as partial sums over
// 2048-entry slices: zpart[b][v][j-1][slice] = sum over the slice of
// max(0, p'_(j-1) - q_v), p'_(j-1) from the sums of the earlier passes.
// Grid (sequences x slices, nodes); nodes with fewer than j children exit.
constexpr int kZThreads = 1024;
constexpr int kZIpt = kTreeSlice / kZThreads;

__global__ __launch_bounds__(kZThreads) void tree_zpass_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ parent, int32_t Q,
    int32_t V, int32_t nslice, float temperature, int32_t probs, const SliceStat* __restrict__ stats,
    double* __restrict__ zpart, int32_t j) {
  __shared__ int s_nc;
  __shared__ RowStat s_rs[2];
  __shared__ double s_z[kZPasses];
  __shared__ double s_d[kZThreads / 64];
  const int b = blockIdx.x / nslice, sl = blockIdx.x % nslice, v = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // Every load is issued before any is waited on: this slice's logits (all
  // threads), the two rows' statistics (waves 0 and 1), the children count
  // (wave 2) and the earlier passes' partial sums (wave 3).
  const float* trow = target + ((size_t)b * Q + v) * V;
  const float* drow = draft + ((size_t)b * Q + v) * V;
  const int v0 = sl * kTreeSlice, v1 = min(V, v0 + kTreeSlice);
  float xp[kZIpt], xq[kZIpt];
#pragma unroll
  for (int k = 0; k < kZIpt; ++k) {
    const int e = min(v0 + k * kZThreads + tid, v1 - 1);
    xp[k] = trow[e];
    xq[k] = drow[e];
  }
  const SliceStat* st = stats + (size_t)b * 2 * kTreeMaxQ * nslice;
  if (w < 2) {
    const RowStat d = merge_row_wave(st + (size_t)(w == 0 ? v : kTreeMaxQ + v) * nslice, nslice, temperature, probs);
    if (lane == 0) s_rs[w] = d;
  } else if (w == 2) {
    bool child = false;
    if (lane >= 1 && lane < Q) {
      const int pc = parent[(size_t)b * Q + lane];
      child = ((pc >= 0 && pc < lane) ? pc : 0) == v;
    }
    const int nc = __popcll(__ballot(child));
    if (lane == 0) s_nc = nc;
  } else if (w == 3 && lane < j - 1) {
    double z = 0.0;
    const double* zp = zpart + (((size_t)b * kTreeMaxQ + v) * kZPasses + lane) * nslice;
    for (int q = 0; q < nslice; ++q) z += zp[q];
    s_z[lane] = z;
  }
  __syncthreads();
  if (s_nc < j) return;
  const RowStat dp = s_rs[0], dq = s_rs[1];
  const double t = (double)temperature;
  double local = 0.0;
#pragma unroll
  for (int k = 0; k < kZIpt; ++k) {
    const int e = v0 + k * kZThreads + tid;
    if (e < v1) {
      const double q = prob_x(xq[k], e, dq, t);
      local += fmax(0.0, chain_value(prob_x(xp[k], e, dp, t), q, s_z, j - 1) - q);
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) local += __shfl_xor(local, off);
  if (lane == 0) s_d[w] = local;
  __syncthreads();
  if (tid == 0) {
    double sum = 0.0;
#pragma unroll
    for (int q = 0; q < kZThreads / 64; ++q) sum += s_d[q];
    zpart[(((size_t)b * kTreeMaxQ + v) * kZPasses + (j - 1)) * nslice + sl] = sum;
  }
}

template <int MODE, bool kDiv>
__device__ __forceinline__ double prob_t(float x, int e, const RowStat& d, double t) {
  if (MODE == 2) return (double)x;
  if (MODE == 1) return e == d.amax ? 1.0 : 0.0;
  return exp(scaled(x, t, kDiv) - d.zmax) * d.invZ;
}

// First rejection at a node: p' = max(0, p_v - q_v) from the logits, written to
// pr (and q_v to qb when store_q); returns this thread's sum.  The next
// batch's loads are issued before the current batch is used (past the end they
// read entry V - 1, unused).
template <int MODE, bool kDiv>
__device__ double first_reject_t(const float* trow, const float* drow, const RowStat& dp, const RowStat& dq,
                                 double t, int V, double* pr, double* qb, bool store_q, const double* z, int vj) {
  constexpr int kStep = kTreeThreads * kTreeBatch;
  const int tid = threadIdx.x;
  double local = 0.0;
  float xp[kTreeBatch], xq[kTreeBatch];
#pragma unroll
  for (int j = 0; j < kTreeBatch; ++j) {
    const int e = min(j * kTreeThreads + tid, V - 1);
    xp[j] = trow[e];
    xq[j] = drow[e];
  }
  for (int e0 = 0; e0 < V; e0 += kStep) {
    float np[kTreeBatch], nq[kTreeBatch];
#pragma unroll
    for (int j = 0; j < kTreeBatch; ++j) {
      const int e = min(e0 + kStep + j * kTreeThreads + tid, V - 1);
      np[j] = trow[e];
      nq[j] = drow[e];
    }
#pragma unroll
    for (int j = 0; j < kTreeBatch; ++j) {
      const int e = e0 + j * kTreeThreads + tid;
      if (e < V) {
        const double q = prob_t<MODE, kDiv>(xq[j], e, dq, t);
        const double r = fmax(0.0, chain_value(prob_t<MODE, kDiv>(xp[j], e, dp, t), q, z, vj) - q);
        pr[e] = r;
        if (store_q) qb[e] = q;
        local += r;
      }
    }
#pragma unroll
    for (int j = 0; j < kTreeBatch; ++j) {
      xp[j] = np[j];
      xq[j] = nq[j];
    }
  }
  return local;
}

__device__ double first_reject(const float* trow, const float* drow, const RowStat& dp, const RowStat& dq, double t,
                               int V, double* pr, double* qb, bool store_q, const double* z, int vj) {
  if (dp.mode == 2) return first_reject_t<2, false>(trow, drow, dp, dq, t, V, pr, qb, store_q, z, vj);
  if (dp.mode == 1) return first_reject_t<1, false>(trow, drow, dp, dq, t, V, pr, qb, store_q, z, vj);
  return t == 1.0 ? first_reject_t<0, false>(trow, drow, dp, dq, t, V, pr, qb, store_q, z, vj)
                  : first_reject_t<0, true>(trow, drow, dp, dq, t, V, pr, qb, store_q, z, vj);
}

// A further rejection at the node: p' = max(0, pr * scale - qb), written back
// (loads pipelined as in first_reject_t).
__device__ double next_reject(double* pr, const double* qb, int V, double scale) {
  constexpr int kStep = kTreeThreads * kTreeBatchD;
  const int tid = threadIdx.x;
  double local = 0.0;
  double pv[kTreeBatchD], qv[kTreeBatchD];
#pragma unroll
  for (int j = 0; j < kTreeBatchD; ++j) {
    const int e = min(j * kTreeThreads + tid, V - 1);
    pv[j] = pr[e];
    qv[j] = qb[e];
  }
  for (int e0 = 0; e0 < V; e0 += kStep) {
    double np[kTreeBatchD], nq[kTreeBatchD];
#pragma unroll
    for (int j = 0; j < kTreeBatchD; ++j) {
      const int e = min(e0 + kStep + j * kTreeThreads + tid, V - 1);
      np[j] = pr[e];
      nq[j] = qb[e];
    }
#pragma unroll
    for (int j = 0; j < kTreeBatchD; ++j) {
      const int e = e0 + j * kTreeThreads + tid;
      if (e < V) {
        const double r = fmax(0.0, pv[j] * scale - qv[j]);
        pr[e] = r;
        local += r;
      }
    }
#pragma unroll
    for (int j = 0; j < kTreeBatchD; ++j) {
      pv[j] = np[j];
      qv[j] = nq[j];
    }
  }
  return local;
}

__device__ __forceinline__ double wave_incl_scan(double x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Values of p' over this wave's segment [s0, s1), 64 entries per step.
template <int MODE, bool kDiv, bool kStored>
struct DrawSrc {
  const float* trow;
  const double* pr;
  RowStat d;
  double t, scale;
  int V;
  __device__ __forceinline__ void load(int e, float& x, double& y) const {
    const int ec = min(e, V - 1);
    if (kStored)
      y = pr[ec];
    else
      x = trow[ec];
  }
  __device__ __forceinline__ double value(int e, float x, double y) const {
    return kStored ? y * scale : prob_t<MODE, kDiv>(x, e, d, t);
  }
};

// Sum of p' over [a, b) by one wave (64 entries per step, kTreeBatchD steps per
// batch, the next batch's loads issued before the current one is used), and
// the last positive entry there.
template <class Src>
__device__ __forceinline__ double wave_range_sum(const Src& src, int a, int b, int& last_pos) {
  const int lane = threadIdx.x & 63;
  double part = 0.0;
  float x[kTreeBatchD];
  double y[kTreeBatchD];
#pragma unroll
  for (int j = 0; j < kTreeBatchD; ++j) src.load(a + 64 * j + lane, x[j], y[j]);
  for (int i0 = a; i0 < b; i0 += 64 * kTreeBatchD) {
    float nx[kTreeBatchD];
    double ny[kTreeBatchD];
#pragma unroll
    for (int j = 0; j < kTreeBatchD; ++j) src.load(i0 + 64 * (kTreeBatchD + j) + lane, nx[j], ny[j]);
#pragma unroll
    for (int j = 0; j < kTreeBatchD; ++j) {
      const int e = i0 + 64 * j + lane;
      if (e < b) {
        const double v = src.value(e, x[j], y[j]);
        part += v;
        if (v > 0.0) last_pos = max(last_pos, e);
      }
    }
#pragma unroll
    for (int j = 0; j < kTreeBatchD; ++j) {
      x[j] = nx[j];
      y[j] = ny[j];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) part += __shfl_xor(part, off);
  return part;
}

// The first of 16 wave partials (in sh.d) whose running sum, from base,
// passes tgt; -1 if none.  *before = the running sum ahead of it.
__device__ __forceinline__ int first_passing(const TreeShared& sh, double base, double tgt, double* before) {
  int wx = -1;
  double run = base;
  *before = base;
#pragma unroll
  for (int q = 0; q < kTreeWaves; ++q) {
    if (wx < 0 && run + sh.d[q] > tgt) {
      wx = q;
      *before = run;
    }
    run += sh.d[q];
  }
  return wx;
}

// Inverse CDF over p' with target fraction uf (strict '>': the first entry
// whose inclusive running sum passes uf * total; when rounding keeps the sum
// from passing it, the last positive entry of the range being searched).  The
// vocabulary is narrowed in three steps: 16 segments (one per wave), 16
// pieces of the segment the CDF passes the target in (one per wave), then the
// wave of the piece scans it in order.
template <class Src>
__device__ int draw(const Src& src, int V, double uf, TreeShared& sh, int* s_found) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int seg = (V + kTreeThreads - 1) / kTreeThreads * 64;  // a multiple of 64; 16 segments cover V
  int last1 = -1;
  const double part1 = wave_range_sum(src, w * seg, min(V, w * seg + seg), last1);
  __syncthreads();
  if (lane == 0) sh.d[w] = part1;
  if (tid == 0) *s_found = 0x7fffffff;
  __syncthreads();
  double total = 0.0;
#pragma unroll
  for (int q = 0; q < kTreeWaves; ++q) total += sh.d[q];
  const double tgt = uf * total;
  double before;
  const int wx = first_passing(sh, 0.0, tgt, &before);
  const int lastV = tree_max_int(last1, sh);
  if (wx < 0) return lastV;
  // pieces of segment wx
  const int a0 = wx * seg, a1 = min(V, a0 + seg);
  const int piece = (seg + kTreeWaves - 1) / kTreeWaves;
  const int p0 = min(a1, a0 + w * piece), p1 = min(a1, p0 + piece);
  int last2 = -1;
  const double part2 = wave_range_sum(src, p0, p1, last2);
  __syncthreads();
  if (lane == 0) sh.d[w] = part2;
  __syncthreads();
  double before2;
  const int wy = first_passing(sh, before, tgt, &before2);
  const int lastS = tree_max_int(last2, sh);  // the segment's last positive entry
  if (wy < 0) return lastS;
  if (w == wy) {
    double run = before2;
    bool done = false;
    int lastP = -1;
    for (int i0 = p0; i0 < p1 && !done; i0 += 64) {
      float x;
      double y;
      src.load(i0 + lane, x, y);
      const int e = i0 + lane;
      const double v = e < p1 ? src.value(e, x, y) : 0.0;
      const double incl = wave_incl_scan(v, lane);
      const unsigned long long hit = __ballot(v > 0.0 && run + incl > tgt);
      const unsigned long long pos = __ballot(v > 0.0);
      if (pos != 0ull) lastP = i0 + 63 - __builtin_clzll(pos);
      if (hit != 0ull) {
        if (lane == 0) *s_found = i0 + __builtin_ctzll(hit);
        done = true;
      }
      run += __shfl(incl, 63);
    }
    if (!done && lane == 0) *s_found = lastP;  // the piece's last positive entry
  }
  __syncthreads();
  return *s_found;
}

__global__ __launch_bounds__(kTreeThreads) void tree_accept_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ parent, const double* __restrict__ uniforms, int32_t Q, int32_t V, int32_t nslice,
    float temperature, int32_t probs, double* __restrict__ ws, const SliceStat* __restrict__ stats,
    const double* __restrict__ zpart, TreeWalk* __restrict__ walk, int32_t* __restrict__ n_acc,
    int32_t* __restrict__ path, int32_t* __restrict__ next) {
  __shared__ int s_par[kTreeMaxQ], s_tok[kTreeMaxQ];
  __shared__ float s_xt[kTreeMaxQ], s_xd[kTreeMaxQ];  // the parent's target / draft logit at each child's token
  __shared__ RowStat s_rs[2 * kTreeMaxQ];
  __shared__ double s_z[kTreeMaxQ][kZPasses];
  __shared__ TreeShared sh;
  __shared__ int s_found;
  const int b = blockIdx.x, tid = threadIdx.x;
  const double t = (double)temperature;
  double* pr = ws + (size_t)b * 2 * V;  // p' = pr[e] * scale once a rejection happened
  double* qb = pr + V;                  // q_v, stored for a further sibling
  const SliceStat* st = stats + (size_t)b * 2 * kTreeMaxQ * nslice;
  // Three independent chains of loads, on different waves: the tree and the
  // parent's logits at each child's token (wave 14), the precomputed
  // normalisers, summed over their slices in order (wave 15; entries of nodes
  // with fewer children hold whatever the workspace held and are never used),
  // and the rows' statistics (every wave, in merge_rows).
  const int lane = tid & 63, w = tid >> 6;
  if (w == kTreeWaves - 2 && lane < Q) {
    const int p = parent[(size_t)b * Q + lane];
    const int pc = (lane > 0 && p >= 0 && p < lane) ? p : (lane > 0 ? 0 : -1);
    const int x = tokens[(size_t)b * Q + lane];
    s_par[lane] = pc;
    s_tok[lane] = x;
    if (lane > 0 && x >= 0 && x < V) {
      s_xt[lane] = target[((size_t)b * Q + pc) * V + x];
      s_xd[lane] = draft[((size_t)b * Q + pc) * V + x];
    }
  } else if (w == kTreeWaves - 1) {
    for (int i = lane; i < Q * kZPasses; i += 64) {
      const double* zp = zpart + ((size_t)b * kTreeMaxQ * kZPasses + i) * nslice;
      double z = 0.0;
      for (int q = 0; q < nslice; ++q) z += zp[q];
      s_z[i / kZPasses][i % kZPasses] = z;
    }
  }
  merge_rows(st, nslice, Q, Q > 1 ? Q : 0, temperature, probs, s_rs);
  __syncthreads();
  const double* u = uniforms + (size_t)b * Q;
  int v = 0, npath = 0;
  // p' = pr * scale when stored; otherwise the chain of vj precomputed
  // normalisers over p_v (p_v itself at vj = 0)
  bool stored = false;
  int vj = 0;
  double scale = 1.0;
  RowStat dp;
  while (true) {
    const float* trow = target + ((size_t)b * Q + v) * V;
    dp = s_rs[v];
    stored = false;
    vj = 0;
    int kept = -1;
    int n_child = 0;
    for (int c = v + 1; c < Q; ++c) n_child += s_par[c] == v;
    if (n_child > 0) {
      const float* drow = draft + ((size_t)b * Q + v) * V;
      const RowStat dq = s_rs[kTreeMaxQ + v];
      for (int c = v + 1; c < Q; ++c) {
        if (s_par[c] != v) continue;
        --n_child;  // siblings still to try after c
        const int x = s_tok[c];
        const bool valid = x >= 0 && x < V;
        // every thread evaluates the test itself (pr entries of other threads
        // are visible: the last pass ended with a block reduction)
        const double qx = !valid ? 0.0 : prob_x(s_xd[c], x, dq, t);
        const double px = !valid ? 0.0 : stored ? pr[x] * scale : chain_value(prob_x(s_xt[c], x, dp, t), qx, s_z[v], vj);
        if (valid && px > 0.0 && u[c - 1] * qx <= px) {
          kept = c;
          break;
        }
        // rejected: p' = max(0, p' - q_v) renormalised (p_v if it vanished);
        // its normaliser is precomputed for the first kZPasses rejections
        if (!stored && vj < kZPasses) {
          ++vj;
          continue;
        }
        double local;
        if (!stored) {
          local = first_reject(trow, drow, dp, dq, t, V, pr, qb, n_child > 0, s_z[v], vj);
        } else {
          local = next_reject(pr, qb, V, scale);
        }
        const double Z = tree_sum(local, sh);
        stored = Z > 0.0;
        scale = stored ? 1.0 / Z : 1.0;
        vj = 0;
      }
    }
    if (kept < 0) break;
    if (tid == 0) path[(size_t)b * (Q - 1) + npath] = kept;
    ++npath;
    v = kept;
    __syncthreads();  // the node's reads of pr / qb are done before the next node writes them
  }

  if (tid == 0) n_acc[b] = npath;
  for (int i = npath + tid; i < Q - 1; i += kTreeThreads) path[(size_t)b * (Q - 1) + i] = -1;
  if (!stored) {
    // p' is p_v or a chain of precomputed normalisers: the draw kernels take it
    if (tid == 0) {
      TreeWalk wk;
      wk.done = 0;
      wk.v = v;
      wk.vj = vj;
      wk.pad = 0;
      walk[b] = wk;
    }
    return;
  }
  // p' stored (more rejections at the node than were precomputed): drawn
  // here; its entries were written by every thread, so they must be visible
  __syncthreads();
  const float* trow = target + ((size_t)b * Q + v) * V;
  const int nx = draw(DrawSrc<2, false, true>{trow, pr, dp, t, scale, V}, V, u[Q - 1], sh, &s_found);
  if (tid == 0) {
    next[b] = nx;
    TreeWalk wk;
    wk.done = 1;
    wk.v = v;
    wk.vj = 0;
    wk.pad = 0;
    walk[b] = wk;
  }
}

// ---- (3) the draw from p' when the walk left it as a chain ----------------
struct DrawSum {
  double s;   // sum of the slice's weights
  int last;   // its last entry with positive weight (or -1)
  int pad;
};

// Weights of one kTreeDraw-entry slice of p' where the walk left each
// sequence (stored for the final scan), their sum and last positive entry.
// Grid (sequences x draw slices).
__global__ __launch_bounds__(kStatThreads) void tree_draw_slice_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, int32_t Q, int32_t V, int32_t nslice,
    int32_t ndraw, float temperature, int32_t probs, const SliceStat* __restrict__ stats,
    const double* __restrict__ zpart, const TreeWalk* __restrict__ walk, double* __restrict__ weights,
    DrawSum* __restrict__ sums) {
  __shared__ RowStat s_rs[2];
  __shared__ double s_z[kZPasses];
  __shared__ double s_d[kStatThreads / 64];
  __shared__ int s_i[kStatThreads / 64];
  const int b = blockIdx.x / ndraw, slice = blockIdx.x % ndraw;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const TreeWalk wk = walk[b];
  if (wk.done) return;
  const int v = wk.v, vj = wk.vj;
  const SliceStat* st = stats + (size_t)b * 2 * kTreeMaxQ * nslice;
  if (w == 0 || (w == 1 && vj > 0)) {
    const RowStat d = merge_row_wave(st + (size_t)(w == 0 ? v : kTreeMaxQ + v) * nslice, nslice, temperature, probs);
    if (lane == 0) s_rs[w] = d;
  }
  if (tid < vj) {
    const double* zp = zpart + (((size_t)b * kTreeMaxQ + v) * kZPasses + tid) * nslice;
    double z = 0.0;
    for (int q = 0; q < nslice; ++q) z += zp[q];
    s_z[tid] = z;
  }
  const float* trow = target + ((size_t)b * Q + v) * V;
  const float* drow = vj > 0 ? draft + ((size_t)b * Q + v) * V : trow;
  const int v0 = slice * kTreeDraw, v1 = min(V, v0 + kTreeDraw);
  float xp[kTreeDrawPer], xq[kTreeDrawPer];
#pragma unroll
  for (int k = 0; k < kTreeDrawPer; ++k) {
    const int e = min(v0 + tid + kStatThreads * k, V - 1);
    xp[k] = trow[e];
    xq[k] = drow[e];
  }
  __syncthreads();
  const RowStat dp = s_rs[0];
  const RowStat dq = vj > 0 ? s_rs[1] : dp;
  const double t = (double)temperature;
  double* wr = weights + (size_t)b * V;
  double sum = 0.0;
  int last = -1;
#pragma unroll
  for (int k = 0; k < kTreeDrawPer; ++k) {
    const int e = v0 + tid + kStatThreads * k;
    if (e >= v1) continue;
    const double p = prob_x(xp[k], e, dp, t);
    const double x = vj > 0 ? chain_value(p, prob_x(xq[k], e, dq, t), s_z, vj) : p;
    wr[e] = x;
    sum += x;
    if (x > 0.0) last = e;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    sum += __shfl_xor(sum, off);
    last = max(last, __shfl_xor(last, off));
  }
  if (lane == 0) {
    s_d[w] = sum;
    s_i[w] = last;
  }
  __syncthreads();
  if (tid == 0) {
    DrawSum o;
    o.s = (s_d[0] + s_d[1]) + (s_d[2] + s_d[3]);
    o.last = max(max(s_i[0], s_i[1]), max(s_i[2], s_i[3]));
    o.pad = 0;
    sums[(size_t)b * ndraw + slice] = o;
  }
}

// Inverse CDF over the stored weights, one workgroup per sequence: wave 0
// finds the draw slice whose running sum first passes u * total (lane s holds
// slice s), then thread t of that slice owns its kTreeDrawPer consecutive
// entries, so a prefix sum in thread order is one in index order (strict
// '>'; when rounding keeps the sum from passing the target, the last
// positive entry of the range searched).
__global__ __launch_bounds__(kStatThreads) void tree_draw_final_kernel(
    const double* __restrict__ uniforms, int32_t Q, int32_t V, int32_t ndraw, const TreeWalk* __restrict__ walk,
    const DrawSum* __restrict__ sums, const double* __restrict__ weights, int32_t* __restrict__ next) {
  __shared__ int s_slice, s_found, s_last;
  __shared__ double s_before, s_tgt;
  __shared__ double s_w[kStatThreads / 64];
  __shared__ int s_l[kStatThreads / 64];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  // (the slice sums are requested with the walk's verdict, not after it)
  const DrawSum o = sums[(size_t)b * ndraw + min(lane, ndraw - 1)];
  if (walk[b].done) return;
  if (w == 0) {
    const bool in = lane < ndraw;
    const double ws = in ? o.s : 0.0;
    double incl = ws;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const double tgt = uniforms[(size_t)b * Q + Q - 1] * __shfl(incl, 63);
    const unsigned long long cross = __ballot(in && incl > tgt);
    int last = in ? o.last : -1;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) last = max(last, __shfl_xor(last, off));
    const int found = cross ? (int)__builtin_ctzll(cross) : -1;
    if (lane == 0) {
      s_slice = found;
      s_tgt = tgt;
      s_last = last;
      s_found = 0x7fffffff;
    }
    if (found >= 0 && lane == found) s_before = incl - ws;
  }
  __syncthreads();
  const int slice = s_slice;
  if (slice < 0) {
    if (tid == 0) next[b] = s_last;
    return;
  }
  const double* wr = weights + (size_t)b * V;
  const int e0 = slice * kTreeDraw + tid * kTreeDrawPer;
  double wv[kTreeDrawPer];
#pragma unroll
  for (int k = 0; k < kTreeDrawPer; ++k) wv[k] = wr[min(e0 + k, V - 1)];
  double local = 0.0;
  int last_pos = -1;
#pragma unroll
  for (int k = 0; k < kTreeDrawPer; ++k) {
    if (e0 + k >= V) wv[k] = 0.0;
    local += wv[k];
    if (wv[k] > 0.0) last_pos = e0 + k;
  }
  double incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_w[w] = incl;
  int lastw = last_pos;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) lastw = max(lastw, __shfl_xor(lastw, off));
  if (lane == 0) s_l[w] = lastw;
  __syncthreads();
  double off_w = 0.0;
  for (int q = 0; q < w; ++q) off_w += s_w[q];
  double run = s_before + off_w + (incl - local);
  const double tgt = s_tgt;
  int hit = -1;
#pragma unroll
  for (int k = 0; k < kTreeDrawPer; ++k) {
    run += wv[k];
    if (hit < 0 && wv[k] > 0.0 && run > tgt) hit = e0 + k;
  }
  if (hit >= 0) atomicMin(&s_found, hit);
  __syncthreads();
  if (tid == 0) {
    const int lastp = max(max(s_l[0], s_l[1]), max(s_l[2], s_l[3]));
    next[b] = s_found != 0x7fffffff ? s_found : (lastp >= 0 ? lastp : s_last);
  }
}

int32_t tree_accept_max_vocab() { return kTreeMaxVocab; }
int32_t tree_accept_max_nodes() { return kTreeMaxQ; }

// Workspace, per sequence: two fp64 rows of V (the stored residual and q_v),
// the slice statistics of up to 64 target and 64 draft rows, the partial
// normalisers of the precomputed rejections, where the walk stopped, the
// draw's fp64 weights (one row of V) and its per-slice sums.
struct TreeWs {
  size_t rows, stats, zpart, walk, weights, sums, total;
};

static TreeWs tree_ws(int32_t B, int32_t V) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t nslice = (V + kTreeSlice - 1) / kTreeSlice;
  const size_t ndraw = (V + kTreeDraw - 1) / kTreeDraw;
  TreeWs w;
  size_t off = 0;
  w.rows = off;
  off += al((size_t)B * 2 * V * sizeof(double));
  w.stats = off;
  off += al((size_t)B * 2 * kTreeMaxQ * nslice * sizeof(SliceStat));
  w.zpart = off;
  off += al((size_t)B * kTreeMaxQ * kZPasses * nslice * sizeof(double));
  w.walk = off;
  off += al((size_t)B * sizeof(TreeWalk));
  w.weights = off;
  off += al((size_t)B * V * sizeof(double));
  w.sums = off;
  off += al((size_t)B * ndraw * sizeof(DrawSum));
  w.total = off;
  return w;
}

size_t tree_accept_ws_bytes(int32_t B, int32_t V) {
  if (B < 1 || V < 1) return 0;
  return tree_ws(B, V).total;
}

hipError_t launch_tree_accept(const float* target, const float* draft, const int32_t* tokens, const int32_t* parent,
                              const double* uniforms, int32_t B, int32_t Q, int32_t V, float temperature,
                              int32_t flags, int32_t* n_acc, int32_t* path, int32_t* next, void* ws,
                              hipStream_t stream) {
  const int probs = (flags & TF_ACCEPT_PROBS) != 0;
  const int nslice = (V + kTreeSlice - 1) / kTreeSlice;
  const int ndraw = (V + kTreeDraw - 1) / kTreeDraw;
  const TreeWs L = tree_ws(B, V);
  char* w = (char*)ws;
  double* rows = (double*)(w + L.rows);
  SliceStat* stats = (SliceStat*)(w + L.stats);
  double* zpart = (double*)(w + L.zpart);
  TreeWalk* walk = (TreeWalk*)(w + L.walk);
  double* weights = (double*)(w + L.weights);
  DrawSum* sums = (DrawSum*)(w + L.sums);
  hipError_t e;
  if (!probs) {
    // target rows 0 .. Q-1, then draft rows Q .. 2Q-1 (none when Q = 1)
    const dim3 grid((unsigned)B * nslice, Q > 1 ? 2 * Q : Q);
    hipLaunchKernelGGL(tree_stats_kernel, grid, dim3(kStatThreads), 0, stream, target, draft, Q, V, nslice,
                       temperature, stats);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (Q > 1) {
    for (int j = 1; j <= kZPasses; ++j) {
      hipLaunchKernelGGL(tree_zpass_kernel, dim3((unsigned)B * nslice, Q), dim3(kZThreads), 0, stream, target,
                         draft, parent, Q, V, nslice, temperature, probs, stats, zpart, j);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL(tree_accept_kernel, dim3(B), dim3(kTreeThreads), 0, stream, target, draft, tokens, parent,
                     uniforms, Q, V, nslice, temperature, probs, rows, stats, zpart, walk, n_acc, path, next);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(tree_draw_slice_kernel, dim3((unsigned)B * ndraw), dim3(kStatThreads), 0, stream, target, draft,
                     Q, V, nslice, ndraw, temperature, probs, stats, zpart, walk, weights, sums);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(tree_draw_final_kernel, dim3(B), dim3(kStatThreads), 0, stream, uniforms, Q, V, ndraw, walk,
                     sums, weights, next);
  return hipGetLastError();
}

}  // namespace tfk
