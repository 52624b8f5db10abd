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
// The walk is sequential per sequence (which child is kept decides the next
// rows), so one 1024-thread workgroup per sequence runs it; thread t owns the
// contiguous vocabulary range [t * ipt, (t + 1) * ipt).  The residual p' is
// kept in fp64 in a caller workspace (one row of V doubles per sequence,
// L2-resident) as stored weights times a running scale, so renormalising costs
// no pass; probabilities are recomputed in fp64 from the logits.  (Holding it
// in registers instead, with the draft probabilities, needed about four
// registers per entry and spilled heavily at V = 32000.)  Everything is fp64
// so decisions are taken in the oracle's precision.
#include "tf_internal.h"

namespace tfk {

constexpr int kTreeThreads = 1024;
constexpr int kTreeWaves = kTreeThreads / 64;
constexpr int kTreeMaxIpt = 64;                 // V <= 65536
constexpr int kTreeMaxQ = 64;

struct TreeDist {
  int mode;     // 0 softmax(x / T), 1 greedy one-hot, 2 probabilities as given
  double zmax;  // max x / T
  double invZ;  // 1 / sum exp(x / T - zmax)
  int amax;     // lowest index of the largest entry
};

__device__ __forceinline__ double tree_val(const TreeDist& d, float x, int v, double t) {
  if (d.mode == 2) return (double)x;
  if (d.mode == 1) return v == d.amax ? 1.0 : 0.0;
  return exp((double)x / t - d.zmax) * d.invZ;
}

struct TreeShared {
  double d[kTreeWaves];
  float f[kTreeWaves];
  int i[kTreeWaves];
};

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

// Distribution parameters of one row (logits, or probabilities with probs).
__device__ TreeDist tree_dist(const float* row, int v0, int v1, float temperature, int probs, TreeShared& sh) {
  TreeDist d;
  d.zmax = 0.0;
  d.invZ = 1.0;
  d.amax = 0;
  if (probs) {
    d.mode = 2;
    return d;
  }
  float bv = -__builtin_huge_valf();
  int bi = 0x7fffffff;
  for (int v = v0; v < v1; ++v) {
    const float x = row[v];
    if (x > bv || (x == bv && v < bi)) {
      bv = x;
      bi = v;
    }
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ov = __shfl_xor(bv, off);
    const int oi = __shfl_xor(bi, off);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  __syncthreads();
  if (lane == 0) {
    sh.f[w] = bv;
    sh.i[w] = bi;
  }
  __syncthreads();
  bv = sh.f[0];
  bi = sh.i[0];
#pragma unroll
  for (int q = 1; q < kTreeWaves; ++q)
    if (sh.f[q] > bv || (sh.f[q] == bv && sh.i[q] < bi)) {
      bv = sh.f[q];
      bi = sh.i[q];
    }
  d.amax = bi;
  if (temperature == 0.f) {
    d.mode = 1;
    return d;
  }
  d.mode = 0;
  const double t = (double)temperature;
  d.zmax = (double)bv / t;
  double z = 0.0;
  for (int v = v0; v < v1; ++v) z += exp((double)row[v] / t - d.zmax);
  d.invZ = 1.0 / tree_sum(z, sh);
  return d;
}

__global__ __launch_bounds__(kTreeThreads) void tree_accept_kernel(
    const float* __restrict__ target, const float* __restrict__ draft, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ parent, const double* __restrict__ uniforms, int32_t Q, int32_t V, float temperature,
    int32_t probs, double* __restrict__ resid, int32_t* __restrict__ n_acc, int32_t* __restrict__ path,
    int32_t* __restrict__ next) {
  __shared__ int s_par[kTreeMaxQ], s_tok[kTreeMaxQ];
  __shared__ TreeShared sh;
  __shared__ double s_px, s_qx;
  __shared__ int s_found;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int ipt = (V + kTreeThreads - 1) / kTreeThreads;
  const int v0 = min(V, tid * ipt), v1 = min(V, v0 + ipt);
  const double t = (double)temperature;
  double* pr = resid + (size_t)b * V;  // p' = pr[v] * scale
  if (tid < Q) {
    const int p = parent[(size_t)b * Q + tid];
    s_par[tid] = (tid > 0 && p >= 0 && p < tid) ? p : (tid > 0 ? 0 : -1);
    s_tok[tid] = tokens[(size_t)b * Q + tid];
  }
  __syncthreads();
  const double* u = uniforms + (size_t)b * Q;
  int v = 0, npath = 0;
  double scale = 1.0;
  while (true) {
    // p' = p_v, the target's distribution for the children of v
    const float* trow = target + ((size_t)b * Q + v) * V;
    const TreeDist dp = tree_dist(trow, v0, v1, temperature, probs, sh);
    for (int e = v0; e < v1; ++e) pr[e] = tree_val(dp, trow[e], e, t);
    scale = 1.0;
    int kept = -1;
    bool has_child = false;
    for (int c = v + 1; c < Q; ++c) has_child = has_child || s_par[c] == v;
    if (has_child) {
      const float* drow = draft + ((size_t)b * Q + v) * V;
      const TreeDist dq = tree_dist(drow, v0, v1, temperature, probs, sh);
      for (int c = v + 1; c < Q; ++c) {
        if (s_par[c] != v) continue;
        const int x = s_tok[c];
        const bool valid = x >= 0 && x < V;
        __syncthreads();  // this thread's own pr writes are visible to itself; the owner of x reads its own
        if (valid && x >= v0 && x < v1) {
          s_px = pr[x] * scale;
          s_qx = tree_val(dq, drow[x], x, t);
        }
        __syncthreads();
        const double px = s_px, qx = s_qx;
        if (valid && px > 0.0 && u[c - 1] * qx <= px) {
          kept = c;
          break;
        }
        // rejected: p' = max(0, p' - q_v) renormalised (p_v if it vanished)
        double local = 0.0;
        for (int e = v0; e < v1; ++e) {
          const double r = fmax(0.0, pr[e] * scale - tree_val(dq, drow[e], e, t));
          pr[e] = r;
          local += r;
        }
        const double Z = tree_sum(local, sh);
        if (Z > 0.0) {
          scale = 1.0 / Z;
        } else {
          for (int e = v0; e < v1; ++e) pr[e] = tree_val(dp, trow[e], e, t);
          scale = 1.0;
        }
      }
    }
    if (kept < 0) break;
    if (tid == 0) path[(size_t)b * (Q - 1) + npath] = kept;
    ++npath;
    v = kept;
    __syncthreads();  // every thread done with this node's rows before pr is rewritten
  }
  // draw the next token from p' (inverse CDF with u[Q - 1], strict '>')
  double local = 0.0;
  int last_pos = -1;
  for (int e = v0; e < v1; ++e) {
    const double r = pr[e] * scale;
    local += r;
    if (r > 0.0) last_pos = e;
  }
  double incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) sh.d[w] = incl;
  if (tid == 0) s_found = 0x7fffffff;
  __syncthreads();
  double off_w = 0.0, total = 0.0;
#pragma unroll
  for (int q = 0; q < kTreeWaves; ++q) {
    if (q < w) off_w += sh.d[q];
    total += sh.d[q];
  }
  const double tgt = u[Q - 1] * total;
  double run = off_w + (incl - local);
  for (int e = v0; e < v1; ++e) {
    const double r = pr[e] * scale;
    run += r;
    if (r > 0.0 && run > tgt) {
      atomicMin(&s_found, e);
      break;
    }
  }
  const int last = tree_max_int(last_pos, sh);  // (its barriers also order the atomicMin before the read)
  if (tid == 0) {
    n_acc[b] = npath;
    // the running sum never passing u * total (rounding): the last positive entry
    next[b] = s_found != 0x7fffffff ? s_found : last;
  }
  for (int i = npath + tid; i < Q - 1; i += kTreeThreads) path[(size_t)b * (Q - 1) + i] = -1;
}

int32_t tree_accept_max_vocab() { return kTreeThreads * kTreeMaxIpt; }
int32_t tree_accept_max_nodes() { return kTreeMaxQ; }

size_t tree_accept_ws_bytes(int32_t B, int32_t V) {
  if (B < 1 || V < 1) return 0;
  return ((size_t)B * V * sizeof(double) + 255) & ~(size_t)255;
}

hipError_t launch_tree_accept(const float* target, const float* draft, const int32_t* tokens, const int32_t* parent,
                              const double* uniforms, int32_t B, int32_t Q, int32_t V, float temperature,
                              int32_t flags, int32_t* n_acc, int32_t* path, int32_t* next, void* ws,
                              hipStream_t stream) {
  const int probs = (flags & TF_ACCEPT_PROBS) != 0;
  hipLaunchKernelGGL(tree_accept_kernel, dim3(B), dim3(kTreeThreads), 0, stream, target, draft, tokens, parent,
                     uniforms, Q, V, temperature, probs, (double*)ws, n_acc, path, next);
  return hipGetLastError();
}

}  // namespace tfk
