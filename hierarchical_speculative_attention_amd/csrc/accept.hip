// Lossless accept / reject of a chain of gamma drafted tokens, after the
// TriForce blog, section "2. Dual Rejection Sampling: Mathematical
// Losslessness": keep draft x while min(1, p(x) / q(x)) >= u; at the first
// rejection draw the next token from max(0, p - q) normalised; if every draft
// is kept, draw a bonus token from the target's next row.
//
// One 1024-thread workgroup per sequence, everything in fp64 so that every
// decision is taken in the same precision as the fp64 reference.  Rows are
// reduced only as far as the chain gets: position i needs the normaliser of
// target row i and draft row i; the final draw needs one more pass over one
// row.  The draw is an inverse CDF: thread t owns a contiguous slice of the
// vocabulary, a block prefix sum of the slice totals gives each slice's
// starting running sum, and the slice holding the crossing scans itself in
// order.
#include "tf_internal.h"

namespace tfk {

constexpr int kAccThreads = 1024;

struct RowDist {
  // p_v = exp(x_v / T - zmax) / Z   (T > 0); one-hot at amax (T == 0);
  // x_v as given (probabilities mode).
  int mode;  // 0 softmax, 1 greedy, 2 probabilities
  double zmax;
  double Z;
  int amax;
};

__device__ __forceinline__ double block_sum_d(double x, double* s_red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if (lane == 0) s_red[w] = x;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x < 64) {
    t = threadIdx.x < kAccThreads / 64 ? s_red[threadIdx.x] : 0.0;
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) t += __shfl_xor(t, off);
    if (threadIdx.x == 0) s_red[32] = t;
  }
  __syncthreads();
  const double r = s_red[32];
  __syncthreads();
  return r;
}

// Max value and its lowest index over the row.
__device__ __forceinline__ void block_argmax(const float* row, int V, double* s_red, int* s_ri, float* mx, int* am) {
  float best = -__builtin_huge_valf();
  int bi = 0x7fffffff;
  for (int v = threadIdx.x; v < V; v += kAccThreads) {
    const float x = row[v];
    if (x > best || (x == best && v < bi)) {
      best = x;
      bi = v;
    }
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const float ob = __shfl_xor(best, off);
    const int oi = __shfl_xor(bi, off);
    if (ob > best || (ob == best && oi < bi)) {
      best = ob;
      bi = oi;
    }
  }
  if (lane == 0) {
    s_red[w] = (double)best;
    s_ri[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double b0 = s_red[0];
    int i0 = s_ri[0];
    for (int j = 1; j < kAccThreads / 64; ++j) {
      if (s_red[j] > b0 || (s_red[j] == b0 && s_ri[j] < i0)) {
        b0 = s_red[j];
        i0 = s_ri[j];
      }
    }
    s_red[33] = b0;
    s_ri[33] = i0;
  }
  __syncthreads();
  *mx = (float)s_red[33];
  *am = s_ri[33];
  __syncthreads();
}

__device__ RowDist make_dist(const float* row, int V, float temperature, int probs, double* s_red, int* s_ri) {
  RowDist d;
  d.zmax = 0.0;
  d.Z = 1.0;
  d.amax = 0;
  if (probs) {
    d.mode = 2;
    return d;
  }
  float mx;
  int am;
  block_argmax(row, V, s_red, s_ri, &mx, &am);
  d.amax = am;
  if (temperature == 0.f) {
    d.mode = 1;
    return d;
  }
  d.mode = 0;
  // z_v = x_v / T; the largest z comes from the largest x (division by T > 0
  // is monotone), so zmax is that value divided by T.
  d.zmax = (double)mx / (double)temperature;
  double s = 0.0;
  for (int v = threadIdx.x; v < V; v += kAccThreads) s += exp((double)row[v] / (double)temperature - d.zmax);
  d.Z = block_sum_d(s, s_red);
  return d;
}

__device__ __forceinline__ double dist_p(const RowDist& d, const float* row, int v, float temperature) {
  if (d.mode == 2) return (double)row[v];
  if (d.mode == 1) return v == d.amax ? 1.0 : 0.0;
  return exp((double)row[v] / (double)temperature - d.zmax) / d.Z;
}

__global__ __launch_bounds__(kAccThreads) void accept_kernel(const float* __restrict__ target,
                                                             const float* __restrict__ draft,
                                                             const int32_t* __restrict__ tokens,
                                                             const double* __restrict__ uniforms, int32_t gamma,
                                                             int32_t V, float temperature, int32_t probs,
                                                             int32_t* __restrict__ n_acc, int32_t* __restrict__ next) {
  __shared__ double s_red[40];
  __shared__ int s_ri[40];
  __shared__ double s_scan[kAccThreads / 64 + 1];
  __shared__ int s_found;
  const int b = blockIdx.x;
  const float* trow0 = target + (size_t)b * (gamma + 1) * V;
  const float* drow0 = draft + (size_t)b * gamma * V;
  const double* u = uniforms + (size_t)b * (gamma + 1);

  int j = gamma;
  RowDist dp, dq;
  for (int i = 0; i < gamma; ++i) {
    const float* tr = trow0 + (size_t)i * V;
    const float* dr = drow0 + (size_t)i * V;
    dp = make_dist(tr, V, temperature, probs, s_red, s_ri);
    dq = make_dist(dr, V, temperature, probs, s_red, s_ri);
    const int x = tokens[(size_t)b * gamma + i];
    const bool in_vocab = x >= 0 && x < V;  // an out-of-range token is rejected
    const double px = in_vocab ? dist_p(dp, tr, x, temperature) : 0.0;
    const double qx = in_vocab ? dist_p(dq, dr, x, temperature) : 0.0;
    bool keep = false;
    if (px > 0.0) {
      const double alpha = (qx == 0.0) ? 1.0 : fmin(1.0, px / qx);
      keep = alpha >= u[i];
    }
    if (!keep) {
      j = i;
      break;
    }
  }

  // Weights of the final draw, evaluated element by element:
  //   rejected at j : r_v = max(0, p_j(v) - q_j(v))   (p_j if that sums to 0)
  //   all kept      : r_v = p_gamma(v)
  const float* tr = trow0 + (size_t)j * V;
  const float* dr = drow0 + (size_t)(j < gamma ? j : 0) * V;
  bool residual = j < gamma;
  if (!residual) dp = make_dist(tr, V, temperature, probs, s_red, s_ri);

  const int ipt = (V + kAccThreads - 1) / kAccThreads;
  const int v0 = threadIdx.x * ipt, v1 = min(V, v0 + ipt);
  double local = 0.0;
  for (int v = v0; v < v1; ++v) {
    const double p = dist_p(dp, tr, v, temperature);
    local += residual ? fmax(0.0, p - dist_p(dq, dr, v, temperature)) : p;
  }
  double total = block_sum_d(local, s_red);
  if (residual && total == 0.0) {
    residual = false;  // fall back to p_j
    local = 0.0;
    for (int v = v0; v < v1; ++v) local += dist_p(dp, tr, v, temperature);
    total = block_sum_d(local, s_red);
  }

  // Exclusive prefix of the slice totals in thread order (fp64).
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  double incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_scan[w] = incl;
  if (threadIdx.x == 0) s_found = 0x7fffffff;
  __syncthreads();
  double excl = __shfl_up(incl, 1);
  if (lane == 0) excl = 0.0;
  double wave_off = 0.0;
  for (int x = 0; x < w; ++x) wave_off += s_scan[x];
  const double run0 = wave_off + excl;
  const double tgt = u[gamma] * total;

  // The crossing: smallest v with running sum > tgt.
  int hit = 0x7fffffff;
  int last_pos = -1;
  double run = run0;
  for (int v = v0; v < v1; ++v) {
    const double p = dist_p(dp, tr, v, temperature);
    const double r = residual ? fmax(0.0, p - dist_p(dq, dr, v, temperature)) : p;
    if (r > 0.0) last_pos = v;
    run += r;
    if (run > tgt && hit == 0x7fffffff) hit = v;
  }
  atomicMin(&s_found, hit);
  // Fallback (running sum never passes u * total through rounding): the last
  // index with positive weight.
  __syncthreads();
  int found = s_found;
  if (found == 0x7fffffff) {
    __syncthreads();
    if (threadIdx.x == 0) s_found = -1;
    __syncthreads();
    atomicMax(&s_found, last_pos);
    __syncthreads();
    found = s_found;
  }
  if (threadIdx.x == 0) {
    n_acc[b] = j;
    next[b] = found;
  }
}

size_t accept_ws_bytes(int32_t, int32_t, int32_t) { return 0; }

hipError_t launch_accept(const float* target, const float* draft, const int32_t* tokens,
                         const double* uniforms, int32_t B, int32_t gamma, int32_t V,
                         float temperature, int32_t flags, int32_t* n_acc, int32_t* next,
                         void*, hipStream_t stream) {
  hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(kAccThreads), 0, stream, target, draft, tokens, uniforms, gamma, V,
                     temperature, (int32_t)((flags & TF_ACCEPT_PROBS) != 0), n_acc, next);
  return hipGetLastError();
}

}  // namespace tfk
