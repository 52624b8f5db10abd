// Tree masks for Force 3, and candidate collection between the two levels of
// the hierarchy's rejection sampling (TriForce blog, "2. Dual Rejection
// Sampling": Force 2 keeps the drafter's candidates with min(1, q/r) >= u1,
// and what it passes on is then verified by Force 3 with min(1, p/q) >= u2).
//
// After each Force 2 round (one tf_accept of gamma1 drafts against q), the
// round emits its n_accepted kept drafts and the token it drew.  They are
// appended to a per-sequence candidate chain of at most gamma2 tokens, each
// with the q row of its position (the distribution level 1 makes it follow,
// which level 2 divides by).  Grid (gamma1 + 1, B): workgroup j copies the q
// row of the round's j-th emitted token; workgroup 0 also writes the tokens
// and the new count.  Counts go from count_in to a different count_out array,
// so no workgroup reads a count another one rewrites.
#include "tf_internal.h"

namespace tfk {

__global__ __launch_bounds__(256) void collect_kernel(const int32_t* __restrict__ draft_tokens,
                                                      const int32_t* __restrict__ n_accepted,
                                                      const int32_t* __restrict__ next_token,
                                                      const float* __restrict__ q_rows, int32_t gamma1, int32_t V,
                                                      const int32_t* __restrict__ count_in,
                                                      int32_t* __restrict__ count_out, int32_t* __restrict__ cand,
                                                      float* __restrict__ cand_q, int32_t gamma2) {
  const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int na = min(max(n_accepted[b], 0), gamma1);
  const int c = min(max(count_in[b], 0), gamma2);
  const int take = min(na + 1, gamma2 - c);  // emitted tokens that still fit
  if (j == 0) {
    for (int i = tid; i < take; i += 256)
      cand[(size_t)b * gamma2 + c + i] = i < na ? draft_tokens[(size_t)b * gamma1 + i] : next_token[b];
    if (tid == 0) count_out[b] = c + take;
  }
  if (j >= take) return;
  const float* src = q_rows + ((size_t)b * (gamma1 + 1) + j) * V;
  float* dst = cand_q + ((size_t)b * gamma2 + c + j) * V;
  if ((V & 3) == 0) {
    const int V4 = V >> 2;
    for (int i = tid; i < V4; i += 256) ((float4*)dst)[i] = ((const float4*)src)[i];
  } else {
    for (int i = tid; i < V; i += 256) dst[i] = src[i];
  }
}

// Visibility masks of candidate trees given by parent pointers (Force 3
// evaluates Force 2's candidate tree with tree attention): one thread per
// node walks to its root; bit m of the mask is set for the node itself and
// each ancestor m.  A parent outside [0, i) hangs node i off the prefix, so
// every walk ends within Q steps.
__global__ __launch_bounds__(256) void tree_masks_kernel(const int32_t* __restrict__ parent, int32_t B, int32_t Q,
                                                         uint64_t* __restrict__ masks) {
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long)B * Q) return;
  const int b = (int)(gid / Q), i = (int)(gid % Q);
  const int32_t* par = parent + (size_t)b * Q;
  uint64_t m = 0;
  int x = i;
  while (x >= 0) {
    m |= 1ull << x;
    const int p = par[x];
    x = (p >= 0 && p < x) ? p : -1;
  }
  masks[gid] = m;
}

hipError_t launch_tree_masks(const int32_t* parent, int32_t B, int32_t Q, uint64_t* masks, hipStream_t stream) {
  const long n = (long)B * Q;
  hipLaunchKernelGGL(tree_masks_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, parent, B, Q, masks);
  return hipGetLastError();
}

hipError_t launch_collect(const int32_t* draft_tokens, const int32_t* n_accepted, const int32_t* next_token,
                          const float* q_rows, int32_t B, int32_t gamma1, int32_t V, const int32_t* count_in,
                          int32_t* count_out, int32_t* cand, float* cand_q, int32_t gamma2, hipStream_t stream) {
  hipLaunchKernelGGL(collect_kernel, dim3(gamma1 + 1, B), dim3(256), 0, stream, draft_tokens, n_accepted, next_token,
                     q_rows, gamma1, V, count_in, count_out, cand, cand_q, gamma2);
  return hipGetLastError();
}

}  // namespace tfk
