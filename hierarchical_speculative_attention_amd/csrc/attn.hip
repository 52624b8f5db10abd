// Split-K decode attention on MFMA for gfx950: the one kernel behind
// full-cache verification (Force 3), attention over retrieved chunks
// (Force 2) and sink + window streaming attention (Force 1) of the TriForce
// blog, section "1. The Three Forces of TriForce".
//
// Work decomposition.  Grid = (splits, KV heads, sequences).  A workgroup of
// four waves owns `tpw` consecutive "virtual" tokens of one (sequence, KV
// head); a virtual token is a cache row (verify), a row of a selected chunk
// (sparse) or a visible streaming position (stream).  Wave w walks 32-token
// tiles w, w+4, w+8, ... of its workgroup's range, keeping an online softmax
// per query row in registers.  The four waves merge through LDS; when a
// (sequence, head) has several splits, each writes an unnormalised partial
// (max, sum, 128 accumulators per row) and the last workgroup to finish
// (device-scope counter) merges them in split order, so results do not
// depend on scheduling.
//
// MFMA mapping (v_mfma_f32_16x16x32_{bf16,f16}; A row / B column = lane % 16,
// k-slots 8 * (lane / 16) + e; C column = lane % 16, C rows 4 * (lane / 16) + r):
//  * S^T = K . Q^T per 16-token subtile: A = 16 key rows straight from HBM
//    (lane (t, g) holds dims 32s + 8g .. +8 of token t for k-step s), B = the
//    query rows (padded to 16 per query tile) held in registers for the whole
//    kernel.  C gives lane (query q, group g) the scores of tokens 4g .. 4g+3.
//  * The value tile must enter the P.V product with tokens on the k axis, but
//    HBM holds it token-major.  A product with a 0/1 selection matrix moves it
//    there without LDS: C = V_tile . Sel puts V[token 4g + r][dim 16b + j] in
//    lane (j, g), register r, which is exactly the A layout of
//    O^T = V^T . P^T with token k-slots 4u + r (u = subtile).  The values are
//    copied exactly (one non-zero product, fp32 accumulate).
//  * P^T comes straight out of the S^T accumulators (same lanes), split into
//    a 16-bit high part and a 16-bit remainder so that the probabilities keep
//    ~16 significant bits; O^T accumulates in fp32 with the query in
//    lane % 16, the same lanes that hold that query's running max and sum.
#include "tf_internal.h"

namespace tfk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct MT;
template <> struct MT<TF_DTYPE_BF16> {
  typedef bf16x8 V8;
  typedef __bf16 S;
  static __device__ __forceinline__ f32x4 mma(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct MT<TF_DTYPE_FP16> {
  typedef f16x8 V8;
  typedef _Float16 S;
  static __device__ __forceinline__ f32x4 mma(V8 a, V8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kNegInf = -__builtin_huge_valf();

// Sequence geometry of one (b) for a mode: virtual length and what a
// virtual token maps to.
struct Geo {
  int n;       // valid cache rows (verify / sparse) or logical length (stream)
  int cap;     // rows allocated per head
  int L;       // virtual tokens
  int s_eff;   // stream: sinks present
  int lo;      // stream: first window position
  int ring;    // stream: ring slots (cap - n_sink)
  int nchunks; // sparse: chunks covering the n valid rows
};

template <int MODE>
__device__ __forceinline__ Geo make_geo(const AttnArgs& a, int b) {
  Geo g;
  g.cap = a.seq_cap[b];
  int n = a.seq_len[b];
  g.s_eff = 0;
  g.lo = 0;
  g.ring = 0;
  g.nchunks = 0;
  if (g.cap <= 0) {
    g.n = 0;
    g.L = 0;
    return g;
  }
  if (MODE == kStream) {
    n = n < 0 ? 0 : n;
    g.n = n;
    g.s_eff = min(a.n_sink, n);
    g.lo = max(a.n_sink, n - a.window);
    g.ring = g.cap - a.n_sink;
    int w = n > g.lo ? n - g.lo : 0;
    if (g.ring <= 0) w = 0;
    g.L = g.s_eff + w;
  } else {
    n = min(max(n, 0), min(g.cap, a.max_len));
    g.n = n;
    g.L = (MODE == kVerify) ? n : a.k * a.cs;
    g.nchunks = (n + a.cs - 1) / a.cs;
  }
  return g;
}

// Virtual token -> cache row, or -1 when nothing valid lives there.
template <int MODE>
__device__ __forceinline__ int map_row(const AttnArgs& a, const Geo& g, int v, int v_end,
                                       const int* s_idx, int chunk_lo) {
  if (v >= v_end) return -1;
  if (MODE == kVerify) return v;
  if (MODE == kSparse) {
    int slot = v / a.cs;
    const int c = s_idx[slot - chunk_lo];
    if (c < 0 || c >= g.nchunks) return -1;  // padding or out of range: nothing read
    const int row = c * a.cs + (v - slot * a.cs);
    return row < g.n ? row : -1;
  }
  // stream
  int slot;
  if (v < g.s_eff) {
    slot = v;
  } else {
    int p = g.lo + (v - g.s_eff);
    slot = a.n_sink + (p - a.n_sink) % g.ring;
  }
  return slot < g.cap ? slot : -1;
}

template <int DT, int MODE, int NQT>
__global__ __launch_bounds__(kThreads) void attn_kernel(const AttnArgs a) {
  using M = MT<DT>;
  using V8 = typename M::V8;
  using S = typename M::S;
  constexpr int kMaxIdx = 4096 / 1 + 2;  // chunk slots per workgroup (tpw <= 4096, cs >= 1)
  __shared__ int s_idx[MODE == kSparse ? kMaxIdx : 1];
  __shared__ float s_o[4][16][132];
  __shared__ float s_m[4][16];
  __shared__ float s_l[4][16];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 15, lg = lane >> 4;
  const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;

  const Geo geo = make_geo<MODE>(a, b);
  const int nsp = max(1, (geo.L + a.tpw - 1) / a.tpw);
  if (split >= nsp) return;
  const int v0 = split * a.tpw;
  const int v1 = min(geo.L, v0 + a.tpw);

  const size_t base = (size_t)a.seq_base[b] + (size_t)hk * (size_t)geo.cap * kHeadDim;
  const uint16_t* __restrict__ Kb = a.K + base;
  const uint16_t* __restrict__ Vb = a.V + base;

  int chunk_lo = 0;
  if (MODE == kSparse) {
    chunk_lo = v0 / a.cs;
    const int chunk_hi = min(a.k, (v1 + a.cs - 1) / a.cs);
    const int32_t* src = a.idx + ((size_t)b * a.Hkv + hk) * a.k;
    for (int j = tid; j < chunk_hi - chunk_lo; j += kThreads) s_idx[j] = src[chunk_lo + j];
    __syncthreads();
  }

  // Query rows of this KV head: heads hk*G .. hk*G+G-1, Qn rows each, contiguous.
  const size_t qrow0 = ((size_t)b * a.Hq + (size_t)hk * a.G) * a.Qn;
  V8 qreg[NQT][4];
  int lim[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int row = qt * 16 + lq;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < a.rows) x = *(const u32x4*)(a.q + (qrow0 + row) * kHeadDim + 32 * s + 8 * lg);
      qreg[qt][s] = __builtin_bit_cast(V8, x);
    }
    lim[qt] = (MODE == kVerify) ? geo.n - a.Qn + (row % a.Qn) : 0x7fffffff;
  }

  // Selection matrices: column j of half h picks dim 16h + j of a 32-dim k-window.
  V8 sel[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[h][e] = (S)((8 * lg + e == 16 * h + lq) ? 1.0f : 0.0f);

  f32x4 acc[NQT][8];
  float m_run[NQT], l_run[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    m_run[qt] = kNegInf;
    l_run[qt] = 0.f;
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) acc[qt][bb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = a.scale_log2;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

  for (int t0 = v0 + kTile * w; t0 < v1; t0 += 4 * kTile) {
    // ---- rows of the two 16-token subtiles, loads of K and V --------------
    const int r0 = map_row<MODE>(a, geo, t0 + lq, v1, s_idx, chunk_lo);
    const int r1 = map_row<MODE>(a, geo, t0 + 16 + lq, v1, s_idx, chunk_lo);
    const unsigned mk0 = (unsigned)(__ballot(r0 >= 0) & 0xFFFFull);
    const unsigned mk1 = (unsigned)(__ballot(r1 >= 0) & 0xFFFFull);
    const uint16_t* k0p = Kb + (size_t)(r0 < 0 ? 0 : r0) * kHeadDim + 8 * lg;
    const uint16_t* k1p = Kb + (size_t)(r1 < 0 ? 0 : r1) * kHeadDim + 8 * lg;
    const uint16_t* v0p = Vb + (size_t)(r0 < 0 ? 0 : r0) * kHeadDim + 8 * lg;
    const uint16_t* v1p = Vb + (size_t)(r1 < 0 ? 0 : r1) * kHeadDim + 8 * lg;
    V8 kr0[4], kr1[4], vr0[4], vr1[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      kr0[s] = __builtin_bit_cast(V8, *(const u32x4*)(k0p + 32 * s));
      kr1[s] = __builtin_bit_cast(V8, *(const u32x4*)(k1p + 32 * s));
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      vr0[s] = __builtin_bit_cast(V8, *(const u32x4*)(v0p + 32 * s));
      vr1[s] = __builtin_bit_cast(V8, *(const u32x4*)(v1p + 32 * s));
    }

    // ---- scores, online softmax, probabilities as MFMA operands ----------
    V8 ph[NQT], pl[NQT];
#pragma unroll
    for (int qt = 0; qt < NQT; ++qt) {
      f32x4 s0 = zero4, s1 = zero4;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        s0 = M::mma(kr0[s], qreg[qt][s], s0);
        s1 = M::mma(kr1[s], qreg[qt][s], s1);
      }
      float mx = kNegInf;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * lg + r;
        const bool vis0 = ((mk0 >> j) & 1u) && (MODE != kVerify || t0 + j <= lim[qt]);
        const bool vis1 = ((mk1 >> j) & 1u) && (MODE != kVerify || t0 + 16 + j <= lim[qt]);
        s0[r] = vis0 ? s0[r] : kNegInf;
        s1[r] = vis1 ? s1[r] : kNegInf;
        mx = fmaxf(mx, fmaxf(s0[r], s1[r]));
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[qt], mx);
      float alpha = 1.f, mc = 0.f;
      if (m_new != kNegInf) {
        alpha = fast_exp2((m_run[qt] - m_new) * c2);
        mc = m_new * c2;
      }
      float psum = 0.f;
      V8 hi, lo;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p0 = fast_exp2(fmaf(s0[r], c2, -mc));
        const float p1 = fast_exp2(fmaf(s1[r], c2, -mc));
        psum += p0 + p1;
        const S h0 = (S)p0, h1 = (S)p1;
        hi[r] = h0;
        hi[4 + r] = h1;
        lo[r] = (S)(p0 - (float)h0);
        lo[4 + r] = (S)(p1 - (float)h1);
      }
      ph[qt] = hi;
      pl[qt] = lo;
      l_run[qt] = l_run[qt] * alpha + psum;
      m_run[qt] = m_new;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) acc[qt][bb] *= alpha;
    }

    // ---- values: move tokens onto the k axis, then O^T += V^T . P^T ------
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const f32x4 t0v = M::mma(vr0[bb >> 1], sel[bb & 1], zero4);
      const f32x4 t1v = M::mma(vr1[bb >> 1], sel[bb & 1], zero4);
      V8 av;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        av[r] = (S)t0v[r];
        av[4 + r] = (S)t1v[r];
      }
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        acc[qt][bb] = M::mma(av, ph[qt], acc[qt][bb]);
        acc[qt][bb] = M::mma(av, pl[qt], acc[qt][bb]);
      }
    }
  }

  // ---- merge the four waves (per query tile) -------------------------------
  const size_t bh = (size_t)b * a.Hkv + hk;
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float lsum = l_run[qt];
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    if (lg == 0) {
      s_m[w][lq] = m_run[qt];
      s_l[w][lq] = lsum;
    }
#pragma unroll
    for (int bb = 0; bb < 8; ++bb)
      *(f32x4*)&s_o[w][lq][16 * bb + 4 * lg] = acc[qt][bb];
    __syncthreads();
    {
      const int q = tid >> 4;          // 0..15
      const int dc = (tid & 15) * 8;   // 8 dims per thread
      const int row = qt * 16 + q;
      float mw[4], ew[4];
      float Mx = kNegInf;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        mw[x] = s_m[x][q];
        Mx = fmaxf(Mx, mw[x]);
      }
      float Ls = 0.f;
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        ew[x] = (mw[x] == kNegInf) ? 0.f : fast_exp2((mw[x] - Mx) * c2);
        Ls += ew[x] * s_l[x][q];
      }
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float t = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) t += ew[x] * s_o[x][q][dc + j];
        o[j] = t;
      }
      if (row < a.rows) {
        if (nsp == 1) {
          const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
          float* dst = a.out + (qrow0 + row) * kHeadDim + dc;
          *(f32x4*)dst = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
          *(f32x4*)(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
          if (a.lse && dc == 0) a.lse[qrow0 + row] = Ls > 0.f ? Mx * a.scale_ln + logf(Ls) : kNegInf;
        } else {
          const size_t pr = (bh * a.nsplit + split) * a.rows_pad + row;
          float* dst = a.part_o + pr * kHeadDim + dc;
          *(f32x4*)dst = f32x4{o[0], o[1], o[2], o[3]};
          *(f32x4*)(dst + 4) = f32x4{o[4], o[5], o[6], o[7]};
          if (dc == 0) {
            a.part_ml[pr * 2 + 0] = Mx;
            a.part_ml[pr * 2 + 1] = Ls;
          }
        }
      }
    }
    __syncthreads();
  }
  if (nsp == 1) return;

  // ---- last workgroup of this (sequence, head) merges the splits -----------
  __threadfence();
  __syncthreads();
  if (tid == 0) {
    const int prev = __hip_atomic_fetch_add(a.counters + bh, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = (prev == nsp - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const size_t pbase = bh * a.nsplit * a.rows_pad;
  for (int item = tid; item < a.rows * 32; item += kThreads) {
    const int row = item >> 5;
    const int dq = (item & 31) * 4;
    float Mx = kNegInf;
    for (int s = 0; s < nsp; ++s) Mx = fmaxf(Mx, a.part_ml[(pbase + (size_t)s * a.rows_pad + row) * 2]);
    float Ls = 0.f;
    f32x4 o = zero4;
    if (Mx != kNegInf) {
      for (int s = 0; s < nsp; ++s) {
        const size_t pr = pbase + (size_t)s * a.rows_pad + row;
        const float ms = a.part_ml[pr * 2];
        const float e = (ms == kNegInf) ? 0.f : fast_exp2((ms - Mx) * c2);
        Ls += e * a.part_ml[pr * 2 + 1];
        o += e * *(const f32x4*)(a.part_o + pr * kHeadDim + dq);
      }
    }
    const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
    *(f32x4*)(a.out + (qrow0 + row) * kHeadDim + dq) = o * inv;
    if (a.lse && dq == 0) a.lse[qrow0 + row] = Ls > 0.f ? Mx * a.scale_ln + logf(Ls) : kNegInf;
  }
  if (tid == 0) a.counters[bh] = 0;
}

SplitPlan plan_splits(int32_t B, int32_t Hkv, int32_t rows, int32_t max_virtual, int32_t target_wgs) {
  SplitPlan p;
  int32_t tpw = 4096;
  const long heads = (long)B * Hkv;
  while (tpw > 128 && heads * (((long)max_virtual + tpw - 1) / tpw) < target_wgs) tpw >>= 1;
  p.tpw = tpw;
  p.nsplit = (int32_t)(((long)max_virtual + tpw - 1) / tpw);
  if (p.nsplit < 1) p.nsplit = 1;
  p.rows_pad = ((rows + 15) / 16) * 16;
  const size_t parts = (size_t)heads * p.nsplit * p.rows_pad;
  if (p.nsplit > 1) {
    p.part_o_bytes = parts * kHeadDim * sizeof(float);
    p.part_ml_bytes = parts * 2 * sizeof(float);
    p.counter_bytes = ((size_t)heads * sizeof(int32_t) + 255) & ~(size_t)255;
  } else {
    p.part_o_bytes = p.part_ml_bytes = p.counter_bytes = 0;
  }
  p.total_bytes = p.counter_bytes + p.part_ml_bytes + p.part_o_bytes;
  return p;
}

template <int DT, int MODE>
static hipError_t launch_nqt(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(a.nsplit, a.Hkv, a.B), block(kThreads);
  const int nqt = (a.rows + 15) / 16;
  switch (nqt) {
    case 1: hipLaunchKernelGGL((attn_kernel<DT, MODE, 1>), grid, block, 0, stream, a); break;
    case 2: hipLaunchKernelGGL((attn_kernel<DT, MODE, 2>), grid, block, 0, stream, a); break;
    case 3: hipLaunchKernelGGL((attn_kernel<DT, MODE, 3>), grid, block, 0, stream, a); break;
    case 4: hipLaunchKernelGGL((attn_kernel<DT, MODE, 4>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DT>
static hipError_t launch_mode(int mode, const AttnArgs& a, hipStream_t stream) {
  switch (mode) {
    case kVerify: return launch_nqt<DT, kVerify>(a, stream);
    case kSparse: return launch_nqt<DT, kSparse>(a, stream);
    case kStream: return launch_nqt<DT, kStream>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn(int dtype, int mode, const AttnArgs& a, hipStream_t stream) {
  if (dtype == TF_DTYPE_BF16) return launch_mode<TF_DTYPE_BF16>(mode, a, stream);
  if (dtype == TF_DTYPE_FP16) return launch_mode<TF_DTYPE_FP16>(mode, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace tfk
