// Split-K decode attention on MFMA for gfx950: the one kernel behind
// full-cache verification of a candidate chain or tree (Force 3), attention
// over retrieved chunks (Force 2) and sink + window streaming attention
// (Force 1) of the TriForce blog, section "1. The Three Forces of TriForce".
//
// Work decomposition.  Grid = (splits, KV heads, sequences).  A workgroup of
// four waves owns `tpw` consecutive "virtual" tokens of one (sequence, KV
// head); a virtual token is a cache row (verify), a row of a selected chunk
// (sparse) or a visible streaming position (stream).  Wave w walks 32-token
// tiles w, w+4, w+8, ... of its workgroup's range, keeping an online softmax
// per query row in registers, with the next tile's loads in flight while it
// consumes the current one.  The four waves merge through LDS; when a
// (sequence, head) has several splits, each writes an unnormalised partial
// (max, sum, 128 accumulators per row) and a small second kernel merges them
// in split order, so results do not depend on scheduling and no device-wide
// fence (an L2 write-back on this chip) is needed.
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
constexpr int kMaxSparseTpw = kSparseMaxTpw;      // virtual tokens per sparse workgroup (host-capped)
constexpr int kMaxSparseIdx = kMaxSparseTpw + 2;  // chunk slots one sparse workgroup can touch

// Sequence geometry of one (b) for a mode: virtual length and what a
// virtual token maps to.
struct Geo {
  int n;       // valid cache rows (verify / sparse) or logical length (stream)
  int cap;     // rows allocated per head
  int L;       // virtual tokens
  int s_eff;   // stream: sinks present
  int lo;      // stream: first window position; sparse with tail: first tail row
  int ring;    // stream: ring slots (cap - n_sink)
  int nchunks; // sparse: chunks covering the n valid rows
};

// The per-sequence descriptor values, read once at kernel entry.
struct SeqDesc {
  int64_t base;
  int cap, len;
};

// Loads the descriptor of sequence b.  The empty asm uses the three values in
// scalar registers at this point, so the loads cannot be sunk past later
// branches: they are issued together, and their one round trip overlaps the
// vector loads already in flight.
__device__ __forceinline__ SeqDesc load_seq(const AttnArgs& a, int b) {
  SeqDesc d;
  d.base = a.seq_base[b];
  d.cap = a.seq_cap[b];
  d.len = a.seq_len[b];
  asm volatile("" : : "s"(d.base), "s"(d.cap), "s"(d.len));
  return d;
}

template <int MODE>
__device__ __forceinline__ Geo make_geo(const AttnArgs& a, const SeqDesc& d) {
  Geo g;
  g.cap = d.cap;
  int n = d.len;
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
    g.L = (MODE == kVerify || MODE == kVerifyTree) ? n : a.k * a.cs;
    g.nchunks = (n + a.cs - 1) / a.cs;
    if (MODE == kSparseTail) {
      g.lo = max(0, n - a.tail);       // first tail row
      g.L = a.k * a.cs + (n - g.lo);   // chunk rows, then the tail
    }
  }
  return g;
}

// A value combined over the four 16-lane rows of a wave (lanes l, l ^ 16,
// l ^ 32, l ^ 48: one column of the MFMA output), first with the row beside
// it, then with the other half.  v_permlane16_swap / v_permlane32_swap with
// one register as both operands leave every lane holding its own value and
// its partner's, so the exchange stays in registers (lane shuffles compile to
// LDS permutes); the partner pairs and their order match x op shfl_xor(x, 16)
// then op shfl_xor(x, 32), so the results are the same bits.
__device__ __forceinline__ float rows4_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Maximum over the 64 lanes of a wave, every lane active: each row of 16
// rotated by 8, 4, 2 and 1 lanes (DPP row_ror), then the four rows combined.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xf, 0xf, false)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xf, 0xf, false)));
  return rows4_max(x);
}

// Inclusive prefix sum over the 64 lanes of a wave (modulo 2^32), every lane
// active: DPP shifts by 1, 2, 4 and 8 lanes within each row of 16, then the
// last lane of rows 0 and 2, and of row 1, broadcast into the rows after them.
__device__ __forceinline__ unsigned wave_incl_scan_u32(unsigned x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return (unsigned)v;
}

// Sparse modes: virtual token v -> cache row, given the chunk index c held by
// v's slot (v / cs), or -1 when nothing valid lives there.  Written without
// branches (every value computed, the invalid ones dropped by selection), so
// that the rows of a tile are mapped together: with a branch per row, each
// row's slot read became a round trip of its own, nine in a row before a
// tile's loads could be issued.  Unsigned arithmetic: v >= 0, and a slot
// holding anything (padding, an index out of range) cannot overflow.
template <int MODE>
__device__ __forceinline__ int sparse_row(const AttnArgs& a, const Geo& g, int v, int v_end, int c) {
  const unsigned cs = (unsigned)a.cs;
  const unsigned slot = (unsigned)v / cs;
  const int row = (int)((unsigned)c * cs + ((unsigned)v - slot * cs));
  // padding or an index out of range reads nothing; with a tail, chunk rows
  // from the tail on are attended as tail rows
  int r = (v < v_end && c >= 0 && c < g.nchunks && row < (MODE == kSparseTail ? g.lo : g.n)) ? row : -1;
  if (MODE == kSparseTail) {
    const int kcs = a.k * a.cs;
    if (v >= kcs) r = v < v_end ? g.lo + (v - kcs) : -1;  // tail row (< n since v < L)
  }
  return r;
}

// Virtual token -> cache row, or -1 when nothing valid lives there.  A sparse
// row's slot is read from the workgroup's slot table, clamped into it: for a
// token inside the workgroup's range it is a slot the workgroup fetched, and
// any other token's row is dropped.
template <int MODE>
__device__ __forceinline__ int map_row(const AttnArgs& a, const Geo& g, int v, int v_end,
                                       const int* s_idx, int chunk_lo) {
  if (MODE == kSparse || MODE == kSparseTail) {
    const unsigned slot = (unsigned)v / (unsigned)a.cs;
    return sparse_row<MODE>(a, g, v, v_end, s_idx[min(slot - (unsigned)chunk_lo, (unsigned)(kMaxSparseIdx - 1))]);
  }
  if (v >= v_end) return -1;
  if (MODE == kVerify || MODE == kVerifyTree) return v;
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

// Two ways to bring a 32-token tile of K and V (16 KB) to the MFMAs:
//
// Staged (verify: long streams, bandwidth-bound).  HBM -> registers -> LDS ->
// MFMA operands.  A 32-token tile of
// K and V (16 KB) is fetched with 16 nontemporal 16-byte loads per lane in
// which each wave instruction covers 1 KB of contiguous memory (4 rows of 256
// bytes): on this chip that pattern streams at about 7.0 TB/s, while loading
// straight into the MFMA operand layout (16 rows x 64 bytes per instruction)
// tops out near 6.3 TB/s.  The tile is staged in a wave-private LDS slab with
// a 288-byte row pitch: consecutive rows start 8 banks apart, so the
// contiguous writes, the 16-row operand reads and the transposing value reads
// (8 bytes from each of four consecutive rows per lane group) are all free
// of bank conflicts (the chip's conflict counter reads 0; a 272-byte pitch
// left 24% of the kernel's LDS cycles to conflicts at one query tile and 36%
// at three, GQA verify 1 us slower; 280 bytes breaks the 16-byte alignment of
// the operand reads: GQA verify 337 -> 593 us).  One tile is in flight while
// the staged one is consumed.
//
// Staged, two deep (sparse: a few gathered tiles per wave, latency-bound).
// The same 1 KB-per-instruction loads and slab, but two register stages
// alternate so that a wave's first two tiles are in flight at once (one
// memory round trip for both); with the value operand read transposed from
// the slab this beat loading straight into the operand layout (sparse pass
// 21.5 -> 20.4 us per 128K layer; the gathers of 2 KB runs stream better in
// 1 KB instructions than in 16 rows x 64 bytes).
//
// Direct (streaming: 256 ring rows per head, one workgroup per head).  Loads
// go straight into the MFMA operand layout (lane (t, g): dims 32 s + 8 g ..
// +8 of token t) and two tiles are in flight at once; staging measured slower
// here (8.6 -> 8.9 us).
constexpr int kPitch = 288;                  // LDS bytes per staged 256-byte row
constexpr int kStageRows = 2 * kTile;        // 32 key rows, then 32 value rows
constexpr int kStageBytes = kStageRows * kPitch;
constexpr int kMergeBytes = 4 * 16 * 132 * 4;  // per-query-tile merge buffer (staged: reuses the slabs)
static_assert(kMergeBytes <= 4 * kStageBytes, "merge buffer must fit in the staging slabs");

struct Stage {
  u32x4 v[16];     // v[i]: staged row 4 i + lane / 16, bytes 16 (lane % 16) .. +16
  unsigned mask;   // bit j: token j of the tile is a valid row
};

// The 16 loads of staged tile t0; rowmap(v, i) gives the cache row of
// virtual token v, for row group i = 0..7 of the lane, or 8 for its
// token-mask row.
template <class RowMap>
__device__ __forceinline__ void load_stage_rows(Stage& st, int t0, const RowMap& rowmap, const uint16_t* Kb,
                                                const uint16_t* Vb, int lane) {
  const int rv = rowmap(t0 + (lane & 31), 8);
  st.mask = (unsigned)(__ballot(rv >= 0) & 0xFFFFFFFFull);
  size_t off[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    // Rows that hold nothing read row 0 (in bounds) and are masked later.
    const int r = rowmap(t0 + 4 * i + (lane >> 4), i);
    off[i] = (size_t)(r < 0 ? 0 : r) * kHeadDim + 8 * (lane & 15);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) st.v[i] = __builtin_nontemporal_load((const u32x4*)(Kb + off[i]));
#pragma unroll
  for (int i = 0; i < 8; ++i) st.v[8 + i] = __builtin_nontemporal_load((const u32x4*)(Vb + off[i]));
}

template <int MODE>
__device__ __forceinline__ void load_stage(Stage& st, const AttnArgs& a, const Geo& geo, int t0, int v1,
                                           const int* s_idx, int chunk_lo, const uint16_t* Kb,
                                           const uint16_t* Vb, int lane) {
  load_stage_rows(st, t0, [&](int v, int) { return map_row<MODE>(a, geo, v, v1, s_idx, chunk_lo); }, Kb, Vb, lane);
}

// The chunk indices one lane needs for staged tile t0 of a sparse workgroup
// (its 8 row groups, then its token-mask row), read straight from the
// (sequence, head)'s k slots, each slot clamped into them: for a token inside
// the workgroup's range the slot is the token's own, any other token's row is
// dropped.
struct TileIdx {
  int c[9];
};

__device__ __forceinline__ void fetch_tile_idx(TileIdx& ti, const AttnArgs& a, const int32_t* slots, int t0,
                                               int lane) {
#pragma unroll
  for (int i = 0; i < 9; ++i) {
    const int v = i < 8 ? t0 + 4 * i + (lane >> 4) : t0 + (lane & 31);
    ti.c[i] = slots[min((unsigned)v / (unsigned)a.cs, (unsigned)(a.k - 1))];
  }
}

__device__ __forceinline__ void write_stage(const Stage& st, unsigned char* slab, int lane) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    *(u32x4*)(slab + (4 * i + (lane >> 4)) * kPitch + 16 * (lane & 15)) = st.v[i];
}

// Direct tile: MFMA operands of both subtiles, in registers.
template <int DT>
struct Tile {
  typename MT<DT>::V8 k0[4], k1[4], v0[4], v1[4];
  unsigned mask;  // bit j: token j of the tile is a valid row
};

template <int DT, int MODE>
__device__ __forceinline__ void load_tile(Tile<DT>& T, const AttnArgs& a, const Geo& geo, int t0, int v1,
                                          const int* s_idx, int chunk_lo, const uint16_t* Kb,
                                          const uint16_t* Vb, int lq, int lg) {
  using V8 = typename MT<DT>::V8;
  const int r0 = map_row<MODE>(a, geo, t0 + lq, v1, s_idx, chunk_lo);
  const int r1 = map_row<MODE>(a, geo, t0 + 16 + lq, v1, s_idx, chunk_lo);
  T.mask = (unsigned)(__ballot(r0 >= 0) & 0xFFFFull) | ((unsigned)(__ballot(r1 >= 0) & 0xFFFFull) << 16);
  // Rows that hold nothing read row 0 (in bounds) and are masked.
  const size_t o0 = (size_t)(r0 < 0 ? 0 : r0) * kHeadDim + 8 * lg;
  const size_t o1 = (size_t)(r1 < 0 ? 0 : r1) * kHeadDim + 8 * lg;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    T.k0[s] = __builtin_bit_cast(V8, *(const u32x4*)(Kb + o0 + 32 * s));
    T.k1[s] = __builtin_bit_cast(V8, *(const u32x4*)(Kb + o1 + 32 * s));
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    T.v0[s] = __builtin_bit_cast(V8, *(const u32x4*)(Vb + o0 + 32 * s));
    T.v1[s] = __builtin_bit_cast(V8, *(const u32x4*)(Vb + o1 + 32 * s));
  }
}

// Operand sources for process_tile: k(u, s) / v(u, s) give the MFMA operand
// of subtile u, k-step s (row 16 u + lane % 16, dims 32 s + 8 (lane / 16) ..).
//
// A staged tile also gives the value operand of the P.V product directly,
// vt(bb): V^T for dims 16 bb .. 16 bb + 15 with the 32 tokens on the k axis,
// in the order the P operand has them (lane (i, g) element j: token 4 g + j,
// then 16 + 4 g + j - 4).  The transposing LDS read (ds_read_b64_tr_b16) gives
// lane i of each 16-lane group element i % 4 of the 8 bytes that lane
// 4 k + i / 4 of the group addressed, as its k-th element; so lane l of group g
// addresses token 4 g + l / 4, dims 16 bb + 4 (l % 4) .. + 3, and two reads, 16
// tokens apart, fill the operand (the lane layout was read off the chip).
// Without a staged tile, V is moved onto the k axis by a product with a 0/1
// selection matrix (an exact copy either way).
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct SlabSource {
  static constexpr bool kTrV = true;
  const unsigned char* kp;   // slab + (lane % 16) * kPitch + 16 (lane / 16)
  const unsigned char* vtp;  // slab + (kTile + 4 (lane / 16) + (lane % 16) / 4) * kPitch + 8 (lane % 4)
  __device__ __forceinline__ SlabSource(const unsigned char* slab, int lane)
      : kp(slab + (lane & 15) * kPitch + 16 * (lane >> 4)),
        vtp(slab + (kTile + 4 * (lane >> 4) + ((lane & 15) >> 2)) * kPitch + 8 * (lane & 3)) {}
  __device__ __forceinline__ typename MT<DT>::V8 k(int u, int s) const {
    return __builtin_bit_cast(typename MT<DT>::V8, *(const u32x4*)(kp + u * 16 * kPitch + 64 * s));
  }
  __device__ __forceinline__ typename MT<DT>::V8 v(int u, int s) const {
    return __builtin_bit_cast(typename MT<DT>::V8, *(const u32x4*)(kp + (kTile + u * 16) * kPitch + 64 * s));
  }
  __device__ __forceinline__ typename MT<DT>::V8 vt(int bb) const {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vtp + 32 * bb));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vtp + 16 * kPitch + 32 * bb));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(typename MT<DT>::V8, u32x4{l2[0], l2[1], h2[0], h2[1]});
  }
};

template <int DT>
struct RegSource {
  static constexpr bool kTrV = false;
  const Tile<DT>& T;
  __device__ __forceinline__ typename MT<DT>::V8 k(int u, int s) const { return u ? T.k1[s] : T.k0[s]; }
  __device__ __forceinline__ typename MT<DT>::V8 v(int u, int s) const { return u ? T.v1[s] : T.v0[s]; }
};

// Online-softmax update of one wave with one tile.
template <int DT, int MODE, int NQT, class Src>
__device__ __forceinline__ void process_tile(const Src& src, unsigned mask, int t0,
                                             const typename MT<DT>::V8 (&qreg)[NQT][4],
                                             const typename MT<DT>::V8 (&sel)[2], const int (&lim)[NQT],
                                             int lim_min, const uint64_t (&tm)[NQT], int tbase,
                                             f32x4 (&acc)[NQT][8], float (&m_run)[NQT],
                                             float (&l_run)[NQT], float c2, int lq, int lg) {
  using M = MT<DT>;
  using V8 = typename M::V8;
  using S = typename M::S;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const unsigned mk0 = mask & 0xFFFFu, mk1 = mask >> 16;
  // Whole tile visible to every row: no per-element masking needed.
  constexpr bool kCausal = MODE == kVerify || MODE == kSparseTail;
  // Tree: rows below tbase (the prefix) are visible to every query row; node
  // m = row - tbase is visible when bit m of the row's mask is set.
  constexpr bool kTree = MODE == kVerifyTree;
  const bool full = mask == 0xFFFFFFFFu && (!kCausal || t0 + 31 <= lim_min) && (!kTree || t0 + 31 < tbase);
  V8 ph[NQT], pl[NQT];
  V8 k0[4], k1[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    k0[s] = src.k(0, s);
    k1[s] = src.k(1, s);
  }
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    f32x4 s0 = zero4, s1 = zero4;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      s0 = M::mma(k0[s], qreg[qt][s], s0);
      s1 = M::mma(k1[s], qreg[qt][s], s1);
    }
    if (!full) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 4 * lg + r;
        bool vis0 = ((mk0 >> j) & 1u) && (!kCausal || t0 + j <= lim[qt]);
        bool vis1 = ((mk1 >> j) & 1u) && (!kCausal || t0 + 16 + j <= lim[qt]);
        if (kTree) {
          const unsigned n0 = (unsigned)(t0 + j - tbase), n1 = (unsigned)(t0 + 16 + j - tbase);
          vis0 = vis0 && (t0 + j < tbase || (n0 < 64u && ((tm[qt] >> n0) & 1ull)));
          vis1 = vis1 && (t0 + 16 + j < tbase || (n1 < 64u && ((tm[qt] >> n1) & 1ull)));
        }
        s0[r] = vis0 ? s0[r] : kNegInf;
        s1[r] = vis1 ? s1[r] : kNegInf;
      }
    }
    float mx = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])), fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
    mx = rows4_max(mx);
    const float m_new = fmaxf(m_run[qt], mx);
    // Rescale only when some row's running max moved (rare once it settles).
    if (__ballot(m_new != m_run[qt]) != 0ull) {
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_run[qt] - m_new) * c2);
      l_run[qt] *= alpha;
#pragma unroll
      for (int bb = 0; bb < 8; ++bb) acc[qt][bb] *= alpha;
      m_run[qt] = m_new;
    }
    const float mc = (m_new == kNegInf) ? 0.f : m_new * c2;
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
    l_run[qt] += psum;
  }
  // Values: tokens on the k axis, then O^T += V^T . P^T.
  if constexpr (Src::kTrV) {
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) {
      const V8 av = src.vt(bb);
#pragma unroll
      for (int qt = 0; qt < NQT; ++qt) {
        acc[qt][bb] = M::mma(av, ph[qt], acc[qt][bb]);
        acc[qt][bb] = M::mma(av, pl[qt], acc[qt][bb]);
      }
    }
  } else {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const V8 v0 = src.v(0, s);
      const V8 v1 = src.v(1, s);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int bb = 2 * s + h;
        const f32x4 t0v = M::mma(v0, sel[h], zero4);
        const f32x4 t1v = M::mma(v1, sel[h], zero4);
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
  }
}

// A work item given explicitly (the equal-work plan of a batch's
// verification): tokens [v0, v1) of one (sequence, KV head); part >= 0 is the
// partial slot its result goes to, part < 0 means the span is the head's
// whole range and its result is the output itself.
struct Span {
  int v0, v1;
  long part;
};

// Verification with 3-4 query tiles, rows split over the waves: wave w < NQT
// owns query tile w over the item's whole token range and holds the register
// state of one tile (~180 registers: two waves per SIMD; all tiles in one wave
// took 410-500 registers, one wave per SIMD, and copied the accumulators
// between register files every tile).  Measured against all tiles in every
// wave (with the transposing V reads): 3 tiles 379 -> 363 us, 4 tiles faster
// too; 2 tiles about equal, so they keep the per-wave path.  Each 32-token K/V
// tile is fetched by all four
// waves together, 16 rows each (1 KB per instruction), two to four tiles in
// flight per workgroup, staged in two shared slabs and consumed after a
// barrier by every owning wave.  A slab is rewritten two tiles later, after
// the barrier that follows its last reads.

template <int DT, int MODE, int NQT>
__device__ __forceinline__ void attn_item_rows(const AttnArgs& a, const int b, const int hk, const int split,
                                               const Span* span, unsigned char* s_stage, float (*s_m)[16],
                                               float (*s_l)[16]) {
  using M = MT<DT>;
  using V8 = typename M::V8;
  using S = typename M::S;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 15, lg = lane >> 4;
  // (with fewer query tiles than waves, the rest would only fetch; a scalar,
  // so that the branch on it is uniform)
  const bool owner = __builtin_amdgcn_readfirstlane(w) < NQT;
  const int qt = owner ? w : 0;
  const int v0 = span ? span->v0 : split * a.tpw;
  const size_t qrow0 = ((size_t)b * a.Hq + (size_t)hk * a.G) * a.Qn;
  const int row = qt * 16 + lq;
  V8 qreg[1][4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (owner && row < a.rows) x = *(const u32x4*)(a.q + (qrow0 + row) * kHeadDim + 32 * s + 8 * lg);
    qreg[0][s] = __builtin_bit_cast(V8, x);
  }
  uint64_t tm[1];
  tm[0] = (MODE == kVerifyTree && owner && row < a.rows) ? a.tmask[(size_t)b * a.Qn + row % a.Qn] : 0ull;

  const SeqDesc sd = load_seq(a, b);
  const Geo geo = make_geo<MODE>(a, sd);
  const int tbase = geo.n - a.Qn;  // tree: cache row of node 0
  const size_t bh = (size_t)b * a.Hkv + hk;
  int nsp, v1;
  long part;  // partial slot (when nsp > 1)
  if (span) {
    nsp = span->part < 0 ? 1 : 2;
    v1 = min(geo.L, span->v1);
    part = span->part;
  } else {
    nsp = max(1, (geo.L + a.tpw - 1) / a.tpw);
    if (split >= nsp) return;
    v1 = min(geo.L, v0 + a.tpw);
    part = (long)(bh * a.nsplit + split);
  }
  const size_t base = (size_t)sd.base + (size_t)hk * (size_t)geo.cap * kHeadDim;
  const uint16_t* __restrict__ Kb = a.K + base;
  const uint16_t* __restrict__ Vb = a.V + base;

  int lim[1];
  lim[0] = (MODE == kVerify) ? geo.n - a.Qn + (row % a.Qn) : 0x7fffffff;
  const int lim_min = (MODE == kVerify) ? geo.n - a.Qn : 0x7fffffff;
  V8 sel[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[h][e] = (S)((8 * lg + e == 16 * h + lq) ? 1.0f : 0.0f);
  f32x4 acc[1][8];
#pragma unroll
  for (int bb = 0; bb < 8; ++bb) acc[0][bb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run[1] = {kNegInf}, l_run[1] = {0.f};
  const float c2 = a.scale_log2;

  // this wave's part of a tile: slab rows 16 w .. 16 w + 15 (K rows 0-31, then V rows 0-31)
  const uint16_t* src = w >= 2 ? Vb : Kb;
  const int rbase = 16 * (w & 1);  // first tile row this wave fetches
  auto fetch = [&](u32x4 (&r)[4], int t0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // rows that hold nothing read row 0 (in bounds) and are masked
      const int rv = map_row<MODE>(a, geo, t0 + rbase + 4 * i + (lane >> 4), v1, nullptr, 0);
      r[i] = __builtin_nontemporal_load((const u32x4*)(src + (size_t)(rv < 0 ? 0 : rv) * kHeadDim + 8 * (lane & 15)));
    }
  };
  auto stage = [&](const u32x4 (&r)[4], unsigned char* slab) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *(u32x4*)(slab + (16 * w + 4 * i + (lane >> 4)) * kPitch + 16 * (lane & 15)) = r[i];
  };
  // (an item with no rows fetches nothing: the sequence may have no row 0)
  const int ntiles = v1 > v0 ? (v1 - v0 + kTile - 1) / kTile : 0;
  auto consume = [&](const u32x4 (&r)[4], int i) {
    const int t = v0 + kTile * i;
    unsigned char* slab = s_stage + (i & 1) * kStageBytes;
    stage(r, slab);
    const unsigned mask =
        (unsigned)(__ballot(map_row<MODE>(a, geo, t + (lane & 31), v1, nullptr, 0) >= 0) & 0xFFFFFFFFull);
    __syncthreads();
    if (owner) {
      __builtin_amdgcn_sched_barrier(0);
      process_tile<DT, MODE, 1>(SlabSource<DT>(slab, lane), mask, t, qreg, sel, lim, lim_min, tm, tbase, acc, m_run,
                                l_run, c2, lq, lg);
    }
  };
  // Two groups of two tiles alternate: while one group's tiles are consumed
  // the other's are in flight, and the group after next is requested before
  // the first of them is staged.  At the loop's head only one group is in
  // flight, so the compiler's waits there (which, with the loop's exits
  // leading back to its head, cover the loads in flight as if any were
  // still pending) hold at most that group; with a ring of four tiles they
  // drained the whole ring every fourth tile.  Fetches past the range read
  // row 0, masked.
  if (ntiles > 0) {
    u32x4 A[2][4], B[2][4];
    fetch(A[0], v0);
    fetch(A[1], v0 + kTile);
    for (int i = 0;; i += 4) {
      __builtin_amdgcn_sched_barrier(0);
      fetch(B[0], v0 + kTile * (i + 2));
      fetch(B[1], v0 + kTile * (i + 3));
      consume(A[0], i);
      if (i + 1 >= ntiles) break;
      consume(A[1], i + 1);
      if (i + 2 >= ntiles) break;
      __builtin_amdgcn_sched_barrier(0);
      fetch(A[0], v0 + kTile * (i + 4));
      fetch(A[1], v0 + kTile * (i + 5));
      consume(B[0], i + 2);
      if (i + 3 >= ntiles) break;
      consume(B[1], i + 3);
      if (i + 4 >= ntiles) break;
    }
  }
  __syncthreads();  // every slab consumed: the results reuse them

  // each owning wave's rows are complete for this split
  float (*s_o)[16][132] = reinterpret_cast<float (*)[16][132]>(s_stage);
  float lsum = l_run[0];
  lsum = rows4_sum(lsum);
  if (owner) {
    if (lg == 0) {
      s_m[w][lq] = m_run[0];
      s_l[w][lq] = lsum;
    }
#pragma unroll
    for (int bb = 0; bb < 8; ++bb) *(f32x4*)&s_o[w][lq][16 * bb + 4 * lg] = acc[0][bb];
  }
  __syncthreads();
  const int q = tid >> 4;          // 0..15
  const int dc = (tid & 15) * 8;   // 8 dims per thread
#pragma unroll
  for (int t2 = 0; t2 < NQT; ++t2) {
    const int r2 = t2 * 16 + q;
    if (r2 < a.rows) {
      const float Mx = s_m[t2][q], Ls = s_l[t2][q];
      float o[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) o[j] = s_o[t2][q][dc + j];
      if (nsp == 1) {
        const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
        float* dst = a.out + (qrow0 + r2) * kHeadDim + dc;
        *(f32x4*)dst = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
        *(f32x4*)(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
        if (a.lse && dc == 0) a.lse[qrow0 + r2] = Ls > 0.f ? Mx * a.scale_ln + logf(Ls) : kNegInf;
      } else {
        const size_t pr = (size_t)part * a.rows_pad + r2;
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
  __syncthreads();  // (LDS reused by the next item of a flat grid)
}

// One work item: split `split` of KV head hk of sequence b, by the whole
// workgroup (the LDS arrays are the kernel's).  SHORT: a sparse item of at
// most 8 tiles (tpw <= 256), so that no wave takes more than two.
template <int DT, int MODE, int NQT, bool SHORT>
__device__ __forceinline__ void attn_item(const AttnArgs& a, const int b, const int hk, const int split,
                                          const Span* span, int* s_idx, unsigned char* s_stage, float (*s_m)[16],
                                          float (*s_l)[16]) {
  using M = MT<DT>;
  using V8 = typename M::V8;
  using S = typename M::S;
  constexpr bool kStaged = MODE == kVerify || MODE == kVerifyTree;
  if constexpr (kStaged && NQT >= 3) {
    attn_item_rows<DT, MODE, NQT>(a, b, hk, split, span, s_stage, s_m, s_l);
    return;
  }
  float (*s_o)[16][132] = reinterpret_cast<float (*)[16][132]>(s_stage);

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int lq = lane & 15, lg = lane >> 4;
  const int v0 = span ? span->v0 : split * a.tpw;

  // Loads that need only the arguments (chunk slots, query rows) are issued
  // before the sequence geometry is read, so their round trips overlap it.
  // The workgroup's slot table (LDS) covers every chunk virtual tokens
  // [v0, v0 + tpw) can touch, clamped to the k slots of the row, so its loads
  // stay in bounds whatever the sequence length turns out to be.  A staged
  // sparse wave also reads the slots of its first two tiles itself, into
  // registers, so that those tiles' loads need no LDS read and no barrier:
  // they follow the slots' one round trip, and the table (used from a wave's
  // third tile on) is waited for after them.  Where no wave has a third
  // tile (SHORT) there is no table, and so no barrier before the first tile.
  constexpr bool kSparseIdx = MODE == kSparse || MODE == kSparseTail;
  constexpr bool kStaged2 = kSparseIdx && NQT <= 2;
  constexpr bool kTable = kSparseIdx && !(kStaged2 && SHORT);
  static_assert(!SHORT || kStaged2, "two tiles per wave: staged sparse items only");
  constexpr int kIdxPerThread = kTable ? (kMaxSparseIdx + kThreads - 1) / kThreads : 1;
  TileIdx ci0, ci1;
  int chunk_lo = 0, n_idx = 0;
  int idx_reg[kIdxPerThread];
  if (kSparseIdx) {
    const int32_t* slots = a.idx + ((size_t)b * a.Hkv + hk) * a.k;
    if (kStaged2) {
      fetch_tile_idx(ci0, a, slots, v0 + kTile * w, lane);
      fetch_tile_idx(ci1, a, slots, v0 + kTile * w + 4 * kTile, lane);
    }
    chunk_lo = v0 / a.cs;
    n_idx = min(a.k, (v0 + a.tpw + a.cs - 1) / a.cs) - chunk_lo;
    // (unconditional loads, each slot clamped into the row: a load under a
    // branch makes the compiler's later waits for it waits for every load)
    if constexpr (kTable) {
#pragma unroll
      for (int u = 0; u < kIdxPerThread; ++u) idx_reg[u] = slots[min(chunk_lo + tid + u * kThreads, a.k - 1)];
    }
  }

  // Query rows of this KV head: heads hk*G .. hk*G+G-1, Qn rows each, contiguous.
  const size_t qrow0 = ((size_t)b * a.Hq + (size_t)hk * a.G) * a.Qn;
  V8 qreg[NQT][4];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int row = qt * 16 + lq;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < a.rows) x = *(const u32x4*)(a.q + (qrow0 + row) * kHeadDim + 32 * s + 8 * lg);
      qreg[qt][s] = __builtin_bit_cast(V8, x);
    }
  }

  uint64_t tm[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int row = qt * 16 + lq;
    tm[qt] = (MODE == kVerifyTree && row < a.rows) ? a.tmask[(size_t)b * a.Qn + row % a.Qn] : 0ull;
  }

  const SeqDesc sd = load_seq(a, b);
  const Geo geo = make_geo<MODE>(a, sd);
  const int tbase = geo.n - a.Qn;  // tree: cache row of node 0
  const size_t bh = (size_t)b * a.Hkv + hk;
  int nsp, v1;
  long part;  // partial slot (when nsp > 1)
  if (span) {
    nsp = span->part < 0 ? 1 : 2;
    v1 = min(geo.L, span->v1);
    part = span->part;
  } else {
    nsp = max(1, (geo.L + a.tpw - 1) / a.tpw);
    if (split >= nsp) return;
    v1 = min(geo.L, v0 + a.tpw);
    part = (long)(bh * a.nsplit + split);
  }

  const size_t base = (size_t)sd.base + (size_t)hk * (size_t)geo.cap * kHeadDim;
  const uint16_t* __restrict__ Kb = a.K + base;
  const uint16_t* __restrict__ Vb = a.V + base;

  // the slot table: written now, waited for (a barrier) before its first
  // use -- here, or after a staged wave's first loads
  if (kTable) {
#pragma unroll
    for (int u = 0; u < kIdxPerThread; ++u) {
      const int j = tid + u * kThreads;
      if (j < n_idx) s_idx[j] = idx_reg[u];
    }
    if (!kStaged2) __syncthreads();
  }

  int lim[NQT];
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    const int row = qt * 16 + lq;
    // Causal limit of this lane's query row i = row % Qn, as a virtual token:
    // verify sees cache rows <= n - Qn + i; with a tail, virtual token
    // k*cs + (r - lo) is cache row r.
    const int causal0 = (MODE == kVerify) ? geo.n - a.Qn : a.k * a.cs + (geo.n - geo.lo) - a.Qn;
    lim[qt] = (MODE == kVerify || MODE == kSparseTail) ? causal0 + (row % a.Qn) : 0x7fffffff;
  }
  const int lim_min = (MODE == kVerify)       ? geo.n - a.Qn
                      : (MODE == kSparseTail) ? a.k * a.cs + (geo.n - geo.lo) - a.Qn
                                              : 0x7fffffff;

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

  // Software pipeline: while a wave consumes the tile staged in its slab, the
  // next tile's 16 loads are in flight.  The prefetch is unconditional (past
  // the end it reads row 0, masked), so every iteration has the same loads
  // outstanding.  LDS operations of one wave complete in order, so a slab is
  // rewritten only after the previous tile's operand reads.
  int t = v0 + kTile * w;
  if constexpr (kStaged2) {
    // two register stages alternate into the slab; the next-but-one tile's
    // loads are issued while the staged one is consumed
    // (issued by every wave, also one with no tile in the range -- its rows
    // are all row 0, masked: a branch around the loads would make the
    // compiler's waits after it count these loads too)
    // (the scheduling barrier keeps the first tile's loads ahead of the
    // second's, so that waiting for them does not wait for both)
    Stage sa, sb;
    load_stage_rows(sa, t, [&](int v, int i) { return sparse_row<MODE>(a, geo, v, v1, ci0.c[i]); }, Kb, Vb, lane);
    __builtin_amdgcn_sched_barrier(0);
    load_stage_rows(sb, t + 4 * kTile, [&](int v, int i) { return sparse_row<MODE>(a, geo, v, v1, ci1.c[i]); }, Kb,
                    Vb, lane);
    if (kTable) __syncthreads();  // the slot table (every wave)
    unsigned char* slab = s_stage + w * kStageBytes;
    const SlabSource<DT> src(slab, lane);
    if (t < v1) {
      // The first tile is consumed outside the loop, where the compiler's
      // waits cover only its own loads (at the loop's head they cover every
      // load in flight, here both tiles').  Its mask is taken before the
      // stage is refilled with the wave's third tile.
      const unsigned mask0 = sa.mask;
      write_stage(sa, slab, lane);
      if (kTable && t + 8 * kTile < v1) load_stage<MODE>(sa, a, geo, t + 8 * kTile, v1, s_idx, chunk_lo, Kb, Vb, lane);
      __builtin_amdgcn_sched_barrier(0);
      process_tile<DT, MODE, NQT>(src, mask0, t, qreg, sel, lim, lim_min, tm, tbase, acc, m_run, l_run, c2, lq, lg);
      t += 4 * kTile;
      while (t < v1) {
        unsigned mask = sb.mask;
        write_stage(sb, slab, lane);
        if (kTable && t + 8 * kTile < v1) load_stage<MODE>(sb, a, geo, t + 8 * kTile, v1, s_idx, chunk_lo, Kb, Vb, lane);
        __builtin_amdgcn_sched_barrier(0);
        process_tile<DT, MODE, NQT>(src, mask, t, qreg, sel, lim, lim_min, tm, tbase, acc, m_run, l_run, c2, lq, lg);
        t += 4 * kTile;
        if (t >= v1) break;
        mask = sa.mask;
        write_stage(sa, slab, lane);
        if (kTable && t + 8 * kTile < v1) load_stage<MODE>(sa, a, geo, t + 8 * kTile, v1, s_idx, chunk_lo, Kb, Vb, lane);
        __builtin_amdgcn_sched_barrier(0);
        process_tile<DT, MODE, NQT>(src, mask, t, qreg, sel, lim, lim_min, tm, tbase, acc, m_run, l_run, c2, lq, lg);
        t += 4 * kTile;
      }
    }
  } else if (kStaged && t < v1) {
    unsigned char* slab = s_stage + w * kStageBytes;
    const SlabSource<DT> src(slab, lane);
    // (one stage in flight, so the wait before staging a tile is exact with or
    // without a prefetch; none is requested past the range)
    Stage st;
    load_stage<MODE>(st, a, geo, t, v1, s_idx, chunk_lo, Kb, Vb, lane);
    unsigned mask = st.mask;
    write_stage(st, slab, lane);
    if (t + 4 * kTile < v1) load_stage<MODE>(st, a, geo, t + 4 * kTile, v1, s_idx, chunk_lo, Kb, Vb, lane);
    while (true) {
      __builtin_amdgcn_sched_barrier(0);
      process_tile<DT, MODE, NQT>(src, mask, t, qreg, sel, lim, lim_min, tm, tbase, acc, m_run, l_run, c2, lq, lg);
      t += 4 * kTile;
      if (t >= v1) break;
      mask = st.mask;
      write_stage(st, slab, lane);
      if (t + 4 * kTile < v1) load_stage<MODE>(st, a, geo, t + 4 * kTile, v1, s_idx, chunk_lo, Kb, Vb, lane);
    }
  } else if (!kStaged && !kStaged2 && t < v1) {
    Tile<DT> A, B;
    load_tile<DT, MODE>(A, a, geo, t, v1, s_idx, chunk_lo, Kb, Vb, lq, lg);
    // A wave with at most two tiles (the 4 + 252 ring: two each) requests
    // nothing past them: the loop below would request a third, past the end
    // (row 0, masked), and that tile's 16 KB through the one compute unit's
    // load path cost 0.45 us of 8.2 (1 or 2 query tiles; with 3-4 the extra
    // copies of the tile step do not fit the registers).
    if (NQT <= 2 && t + 8 * kTile >= v1) {
      load_tile<DT, MODE>(B, a, geo, t + 4 * kTile, v1, s_idx, chunk_lo, Kb, Vb, lq, lg);
      __builtin_amdgcn_sched_barrier(0);
      process_tile<DT, MODE, NQT>(RegSource<DT>{A}, A.mask, t, qreg, sel, lim, lim_min, tm, tbase, acc, m_run,
                                  l_run, c2, lq, lg);
      if (t + 4 * kTile < v1) {
        __builtin_amdgcn_sched_barrier(0);
        process_tile<DT, MODE, NQT>(RegSource<DT>{B}, B.mask, t + 4 * kTile, qreg, sel, lim, lim_min, tm, tbase, acc,
                                    m_run, l_run, c2, lq, lg);
      }
    } else while (true) {
      load_tile<DT, MODE>(B, a, geo, t + 4 * kTile, v1, s_idx, chunk_lo, Kb, Vb, lq, lg);
      __builtin_amdgcn_sched_barrier(0);
      process_tile<DT, MODE, NQT>(RegSource<DT>{A}, A.mask, t, qreg, sel, lim, lim_min, tm, tbase, acc, m_run,
                                  l_run, c2, lq, lg);
      t += 4 * kTile;
      if (t >= v1) break;
      load_tile<DT, MODE>(A, a, geo, t + 4 * kTile, v1, s_idx, chunk_lo, Kb, Vb, lq, lg);
      __builtin_amdgcn_sched_barrier(0);
      process_tile<DT, MODE, NQT>(RegSource<DT>{B}, B.mask, t, qreg, sel, lim, lim_min, tm, tbase, acc, m_run,
                                  l_run, c2, lq, lg);
      t += 4 * kTile;
      if (t >= v1) break;
    }
  }
  if (kStaged || kStaged2) __syncthreads();  // every slab consumed: the merge reuses them

  // ---- merge the four waves (per query tile) -------------------------------
#pragma unroll
  for (int qt = 0; qt < NQT; ++qt) {
    float lsum = l_run[qt];
    lsum = rows4_sum(lsum);
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
        float acc_o = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) acc_o += ew[x] * s_o[x][q][dc + j];
        o[j] = acc_o;
      }
      if (row < a.rows) {
        if (nsp == 1) {
          const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
          float* dst = a.out + (qrow0 + row) * kHeadDim + dc;
          *(f32x4*)dst = f32x4{o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv};
          *(f32x4*)(dst + 4) = f32x4{o[4] * inv, o[5] * inv, o[6] * inv, o[7] * inv};
          if (a.lse && dc == 0) a.lse[qrow0 + row] = Ls > 0.f ? Mx * a.scale_ln + logf(Ls) : kNegInf;
        } else {
          const size_t pr = (size_t)part * a.rows_pad + row;
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
}

// Tiles of a batch's verification: sequence b has Hkv * ceil(L_b / 32)
// 32-token tiles (L_b its virtual length), head-major; s_pre[b] = the tiles
// of sequences 0 .. b-1.  Computed by wave 0 from the device-resident lengths
// (the host checks that the total fits an int).
template <int MODE>
__device__ __forceinline__ void flat_prefix(const AttnArgs& a, int* s_pre) {
  const int lane = threadIdx.x & 63;
  if (threadIdx.x >= 64) return;
  int carry = 0;
  for (int b0 = 0; b0 < a.B; b0 += 64) {
    const int b = b0 + lane;
    int tiles = 0;
    if (b < a.B) {
      SeqDesc sd;
      sd.base = 0;
      sd.cap = a.seq_cap[b];
      sd.len = a.seq_len[b];
      const Geo g = make_geo<MODE>(a, sd);
      tiles = a.Hkv * ((g.L + kTile - 1) / kTile);
    }
    const int incl = (int)wave_incl_scan_u32((unsigned)tiles);
    if (b < a.B) s_pre[b + 1] = carry + incl;
    carry += __builtin_amdgcn_readlane(incl, 63);
  }
  if (lane == 0) s_pre[0] = 0;
}

// Equal work per workgroup: of a batch's TT tiles (in sequence, head, tile
// order) workgroup g of G = min(grid, TT) takes tiles [floor(g TT / G),
// floor((g + 1) TT / G)), at least one each (the rest of the grid idles),
// so all G finish together whatever the lengths (items of one split size
// filled 3.7 rounds of the 512 resident workgroups on the 8-sequence batch,
// the last one 69% full).  The workgroup holding tile x is
// floor(((x + 1) G - 1) / TT).  A workgroup's range crosses (sequence, head)
// segments; its part of segment s is written to partial slot g + s (unique:
// along the tile order each cut advances g, s or both), so a segment's parts
// are consecutive slots, merged in order by combine_kernel; a segment inside
// one workgroup is written as output directly.
__device__ __forceinline__ long flat_wg_of(long x, long TT, long G) { return ((x + 1) * G - 1) / TT; }


// One query tile fits two waves per SIMD (<= 256 registers, no spills);
// more query tiles run one wave per SIMD.  Either one work item per
// workgroup (grid = splits x KV heads x sequences), or, for the verification
// of a ragged batch (FLAT), a one-dimensional grid whose workgroups take
// items i, i + gridDim.x, ... of the batch's actual items: with a grid sized
// for the longest sequence, the items of short sequences would leave most
// workgroups empty and, since workgroups go to the XCDs in index order, load
// the XCDs unevenly.  SHORT: sparse items of at most 8 tiles (see attn_item),
// which keep no slot table.
template <int DT, int MODE, int NQT, bool FLAT, bool SHORT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(
    (NQT == 1 || ((MODE == kVerify || MODE == kVerifyTree) && NQT >= 3)) ? 2 : 1,
    (NQT == 1 || ((MODE == kVerify || MODE == kVerifyTree) && NQT >= 3)) ? 2 : 1)))
void attn_kernel(const AttnArgs a) {
  constexpr bool kStaged = MODE == kVerify || MODE == kVerifyTree;
  // four wave-private slabs (verify and sparse with up to two query tiles),
  // the two shared slabs of the row split (verify, 3-4 tiles), or the merge
  // buffer alone (direct loads)
  constexpr bool kSlabs4 = (kStaged && NQT <= 2) || ((MODE == kSparse || MODE == kSparseTail) && NQT <= 2);
  constexpr int kStageLds = kSlabs4 ? 4 * kStageBytes : (kStaged ? 2 * kStageBytes : kMergeBytes);
  static_assert(kMergeBytes <= 2 * kStageBytes, "results must fit in two slabs");
  __shared__ int s_idx[(MODE == kSparse || MODE == kSparseTail) && !SHORT ? kMaxSparseIdx : 1];
  __shared__ __attribute__((aligned(16))) unsigned char s_stage[kStageLds];
  __shared__ float s_m[4][16];
  __shared__ float s_l[4][16];
  __shared__ int s_pre[FLAT ? kMaxFlatSeqs + 1 : 1];
  if (FLAT) {
    flat_prefix<MODE>(a, s_pre);
    __syncthreads();
    if (blockIdx.x == 0)  // for the merge kernel
      for (int j = threadIdx.x; j <= a.B; j += kThreads) a.flat_prefix[j] = s_pre[j];
    // (G <= TT: with more workgroups than tiles some would get none, and the
    // merge's consecutive slots would skip theirs)
    const long TT = s_pre[a.B], G = min((long)gridDim.x, TT);
    long x = (long)blockIdx.x * TT / max(G, 1L);
    const long xe = blockIdx.x < G ? ((long)blockIdx.x + 1) * TT / G : x;
    while (x < xe) {
      int lo = 0, hi = a.B;  // the sequence: largest b with s_pre[b] <= x (its tiles are not empty)
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pre[mid] <= x) lo = mid; else hi = mid;
      }
      const long T = (s_pre[lo + 1] - s_pre[lo]) / a.Hkv;  // tiles per head of sequence lo
      const long rel = x - s_pre[lo];
      const int hk = (int)(rel / T);
      const long seg0 = s_pre[lo] + (long)hk * T, seg1 = seg0 + T;
      const long x1 = min(xe, seg1);
      Span sp;
      sp.v0 = (int)((x - seg0) * kTile);
      sp.v1 = (int)((x1 - seg0) * kTile);
      sp.part = flat_wg_of(seg0, TT, G) == flat_wg_of(seg1 - 1, TT, G) ? -1L
                                                                           : (long)blockIdx.x + (long)lo * a.Hkv + hk;
      attn_item<DT, MODE, NQT, SHORT>(a, lo, hk, 0, &sp, s_idx, s_stage, s_m, s_l);
      x = x1;
    }
  } else {
    // One item per workgroup: grid (splits, KV heads, sequences), or, when
    // the plan ends in a short split per (sequence, KV head), a 1-D grid that
    // puts those splits after all the others.  Workgroups are dispatched in
    // index order, so the grid's second round is then made of the short
    // items, not of full splits of the last heads.
    if (a.tail_last) {
      const int heads = a.B * a.Hkv;
      const int full = a.nsplit - 1;
      const int L = blockIdx.x;
      const int split = L < full * heads ? L % full : full;
      const int head = L < full * heads ? L / full : L - full * heads;
      attn_item<DT, MODE, NQT, SHORT>(a, head / a.Hkv, head % a.Hkv, split, nullptr, s_idx, s_stage, s_m, s_l);
    } else {
      attn_item<DT, MODE, NQT, SHORT>(a, blockIdx.z, blockIdx.y, blockIdx.x, nullptr, s_idx, s_stage, s_m, s_l);
    }
  }
}

// Merge of the split partials of every (sequence, KV head, query row) whose
// sequence needed more than one split: one wave per row, two dims per lane,
// splits in order.  Runs as its own launch so that no device-wide fence is
// needed inside the attention kernel.  Splits are taken in groups of GROUP
// (4, 8, 16 or 32: the smallest that holds the plan's split count; 32 for a
// batch on the equal-work grid): the group's (max, sum) pairs and its
// accumulator rows are all requested before any is used, so a group costs
// one memory round trip; groups are folded with an online rescale.  (Groups
// of 32 for 16 splits requested 16 clamped duplicates per lane: the sparse
// call at the Llama2-7B-128K shape took 0.6 us more, the 8-sequence batch's
// 1.1 us more, outputs bitwise equal since the extra terms are zeros.)  The first group is requested before the
// sequence geometry is known: every split index below the planned split count
// lies inside the workspace, and splits past this sequence's own count are
// dropped by selection (their contents are never combined arithmetically).
// Lane s of the wave holds split s's (max, sum): the group's max is a
// register reduction, lane s computes split s's weight (one exponential per
// lane), and the (weight, sum) pairs reach every lane through GROUP / 2
// broadcast LDS reads; the weighted sum and the accumulators are then folded in split
// order.  (This replaced ~128 readlane broadcasts per group, each followed
// by hazard waits: bit-identical results, the sparse call 19.92 -> 19.82 us.)

template <int MODE, bool FLAT, int GROUP>
__global__ __launch_bounds__(64) void combine_kernel(const AttnArgs a) {
  constexpr int kGroup = GROUP;
  __shared__ __attribute__((aligned(16))) float2 s_el[kGroup];
  const int row = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const float c2 = a.scale_log2;
  const size_t bh = (size_t)b * a.Hkv + hk;
  const float2* ml = (const float2*)a.part_ml;
  size_t pbase = bh * a.nsplit * a.rows_pad + row;  // (the equal-work plan sets it below)

  float2 mlv;
  float2 v[kGroup];
  // Loads are unconditional, from split indices clamped into [0, bound):
  // a conditional load becomes a branch of its own and waits on its result.
  auto load_group = [&](int s0, int bound) {
    const int sl = min(s0 + (lane & (kGroup - 1)), bound - 1);
    mlv = ml[pbase + (size_t)sl * a.rows_pad];
#pragma unroll
    for (int u = 0; u < kGroup; ++u)
      v[u] = *(const float2*)(a.part_o + (pbase + (size_t)min(s0 + u, bound - 1) * a.rows_pad) * kHeadDim + 2 * lane);
  };
  int nsp;
  if constexpr (FLAT) {
    // the segment's parts: consecutive slots from (its first workgroup) + s,
    // located from the tile prefix the attention kernel stored
    if (row >= a.rows) return;
    const long p0 = a.flat_prefix[b], p1 = a.flat_prefix[b + 1], TT = a.flat_prefix[a.B];
    const long T = (p1 - p0) / a.Hkv;
    if (T == 0) {  // no rows: nothing attended
      const size_t qrow0 = ((size_t)b * a.Hq + (size_t)hk * a.G) * a.Qn;
      *(float2*)(a.out + (qrow0 + row) * kHeadDim + 2 * lane) = make_float2(0.f, 0.f);
      if (a.lse && lane == 0) a.lse[qrow0 + row] = kNegInf;
      return;
    }
    const long seg0 = p0 + (long)hk * T, G = min((long)a.flat_wgs, TT);
    const long g0 = flat_wg_of(seg0, TT, G);
    nsp = (int)(flat_wg_of(seg0 + T - 1, TT, G) - g0 + 1);
    if (nsp == 1) return;  // written directly by the attention kernel
    pbase = (size_t)(g0 + (long)bh) * a.rows_pad + row;
    load_group(0, nsp);
  } else {
    SeqDesc sd;
    sd.base = 0;  // not used by the geometry
    sd.cap = a.seq_cap[b];
    sd.len = a.seq_len[b];
    load_group(0, a.nsplit);
    // Every load above is consumed here, before the geometry decides whether
    // this row merges at all: otherwise the compiler sinks the group's loads
    // past that branch and the descriptor read and the group become two
    // serial round trips instead of one.
    asm volatile("" : : "v"(sd.cap), "v"(sd.len), "v"(mlv.x), "v"(mlv.y));
#pragma unroll
    for (int u = 0; u < kGroup; ++u) asm volatile("" : : "v"(v[u].x), "v"(v[u].y));
    const Geo geo = make_geo<MODE>(a, sd);
    nsp = max(1, (geo.L + a.tpw - 1) / a.tpw);
    if (nsp == 1 || row >= a.rows) return;  // written directly by the attention kernel
  }

  float Mx = kNegInf, Ls = 0.f, o0 = 0.f, o1 = 0.f;
  for (int s0 = 0; s0 < nsp; s0 += kGroup) {
    if (s0 > 0) {
      __syncthreads();  // (the previous group's reads of s_el are done)
      load_group(s0, nsp);
    }
    if (s0 + (lane & (kGroup - 1)) >= nsp) mlv = make_float2(kNegInf, 0.f);
#pragma unroll
    for (int u = 0; u < kGroup; ++u)
      if (s0 + u >= nsp) v[u] = make_float2(0.f, 0.f);
    const float gm = wave_max(mlv.x);  // (lanes 32-63 repeat lanes 0-31)
    const float Mn = fmaxf(Mx, gm);
    if (Mn == kNegInf) continue;  // nothing seen yet
    const float r = (Mx == kNegInf) ? 0.f : fast_exp2((Mx - Mn) * c2);
    const float e = (mlv.x == kNegInf) ? 0.f : fast_exp2((mlv.x - Mn) * c2);
    // every lane needs every split's (weight, sum): lane s publishes split
    // s's, and all lanes read them back with broadcast LDS reads
    if (lane < kGroup) s_el[lane] = make_float2(e, mlv.y);
    __syncthreads();
    float2 el[kGroup];
#pragma unroll
    for (int q = 0; q < kGroup / 2; ++q) {
      const float4 t = ((const float4*)s_el)[q];
      el[2 * q] = make_float2(t.x, t.y);
      el[2 * q + 1] = make_float2(t.z, t.w);
    }
    float le = 0.f;
#pragma unroll
    for (int u = 0; u < kGroup; ++u) le += el[u].x * el[u].y;
    Ls = Ls * r + le;
    o0 *= r;
    o1 *= r;
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      o0 += el[u].x * v[u].x;
      o1 += el[u].x * v[u].y;
    }
    Mx = Mn;
  }
  const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
  const size_t qrow0 = ((size_t)b * a.Hq + (size_t)hk * a.G) * a.Qn;
  *(float2*)(a.out + (qrow0 + row) * kHeadDim + 2 * lane) = make_float2(o0 * inv, o1 * inv);
  if (a.lse && lane == 0) a.lse[qrow0 + row] = Ls > 0.f ? Mx * a.scale_ln + logf(Ls) : kNegInf;
}

SplitPlan plan_splits(int32_t B, int32_t Hkv, int32_t rows, int32_t max_virtual, int32_t target_wgs,
                      int32_t max_tpw, int32_t min_tpw) {
  SplitPlan p;
  const long heads = (long)B * Hkv;
  const long per_head = target_wgs / heads;  // splits per (sequence, KV head) that keep the grid within target
  long tpw = max_tpw;
  p.tail_last = 0;
  if (per_head >= 1 && (long)max_virtual > per_head * max_tpw &&
      (long)max_virtual - per_head * max_tpw <= max_tpw / 8) {
    p.tail_last = 1;
    // one round of full splits and a tail split of at most max_tpw / 8
    // virtual tokens per (sequence, head): the tails are dispatched last
    // (short items, run as the first full splits finish), cheaper than two
    // rounds of half-size splits (a cache allocated a little past its
    // length: Llama2-7B-128K with 512 spare rows, verify 322 -> 318 us)
  } else if (per_head >= 1) {
    // whole rounds of per_head splits: one when the splits fit max_tpw, else
    // as few as do (a last round of a few long splits would run on its own)
    const long rounds = ((long)max_virtual + per_head * max_tpw - 1) / (per_head * max_tpw);
    const long n = per_head * max(1L, rounds);
    long fit = ((long)max_virtual + n - 1) / n;
    fit = max((long)min_tpw, (fit + kTile - 1) / kTile * kTile);
    if (fit < tpw) tpw = fit;
  }
  p.flat_wgs = 0;
  p.flat_prefix_bytes = 0;
  p.tpw = (int32_t)tpw;
  p.nsplit = (int32_t)(((long)max_virtual + tpw - 1) / tpw);
  if (p.nsplit < 1) p.nsplit = 1;
  p.rows_pad = ((rows + 15) / 16) * 16;
  const size_t parts = (size_t)heads * p.nsplit * p.rows_pad;
  if (p.nsplit > 1) {
    p.part_ml_bytes = (parts * 2 * sizeof(float) + 255) & ~(size_t)255;
    p.part_o_bytes = parts * kHeadDim * sizeof(float);
  } else {
    p.part_o_bytes = p.part_ml_bytes = 0;
  }
  p.total_bytes = p.part_ml_bytes + p.part_o_bytes;
  return p;
}

bool flat_eligible(int32_t B, int32_t Hkv, int32_t max_len) {
  const long tiles = (long)B * Hkv * (((long)max_len + kTile - 1) / kTile);
  return B > 1 && B <= kMaxFlatSeqs && tiles < 0x7fffffffL;
}

SplitPlan plan_flat(int32_t B, int32_t Hkv, int32_t rows, int32_t G) {
  SplitPlan p;
  p.tail_last = 0;
  p.flat_wgs = G;
  p.tpw = 0;  // (spans come from the tile ranges)
  p.nsplit = G + B * Hkv;
  p.rows_pad = ((rows + 15) / 16) * 16;
  const size_t parts = (size_t)p.nsplit * p.rows_pad;
  p.part_ml_bytes = (parts * 2 * sizeof(float) + 255) & ~(size_t)255;
  p.part_o_bytes = parts * kHeadDim * sizeof(float);
  p.flat_prefix_bytes = ((size_t)(B + 1) * sizeof(int32_t) + 255) & ~(size_t)255;
  p.total_bytes = p.part_ml_bytes + p.part_o_bytes + p.flat_prefix_bytes;
  return p;
}

template <int DT, int MODE, int NQT, bool FLAT, bool MAY_SHORT>
static void launch_kernel(bool short_items, dim3 grid, dim3 block, hipStream_t stream, const AttnArgs& a) {
  if constexpr (MAY_SHORT) {
    if (short_items) {
      hipLaunchKernelGGL((attn_kernel<DT, MODE, NQT, FLAT, true>), grid, block, 0, stream, a);
      return;
    }
  }
  hipLaunchKernelGGL((attn_kernel<DT, MODE, NQT, FLAT, false>), grid, block, 0, stream, a);
}

template <int DT, int MODE, bool FLAT>
static hipError_t launch_tiles(const AttnArgs& a, hipStream_t stream) {
  dim3 grid(a.nsplit, a.Hkv, a.B), block(kThreads);
  if (a.tail_last) {
    if ((long)a.nsplit * a.Hkv * a.B > 0x7fffffffL) return hipErrorInvalidConfiguration;
    grid = dim3((unsigned)((long)a.nsplit * a.Hkv * a.B), 1, 1);
  }
  if (FLAT) grid = dim3((unsigned)a.flat_wgs, 1, 1);
  const int nqt = (a.rows + 15) / 16;
  // sparse items of at most 8 tiles (two per wave) keep no slot table
  constexpr bool kMayShort = (MODE == kSparse || MODE == kSparseTail) && !FLAT;
  const bool short_items = kMayShort && a.tpw <= 8 * kTile;
  switch (nqt) {
    case 1: launch_kernel<DT, MODE, 1, FLAT, kMayShort>(short_items, grid, block, stream, a); break;
    case 2: launch_kernel<DT, MODE, 2, FLAT, kMayShort>(short_items, grid, block, stream, a); break;
    case 3: launch_kernel<DT, MODE, 3, FLAT, false>(false, grid, block, stream, a); break;
    case 4: launch_kernel<DT, MODE, 4, FLAT, false>(false, grid, block, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (!FLAT && a.nsplit == 1)) return e;
  const dim3 cgrid(a.rows, a.Hkv, a.B);
  if (!FLAT && a.nsplit <= 4)
    hipLaunchKernelGGL((combine_kernel<MODE, FLAT, 4>), cgrid, dim3(64), 0, stream, a);
  else if (!FLAT && a.nsplit <= 8)
    hipLaunchKernelGGL((combine_kernel<MODE, FLAT, 8>), cgrid, dim3(64), 0, stream, a);
  else if (!FLAT && a.nsplit <= 16)
    hipLaunchKernelGGL((combine_kernel<MODE, FLAT, 16>), cgrid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL((combine_kernel<MODE, FLAT, 32>), cgrid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

// Verification of a batch takes the equal-work grid when its plan says so;
// everything else one item per workgroup.
template <int DT, int MODE>
static hipError_t launch_nqt(const AttnArgs& a, hipStream_t stream) {
  if constexpr (MODE == kVerify || MODE == kVerifyTree) {
    if (a.flat_wgs > 0) return launch_tiles<DT, MODE, true>(a, stream);
  }
  return launch_tiles<DT, MODE, false>(a, stream);
}

template <int DT>
static hipError_t launch_mode(int mode, const AttnArgs& a, hipStream_t stream) {
  switch (mode) {
    case kVerify: return launch_nqt<DT, kVerify>(a, stream);
    case kSparse: return launch_nqt<DT, kSparse>(a, stream);
    case kStream: return launch_nqt<DT, kStream>(a, stream);
    case kSparseTail: return launch_nqt<DT, kSparseTail>(a, stream);
    case kVerifyTree: return launch_nqt<DT, kVerifyTree>(a, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn(int dtype, int mode, const AttnArgs& a, hipStream_t stream) {
  if (dtype == TF_DTYPE_BF16) return launch_mode<TF_DTYPE_BF16>(mode, a, stream);
  if (dtype == TF_DTYPE_FP16) return launch_mode<TF_DTYPE_FP16>(mode, a, stream);
  return hipErrorInvalidValue;
}

}  // namespace tfk
