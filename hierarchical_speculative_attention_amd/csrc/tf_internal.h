// Internal declarations shared by the HIP translation units of libtfattn.
// Nothing here is part of the public C ABI (include/tf_attn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "tf_attn.h"

namespace tfk {

constexpr int kHeadDim = 128;
constexpr int kThreads = 256;          // 4 waves of 64 lanes
constexpr int kTile = 32;              // virtual tokens per wave iteration
constexpr int kMaxRows = 64;           // query rows per KV head (4 MFMA query tiles)

enum AttnMode { kVerify = 0, kSparse = 1, kStream = 2, kSparseTail = 3, kVerifyTree = 4 };

struct AttnArgs {
  const uint16_t* q;        // [B][Hq][Qn][d]
  const uint16_t* K;
  const uint16_t* V;
  const int64_t* seq_base;
  const int32_t* seq_cap;
  const int32_t* seq_len;
  int32_t max_len;
  int32_t B, Hq, Hkv, G, Qn, rows;  // rows = G * Qn query rows per KV head
  // sparse
  const int32_t* idx;       // [B][Hkv][k]
  int32_t k, cs;
  int32_t tail;             // sparse with tail: most recent rows attended causally
  // stream
  int32_t n_sink, window;
  // verification over a candidate tree
  const uint64_t* tmask;    // [B][Qn]: bit m = the row sees tree node m (cache row n - Qn + m)
  // split-K
  int32_t tpw;              // virtual tokens per workgroup (multiple of 128)
  int32_t nsplit;           // splits of the longest sequence (partial-buffer stride; the 3-D grid's x)
  int32_t rows_pad;         // 16 * query tiles
  int32_t tail_last;        // the plan ends with a short split per (sequence, head), dispatched after the rest
  int32_t flat_wgs;         // > 0: a batch's verification with equal work per workgroup, on this many
  int32_t* flat_prefix;     // [B + 1] tiles before each sequence, stored by the attention kernel for the merge
  float* out;               // [B][Hq][Qn][d]
  float* lse;               // [B][Hq][Qn] or null
  float* part_o;            // [B][Hkv][nsplit][rows_pad][d]
  float* part_ml;           // [B][Hkv][nsplit][rows_pad][2]
  float scale_log2;         // log2(e) / sqrt(d)
  float scale_ln;           // 1 / sqrt(d)
};

// Split plan shared by the workspace-size functions and the launches.
struct SplitPlan {
  int32_t tpw;
  int32_t nsplit;
  int32_t rows_pad;
  int32_t tail_last;  // one round of full splits and a short last split per (sequence, head)
  int32_t flat_wgs;   // > 0: equal work per workgroup over a batch's tiles (nsplit = partial slots)
  size_t part_o_bytes, part_ml_bytes, flat_prefix_bytes, total_bytes;
};

// Virtual tokens per workgroup: the fewest (a multiple of the tile, at least
// min_tpw, at most max_tpw) that give the grid a whole number of rounds of
// target_wgs workgroups, the number resident at once -- one round when
// max_tpw allows.  A grid a little past a whole round would leave its last
// workgroups to start only when the first ones finish.
constexpr int32_t kVerifyMaxTpw = 8192;
constexpr int32_t kSparseMaxTpw = 1024;
// At least 256 gathered tokens (128 KB of K and V) per workgroup: GQA 512K
// (8 KV heads x 8192 tokens) in 64 splits of 128 took 16.8 us, in 32 of 256
// 15.2 us (one group of partials to merge), in 16 of 512 18.0 us; the
// Llama2-7B-128K layer already takes 256 per split.
constexpr int32_t kVerifyMinTpw = 128;
constexpr int32_t kSparseMinTpw = 256;
SplitPlan plan_splits(int32_t B, int32_t Hkv, int32_t rows, int32_t max_virtual, int32_t target_wgs,
                      int32_t max_tpw, int32_t min_tpw);
// Verification of a batch of 2 .. kMaxFlatSeqs sequences whose tiles
// (B * Hkv * ceil(max_len / 32)) fit an int: every one of G workgroups takes
// an equal share of the batch's tiles, with G + B * Hkv partial slots.
constexpr int kMaxFlatSeqs = 1024;
bool flat_eligible(int32_t B, int32_t Hkv, int32_t max_len);
SplitPlan plan_flat(int32_t B, int32_t Hkv, int32_t rows, int32_t G);

hipError_t launch_attn(int dtype, int mode, const AttnArgs& a, hipStream_t stream);

// chunk keys / scores
hipError_t launch_chunk_keys(const uint16_t* K, const tf_kv_desc& kv, int32_t cs,
                             const int32_t* chunk_begin, int32_t max_chunks,
                             void* ck, const tf_kv_desc& ckd, hipStream_t stream);
hipError_t launch_scores(const uint16_t* q, int32_t q_dtype, int32_t Hq, const void* ck,
                         const tf_kv_desc& ckd, float* scores, int32_t c_max, hipStream_t stream);
// top-k
// Top-k: rows of more than 16384 chunks, at most kTopkSplitMaxRows of them
// per call, are selected in kTopkSlices slices per row and then merged.
constexpr int kTopkSlices = 8;
constexpr int kTopkSplitMaxRows = 16;
struct TopkSplit {
  int S;  // slices per row (1: one workgroup per row)
  int L;  // chunks per slice
};
TopkSplit plan_topk(int32_t B, int32_t rows, int32_t c_max, int32_t k);
size_t topk_workspace_bytes(int32_t B, int32_t rows, int32_t c_max, int32_t k);
hipError_t launch_topk(const float* scores, int32_t B, int32_t rows, int32_t c_max, const int32_t* n_chunks,
                       int32_t k, int32_t* idx, void* ws, hipStream_t stream);
// accept
size_t accept_ws_bytes(int32_t B, int32_t gamma, int32_t V);
int32_t accept_max_vocab();
hipError_t launch_accept(const float* target, const float* draft, const int32_t* tokens,
                         const double* uniforms, int32_t B, int32_t gamma, int32_t V,
                         float temperature, int32_t flags, int32_t* n_acc, int32_t* next,
                         void* ws, hipStream_t stream);

// cache maintenance
hipError_t launch_append(const uint16_t* Knew, const uint16_t* Vnew, int32_t R, uint16_t* K, uint16_t* V,
                         const tf_kv_desc& kv, int32_t mode, int32_t n_sink, int32_t window, int32_t reserve,
                         int32_t* status, hipStream_t stream);
hipError_t launch_commit(int32_t* seq_len, int32_t B, int32_t add, int32_t gamma, const int32_t* n_accepted,
                         hipStream_t stream);

// tree visibility masks from parent pointers
hipError_t launch_tree_masks(const int32_t* parent, int32_t B, int32_t Q, uint64_t* masks, hipStream_t stream);
// accept over a candidate tree
int32_t tree_accept_max_vocab();
int32_t tree_accept_max_nodes();
size_t tree_accept_ws_bytes(int32_t B, int32_t V);
hipError_t launch_tree_accept(const float* target, const float* draft, const int32_t* tokens, const int32_t* parent,
                              const double* uniforms, int32_t B, int32_t Q, int32_t V, float temperature,
                              int32_t flags, int32_t* n_acc, int32_t* path, int32_t* next, void* ws,
                              hipStream_t stream);
// two-level accept: candidate collection
hipError_t launch_collect(const int32_t* draft_tokens, const int32_t* n_accepted, const int32_t* next_token,
                          const float* q_rows, int32_t B, int32_t gamma1, int32_t V, const int32_t* count_in,
                          int32_t* count_out, int32_t* cand, float* cand_q, int32_t gamma2, hipStream_t stream);

}  // namespace tfk
