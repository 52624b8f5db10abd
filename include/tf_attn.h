/*
 * tf_attn.h - C ABI of the MI355X (gfx950) decode-step attention library of
 * hierarchical speculative decoding (TriForce).
 *
 * The operations come from two web pages:
 *   [blog] aifetchly, "TriForce: Hierarchical Speculative Decoding for LLMs",
 *          section "1. The Three Forces of TriForce" (Force 1: a drafter on a
 *          streaming cache of initial sinks plus the most recent W tokens;
 *          Force 2: the target on a retrieval-sparse cache of the top-k KV
 *          blocks chosen by key-query similarity; Force 3: the target on the
 *          full cache verifying the candidates in one pass) and section
 *          "2. Dual Rejection Sampling: Mathematical Losslessness" (accept x
 *          when min(1, p(x)/q(x)) >= u, else draw from the normalised
 *          max(0, p - q)).
 *   [abs]  mlsanity / fugumt pages on arXiv 2404.11912, "Abstract": the whole
 *          KV cache is read for every generated token; a retrieval-based
 *          sparse KV cache acts as draft; robust across temperatures.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every function returns a tf_status.  Arguments are validated on the host
 *    before anything is enqueued; on any error nothing is launched and the
 *    outputs are untouched.  tf_last_error_detail() then describes the error
 *    (thread-local, valid until the next call on that thread).
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *    never allocates, frees or synchronises; scratch memory is a caller-owned
 *    workspace whose size the matching *_workspace_size() function returns.
 *  - Work is enqueued asynchronously on the caller's stream (0 = null stream).
 *  - Results are deterministic: split counts and combine order depend only on
 *    the arguments, so repeated calls give bitwise identical outputs.
 *  - Head dimension d must be 128.  K/V storage is fp16 or bf16; all
 *    attention arithmetic accumulates in fp32 and outputs are fp32.
 *  - Pointers must be 16-byte aligned, and every row offset a descriptor
 *    implies (seq_base[b] and seq_cap[b] * d) a multiple of 8 elements.
 *  - Calls that share one workspace must not overlap in time (same stream or
 *    explicitly ordered).  A workspace needs no initialisation: it only holds
 *    per-split partial results (and, for the verification of a batch, each
 *    sequence's tile count) that each call writes before reading.
 *  - Caches must hold finite values.
 *  - With TF_LOG set to anything but "0" in the environment, every rejected
 *    call prints its status and detail, and every attention call its launch
 *    shape (tokens per workgroup, split count), to stderr as "[tf] ..." lines.
 */
#ifndef TF_ATTN_H
#define TF_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* tf_stream_t; /* a hipStream_t */

typedef enum {
  TF_OK = 0,
  TF_ERR_INVALID_ARG = 1, /* null pointer, negative size, misalignment, bad combination */
  TF_ERR_UNSUPPORTED = 2, /* valid but not implemented (d != 128, too many query rows, ...) */
  TF_ERR_WORKSPACE = 3,   /* workspace missing or smaller than *_workspace_size() */
  TF_ERR_HIP = 4          /* a HIP launch failed; see tf_last_error_detail() */
} tf_status;

typedef enum { TF_DTYPE_FP16 = 1, TF_DTYPE_BF16 = 2, TF_DTYPE_FP32 = 3 } tf_dtype;

/*
 * Head-major ragged cache descriptor.  Row t of head g of sequence b starts
 * at element  seq_base[b] + (g * seq_cap[b] + t) * d  of the buffer it
 * describes.  seq_base / seq_cap / seq_len are DEVICE arrays of length B;
 * the other fields are host values.  Kernels clamp each seq_len[b] into
 * [0, min(seq_cap[b], max_len)], so a wrong length can drop rows but never
 * reads outside the rows the descriptor declares.
 */
typedef struct {
  int32_t B;                /* sequences */
  int32_t H;                /* KV heads */
  int32_t d;                /* head dimension (128) */
  int32_t dtype;            /* tf_dtype of the described buffer */
  const int64_t* seq_base;  /* device [B]: element offset of (b, head 0, row 0) */
  const int32_t* seq_cap;   /* device [B]: rows allocated per head */
  const int32_t* seq_len;   /* device [B]: valid rows */
  int32_t max_len;          /* host: upper bound of every seq_len[b]; sizes the grid */
} tf_kv_desc;

const char* tf_status_string(int status);
const char* tf_last_error_detail(void);

/*
 * a1  Chunk-mean keys.  [blog] Force 2 retrieves KV blocks by key-query
 * similarity; a block is summarised by the mean of its keys.
 *   ck[b][g][c] = mean of K[b][g][t] over t in [c*cs, min((c+1)*cs, n_b)),
 * summed in fp32 and rounded once (nearest even) to ckd->dtype, which is the
 * K dtype or TF_DTYPE_FP32.  Only chunks c in
 * [chunk_begin[b], min(chunk_begin[b] + max_chunks, ceil(n_b / cs))) are
 * written, so a decode loop refreshes just the chunks new rows fell into.
 *   K          : device, described by kv.
 *   chunk_begin: device int32 [B], or NULL for 0.
 *   max_chunks : host, > 0; chunks per sequence this call may write.
 *   ck         : device, described by ckd (rows are chunks; ckd->seq_len is
 *                not read; ckd->seq_cap[b] must be >= ceil(n_b / cs)).
 */
int tf_build_chunk_keys(const void* K, const tf_kv_desc* kv, int32_t chunk_size,
                        const int32_t* chunk_begin, int32_t max_chunks,
                        void* ck, const tf_kv_desc* ckd, tf_stream_t stream);

/*
 * a2  Query-to-chunk scores.  [blog] Force 2, "Key-Query similarity".
 *   scores[b][g][c] = sum over the G = Hq / H query heads h = g*G .. g*G+G-1
 *                     of q[b][h] . ck[b][g][c]      (unscaled, fp32)
 * for c < C_b = ckd->seq_len[b] (chunk count), and -inf for C_b <= c < c_max.
 *   q      : device [B][Hq][d], ckd->dtype must equal the q dtype `q_dtype`
 *            unless ckd->dtype is TF_DTYPE_FP32.
 *   ck     : device, described by ckd (seq_len = chunk counts, max_len <= c_max).
 *   scores : device fp32 [B][H][c_max].
 * c_max above 1 << 22 (4,194,304 chunks) returns TF_ERR_UNSUPPORTED.
 */
int tf_score_chunks(const void* q, int32_t q_dtype, int32_t Hq,
                    const void* ck, const tf_kv_desc* ckd,
                    float* scores, int32_t c_max, tf_stream_t stream);

/*
 * a3  Top-k chunk selection under a token budget.  [blog] Force 2 keeps a
 * small subset of the most critical blocks ("top k = 2,048 tokens").
 * For each row (b, g): the k = budget / cs chunk indices with the largest
 * scores among c < n_chunks[b]; ties go to the lower index; NaN ranks as
 * -inf and -0.0 as +0.0; written ascending; padded with -1 when
 * n_chunks[b] < k.  Bit-exact for a given score array.
 *   scores  : device fp32 [B][rows_per_seq][c_max].
 *   n_chunks: device int32 [B] (clamped into [0, c_max]).
 *   idx     : device int32 [B][rows_per_seq][k].
 *   ws      : tf_select_topk_workspace_size(B, rows_per_seq, c_max, k) bytes
 *             (256-byte aligned; no initialisation).  It is nonzero only for
 *             at most 16 rows (B * rows_per_seq) of 16385 to 65536 chunks
 *             with k <= 2048 and 2 k <= the slice length (c_max / 8 rounded
 *             up to a multiple of 4): these are selected in 8 slices per row
 *             (each slice's k best as 8-byte candidates) and then merged.
 *             Otherwise ws may be NULL.  Too small a workspace returns
 *             TF_ERR_WORKSPACE.
 *   c_max <= 1 << 20.
 */
int tf_select_topk(const float* scores, int32_t B, int32_t rows_per_seq, int32_t c_max,
                   const int32_t* n_chunks, int32_t k, int32_t* idx,
                   void* ws, size_t ws_bytes, tf_stream_t stream);
size_t tf_select_topk_workspace_size(int32_t B, int32_t rows_per_seq, int32_t c_max, int32_t k);

/*
 * a4  Attention over the gathered chunks.  [blog] Force 2 runs on the
 * retrieval-sparse cache; [abs] sparse KV cache via retrieval as draft.
 *   out[b][h] = sum_t softmax_t(q[b][h] . K_t / sqrt(d)) V_t over the rows t of
 *   the chunks idx[b][g][0..k) (g = h / G; entries < 0 skipped; rows >= n_b
 *   skipped), lse[b][h] = log sum_t exp(q . K_t / sqrt(d)); a head with no
 *   row gets out = 0, lse = -inf.
 *   q  : device [B][Hq][d] in kv->dtype.   out: device fp32 [B][Hq][d].
 *   lse: device fp32 [B][Hq] or NULL.      idx: device int32 [B][H][k].
 *   ws : tf_sparse_attn_workspace_size(kv->B, Hq, kv->H, k, chunk_size) bytes.
 */
int tf_sparse_attn(const void* q, int32_t Hq, const void* K, const void* V,
                   const tf_kv_desc* kv, const int32_t* idx, int32_t k, int32_t chunk_size,
                   float* out, float* lse, void* ws, size_t ws_bytes, tf_stream_t stream);
size_t tf_sparse_attn_workspace_size(int32_t B, int32_t Hq, int32_t H, int32_t k, int32_t chunk_size);

/*
 * a4, multi-query form: Force 2 verifying the small drafter's tokens on the
 * sparse cache ([blog] Force 2 evaluates the candidates from Force 1;
 * "2. Dual Rejection Sampling" then tests them r -> q).  The cache already
 * holds the Q drafted rows as its last Q rows (as for tf_verify_attn).  With
 * n = n_b and t0 = max(0, n - tail), query row i (0 <= i < Q) of head h sees
 *   { rows of the chunks idx[b][g][0..k) below t0 }  U  [t0, n - Q + i]
 * (g = h / G; entries < 0 skipped).  With every chunk selected, or tail >= n,
 * this is tf_verify_attn.  Requires tail >= Q.
 *   q  : device [B][Hq][Q][d] in kv->dtype.  out: device fp32 [B][Hq][Q][d].
 *   lse: device fp32 [B][Hq][Q] or NULL.     idx: device int32 [B][H][k].
 *   ws : tf_sparse_verify_attn_workspace_size(kv->B, Hq, kv->H, Q, k, chunk_size, tail).
 */
int tf_sparse_verify_attn(const void* q, int32_t Hq, int32_t Q, const void* K, const void* V,
                          const tf_kv_desc* kv, const int32_t* idx, int32_t k, int32_t chunk_size,
                          int32_t tail, float* out, float* lse, void* ws, size_t ws_bytes,
                          tf_stream_t stream);
size_t tf_sparse_verify_attn_workspace_size(int32_t B, int32_t Hq, int32_t H, int32_t Q, int32_t k,
                                            int32_t chunk_size, int32_t tail);

/*
 * a5  Sink + window streaming attention.  [blog] Force 1 drafts on a cache of
 * the initial sink tokens plus the most recent W tokens (StreamingLLM).
 * With n = sd->seq_len[b] the logical length, the visible positions are
 *   [0, min(n_sink, n))  U  [max(n_sink, n - window), n).
 * Ring layout: position p < n_sink is in slot p; p >= n_sink is in slot
 *   n_sink + (p - n_sink) mod (seq_cap[b] - n_sink),
 * and seq_cap[b] >= n_sink + window is the caller's contract.  seq_len here
 * is the LOGICAL length (it may exceed seq_cap; it is not clamped to it).
 *   q: device [B][Hq][d]; out: device fp32 [B][Hq][d]; lse: [B][Hq] or NULL.
 *   No workspace.
 */
int tf_stream_attn(const void* q, int32_t Hq, const void* Ks, const void* Vs,
                   const tf_kv_desc* sd, int32_t n_sink, int32_t window,
                   float* out, float* lse, tf_stream_t stream);

/*
 * a6  Full-cache multi-query verification.  [blog] Force 3 verifies all
 * candidates against the complete cache in one parallel pass; [abs] the
 * whole KV cache is loaded for every generated token.  Chain form: the last
 * Q rows of the cache are the draft positions, so query row i (0 <= i < Q)
 * of head h sees rows j <= n_b - Q + i:
 *   out[b][h][i] = sum_{j <= n_b - Q + i} softmax_j(q[b][h][i] . K_j / sqrt(d)) V_j
 * (a row that sees nothing gets out = 0, lse = -inf).
 *   q  : device [B][Hq][Q][d] in kv->dtype.  out: device fp32 [B][Hq][Q][d].
 *   lse: device fp32 [B][Hq][Q] or NULL.     G * Q <= 64.
 *   ws : tf_verify_attn_workspace_size(kv->B, Hq, kv->H, Q, kv->max_len) bytes
 *        (for a batch of 2 to 1024 sequences: (512 + B * H) partial slots of
 *        the query rows, whatever max_len, work being shared equally by 512
 *        workgroups; for one sequence: its splits' partials, which grow with
 *        max_len).
 */
int tf_verify_attn(const void* q, int32_t Hq, int32_t Q, const void* K, const void* V,
                   const tf_kv_desc* kv, float* out, float* lse,
                   void* ws, size_t ws_bytes, tf_stream_t stream);
size_t tf_verify_attn_workspace_size(int32_t B, int32_t Hq, int32_t H, int32_t Q, int32_t max_len);

/*
 * a6 without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops or harnesses that forbid
 * allocation).  Same arguments, semantics and results as tf_verify_attn
 * (bitwise: the same kernels and split plan) except that the split partials
 * go to a scratch array built into the library: every GPU the library runs
 * on holds tf_verify_attn_noalloc_max_bytes() = 48 MiB of it until the process
 * ends, and a call whose partials need more (tf_verify_attn_workspace_size
 * above that; e.g. one sequence of 32 KV heads, G * Q = 7 and room for 4M
 * rows) is refused with TF_ERR_WORKSPACE before anything is enqueued.  The
 * call allocates nothing.
 * The scratch is shared by every call on that GPU: calls that overlap on one
 * GPU (other streams, other host threads) race and must be serialised by
 * the caller.  stream must belong to the current device (TF_ERR_INVALID_ARG
 * otherwise); the scratch's device address is looked up on the first call on
 * each device.
 */
int tf_verify_attn_noalloc(const void* q, int32_t Hq, int32_t Q, const void* K, const void* V,
                           const tf_kv_desc* kv, float* out, float* lse, tf_stream_t stream);
size_t tf_verify_attn_noalloc_max_bytes(void);

/*
 * a6 over a candidate tree.  [blog] Force 3 evaluates the candidate tree that
 * Force 2 assembles in one parallel pass with tree attention.  The last Q
 * cache rows hold the tree's nodes in order: node m is row n_b - Q + m.
 * Query row i (0 <= i < Q) of head h sees every row below n_b - Q and node m
 * when bit m of tree_mask[b][i] is set:
 *   out[b][h][i] = sum over those rows j of softmax_j(q[b][h][i] . K_j / sqrt(d)) V_j
 * (a row that sees nothing gets out = 0, lse = -inf).  Masks with bits 0..i of
 * row i (a chain) give exactly tf_verify_attn.
 *   tree_mask: device uint64 [B][Q] (tf_tree_masks builds it from parents).
 *   Other arguments as for tf_verify_attn; 1 <= Q <= 64; the workspace is
 *   tf_verify_attn_workspace_size(kv->B, Hq, kv->H, Q, kv->max_len) bytes.
 */
int tf_verify_tree_attn(const void* q, int32_t Hq, int32_t Q, const void* K, const void* V,
                        const tf_kv_desc* kv, const uint64_t* tree_mask, float* out, float* lse,
                        void* ws, size_t ws_bytes, tf_stream_t stream);

/*
 * Tree masks from parent pointers: tree_mask[b][i] has bit m set when node m
 * is node i or one of its ancestors.  parent: device int32 [B][Q]; parent[b]
 * [i] = -1 hangs node i off the committed prefix, and a value outside [0, i)
 * is read as -1 (nodes come in topological order).  tree_mask: device uint64
 * [B][Q].  1 <= Q <= 64.
 */
int tf_tree_masks(const int32_t* parent, int32_t B, int32_t Q, uint64_t* tree_mask, tf_stream_t stream);

/*
 * a7  Lossless accept / reject.  [blog] "2. Dual Rejection Sampling".
 * Per sequence b, with p_i = softmax(target[b][i] / T), q_i =
 * softmax(draft[b][i] / T) in fp64 (T = 0: one-hot at the lowest-index
 * argmax; flag TF_ACCEPT_PROBS: the rows already are probabilities, used as
 * given):
 *   for i = 0 .. gamma-1, x = draft_tokens[b][i]: keep x when p_i(x) > 0 and
 *   min(1, p_i(x) / q_i(x)) >= uniforms[b][i] (q_i(x) = 0 counts as 1);
 *   stop at the first rejection j.
 *   next_token[b] is drawn with u = uniforms[b][gamma] by inverse CDF (the
 *   smallest t whose running sum exceeds u * total, strictly) from
 *   max(0, p_j - q_j) (p_j if that sums to 0) after a rejection, or from
 *   p_gamma when every draft was kept.  n_accepted[b] = j (gamma if none was
 *   rejected).  Emitted tokens: draft_tokens[b][0 .. n_accepted) then next.
 *   target: device fp32 [B][gamma+1][V]; draft: device fp32 [B][gamma][V];
 *   draft_tokens: device int32 [B][gamma] (each in [0, V)); uniforms: device
 *   fp64 [B][gamma+1] in (0, 1).  Outputs: device int32 [B].
 *   ws: tf_accept_workspace_size(B, gamma, V) bytes (per-row statistics and
 *       the draw's fp64 weights, 16 V bytes per sequence).
 *   Limits: V <= 65536, gamma <= 1024, B * (2 gamma + 1) * ceil(V / 4096) < 2^31.
 */
#define TF_ACCEPT_PROBS 1
int tf_accept(const float* target, const float* draft, const int32_t* draft_tokens,
              const double* uniforms, int32_t B, int32_t gamma, int32_t V, float temperature,
              int32_t flags, int32_t* n_accepted, int32_t* next_token,
              void* ws, size_t ws_bytes, tf_stream_t stream);
size_t tf_accept_workspace_size(int32_t B, int32_t gamma, int32_t V);

/*
 * Cache maintenance around the step.  Drafted rows enter the caches before
 * they are verified and the rejected ones leave again ([blog] Force 3 reads
 * the complete cache; Force 1 keeps the sinks plus a rolling window of the
 * most recent tokens; "2. Dual Rejection Sampling" discards every draft after
 * the first rejection).  Lengths stay on the device, so a decode loop of
 * append / attention / accept / commit needs no host round trip.
 *
 * tf_append_kv: copies R new rows per (sequence, head) into K and V.
 *   K_new, V_new: device [kv->B][kv->H][R][d] in kv->dtype (fp16 / bf16).
 *   K, V        : device caches described by kv; kv->seq_len[b] = n_b is the
 *                 current length (read, not changed: see tf_commit_length).
 *   mode TF_APPEND_FULL: the rows become positions n_b .. n_b + R - 1 in rows
 *     n_b .. n_b + R - 1; a sequence with n_b + R > seq_cap[b] gets
 *     TF_APPEND_NO_ROOM and is left as it is.
 *   mode TF_APPEND_RING (the streaming cache of tf_stream_attn; n_b is the
 *     logical length): position p goes to slot p if p < n_sink, else to slot
 *     n_sink + (p - n_sink) mod (seq_cap[b] - n_sink).  `reserve` (>= R)
 *     bounds the rows appended since the last length that can no longer be
 *     rolled back; a ring with seq_cap[b] - n_sink < window + reserve gets
 *     TF_APPEND_RING_TOO_SMALL and is left as it is (with fewer slots, a
 *     rollback could expose a visible position whose slot a newer row took).
 *   n_b < 0 gives TF_APPEND_BAD_LENGTH.  status: device int32 [B] (per
 *   sequence, one of tf_append_status) or NULL.  R = 0 enqueues nothing.
 *   kv->max_len is not used.
 *
 * tf_commit_length: seq_len[b] = max(0, seq_len[b] + add - drop_b), with
 *   drop_b = gamma - clamp(n_accepted[b], 0, gamma) when n_accepted (device
 *   int32 [B], e.g. the output of tf_accept) is given, else 0.  seq_len is a
 *   device int32 [B] array (a descriptor's seq_len), updated in place.
 *   add >= 0, gamma >= 0.
 */
typedef enum { TF_APPEND_FULL = 0, TF_APPEND_RING = 1 } tf_append_mode;
typedef enum {
  TF_APPEND_OK = 0,
  TF_APPEND_NO_ROOM = 1,
  TF_APPEND_RING_TOO_SMALL = 2,
  TF_APPEND_BAD_LENGTH = 3
} tf_append_status;
int tf_append_kv(const void* K_new, const void* V_new, int32_t R, void* K, void* V, const tf_kv_desc* kv,
                 int32_t mode, int32_t n_sink, int32_t window, int32_t reserve, int32_t* status,
                 tf_stream_t stream);
int tf_commit_length(int32_t* seq_len, int32_t B, int32_t add, int32_t gamma, const int32_t* n_accepted,
                     tf_stream_t stream);

/*
 * a7 over a candidate tree.  [blog] Force 3 verifies the candidate tree Force
 * 2 assembles; acceptance and residual as in "2. Dual Rejection Sampling".
 * Per sequence b, Q nodes: node 0 is the last committed token, nodes
 * 1 .. Q-1 candidates with token tokens[b][c] and parent[b][c] in [0, c) (any
 * other value hangs c off node 0).  target[b][v] holds the target's logits
 * (or probabilities, flag TF_ACCEPT_PROBS) for the children of node v,
 * draft[b][v] the distribution they were drafted from (rows of leaves are not
 * read).  From node 0, the children of the current node v are tried in index
 * order: child c with token x is kept when p'(x) > 0 and
 * uniforms[b][c - 1] * q_v(x) <= p'(x), where p' starts as p_v and after
 * each rejected sibling becomes max(0, p' - q_v) renormalised (p_v if that
 * vanishes through rounding); a kept child becomes v.  When no child is kept,
 * or v has none, next_token[b] is drawn from p' by inverse CDF with
 * uniforms[b][Q - 1] (the rule of tf_accept).  With siblings drafted
 * independently from q_v the emitted tokens follow the target; a chain
 * (parent[c] = c - 1) gives exactly tf_accept.  T = 0 is greedy as there.
 *   target, draft: device fp32 [B][Q][V]; tokens, parent: device int32
 *   [B][Q] (tokens[b][0] not read); uniforms: device fp64 [B][Q] in (0, 1).
 *   Outputs: n_accepted[b] = kept nodes; path[b][0 .. Q-2] = the kept nodes
 *   in order, then -1 (NULL allowed when Q = 1); next_token[b].
 *   ws: tf_tree_accept_workspace_size(B, V) bytes (per sequence three fp64
 *     rows of V -- a stored residual, the current node's draft distribution
 *     and the draw's weights -- the per-slice statistics of up to 64 target
 *     and 64 draft rows, and the residuals' partial normalisers).
 *   Limits: Q <= 64, V <= 65536.
 */
int tf_tree_accept(const float* target, const float* draft, const int32_t* tokens, const int32_t* parent,
                   const double* uniforms, int32_t B, int32_t Q, int32_t V, float temperature, int32_t flags,
                   int32_t* n_accepted, int32_t* path, int32_t* next_token, void* ws, size_t ws_bytes,
                   tf_stream_t stream);
size_t tf_tree_accept_workspace_size(int32_t B, int32_t V);

/*
 * Two-level accept, r -> q -> p ([blog] "2. Dual Rejection Sampling": Force 2
 * keeps a drafter candidate x when min(1, q(x)/r(x)) >= u1; what Force 2
 * passes on is verified by Force 3 with min(1, p(x)/q(x)) >= u2, a rejection
 * there drawing from max(0, p - q)).  Both levels are tf_accept calls (the
 * drafter's own sampling is tf_accept with gamma = 0); between them, after
 * each Force 2 round of gamma1 drafts (target q_rows, draft r rows),
 * tf_collect_candidates appends the round's emitted tokens -- draft_tokens[b]
 * [0 .. n_accepted[b]) then next_token[b] -- to sequence b's chain, as long as
 * fewer than gamma2 are there, together with the q row of each token's
 * position (q_rows[b][j] for the round's j-th emitted token).  Force 3 then
 * calls tf_accept(target = p rows [B][gamma2 + 1][V], draft = cand_q,
 * draft_tokens = cand).
 *   draft_tokens: device int32 [B][gamma1]; n_accepted, next_token: device
 *     int32 [B] (clamped: n_accepted into [0, gamma1]).
 *   q_rows: device fp32 [B][gamma1 + 1][V] (logits or probabilities: copied).
 *   count_in: device int32 [B], candidates already collected (clamped into
 *     [0, gamma2]); count_out: device int32 [B], a DIFFERENT array, receives
 *     count_in[b] + the tokens taken (alternate the two arrays between rounds).
 *   cand: device int32 [B][gamma2]; cand_q: device fp32 [B][gamma2][V]; slots
 *     at and past count_out[b] are not written.
 *   1 <= gamma2 <= 1024, 0 <= gamma1 <= 1024, V >= 1.  No workspace.
 */
int tf_collect_candidates(const int32_t* draft_tokens, const int32_t* n_accepted, const int32_t* next_token,
                          const float* q_rows, int32_t B, int32_t gamma1, int32_t V, const int32_t* count_in,
                          int32_t* count_out, int32_t* cand, float* cand_q, int32_t gamma2, tf_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* TF_ATTN_H */
