// C ABI of libtfattn (declared in include/tf_attn.h): host-side validation,
// split planning and kernel launches.  Nothing is enqueued unless every
// argument check passes.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "tf_internal.h"

#define TF_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_detail[512] = "";

// TF_LOG set (and not "0") in the environment: every rejected call prints its
// status and detail, and every attention call its launch shape, to stderr.
bool log_on() {
  static const bool on = [] {
    const char* e = std::getenv("TF_LOG");
    return e && e[0] && std::strcmp(e, "0") != 0;
  }();
  return on;
}

void log_line(const char* fmt, ...) {
  if (!log_on()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[tf] %s\n", buf);
}

const char* status_name(int status);

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  log_line("%s: %s", status_name(status), g_detail);
  return status;
}

int ok() {
  g_detail[0] = '\0';
  return TF_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TF_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool is16(int dt) { return dt == TF_DTYPE_FP16 || dt == TF_DTYPE_BF16; }

// Checks shared by every cache descriptor.
int check_desc(const tf_kv_desc* kv, const char* name, bool allow_fp32) {
  if (!kv) return fail(TF_ERR_INVALID_ARG, "%s is NULL", name);
  if (kv->B < 0 || kv->H < 1 || kv->max_len < 0)
    return fail(TF_ERR_INVALID_ARG, "%s: B=%d H=%d max_len=%d out of range", name, kv->B, kv->H, kv->max_len);
  if (kv->d != tfk::kHeadDim) return fail(TF_ERR_UNSUPPORTED, "%s: head dim %d (only 128)", name, kv->d);
  if (!(is16(kv->dtype) || (allow_fp32 && kv->dtype == TF_DTYPE_FP32)))
    return fail(allow_fp32 ? TF_ERR_INVALID_ARG : TF_ERR_UNSUPPORTED, "%s: dtype %d not supported", name, kv->dtype);
  if (kv->B > 0 && (!kv->seq_base || !kv->seq_cap || !kv->seq_len))
    return fail(TF_ERR_INVALID_ARG, "%s: seq_base/seq_cap/seq_len must be device arrays", name);
  if (kv->B > 65535 || kv->H > 65535) return fail(TF_ERR_UNSUPPORTED, "%s: B or H above 65535", name);
  return TF_OK;
}

int check_ptr(const void* p, const char* name, size_t align) {
  if (!p) return fail(TF_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(TF_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return TF_OK;
}

int check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return TF_OK;
  if (!ws) return fail(TF_ERR_WORKSPACE, "workspace of %zu bytes required, got NULL", need);
  if (!aligned(ws, 256)) return fail(TF_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  if (have < need) return fail(TF_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
  return TF_OK;
}

#define TRY(x)              \
  do {                      \
    const int _s = (x);     \
    if (_s != TF_OK) return _s; \
  } while (0)

// Target number of workgroups per launch: two per compute unit (256 CUs),
// one resident round at two waves per SIMD.
constexpr int kVerifyTargetWgs = 512;
constexpr int kSparseTargetWgs = 512;

// Split plan of a verification call (chain or tree): a batch of several
// sequences takes equal work per workgroup over its tiles, one sequence the
// split grid.
static tfk::SplitPlan verify_plan(int32_t B, int32_t H, int32_t rows, int32_t max_len) {
  if (tfk::flat_eligible(B, H, max_len)) return tfk::plan_flat(B, H, rows, kVerifyTargetWgs);
  return tfk::plan_splits(B, H, rows, max_len, kVerifyTargetWgs, tfk::kVerifyMaxTpw, tfk::kVerifyMinTpw);
}

void fill_common(tfk::AttnArgs& a, const void* q, const void* K, const void* V, const tf_kv_desc* kv, int Hq, int Qn,
                 float* out, float* lse) {
  a.q = (const uint16_t*)q;
  a.K = (const uint16_t*)K;
  a.V = (const uint16_t*)V;
  a.seq_base = kv->seq_base;
  a.seq_cap = kv->seq_cap;
  a.seq_len = kv->seq_len;
  a.max_len = kv->max_len;
  a.B = kv->B;
  a.Hq = Hq;
  a.Hkv = kv->H;
  a.G = Hq / kv->H;
  a.Qn = Qn;
  a.rows = a.G * Qn;
  a.idx = nullptr;
  a.k = 0;
  a.cs = 1;
  a.tail = 0;
  a.n_sink = 0;
  a.window = 0;
  a.out = out;
  a.lse = lse;
  a.part_o = nullptr;
  a.part_ml = nullptr;
  a.tmask = nullptr;
  a.scale_ln = 1.0f / std::sqrt((float)tfk::kHeadDim);
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)tfk::kHeadDim));
}

void fill_plan(tfk::AttnArgs& a, const tfk::SplitPlan& p, void* ws) {
  a.tpw = p.tpw;
  a.nsplit = p.nsplit;
  a.rows_pad = p.rows_pad;
  a.tail_last = p.tail_last;
  a.flat_wgs = p.flat_wgs;
  a.flat_prefix = nullptr;
  if (p.total_bytes) {
    char* w = (char*)ws;
    a.part_ml = (float*)w;
    a.part_o = (float*)(w + p.part_ml_bytes);
    if (p.flat_wgs > 0) a.flat_prefix = (int32_t*)(w + p.part_ml_bytes + p.part_o_bytes);
  }
}

const char* status_name(int status) {
  switch (status) {
    case TF_OK: return "TF_OK";
    case TF_ERR_INVALID_ARG: return "TF_ERR_INVALID_ARG";
    case TF_ERR_UNSUPPORTED: return "TF_ERR_UNSUPPORTED";
    case TF_ERR_WORKSPACE: return "TF_ERR_WORKSPACE";
    case TF_ERR_HIP: return "TF_ERR_HIP";
  }
  return "TF_ERR_UNKNOWN";
}

// Launch of an attention call (after its checks passed), logged when TF_LOG is set.
int attn_call(const char* fn, int dtype, int mode, const tfk::AttnArgs& a, hipStream_t stream) {
  if (a.flat_wgs > 0)
    log_line("%s: B=%d Hq=%d H=%d rows/head=%d max_len=%d equal work on %d workgroups, %d partial slots "
             "(+ split merge)", fn, a.B, a.Hq, a.Hkv, a.rows, a.max_len, a.flat_wgs, a.nsplit);
  else
    log_line("%s: B=%d Hq=%d H=%d rows/head=%d max_len=%d tokens/workgroup=%d splits=%d%s", fn, a.B, a.Hq, a.Hkv,
             a.rows, a.max_len, a.tpw, a.nsplit, a.nsplit > 1 ? " (+ split merge)" : "");
  return check_hip(tfk::launch_attn(dtype, mode, a, stream), fn);
}

}  // namespace

TF_EXPORT const char* tf_status_string(int status) { return status_name(status); }

TF_EXPORT const char* tf_last_error_detail(void) { return g_detail; }

// ---------------------------------------------------------------------------
// a1
// ---------------------------------------------------------------------------
TF_EXPORT int tf_build_chunk_keys(const void* K, const tf_kv_desc* kv, int32_t chunk_size,
                                  const int32_t* chunk_begin, int32_t max_chunks, void* ck,
                                  const tf_kv_desc* ckd, tf_stream_t stream) {
  TRY(check_desc(kv, "kv", false));
  TRY(check_desc(ckd, "ckd", true));
  if (ckd->B != kv->B || ckd->H != kv->H) return fail(TF_ERR_INVALID_ARG, "ckd B/H differ from kv");
  if (ckd->dtype != TF_DTYPE_FP32 && ckd->dtype != kv->dtype)
    return fail(TF_ERR_INVALID_ARG, "chunk keys are stored in the K dtype or fp32");
  if (chunk_size < 1 || chunk_size > 4096) return fail(TF_ERR_INVALID_ARG, "chunk_size %d out of [1, 4096]", chunk_size);
  if (max_chunks < 1) return fail(TF_ERR_INVALID_ARG, "max_chunks must be >= 1");
  if (kv->B == 0) return ok();
  TRY(check_ptr(K, "K", 16));
  TRY(check_ptr(ck, "ck", 16));
  if (chunk_begin) TRY(check_ptr(chunk_begin, "chunk_begin", 4));
  if ((max_chunks + 15) / 16 > 0x7fffffff) return fail(TF_ERR_UNSUPPORTED, "max_chunks too large");
  return check_hip(tfk::launch_chunk_keys((const uint16_t*)K, *kv, chunk_size, chunk_begin, max_chunks, ck, *ckd,
                                          (hipStream_t)stream),
                   "tf_build_chunk_keys");
}

// ---------------------------------------------------------------------------
// a2
// ---------------------------------------------------------------------------
TF_EXPORT int tf_score_chunks(const void* q, int32_t q_dtype, int32_t Hq, const void* ck, const tf_kv_desc* ckd,
                              float* scores, int32_t c_max, tf_stream_t stream) {
  TRY(check_desc(ckd, "ckd", true));
  if (!is16(q_dtype)) return fail(TF_ERR_UNSUPPORTED, "q dtype %d not supported", q_dtype);
  if (ckd->dtype != TF_DTYPE_FP32 && ckd->dtype != q_dtype)
    return fail(TF_ERR_INVALID_ARG, "16-bit chunk keys must share the query dtype");
  if (Hq < 1 || Hq % ckd->H != 0) return fail(TF_ERR_INVALID_ARG, "Hq=%d is not a multiple of H=%d", Hq, ckd->H);
  if (c_max < 1) return fail(TF_ERR_INVALID_ARG, "c_max must be >= 1");
  // (the key loads address a head's row with 32-bit byte offsets)
  if (c_max > (1 << 22)) return fail(TF_ERR_UNSUPPORTED, "c_max %d above 1<<22", c_max);
  if (ckd->max_len > c_max) return fail(TF_ERR_INVALID_ARG, "ckd->max_len %d exceeds c_max %d", ckd->max_len, c_max);
  if (ckd->B == 0) return ok();
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(ck, "ck", 16));
  TRY(check_ptr(scores, "scores", 4));
  return check_hip(tfk::launch_scores((const uint16_t*)q, q_dtype, Hq, ck, *ckd, scores, c_max, (hipStream_t)stream),
                   "tf_score_chunks");
}

// ---------------------------------------------------------------------------
// a3
// ---------------------------------------------------------------------------
TF_EXPORT size_t tf_select_topk_workspace_size(int32_t B, int32_t rows_per_seq, int32_t c_max, int32_t k) {
  if (B < 1 || rows_per_seq < 1 || c_max < 1 || k < 1 || c_max > (1 << 20) || B > 65535) return 0;
  return tfk::topk_workspace_bytes(B, rows_per_seq, c_max, k);
}

TF_EXPORT int tf_select_topk(const float* scores, int32_t B, int32_t rows_per_seq, int32_t c_max,
                             const int32_t* n_chunks, int32_t k, int32_t* idx, void* ws, size_t ws_bytes,
                             tf_stream_t stream) {
  if (B < 0 || rows_per_seq < 1 || c_max < 1 || k < 1)
    return fail(TF_ERR_INVALID_ARG, "B=%d rows=%d c_max=%d k=%d out of range", B, rows_per_seq, c_max, k);
  if (c_max > (1 << 20)) return fail(TF_ERR_UNSUPPORTED, "c_max %d above 1<<20", c_max);
  if (B > 65535) return fail(TF_ERR_UNSUPPORTED, "B above 65535");
  if (B == 0) return ok();
  TRY(check_ptr(scores, "scores", 4));
  TRY(check_ptr(n_chunks, "n_chunks", 4));
  TRY(check_ptr(idx, "idx", 4));
  TRY(check_ws(ws, ws_bytes, tfk::topk_workspace_bytes(B, rows_per_seq, c_max, k)));
  const tfk::TopkSplit p = tfk::plan_topk(B, rows_per_seq, c_max, k);
  log_line("tf_select_topk: B=%d rows=%d c_max=%d k=%d slices=%d%s", B, rows_per_seq, c_max, k, p.S,
           p.S > 1 ? " (+ merge)" : "");
  return check_hip(tfk::launch_topk(scores, B, rows_per_seq, c_max, n_chunks, k, idx, ws, (hipStream_t)stream),
                   "tf_select_topk");
}

// ---------------------------------------------------------------------------
// a4
// ---------------------------------------------------------------------------
TF_EXPORT size_t tf_sparse_attn_workspace_size(int32_t B, int32_t Hq, int32_t H, int32_t k, int32_t chunk_size) {
  if (B < 1 || H < 1 || Hq < 1 || k < 1 || chunk_size < 1) return 0;
  const long virt = (long)k * chunk_size;
  if (virt > 0x7fffffffL) return 0;
  return tfk::plan_splits(B, H, Hq / H, (int32_t)virt, kSparseTargetWgs, tfk::kSparseMaxTpw, tfk::kSparseMinTpw).total_bytes;
}

TF_EXPORT int tf_sparse_attn(const void* q, int32_t Hq, const void* K, const void* V, const tf_kv_desc* kv,
                             const int32_t* idx, int32_t k, int32_t chunk_size, float* out, float* lse, void* ws,
                             size_t ws_bytes, tf_stream_t stream) {
  TRY(check_desc(kv, "kv", false));
  if (Hq < 1 || Hq % kv->H != 0) return fail(TF_ERR_INVALID_ARG, "Hq=%d is not a multiple of H=%d", Hq, kv->H);
  if (Hq / kv->H > tfk::kMaxRows) return fail(TF_ERR_UNSUPPORTED, "more than %d query heads per KV head", tfk::kMaxRows);
  if (k < 1 || chunk_size < 1 || chunk_size > 4096) return fail(TF_ERR_INVALID_ARG, "k=%d chunk_size=%d", k, chunk_size);
  if ((long)k * chunk_size > 0x7fffffffL) return fail(TF_ERR_UNSUPPORTED, "k * chunk_size too large");
  if (kv->B == 0) return ok();
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(K, "K", 16));
  TRY(check_ptr(V, "V", 16));
  TRY(check_ptr(idx, "idx", 4));
  TRY(check_ptr(out, "out", 16));
  if (lse) TRY(check_ptr(lse, "lse", 4));
  const tfk::SplitPlan plan =
      tfk::plan_splits(kv->B, kv->H, Hq / kv->H, k * chunk_size, kSparseTargetWgs, tfk::kSparseMaxTpw, tfk::kSparseMinTpw);
  TRY(check_ws(ws, ws_bytes, plan.total_bytes));
  tfk::AttnArgs a;
  fill_common(a, q, K, V, kv, Hq, 1, out, lse);
  a.idx = idx;
  a.k = k;
  a.cs = chunk_size;
  fill_plan(a, plan, ws);
  return attn_call("tf_sparse_attn", kv->dtype, tfk::kSparse, a, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// a4, multi-query form with a causal tail (Force 2 verifying Force 1's drafts)
// ---------------------------------------------------------------------------
TF_EXPORT size_t tf_sparse_verify_attn_workspace_size(int32_t B, int32_t Hq, int32_t H, int32_t Q, int32_t k,
                                                      int32_t chunk_size, int32_t tail) {
  if (B < 1 || H < 1 || Hq < 1 || Q < 1 || k < 1 || chunk_size < 1 || tail < 1) return 0;
  const long virt = (long)k * chunk_size + tail;
  if (virt > 0x7fffffffL) return 0;
  return tfk::plan_splits(B, H, (Hq / H) * Q, (int32_t)virt, kSparseTargetWgs, tfk::kSparseMaxTpw, tfk::kSparseMinTpw).total_bytes;
}

TF_EXPORT int tf_sparse_verify_attn(const void* q, int32_t Hq, int32_t Q, const void* K, const void* V,
                                    const tf_kv_desc* kv, const int32_t* idx, int32_t k, int32_t chunk_size,
                                    int32_t tail, float* out, float* lse, void* ws, size_t ws_bytes,
                                    tf_stream_t stream) {
  TRY(check_desc(kv, "kv", false));
  if (Hq < 1 || Hq % kv->H != 0) return fail(TF_ERR_INVALID_ARG, "Hq=%d is not a multiple of H=%d", Hq, kv->H);
  if (Q < 1) return fail(TF_ERR_INVALID_ARG, "Q must be >= 1");
  if ((long)(Hq / kv->H) * Q > tfk::kMaxRows)
    return fail(TF_ERR_UNSUPPORTED, "G*Q = %ld query rows per KV head (at most %d)", (long)(Hq / kv->H) * Q,
                tfk::kMaxRows);
  if (k < 1 || chunk_size < 1 || chunk_size > 4096) return fail(TF_ERR_INVALID_ARG, "k=%d chunk_size=%d", k, chunk_size);
  if (tail < Q) return fail(TF_ERR_INVALID_ARG, "tail=%d must cover the Q=%d drafted rows", tail, Q);
  if ((long)k * chunk_size + tail > 0x7fffffffL) return fail(TF_ERR_UNSUPPORTED, "k * chunk_size + tail too large");
  if (kv->B == 0) return ok();
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(K, "K", 16));
  TRY(check_ptr(V, "V", 16));
  TRY(check_ptr(idx, "idx", 4));
  TRY(check_ptr(out, "out", 16));
  if (lse) TRY(check_ptr(lse, "lse", 4));
  const tfk::SplitPlan plan = tfk::plan_splits(kv->B, kv->H, (Hq / kv->H) * Q, k * chunk_size + tail,
                                               kSparseTargetWgs, tfk::kSparseMaxTpw, tfk::kSparseMinTpw);
  TRY(check_ws(ws, ws_bytes, plan.total_bytes));
  tfk::AttnArgs a;
  fill_common(a, q, K, V, kv, Hq, Q, out, lse);
  a.idx = idx;
  a.k = k;
  a.cs = chunk_size;
  a.tail = tail;
  fill_plan(a, plan, ws);
  return attn_call("tf_sparse_verify_attn", kv->dtype, tfk::kSparseTail, a, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// a5
// ---------------------------------------------------------------------------
TF_EXPORT int tf_stream_attn(const void* q, int32_t Hq, const void* Ks, const void* Vs, const tf_kv_desc* sd,
                             int32_t n_sink, int32_t window, float* out, float* lse, tf_stream_t stream) {
  TRY(check_desc(sd, "sd", false));
  if (Hq < 1 || Hq % sd->H != 0) return fail(TF_ERR_INVALID_ARG, "Hq=%d is not a multiple of H=%d", Hq, sd->H);
  if (Hq / sd->H > tfk::kMaxRows) return fail(TF_ERR_UNSUPPORTED, "more than %d query heads per KV head", tfk::kMaxRows);
  if (n_sink < 0 || window < 0 || (long)n_sink + window > (1L << 24))
    return fail(TF_ERR_INVALID_ARG, "n_sink=%d window=%d out of range", n_sink, window);
  if (sd->B == 0) return ok();
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(Ks, "Ks", 16));
  TRY(check_ptr(Vs, "Vs", 16));
  TRY(check_ptr(out, "out", 16));
  if (lse) TRY(check_ptr(lse, "lse", 4));
  tfk::AttnArgs a;
  fill_common(a, q, Ks, Vs, sd, Hq, 1, out, lse);
  a.n_sink = n_sink;
  a.window = window;
  // One workgroup per (sequence, head): every visible position in one split.
  tfk::SplitPlan plan;
  plan.tpw = ((n_sink + window + 127) / 128) * 128;
  if (plan.tpw < 128) plan.tpw = 128;
  plan.nsplit = 1;
  plan.rows_pad = ((a.rows + 15) / 16) * 16;
  plan.tail_last = 0;
  plan.part_o_bytes = plan.part_ml_bytes = plan.total_bytes = 0;
  fill_plan(a, plan, nullptr);
  return attn_call("tf_stream_attn", sd->dtype, tfk::kStream, a, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// a6
// ---------------------------------------------------------------------------
TF_EXPORT size_t tf_verify_attn_workspace_size(int32_t B, int32_t Hq, int32_t H, int32_t Q, int32_t max_len) {
  if (B < 1 || H < 1 || Hq < 1 || Q < 1 || max_len < 0) return 0;
  return verify_plan(B, H, (Hq / H) * Q, max_len).total_bytes;
}

TF_EXPORT int tf_verify_attn(const void* q, int32_t Hq, int32_t Q, const void* K, const void* V,
                             const tf_kv_desc* kv, float* out, float* lse, void* ws, size_t ws_bytes,
                             tf_stream_t stream) {
  TRY(check_desc(kv, "kv", false));
  if (Hq < 1 || Hq % kv->H != 0) return fail(TF_ERR_INVALID_ARG, "Hq=%d is not a multiple of H=%d", Hq, kv->H);
  if (Q < 1) return fail(TF_ERR_INVALID_ARG, "Q must be >= 1");
  if ((long)(Hq / kv->H) * Q > tfk::kMaxRows)
    return fail(TF_ERR_UNSUPPORTED, "G*Q = %ld query rows per KV head (at most %d)", (long)(Hq / kv->H) * Q,
                tfk::kMaxRows);
  if (kv->B == 0) return ok();
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(K, "K", 16));
  TRY(check_ptr(V, "V", 16));
  TRY(check_ptr(out, "out", 16));
  if (lse) TRY(check_ptr(lse, "lse", 4));
  const tfk::SplitPlan plan =
      verify_plan(kv->B, kv->H, (Hq / kv->H) * Q, kv->max_len);
  TRY(check_ws(ws, ws_bytes, plan.total_bytes));
  tfk::AttnArgs a;
  fill_common(a, q, K, V, kv, Hq, Q, out, lse);
  fill_plan(a, plan, ws);
  return attn_call("tf_verify_attn", kv->dtype, tfk::kVerify, a, (hipStream_t)stream);
}

// ---------------------------------------------------------------------------
// a6 without a caller workspace, for callers that cannot allocate (code under
// graph capture, serving loops that forbid allocation).  The split partials
// live in `scratch`, a file-scope device array of kNoAllocScratchBytes that
// every GPU the library runs on holds until the process ends.  Host code
// never passes the array's name to a kernel (in host code it names a
// host-side stand-in): its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and that address is what the
// kernels get.  Every call on a GPU shares that GPU's copy, so calls that
// overlap on one GPU (different streams, or different host threads) race.
// The partials need no clearing: each split writes every value it is later
// read for.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = size_t(48) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's copy of `scratch` (looked up on the
// first call made with the device current); TF_ERR_* on failure.
int scratch_on_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  TRY(check_hip(hipGetDevice(&dev), "hipGetDevice"));
  if (stream) {
    hipDevice_t sdev = -1;
    TRY(check_hip(hipStreamGetDevice(stream, &sdev), "hipStreamGetDevice"));
    if (sdev != dev) return fail(TF_ERR_INVALID_ARG, "stream is on device %d but device %d is current", (int)sdev, dev);
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(TF_ERR_UNSUPPORTED, "device %d (at most %d devices)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    TRY(check_hip(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (!ptr || !aligned(ptr, 256)) return fail(TF_ERR_HIP, "scratch address %p is not 256-byte aligned", ptr);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return ok();
}
}  // namespace

TF_EXPORT size_t tf_verify_attn_noalloc_max_bytes(void) { return kNoAllocScratchBytes; }

TF_EXPORT int tf_verify_attn_noalloc(const void* q, int32_t Hq, int32_t Q, const void* K, const void* V,
                                     const tf_kv_desc* kv, float* out, float* lse, tf_stream_t stream) {
  TRY(check_desc(kv, "kv", false));
  if (Hq < 1 || Hq % kv->H != 0) return fail(TF_ERR_INVALID_ARG, "Hq=%d is not a multiple of H=%d", Hq, kv->H);
  if (Q < 1) return fail(TF_ERR_INVALID_ARG, "Q must be >= 1");
  if ((long)(Hq / kv->H) * Q > tfk::kMaxRows)
    return fail(TF_ERR_UNSUPPORTED, "G*Q = %ld query rows per KV head (at most %d)", (long)(Hq / kv->H) * Q,
                tfk::kMaxRows);
  if (kv->B == 0) return ok();
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(K, "K", 16));
  TRY(check_ptr(V, "V", 16));
  TRY(check_ptr(out, "out", 16));
  if (lse) TRY(check_ptr(lse, "lse", 4));
  const tfk::SplitPlan plan =
      verify_plan(kv->B, kv->H, (Hq / kv->H) * Q, kv->max_len);
  if (plan.total_bytes > kNoAllocScratchBytes)
    return fail(TF_ERR_WORKSPACE, "this call needs %zu bytes of split partials; the built-in scratch holds %zu "
                "(use tf_verify_attn with a workspace)", plan.total_bytes, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (plan.total_bytes) TRY(scratch_on_current_device((hipStream_t)stream, &ws));
  tfk::AttnArgs a;
  fill_common(a, q, K, V, kv, Hq, Q, out, lse);
  fill_plan(a, plan, ws);
  return attn_call("tf_verify_attn_noalloc", kv->dtype, tfk::kVerify, a, (hipStream_t)stream);
}

TF_EXPORT int tf_verify_tree_attn(const void* q, int32_t Hq, int32_t Q, const void* K, const void* V,
                                  const tf_kv_desc* kv, const uint64_t* tree_mask, float* out, float* lse, void* ws,
                                  size_t ws_bytes, tf_stream_t stream) {
  TRY(check_desc(kv, "kv", false));
  if (Hq < 1 || Hq % kv->H != 0) return fail(TF_ERR_INVALID_ARG, "Hq=%d is not a multiple of H=%d", Hq, kv->H);
  if (Q < 1 || Q > 64) return fail(TF_ERR_INVALID_ARG, "Q=%d must be in [1, 64]", Q);
  if ((long)(Hq / kv->H) * Q > tfk::kMaxRows)
    return fail(TF_ERR_UNSUPPORTED, "G*Q = %ld query rows per KV head (at most %d)", (long)(Hq / kv->H) * Q,
                tfk::kMaxRows);
  if (kv->B == 0) return ok();
  TRY(check_ptr(q, "q", 16));
  TRY(check_ptr(K, "K", 16));
  TRY(check_ptr(V, "V", 16));
  TRY(check_ptr(tree_mask, "tree_mask", 8));
  TRY(check_ptr(out, "out", 16));
  if (lse) TRY(check_ptr(lse, "lse", 4));
  const tfk::SplitPlan plan =
      verify_plan(kv->B, kv->H, (Hq / kv->H) * Q, kv->max_len);
  TRY(check_ws(ws, ws_bytes, plan.total_bytes));
  tfk::AttnArgs a;
  fill_common(a, q, K, V, kv, Hq, Q, out, lse);
  fill_plan(a, plan, ws);
  a.tmask = tree_mask;
  return attn_call("tf_verify_tree_attn", kv->dtype, tfk::kVerifyTree, a, (hipStream_t)stream);
}

TF_EXPORT int tf_tree_masks(const int32_t* parent, int32_t B, int32_t Q, uint64_t* tree_mask, tf_stream_t stream) {
  if (B < 0 || Q < 1 || Q > 64) return fail(TF_ERR_INVALID_ARG, "B=%d Q=%d (need B >= 0, 1 <= Q <= 64)", B, Q);
  if (B == 0) return ok();
  TRY(check_ptr(parent, "parent", 4));
  TRY(check_ptr(tree_mask, "tree_mask", 8));
  return check_hip(tfk::launch_tree_masks(parent, B, Q, tree_mask, (hipStream_t)stream), "tf_tree_masks");
}

// ---------------------------------------------------------------------------
// a7
// ---------------------------------------------------------------------------
TF_EXPORT size_t tf_accept_workspace_size(int32_t B, int32_t gamma, int32_t V) {
  return tfk::accept_ws_bytes(B, gamma, V);
}

TF_EXPORT int tf_accept(const float* target, const float* draft, const int32_t* draft_tokens,
                        const double* uniforms, int32_t B, int32_t gamma, int32_t V, float temperature,
                        int32_t flags, int32_t* n_accepted, int32_t* next_token, void* ws, size_t ws_bytes,
                        tf_stream_t stream) {
  if (B < 0 || gamma < 0 || V < 1) return fail(TF_ERR_INVALID_ARG, "B=%d gamma=%d V=%d out of range", B, gamma, V);
  if (!(temperature >= 0.f) || std::isinf(temperature))
    return fail(TF_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  if (flags & ~TF_ACCEPT_PROBS) return fail(TF_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (V > tfk::accept_max_vocab()) return fail(TF_ERR_UNSUPPORTED, "V=%d above %d", V, tfk::accept_max_vocab());
  if (gamma > 1024) return fail(TF_ERR_UNSUPPORTED, "gamma above 1024");
  if ((long)B * (2 * gamma + 1) * ((V + 4095) / 4096) > 0x7fffffffL)
    return fail(TF_ERR_UNSUPPORTED, "B * (2 * gamma + 1) * ceil(V / 4096) above 2^31 - 1");
  if (B == 0) return ok();
  TRY(check_ptr(target, "target", 4));
  if (gamma > 0) {
    TRY(check_ptr(draft, "draft", 4));
    TRY(check_ptr(draft_tokens, "draft_tokens", 4));
  }
  TRY(check_ptr(uniforms, "uniforms", 8));
  TRY(check_ptr(n_accepted, "n_accepted", 4));
  TRY(check_ptr(next_token, "next_token", 4));
  TRY(check_ws(ws, ws_bytes, tfk::accept_ws_bytes(B, gamma, V)));
  return check_hip(tfk::launch_accept(target, draft, draft_tokens, uniforms, B, gamma, V, temperature, flags,
                                      n_accepted, next_token, ws, (hipStream_t)stream),
                   "tf_accept");
}

// ---------------------------------------------------------------------------
// Cache maintenance
// ---------------------------------------------------------------------------
TF_EXPORT int tf_append_kv(const void* K_new, const void* V_new, int32_t R, void* K, void* V, const tf_kv_desc* kv,
                           int32_t mode, int32_t n_sink, int32_t window, int32_t reserve, int32_t* status,
                           tf_stream_t stream) {
  TRY(check_desc(kv, "kv", false));
  if (R < 0 || R > (1 << 20)) return fail(TF_ERR_INVALID_ARG, "R=%d out of range", R);
  if (mode != TF_APPEND_FULL && mode != TF_APPEND_RING) return fail(TF_ERR_INVALID_ARG, "mode %d unknown", mode);
  if (mode == TF_APPEND_RING && (n_sink < 0 || window < 0 || reserve < R))
    return fail(TF_ERR_INVALID_ARG, "ring: n_sink=%d window=%d reserve=%d (need >= 0, >= 0, >= R=%d)", n_sink,
                window, reserve, R);
  if (kv->B == 0 || R == 0) return ok();
  TRY(check_ptr(K_new, "K_new", 16));
  TRY(check_ptr(V_new, "V_new", 16));
  TRY(check_ptr(K, "K", 16));
  TRY(check_ptr(V, "V", 16));
  if (status) TRY(check_ptr(status, "status", 4));
  return check_hip(tfk::launch_append((const uint16_t*)K_new, (const uint16_t*)V_new, R, (uint16_t*)K, (uint16_t*)V,
                                      *kv, mode, n_sink, window, reserve, status, (hipStream_t)stream),
                   "tf_append_kv");
}

TF_EXPORT int tf_commit_length(int32_t* seq_len, int32_t B, int32_t add, int32_t gamma, const int32_t* n_accepted,
                               tf_stream_t stream) {
  if (B < 0 || add < 0 || gamma < 0) return fail(TF_ERR_INVALID_ARG, "B=%d add=%d gamma=%d must be >= 0", B, add, gamma);
  if (B == 0) return ok();
  TRY(check_ptr(seq_len, "seq_len", 4));
  if (n_accepted) TRY(check_ptr(n_accepted, "n_accepted", 4));
  return check_hip(tfk::launch_commit(seq_len, B, add, gamma, n_accepted, (hipStream_t)stream), "tf_commit_length");
}

// ---------------------------------------------------------------------------
// Two-level accept: candidate collection between the levels
// ---------------------------------------------------------------------------
TF_EXPORT int tf_collect_candidates(const int32_t* draft_tokens, const int32_t* n_accepted, const int32_t* next_token,
                                    const float* q_rows, int32_t B, int32_t gamma1, int32_t V,
                                    const int32_t* count_in, int32_t* count_out, int32_t* cand, float* cand_q,
                                    int32_t gamma2, tf_stream_t stream) {
  if (B < 0 || gamma1 < 0 || gamma1 > 1024 || V < 1 || gamma2 < 1 || gamma2 > 1024)
    return fail(TF_ERR_INVALID_ARG, "B=%d gamma1=%d V=%d gamma2=%d out of range", B, gamma1, V, gamma2);
  if (B == 0) return ok();
  if (gamma1 > 0) TRY(check_ptr(draft_tokens, "draft_tokens", 4));
  TRY(check_ptr(n_accepted, "n_accepted", 4));
  TRY(check_ptr(next_token, "next_token", 4));
  TRY(check_ptr(q_rows, "q_rows", 16));
  TRY(check_ptr(count_in, "count_in", 4));
  TRY(check_ptr(count_out, "count_out", 4));
  TRY(check_ptr(cand, "cand", 4));
  TRY(check_ptr(cand_q, "cand_q", 16));
  if ((const void*)count_in == (const void*)count_out)
    return fail(TF_ERR_INVALID_ARG, "count_in and count_out must be different arrays");
  return check_hip(tfk::launch_collect(draft_tokens, n_accepted, next_token, q_rows, B, gamma1, V, count_in,
                                       count_out, cand, cand_q, gamma2, (hipStream_t)stream),
                   "tf_collect_candidates");
}

// ---------------------------------------------------------------------------
// Accept over a candidate tree
// ---------------------------------------------------------------------------
TF_EXPORT size_t tf_tree_accept_workspace_size(int32_t B, int32_t V) { return tfk::tree_accept_ws_bytes(B, V); }

TF_EXPORT int tf_tree_accept(const float* target, const float* draft, const int32_t* tokens, const int32_t* parent,
                             const double* uniforms, int32_t B, int32_t Q, int32_t V, float temperature,
                             int32_t flags, int32_t* n_accepted, int32_t* path, int32_t* next_token, void* ws,
                             size_t ws_bytes, tf_stream_t stream) {
  if (B < 0 || Q < 1 || V < 1) return fail(TF_ERR_INVALID_ARG, "B=%d Q=%d V=%d out of range", B, Q, V);
  if (!(temperature >= 0.f) || std::isinf(temperature))
    return fail(TF_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  if (flags & ~TF_ACCEPT_PROBS) return fail(TF_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (Q > tfk::tree_accept_max_nodes()) return fail(TF_ERR_UNSUPPORTED, "Q=%d above %d", Q, tfk::tree_accept_max_nodes());
  if (V > tfk::tree_accept_max_vocab()) return fail(TF_ERR_UNSUPPORTED, "V=%d above %d", V, tfk::tree_accept_max_vocab());
  if (B == 0) return ok();
  TRY(check_ptr(target, "target", 4));
  if (Q > 1) {
    TRY(check_ptr(draft, "draft", 4));
    TRY(check_ptr(path, "path", 4));
  }
  TRY(check_ptr(tokens, "tokens", 4));
  TRY(check_ptr(parent, "parent", 4));
  TRY(check_ptr(uniforms, "uniforms", 8));
  TRY(check_ptr(n_accepted, "n_accepted", 4));
  TRY(check_ptr(next_token, "next_token", 4));
  TRY(check_ws(ws, ws_bytes, tfk::tree_accept_ws_bytes(B, V)));
  return check_hip(tfk::launch_tree_accept(target, draft, tokens, parent, uniforms, B, Q, V, temperature, flags,
                                           n_accepted, path, next_token, ws, (hipStream_t)stream),
                   "tf_tree_accept");
}

