// C ABI of the QLoRA NF4 library: argument validation (host only, before any
// launch), workspace layout and kernel dispatch.  See include/qlora_nf4.h for
// the contract of each entry point.
#include "qlora_nf4.h"
#include "qlora_nf4_profile.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "launch.h"

using namespace qlora;

namespace {

thread_local char g_err[512] = "";

// Per-thread event pairs attached with qlora_profile_events.
struct ProfPair {
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local ProfPair g_prof[QLORA_KERNEL_COUNT];

// Brackets one kernel launch with the attached events (if any).
struct ProfScope {
  const ProfPair& p;
  hipStream_t s;
  ProfScope(int id, hipStream_t stream) : p(g_prof[id]), s(stream) {
    if (p.start) (void)hipEventRecord(p.start, s);
  }
  ~ProfScope() {
    if (p.stop) (void)hipEventRecord(p.stop, s);
  }
};

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(QLORA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int64_t kMaxNumel = (int64_t)1 << 37;
constexpr int64_t kAlign = 256;  // alignment of workspace regions
constexpr int kMaxBatch = 4096;  // tensors per batched quantisation call

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

int64_t nblocks(int64_t numel) { return ceil_div(numel, QLORA_NF4_BLOCKSIZE); }
int64_t ngroups(int64_t numel) { return ceil_div(nblocks(numel), QLORA_NF4_BLOCKSIZE2); }

// Validate the descriptor itself (shape, flags, buffer pointers).
int check_desc(const qlora_nf4_t* q, const char* fn) {
  if (!q) return fail(QLORA_ERR_INVALID_ARG, "%s: descriptor is NULL", fn);
  if (q->rows < 0 || q->cols < 0) return fail(QLORA_ERR_INVALID_ARG, "%s: negative shape", fn);
  if (q->cols > 0 && q->rows > kMaxNumel / q->cols)
    return fail(QLORA_ERR_INVALID_ARG, "%s: rows*cols must be below 2^37", fn);
  if (q->blocksize != QLORA_NF4_BLOCKSIZE || q->blocksize2 != QLORA_NF4_BLOCKSIZE2)
    return fail(QLORA_ERR_INVALID_ARG, "%s: blocksize must be 64 and blocksize2 256", fn);
  if (q->double_quant != 0 && q->double_quant != 1)
    return fail(QLORA_ERR_INVALID_ARG, "%s: double_quant must be 0 or 1", fn);
  if (q->code_type < 0 || q->code_type > CODE_INT8)
    return fail(QLORA_ERR_INVALID_ARG, "%s: code_type must be one of the qlora_code_type values", fn);
  if (q->rows * q->cols == 0) return QLORA_OK;
  if (!q->codes) return fail(QLORA_ERR_INVALID_ARG, "%s: codes is NULL", fn);
  if (!aligned16(q->codes)) return fail(QLORA_ERR_MISALIGNED, "%s: codes not 16-byte aligned", fn);
  if (q->double_quant) {
    if (!q->absmax_q || !q->scale2 || !q->offset)
      return fail(QLORA_ERR_INVALID_ARG, "%s: absmax_q, scale2 and offset are required with double_quant", fn);
    if (!aligned16(q->absmax_q) || !aligned16(q->scale2) || !aligned16(q->offset))
      return fail(QLORA_ERR_MISALIGNED, "%s: constant buffers must be 16-byte aligned", fn);
  } else {
    if (!q->absmax) return fail(QLORA_ERR_INVALID_ARG, "%s: absmax is required without double_quant", fn);
    if (!aligned16(q->absmax)) return fail(QLORA_ERR_MISALIGNED, "%s: absmax not 16-byte aligned", fn);
  }
  return QLORA_OK;
}

DQParams dq_params(const qlora_nf4_t* q) {
  DQParams p;
  p.absmax_q = q->absmax_q;
  p.absmax = q->absmax;
  p.scale2 = q->scale2;
  p.offset = q->offset;
  p.double_quant = q->double_quant;
  p.code_type = q->code_type;
  return p;
}

// Workspace layouts ------------------------------------------------------

int64_t quant_ws(int64_t numel, int dq) {
  if (!dq || numel == 0) return 0;
  const int64_t nb = nblocks(numel);
  return round_up(nb * 4, kAlign) + round_up((int64_t)quantize_parts(numel) * kMeanDigits * 8, kAlign);
}

// Shapes the small-token path can take (it also needs 4-bit codes); the
// workspace layouts are sized for it whatever the code type.
bool small_token_shape(int64_t M, int64_t N, int64_t r) {
  return M >= 1 && M <= kGemvMaxM && N % 4 == 0 && r <= 256;
}

struct FwdWs {
  // byte offsets: fp32 partials of X A (split partials, or on the
  // small-token path one slice per 256-wide reduction chunk), bf16 s*XA
  // [M, rp], then one region for the small-token path's fp32 partials of
  // X W^T [gemv_splits][M][N] or the main product's split tiles
  int64_t part, xas, gv, total;
  int splits, gemv_splits;
};
FwdWs fwd_ws(int64_t M, int64_t N, int64_t K, int64_t r) {
  const int64_t rp = round_up(r, 64);
  FwdWs w;
  const bool small = small_token_shape(M, N, r);
  w.gemv_splits = small ? gemv_splits(M, N, K) : 0;
  w.splits = skinny_splits(M, r, K);
  if (small && xa_chunks(K) > w.splits) w.splits = xa_chunks(K);
  w.part = 0;
  w.xas = w.part + round_up((int64_t)w.splits * M * rp * 4, kAlign);
  w.gv = w.xas + round_up(M * rp * 2, kAlign);
  // the small-token region also holds the split tiles of the 256 x 256
  // kernel, which takes Int8 weights at any token count
  const int64_t st_bytes = main_split_bytes(M, N, K);
  const int64_t gm_bytes = w.gemv_splits > 0 ? (int64_t)w.gemv_splits * M * N * 4 : 0;
  const int64_t gv_bytes = gm_bytes > st_bytes ? gm_bytes : st_bytes;
  w.total = w.gv + round_up(gv_bytes, kAlign);
  return w;
}

// The forward takes the small-token path (weight-streaming kernel) for these
// shapes; the backward's recomputation of XA follows the same path.
bool small_token_path(int64_t M, int64_t N, int64_t r, int32_t code_type) {
  return small_token_shape(M, N, r) && code_type != CODE_INT8;
}

struct BwdWs {
  // fp32 partials of dY B^T (and before them, when XA is recomputed, those of
  // X A), bf16 s*T [M, rp], the recomputed bf16 XA [M, r], fp32 partials of
  // the token reductions and of the main product's split tiles (one region,
  // used in turn)
  int64_t part_t, ts, xa, part, part_b, total;
  int splits_t, splits_x, splits_a, splits_b;
};
BwdWs bwd_ws(int64_t M, int64_t N, int64_t K, int64_t r) {
  const int64_t rp = round_up(r, 64);
  BwdWs w;
  w.splits_t = skinny_splits(M, r, N);
  w.splits_x = skinny_splits(M, r, K);  // as the forward's X A
  if (small_token_shape(M, N, r) && xa_chunks(K) > w.splits_x) w.splits_x = xa_chunks(K);
  w.splits_a = tn_splits(M, K, r);
  w.splits_b = tn_splits(M, N, r);  // dB is formed as dB^T [N, r]
  // the two token reductions run together (dA partials at part, dB^T
  // partials at part + part_b); the main product's split tiles use the
  // same space before them
  w.part_b = round_up((int64_t)w.splits_a * K * r * 4, kAlign);
  int64_t pbytes = w.part_b + (int64_t)w.splits_b * N * r * 4;
  const int64_t pm = main_split_bytes(M, K, N);
  if (pm > pbytes) pbytes = pm;
  const int64_t st = w.splits_t > w.splits_x ? w.splits_t : w.splits_x;
  w.part_t = 0;
  w.ts = w.part_t + round_up(st * M * rp * 4, kAlign);
  w.xa = w.ts + round_up(M * rp * 2, kAlign);
  w.part = w.xa + round_up(M * r * 2, kAlign);
  w.total = w.part + round_up(pbytes, kAlign);
  return w;
}

int check_linear_shape(const qlora_nf4_t* W, int64_t M, int32_t r, const char* fn) {
  int st = check_desc(W, fn);
  if (st) return st;
  if (M < 0) return fail(QLORA_ERR_INVALID_ARG, "%s: M < 0", fn);
  if (W->rows <= 0 || W->cols <= 0 || W->rows % 64 || W->cols % 64)
    return fail(QLORA_ERR_INVALID_ARG, "%s: weight [N, K] needs N, K > 0 and multiples of 64 (got %lld x %lld)",
                fn, (long long)W->rows, (long long)W->cols);
  if (r < 1 || r > QLORA_MAX_RANK) return fail(QLORA_ERR_INVALID_ARG, "%s: rank r must be in [1, 256]", fn);
  if (M > kMaxNumel / (W->rows > W->cols ? W->rows : W->cols))
    return fail(QLORA_ERR_INVALID_ARG, "%s: M too large", fn);
  return QLORA_OK;
}

int check_ptr(const void* p, const char* name, const char* fn) {
  if (!p) return fail(QLORA_ERR_INVALID_ARG, "%s: %s is NULL", fn, name);
  if (!aligned16(p)) return fail(QLORA_ERR_MISALIGNED, "%s: %s not 16-byte aligned", fn, name);
  return QLORA_OK;
}

}  // namespace

extern "C" {

const char* qlora_status_string(int32_t status) {
  switch (status) {
    case QLORA_OK: return "ok";
    case QLORA_ERR_INVALID_ARG: return "invalid argument";
    case QLORA_ERR_UNSUPPORTED_DTYPE: return "unsupported dtype";
    case QLORA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case QLORA_ERR_MISALIGNED: return "pointer not 16-byte aligned";
    case QLORA_ERR_HIP: return "HIP launch error";
    case QLORA_ERR_INTERNAL: return "internal consistency check failed";
    default: return "unknown status";
  }
}

const char* qlora_last_error(void) { return g_err; }

}  // extern "C"

// Records a failure message for the calling thread (for entry points defined
// in other files of the library) and returns `status`.
int qlora::record_failure(int status, const char* msg) {
  snprintf(g_err, sizeof(g_err), "%s", msg);
  return status;
}

extern "C" {

int qlora_profile_events(int32_t kernel_id, void* start_event, void* stop_event) {
  if (kernel_id < 0 || kernel_id >= QLORA_KERNEL_COUNT)
    return fail(QLORA_ERR_INVALID_ARG, "qlora_profile_events: unknown kernel id %d", kernel_id);
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(QLORA_ERR_INVALID_ARG, "qlora_profile_events: give both events or neither");
  g_prof[kernel_id].start = (hipEvent_t)start_event;
  g_prof[kernel_id].stop = (hipEvent_t)stop_event;
  return QLORA_OK;
}

int qlora_nf4_codebook(float* out) {
  if (!out) return fail(QLORA_ERR_INVALID_ARG, "qlora_nf4_codebook: out is NULL");
  memcpy(out, nf4_values().v, sizeof(float) * 16);
  return QLORA_OK;
}

int qlora_codebook(int32_t code_type, float* out) {
  if (!out) return fail(QLORA_ERR_INVALID_ARG, "qlora_codebook: out is NULL");
  if (code_type < 0 || code_type > CODE_INT8)
    return fail(QLORA_ERR_INVALID_ARG, "qlora_codebook: code_type must be one of the qlora_code_type values");
  if (code_type == CODE_INT8) memcpy(out, int8_tables().value, sizeof(float) * 256);
  else memcpy(out, code_values(code_type).v, sizeof(float) * 16);
  return QLORA_OK;
}

int qlora_storage_bytes(int64_t numel, int32_t double_quant, int32_t code_type, int64_t* bytes) {
  if (code_type < 0 || code_type > CODE_INT8)
    return fail(QLORA_ERR_INVALID_ARG, "qlora_storage_bytes: code_type must be one of the qlora_code_type values");
  if (!bytes) return fail(QLORA_ERR_INVALID_ARG, "qlora_storage_bytes: bytes is NULL");
  if (numel < 0 || numel >= kMaxNumel) return fail(QLORA_ERR_INVALID_ARG, "qlora_storage_bytes: bad numel");
  if (double_quant != 0 && double_quant != 1)
    return fail(QLORA_ERR_INVALID_ARG, "qlora_storage_bytes: double_quant must be 0 or 1");
  qlora_nf4_storage_bytes(numel, double_quant, bytes);
  if (code_type == CODE_INT8) bytes[0] = numel;
  return QLORA_OK;
}

int qlora_nf4_storage_bytes(int64_t numel, int32_t double_quant, int64_t* bytes) {
  if (!bytes) return fail(QLORA_ERR_INVALID_ARG, "qlora_nf4_storage_bytes: bytes is NULL");
  if (numel < 0 || numel >= kMaxNumel) return fail(QLORA_ERR_INVALID_ARG, "qlora_nf4_storage_bytes: bad numel");
  if (double_quant != 0 && double_quant != 1)
    return fail(QLORA_ERR_INVALID_ARG, "qlora_nf4_storage_bytes: double_quant must be 0 or 1");
  bytes[0] = ceil_div(numel, 2);
  bytes[1] = double_quant ? nblocks(numel) : 0;
  bytes[2] = double_quant ? 0 : 4 * nblocks(numel);
  bytes[3] = double_quant ? 4 * ngroups(numel) : 0;
  bytes[4] = double_quant ? 4 : 0;
  return QLORA_OK;
}

int qlora_nf4_quantize_workspace(int64_t numel, int32_t double_quant, int64_t* ws_bytes) {
  if (!ws_bytes) return fail(QLORA_ERR_INVALID_ARG, "qlora_nf4_quantize_workspace: ws_bytes is NULL");
  if (numel < 0 || numel >= kMaxNumel) return fail(QLORA_ERR_INVALID_ARG, "qlora_nf4_quantize_workspace: bad numel");
  if (double_quant != 0 && double_quant != 1)
    return fail(QLORA_ERR_INVALID_ARG, "qlora_nf4_quantize_workspace: double_quant must be 0 or 1");
  *ws_bytes = quant_ws(numel, double_quant);
  return QLORA_OK;
}

int qlora_linear_workspace(int64_t M, int64_t N, int64_t K, int32_t r, int64_t* fwd_bytes, int64_t* bwd_bytes) {
  if (M < 0 || N <= 0 || K <= 0 || N % 64 || K % 64 || r < 1 || r > QLORA_MAX_RANK)
    return fail(QLORA_ERR_INVALID_ARG, "qlora_linear_workspace: bad shape or rank");
  if (fwd_bytes) *fwd_bytes = fwd_ws(M, N, K, r).total;
  if (bwd_bytes) *bwd_bytes = bwd_ws(M, N, K, r).total;
  return QLORA_OK;
}

int qlora_nf4_quantize(const void* w, int32_t w_dtype, const qlora_nf4_t* q, void* ws, int64_t ws_bytes,
                       void* stream) {
  static const char* fn = "qlora_nf4_quantize";
  int st = check_desc(q, fn);
  if (st) return st;
  if (w_dtype != QLORA_DTYPE_F32 && w_dtype != QLORA_DTYPE_BF16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: w_dtype must be F32 or BF16", fn);
  const int64_t numel = q->rows * q->cols;
  if (numel == 0) return QLORA_OK;
  if ((st = check_ptr(w, "w", fn))) return st;
  const int64_t need = quant_ws(numel, q->double_quant);
  if (ws_bytes < need) return fail(QLORA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %lld bytes", fn, (long long)need);
  if (need > 0 && (st = check_ptr(ws, "ws", fn))) return st;
  if (!quant_tables_ok(q->code_type))
    return fail(QLORA_ERR_INTERNAL, "%s: the quantisation table of code type %d is inconsistent", fn, q->code_type);
  hipStream_t s = (hipStream_t)stream;
  const int64_t nb = nblocks(numel);
  float* c2 = q->double_quant ? (float*)ws : q->absmax;
  uint64_t* parts = q->double_quant ? (uint64_t*)((char*)ws + round_up(nb * 4, kAlign)) : nullptr;
  hipError_t e;
  {
    ProfScope ps(QLORA_KERNEL_QUANTIZE, s);
    e = launch_quantize(w, w_dtype == QLORA_DTYPE_BF16, numel, q->code_type, q->codes, c2, parts, s);
  }
  if (e != hipSuccess) return hip_fail(e, fn);
  if (q->double_quant) {
    e = launch_double_quant(c2, nb, parts, quantize_parts(numel), q->absmax_q, q->scale2, q->offset, s);
    if (e != hipSuccess) return hip_fail(e, fn);
  }
  return QLORA_OK;
}

int qlora_nf4_quantize_batched_workspace(const qlora_nf4_t* q, int32_t count, int64_t* ws_bytes) {
  static const char* fn = "qlora_nf4_quantize_batched_workspace";
  if (!ws_bytes) return fail(QLORA_ERR_INVALID_ARG, "%s: ws_bytes is NULL", fn);
  if (count < 0 || count > kMaxBatch) return fail(QLORA_ERR_INVALID_ARG, "%s: count must be in [0, %d]", fn, kMaxBatch);
  if (count > 0 && !q) return fail(QLORA_ERR_INVALID_ARG, "%s: q is NULL", fn);
  int64_t total = 0;
  for (int32_t i = 0; i < count; ++i) {
    int st = check_desc(&q[i], fn);
    if (st) return st;
    total += quant_ws(q[i].rows * q[i].cols, q[i].double_quant);
  }
  *ws_bytes = total;
  return QLORA_OK;
}

int qlora_nf4_quantize_batched(const void* const* w, int32_t w_dtype, const qlora_nf4_t* q, int32_t count, void* ws,
                               int64_t ws_bytes, void* stream) {
  static const char* fn = "qlora_nf4_quantize_batched";
  if (count < 0 || count > kMaxBatch) return fail(QLORA_ERR_INVALID_ARG, "%s: count must be in [0, %d]", fn, kMaxBatch);
  if (count == 0) return QLORA_OK;
  if (!w || !q) return fail(QLORA_ERR_INVALID_ARG, "%s: w and q must be host arrays of count entries", fn);
  if (w_dtype != QLORA_DTYPE_F32 && w_dtype != QLORA_DTYPE_BF16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: w_dtype must be F32 or BF16", fn);
  int st;
  int64_t need = 0;
  for (int32_t i = 0; i < count; ++i) {
    if ((st = check_desc(&q[i], fn))) return st;
    if (q[i].code_type != q[0].code_type || q[i].double_quant != q[0].double_quant)
      return fail(QLORA_ERR_INVALID_ARG, "%s: every descriptor must share code_type and double_quant", fn);
    if (q[i].rows * q[i].cols > 0 && (st = check_ptr(w[i], "w[i]", fn))) return st;
    need += quant_ws(q[i].rows * q[i].cols, q[i].double_quant);
  }
  if (ws_bytes < need) return fail(QLORA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %lld bytes", fn, (long long)need);
  if (need > 0 && (st = check_ptr(ws, "ws", fn))) return st;
  if (!quant_tables_ok(q[0].code_type))
    return fail(QLORA_ERR_INTERNAL, "%s: the quantisation table of code type %d is inconsistent", fn, q[0].code_type);
  // each non-empty tensor's workspace regions, in order, laid out as qlora_nf4_quantize lays out its own
  QuantJob jobs[kMaxBatch];
  int n = 0;
  char* base = (char*)ws;
  for (int32_t i = 0; i < count; ++i) {
    const int64_t numel = q[i].rows * q[i].cols;
    const int64_t wsi = quant_ws(numel, q[i].double_quant);
    if (numel > 0) {
      QuantJob& jb = jobs[n++];
      const int64_t nb = nblocks(numel);
      jb.w = w[i];
      jb.numel = numel;
      jb.codes = q[i].codes;
      jb.c2 = q[i].double_quant ? (float*)base : q[i].absmax;
      jb.partials = q[i].double_quant ? (uint64_t*)(base + round_up(nb * 4, kAlign)) : nullptr;
      jb.absmax_q = q[i].absmax_q;
      jb.scale2 = q[i].scale2;
      jb.offset = q[i].offset;
    }
    base += wsi;
  }
  const hipError_t e = launch_quantize_batched(jobs, n, w_dtype == QLORA_DTYPE_BF16, q[0].code_type,
                                               q[0].double_quant != 0, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}

int qlora_nf4_dequantize(const qlora_nf4_t* q, void* out, int32_t out_dtype, void* stream) {
  static const char* fn = "qlora_nf4_dequantize";
  int st = check_desc(q, fn);
  if (st) return st;
  if (out_dtype != QLORA_DTYPE_F32 && out_dtype != QLORA_DTYPE_BF16)
    return fail(QLORA_ERR_UNSUPPORTED_DTYPE, "%s: out_dtype must be F32 or BF16", fn);
  const int64_t numel = q->rows * q->cols;
  if (numel == 0) return QLORA_OK;
  if ((st = check_ptr(out, "out", fn))) return st;
  hipError_t e;
  {
    ProfScope ps(QLORA_KERNEL_DEQUANTIZE, (hipStream_t)stream);
    e = launch_dequantize(q->codes, numel, q->code_type, q->double_quant != 0, q->absmax_q, q->absmax, q->scale2, q->offset, out,
                          out_dtype == QLORA_DTYPE_BF16, (hipStream_t)stream);
  }
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}

}  // extern "C"

namespace {

// 1 / (1 - p) in fp32: the inverted-dropout scale of the kept elements.
float keep_scale_of(float p) { return (float)(1.0 / (1.0 - (double)p)); }

int check_dropout(const void* keep, float p, const char* fn) {
  if (!keep) return QLORA_OK;
  if (!(p >= 0.0f && p < 1.0f)) return fail(QLORA_ERR_INVALID_ARG, "%s: dropout p must be in [0, 1)", fn);
  return check_ptr(keep, "keep_mask", fn);
}

// The forward with optional LoRA dropout (keep = null: none).
int linear_fwd_impl(const void* X, int64_t M, const qlora_nf4_t* W, const void* A, const void* B, int32_t r, float s,
                    const void* keep, float p, void* Y, void* XA, void* ws, int64_t ws_bytes, void* stream,
                    const char* fn) {
  int st = check_linear_shape(W, M, r, fn);
  if (st) return st;
  if ((st = check_dropout(keep, p, fn))) return st;
  if (M == 0) return QLORA_OK;
  const uint8_t* km = (const uint8_t*)keep;
  const float d = km ? keep_scale_of(p) : 1.0f;
  if ((st = check_ptr(X, "X", fn)) || (st = check_ptr(A, "A", fn)) || (st = check_ptr(B, "B", fn)) ||
      (st = check_ptr(Y, "Y", fn)))
    return st;
  if (XA && !aligned16(XA)) return fail(QLORA_ERR_MISALIGNED, "%s: XA not 16-byte aligned", fn);
  const int64_t N = W->rows, K = W->cols, rp = round_up(r, 64);
  const FwdWs L = fwd_ws(M, N, K, r);
  if (ws_bytes < L.total) return fail(QLORA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %lld bytes", fn, (long long)L.total);
  if ((st = check_ptr(ws, "ws", fn))) return st;
  hipStream_t hs = (hipStream_t)stream;
  char* base = (char*)ws;
  float* part = (float*)(base + L.part);
  uint16_t* xas = (uint16_t*)(base + L.xas);
  hipError_t e;
  if (small_token_path(M, N, r, W->code_type)) {  // the weight-streaming kernel takes 4-bit codes
    // few tokens: the weight-streaming product, which also writes the X A
    // partials per reduction chunk, then one kernel that adds both sets of
    // partials and the adapter term
    float* gv = (float*)(base + L.gv);
    {
      ProfScope ps(QLORA_KERNEL_FWD_MAIN, hs);
      e = launch_gemv((const uint16_t*)X, M, K, W->codes, dq_params(W), N, gv, L.gemv_splits, (const uint16_t*)A, r,
                      rp, km, part, hs);
    }
    if (e != hipSuccess) return hip_fail(e, fn);
    e = launch_gemv_reduce(gv, L.gemv_splits, M, N, part, xa_chunks(K), rp, s * d, d, (const uint16_t*)B, r,
                           (uint16_t*)Y, (uint16_t*)XA, hs);
    if (e != hipSuccess) return hip_fail(e, fn);
    return QLORA_OK;
  }
  // XA = X A [M, r]: bf16 copy for the backward, bf16(s XA) padded to rp for the adapter steps
  if ((e = launch_skinny((const uint16_t*)X, (const uint16_t*)A, true, M, r, K, part, L.splits, (uint16_t*)XA, xas, rp,
                         s * d, d, km, hs)) != hipSuccess)
    return hip_fail(e, fn);
  {
    ProfScope ps(QLORA_KERNEL_FWD_MAIN, hs);
    e = launch_fwd_main((const uint16_t*)X, M, K, W->codes, dq_params(W), N, xas, (const uint16_t*)B, r, rp,
                        (uint16_t*)Y, (float*)(base + L.gv), hs);
  }
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}

// The backward with optional LoRA dropout (keep = null: none).
int linear_bwd_impl(const void* dY, const void* X, const void* XA, int64_t M, const qlora_nf4_t* W, const void* A,
                    const void* B, int32_t r, float s, const void* keep, float p, void* dX, void* dA, void* dB,
                    int32_t accumulate, void* ws, int64_t ws_bytes, void* stream, const char* fn) {
  int st = check_linear_shape(W, M, r, fn);
  if (st) return st;
  if ((st = check_dropout(keep, p, fn))) return st;
  if (accumulate != 0 && accumulate != 1) return fail(QLORA_ERR_INVALID_ARG, "%s: accumulate must be 0 or 1", fn);
  const uint8_t* km = (const uint8_t*)keep;
  const float d = km ? keep_scale_of(p) : 1.0f;
  if ((st = check_ptr(dA, "dA", fn)) || (st = check_ptr(dB, "dB", fn))) return st;
  const int64_t N = W->rows, K = W->cols, rp = round_up(r, 64);
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e;
  if (M == 0) {  // no tokens: the gradients are zero (nothing to add when accumulating)
    if (accumulate) return QLORA_OK;
    if ((e = launch_fill_zero_u16((uint16_t*)dA, K * r, hs)) != hipSuccess) return hip_fail(e, fn);
    if ((e = launch_fill_zero_u16((uint16_t*)dB, (int64_t)r * N, hs)) != hipSuccess) return hip_fail(e, fn);
    return QLORA_OK;
  }
  if ((st = check_ptr(dY, "dY", fn)) || (st = check_ptr(X, "X", fn)) || (st = check_ptr(A, "A", fn)) ||
      (st = check_ptr(B, "B", fn)))
    return st;
  if (XA && !aligned16(XA)) return fail(QLORA_ERR_MISALIGNED, "%s: XA not 16-byte aligned", fn);
  if (dX && !aligned16(dX)) return fail(QLORA_ERR_MISALIGNED, "%s: dX not 16-byte aligned", fn);
  const BwdWs L = bwd_ws(M, N, K, r);
  if (ws_bytes < L.total) return fail(QLORA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %lld bytes", fn, (long long)L.total);
  if ((st = check_ptr(ws, "ws", fn))) return st;
  char* base = (char*)ws;
  float* part_t = (float*)(base + L.part_t);
  uint16_t* ts = (uint16_t*)(base + L.ts);
  float* part = (float*)(base + L.part);
  if (!XA) {
    // recompute XA = (drop(X)) A exactly as the forward writes it: the same
    // split partials, then the forward's own reduction for its path
    uint16_t* xa = (uint16_t*)(base + L.xa);
    if (small_token_path(M, N, r, W->code_type)) {
      if ((e = launch_xa_chunks((const uint16_t*)X, M, K, (const uint16_t*)A, r, rp, km, part_t, hs)) != hipSuccess)
        return hip_fail(e, fn);
      if ((e = launch_xa_reduce(part_t, xa_chunks(K), M, rp, d, r, xa, hs)) != hipSuccess) return hip_fail(e, fn);
    } else if ((e = launch_skinny((const uint16_t*)X, (const uint16_t*)A, true, M, r, K, part_t, L.splits_x, xa,
                                  nullptr, rp, s * d, d, km, hs)) != hipSuccess) {
      return hip_fail(e, fn);
    }
    XA = xa;
  }
  // s*T = s * dY B^T  [M, rp]
  if ((e = launch_skinny((const uint16_t*)dY, (const uint16_t*)B, false, M, r, N, part_t, L.splits_t, nullptr, ts, rp,
                         s, 1.0f, nullptr, hs)) != hipSuccess)
    return hip_fail(e, fn);
  if (dX) {
    {
      ProfScope ps(QLORA_KERNEL_BWD_DX, hs);
      e = launch_bwd_dx((const uint16_t*)dY, M, N, W->codes, dq_params(W), K, ts, (const uint16_t*)A, r, rp,
                        (uint16_t*)dX, part, km, d, hs);
    }
    if (e != hipSuccess) return hip_fail(e, fn);
  }
  // dA = X^T (s T) [K, r] and dB^T = s dY^T XA [N, r] (written as dB [r, N])
  if ((e = launch_tn_pair((const uint16_t*)X, K, K, km, ts, rp, r, part, L.splits_a, (uint16_t*)dA, d,
                          (const uint16_t*)dY, N, N, (const uint16_t*)XA, r, r,
                          (float*)((char*)part + L.part_b), L.splits_b, (uint16_t*)dB, s, M, accumulate != 0,
                          hs)) != hipSuccess)
    return hip_fail(e, fn);
  return QLORA_OK;
}

}  // namespace

extern "C" {

int qlora_linear_fwd(const void* X, int64_t M, const qlora_nf4_t* W, const void* A, const void* B, int32_t r, float s,
                     void* Y, void* XA, void* ws, int64_t ws_bytes, void* stream) {
  return linear_fwd_impl(X, M, W, A, B, r, s, nullptr, 0.0f, Y, XA, ws, ws_bytes, stream, "qlora_linear_fwd");
}

int qlora_linear_fwd_dropout(const void* X, int64_t M, const qlora_nf4_t* W, const void* A, const void* B, int32_t r,
                             float s, const void* keep_mask, float p, void* Y, void* XA, void* ws, int64_t ws_bytes,
                             void* stream) {
  static const char* fn = "qlora_linear_fwd_dropout";
  if (!keep_mask) return fail(QLORA_ERR_INVALID_ARG, "%s: keep_mask is NULL", fn);
  return linear_fwd_impl(X, M, W, A, B, r, s, keep_mask, p, Y, XA, ws, ws_bytes, stream, fn);
}

int qlora_linear_bwd(const void* dY, const void* X, const void* XA, int64_t M, const qlora_nf4_t* W, const void* A,
                     const void* B, int32_t r, float s, void* dX, void* dA, void* dB, int32_t accumulate, void* ws,
                     int64_t ws_bytes, void* stream) {
  return linear_bwd_impl(dY, X, XA, M, W, A, B, r, s, nullptr, 0.0f, dX, dA, dB, accumulate, ws, ws_bytes, stream,
                         "qlora_linear_bwd");
}

int qlora_linear_bwd_dropout(const void* dY, const void* X, const void* XA, int64_t M, const qlora_nf4_t* W,
                             const void* A, const void* B, int32_t r, float s, const void* keep_mask, float p,
                             void* dX, void* dA, void* dB, int32_t accumulate, void* ws, int64_t ws_bytes,
                             void* stream) {
  static const char* fn = "qlora_linear_bwd_dropout";
  if (!keep_mask) return fail(QLORA_ERR_INVALID_ARG, "%s: keep_mask is NULL", fn);
  return linear_bwd_impl(dY, X, XA, M, W, A, B, r, s, keep_mask, p, dX, dA, dB, accumulate, ws, ws_bytes, stream,
                         fn);
}

int qlora_dropout_mask(uint64_t seed, uint64_t offset, int64_t M, int64_t K, float p, void* keep_mask,
                       void* stream) {
  static const char* fn = "qlora_dropout_mask";
  if (M < 0 || K <= 0 || K % 8) return fail(QLORA_ERR_INVALID_ARG, "%s: need M >= 0, K > 0 and K %% 8 == 0", fn);
  if (M > kMaxNumel / K) return fail(QLORA_ERR_INVALID_ARG, "%s: M * K must be below 2^37", fn);
  if (!(p >= 0.0f && p < 1.0f)) return fail(QLORA_ERR_INVALID_ARG, "%s: dropout p must be in [0, 1)", fn);
  if (M == 0) return QLORA_OK;
  int st;
  if ((st = check_ptr(keep_mask, "keep_mask", fn))) return st;
  // T = floor(p * 2^32), exact in double (p has 24 significant bits)
  const uint32_t T = (uint32_t)floor((double)p * 4294967296.0);
  const hipError_t e = launch_dropout_mask((uint8_t*)keep_mask, M * (K / 8), seed, offset, T, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}

int qlora_clip_scale_workspace(int64_t n, int64_t* ws_bytes) {
  if (!ws_bytes) return fail(QLORA_ERR_INVALID_ARG, "qlora_clip_scale_workspace: ws_bytes is NULL");
  if (n < 0) return fail(QLORA_ERR_INVALID_ARG, "qlora_clip_scale_workspace: n < 0");
  *ws_bytes = round_up((int64_t)clip_parts(n) * 8, kAlign);
  return QLORA_OK;
}

int qlora_clip_scale(const void* grad, int64_t n, float max_norm, float* scale, void* ws, int64_t ws_bytes,
                     void* stream) {
  static const char* fn = "qlora_clip_scale";
  int st;
  if (n < 0) return fail(QLORA_ERR_INVALID_ARG, "%s: n < 0", fn);
  if (!(max_norm > 0.0f)) return fail(QLORA_ERR_INVALID_ARG, "%s: max_norm must be > 0", fn);
  if ((st = check_ptr(scale, "scale", fn))) return st;
  if (n > 0 && (st = check_ptr(grad, "grad", fn))) return st;
  const int64_t need = round_up((int64_t)clip_parts(n) * 8, kAlign);
  if (ws_bytes < need) return fail(QLORA_ERR_WORKSPACE_TOO_SMALL, "%s: workspace needs %lld bytes", fn, (long long)need);
  if ((st = check_ptr(ws, "ws", fn))) return st;
  const hipError_t e = launch_clip_scale((const uint16_t*)grad, n, max_norm, scale, (double*)ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}

int qlora_adamw_step_paged(float* param, void* param_bf16, const void* grad, float* exp_avg, float* exp_avg_sq,
                           int64_t n, const float* grad_scale, float lr, float beta1, float beta2, float eps,
                           float weight_decay, int32_t step, void* staging, int64_t staging_bytes, void* stream,
                           void* copy_stream) {
  static const char* fn = "qlora_adamw_step_paged";
  int st;
  if (n < 0) return fail(QLORA_ERR_INVALID_ARG, "%s: n < 0", fn);
  if (step < 1) return fail(QLORA_ERR_INVALID_ARG, "%s: step counts from 1", fn);
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
    return fail(QLORA_ERR_INVALID_ARG, "%s: betas must be in [0, 1)", fn);
  if (!(eps > 0.0f) || !(lr >= 0.0f) || !(weight_decay >= 0.0f))
    return fail(QLORA_ERR_INVALID_ARG, "%s: need eps > 0, lr >= 0, weight_decay >= 0", fn);
  // chunk: floats per state and slot, a multiple of 256 (staging = 2 slots x 2 states)
  const int64_t chunk = staging_bytes / 16 / 256 * 256;
  if (chunk < 256) return fail(QLORA_ERR_WORKSPACE_TOO_SMALL, "%s: staging needs at least 4096 bytes", fn);
  if (n == 0) return QLORA_OK;
  if ((st = check_ptr(param, "param", fn)) || (st = check_ptr(grad, "grad", fn)) ||
      (st = check_ptr(exp_avg, "exp_avg", fn)) || (st = check_ptr(exp_avg_sq, "exp_avg_sq", fn)) ||
      (st = check_ptr(staging, "staging", fn)))
    return st;
  if (param_bf16 && !aligned16(param_bf16)) return fail(QLORA_ERR_MISALIGNED, "%s: param_bf16 not 16-byte aligned", fn);
  if (grad_scale && !aligned16(grad_scale))
    return fail(QLORA_ERR_MISALIGNED, "%s: grad_scale not 16-byte aligned", fn);
  const hipError_t e =
      launch_adamw_paged(param, (uint16_t*)param_bf16, (const uint16_t*)grad, exp_avg, exp_avg_sq, n, grad_scale, lr,
                         beta1, beta2, eps, weight_decay, step, (float*)staging, chunk, (hipStream_t)stream,
                         (hipStream_t)copy_stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}

int qlora_adamw_step(float* param, void* param_bf16, const void* grad, float* exp_avg, float* exp_avg_sq, int64_t n,
                     const float* grad_scale, float lr, float beta1, float beta2, float eps, float weight_decay,
                     int32_t step, void* stream) {
  static const char* fn = "qlora_adamw_step";
  int st;
  if (n < 0) return fail(QLORA_ERR_INVALID_ARG, "%s: n < 0", fn);
  if (step < 1) return fail(QLORA_ERR_INVALID_ARG, "%s: step counts from 1", fn);
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f))
    return fail(QLORA_ERR_INVALID_ARG, "%s: betas must be in [0, 1)", fn);
  if (!(eps > 0.0f) || !(lr >= 0.0f) || !(weight_decay >= 0.0f))
    return fail(QLORA_ERR_INVALID_ARG, "%s: need eps > 0, lr >= 0, weight_decay >= 0", fn);
  if (n == 0) return QLORA_OK;
  if ((st = check_ptr(param, "param", fn)) || (st = check_ptr(grad, "grad", fn)) ||
      (st = check_ptr(exp_avg, "exp_avg", fn)) || (st = check_ptr(exp_avg_sq, "exp_avg_sq", fn)))
    return st;
  if (param_bf16 && !aligned16(param_bf16)) return fail(QLORA_ERR_MISALIGNED, "%s: param_bf16 not 16-byte aligned", fn);
  if (grad_scale && !aligned16(grad_scale))
    return fail(QLORA_ERR_MISALIGNED, "%s: grad_scale not 16-byte aligned", fn);
  const hipError_t e = launch_adamw(param, (uint16_t*)param_bf16, (const uint16_t*)grad, exp_avg, exp_avg_sq, n,
                                    grad_scale, lr, beta1, beta2, eps, weight_decay, step, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, fn);
  return QLORA_OK;
}

}  // extern "C"
