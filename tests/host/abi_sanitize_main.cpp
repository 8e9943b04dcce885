// CPU-only driver of the C ABI for the sanitizer build (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code): argument validation, the
// workspace and storage size arithmetic and the host planning, with the
// kernel launchers replaced by stubs that check every workspace region a
// kernel would write (launch_stubs.cpp).  Pointers are fake, 16-byte aligned
// addresses that are never dereferenced.  Prints "ok" and exits 0 when every
// expectation holds.
#include <stdio.h>
#include <string.h>

#include "launch_stubs.h"
#include "qlora_nf4.h"

static int fails = 0;
#define EXPECT(cond)                                                               \
  do {                                                                             \
    if (!(cond)) {                                                                 \
      fprintf(stderr, "FAIL line %d: %s (%s)\n", __LINE__, #cond, qlora_last_error()); \
      ++fails;                                                                     \
    }                                                                              \
  } while (0)

static void* P(uintptr_t a) { return (void*)a; }
static const uintptr_t kWs = (uintptr_t)1 << 44;   // fake workspace base
static const uintptr_t kBuf = (uintptr_t)1 << 40;  // fake caller buffers (far below the workspace)

static qlora_nf4_t desc(int64_t rows, int64_t cols, int dq, int ct) {
  qlora_nf4_t d;
  memset(&d, 0, sizeof(d));
  d.rows = rows;
  d.cols = cols;
  d.blocksize = 64;
  d.blocksize2 = 256;
  d.double_quant = dq;
  d.code_type = ct;
  d.codes = (uint8_t*)P(kBuf + 0x1000);
  d.absmax_q = (uint8_t*)P(kBuf + 0x2000);
  d.absmax = (float*)P(kBuf + 0x3000);
  d.scale2 = (float*)P(kBuf + 0x4000);
  d.offset = (float*)P(kBuf + 0x5000);
  return d;
}

static void use_ws(int64_t bytes) {
  stub::ws_lo = kWs;
  stub::ws_hi = kWs + (uintptr_t)bytes;
}

static void linear_case(int64_t M, int64_t N, int64_t K, int r, int ct) {
  int64_t fb = -1, bb = -1;
  EXPECT(qlora_linear_workspace(M, N, K, r, &fb, &bb) == QLORA_OK);
  EXPECT(fb >= 0 && bb >= 0);
  const qlora_nf4_t d = desc(N, K, 1, ct);
  void *X = P(kBuf + 0x10000), *A = P(kBuf + 0x20000), *B = P(kBuf + 0x30000), *Y = P(kBuf + 0x40000);
  void *XA = P(kBuf + 0x50000), *dY = P(kBuf + 0x60000), *dX = P(kBuf + 0x70000), *dA = P(kBuf + 0x80000);
  void *dB = P(kBuf + 0x90000), *keep = P(kBuf + 0xA0000);
  const float s = 16.0f / r;
  use_ws(fb);
  EXPECT(qlora_linear_fwd(X, M, &d, A, B, r, s, Y, XA, P(kWs), fb, nullptr) == QLORA_OK);
  EXPECT(qlora_linear_fwd_dropout(X, M, &d, A, B, r, s, keep, 0.1f, Y, nullptr, P(kWs), fb, nullptr) == QLORA_OK);
  if (M > 0) EXPECT(qlora_linear_fwd(X, M, &d, A, B, r, s, Y, XA, P(kWs), fb - 1, nullptr) ==
                    QLORA_ERR_WORKSPACE_TOO_SMALL);
  use_ws(bb);
  for (int acc = 0; acc <= 1; ++acc) {
    EXPECT(qlora_linear_bwd(dY, X, XA, M, &d, A, B, r, s, dX, dA, dB, acc, P(kWs), bb, nullptr) == QLORA_OK);
    EXPECT(qlora_linear_bwd(dY, X, nullptr, M, &d, A, B, r, s, nullptr, dA, dB, acc, P(kWs), bb, nullptr) ==
           QLORA_OK);
    EXPECT(qlora_linear_bwd_dropout(dY, X, nullptr, M, &d, A, B, r, s, keep, 0.05f, dX, dA, dB, acc, P(kWs), bb,
                                    nullptr) == QLORA_OK);
  }
  if (M > 0) EXPECT(qlora_linear_bwd(dY, X, XA, M, &d, A, B, r, s, dX, dA, dB, 0, P(kWs), bb - 1, nullptr) ==
                    QLORA_ERR_WORKSPACE_TOO_SMALL);
}

static void quant_case(int64_t rows, int64_t cols, int ct) {
  for (int dq = 0; dq <= 1; ++dq) {
    const qlora_nf4_t d = desc(rows, cols, dq, ct);
    int64_t ws = -1, bytes[5];
    EXPECT(qlora_nf4_quantize_workspace(rows * cols, dq, &ws) == QLORA_OK && ws >= 0);
    EXPECT(qlora_storage_bytes(rows * cols, dq, ct, bytes) == QLORA_OK);
    use_ws(ws);
    for (int dt = 0; dt <= 1; ++dt)
      EXPECT(qlora_nf4_quantize(P(kBuf + 0xB0000), dt, &d, ws ? P(kWs) : nullptr, ws, nullptr) == QLORA_OK);
    if (ws > 0) EXPECT(qlora_nf4_quantize(P(kBuf + 0xB0000), 0, &d, P(kWs), ws - 1, nullptr) ==
                       QLORA_ERR_WORKSPACE_TOO_SMALL);
    for (int dt = 0; dt <= 1; ++dt) EXPECT(qlora_nf4_dequantize(&d, P(kBuf + 0xC0000), dt, nullptr) == QLORA_OK);
  }
}

int main() {
  // the workload shapes, ragged and tiny ones, every code type of the linear
  const int64_t shapes[][4] = {{16, 256, 256, 8},      {4096, 4096, 4096, 64},   {2048, 11008, 4096, 64},
                               {2048, 4096, 11008, 64}, {8192, 22016, 8192, 64},  {8192, 8192, 22016, 64},
                               {1, 8192, 22016, 64},    {4, 8192, 22016, 64},     {16, 8192, 22016, 64},
                               {17, 128, 704, 100},     {200, 192, 320, 8},       {1, 64, 64, 1},
                               {300, 256, 192, 256},    {0, 256, 256, 8},         {1 << 20, 64, 64, 17},
                               {129, 640, 256, 17},     {5, 256, 64 * 12, 256},   {65536, 64, 64 * 1000, 3}};
  for (const auto& sh : shapes)
    for (int ct : {0, 1, 4}) linear_case(sh[0], sh[1], sh[2], (int)sh[3], ct);
  // quantisation sizes: tiny, ragged tails, the workload matrices
  const int64_t qs[][2] = {{1, 1},       {1, 63},      {1, 64},       {3, 65},      {256, 256}, {1, 16384 * 3 + 5},
                           {4096, 4096}, {11008, 4096}, {22016, 8192}, {7, 1 << 20}};
  for (const auto& q : qs)
    for (int ct = 0; ct <= 4; ++ct) quant_case(q[0], q[1], ct);
  // batched quantisation of every quantisation size at once (and a
  // mismatched batch)
  for (int ct = 0; ct <= 4; ++ct) {
    for (int dq = 0; dq <= 1; ++dq) {
      const int n = (int)(sizeof(qs) / sizeof(qs[0]));
      qlora_nf4_t ds[16];
      const void* ws_ptrs[16];
      for (int i = 0; i < n; ++i) {
        ds[i] = desc(qs[i][0], qs[i][1], dq, ct);
        ws_ptrs[i] = P(kBuf + 0xD0000 + 0x1000 * i);
      }
      int64_t need = -1;
      EXPECT(qlora_nf4_quantize_batched_workspace(ds, n, &need) == QLORA_OK && need >= 0);
      use_ws(need);
      EXPECT(qlora_nf4_quantize_batched(ws_ptrs, 0, ds, n, need ? P(kWs) : nullptr, need, nullptr) == QLORA_OK);
      if (need > 0) EXPECT(qlora_nf4_quantize_batched(ws_ptrs, 0, ds, n, P(kWs), need - 1, nullptr) ==
                           QLORA_ERR_WORKSPACE_TOO_SMALL);
      ds[1].code_type = (ct + 1) % 5;
      EXPECT(qlora_nf4_quantize_batched(ws_ptrs, 0, ds, n, P(kWs), need, nullptr) == QLORA_ERR_INVALID_ARG);
    }
  }
  // storage and workspace queries at the size limits
  int64_t bytes[5], ws;
  EXPECT(qlora_nf4_storage_bytes(((int64_t)1 << 37) - 1, 1, bytes) == QLORA_OK);
  EXPECT(qlora_nf4_storage_bytes((int64_t)1 << 37, 1, bytes) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_storage_bytes(((int64_t)1 << 37) - 1, 0, 4, bytes) == QLORA_OK);
  EXPECT(qlora_nf4_quantize_workspace(((int64_t)1 << 37) - 1, 1, &ws) == QLORA_OK);
  EXPECT(qlora_nf4_quantize_workspace(-1, 1, &ws) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_linear_workspace(-1, 64, 64, 8, &ws, &ws) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_linear_workspace(((int64_t)1 << 37) / 64, 64, 64, 256, &ws, &ws) == QLORA_OK);
  // a descriptor beyond the element limit, and bad descriptors
  qlora_nf4_t big = desc((int64_t)1 << 20, (int64_t)1 << 20, 1, 0);
  EXPECT(qlora_nf4_quantize(P(kBuf), 0, &big, P(kWs), 1 << 30, nullptr) == QLORA_ERR_INVALID_ARG);
  qlora_nf4_t neg = desc(-1, 64, 1, 0);
  EXPECT(qlora_nf4_dequantize(&neg, P(kBuf), 0, nullptr) == QLORA_ERR_INVALID_ARG);
  qlora_nf4_t huge_m = desc(64, 64, 1, 0);
  int64_t fb, bb;
  EXPECT(qlora_linear_workspace(8, 64, 64, 8, &fb, &bb) == QLORA_OK);
  EXPECT(qlora_linear_fwd(P(kBuf), (int64_t)1 << 40, &huge_m, P(kBuf), P(kBuf), 8, 1.0f, P(kBuf), nullptr, P(kWs),
                          fb, nullptr) == QLORA_ERR_INVALID_ARG);
  // the codebooks and every status text
  float cb[256];
  for (int ct = 0; ct <= 4; ++ct) EXPECT(qlora_codebook(ct, cb) == QLORA_OK);
  EXPECT(qlora_codebook(5, cb) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_nf4_codebook(cb) == QLORA_OK && cb[7] == 0.0f && cb[15] == 1.0f);
  for (int st = -7; st <= 0; ++st) EXPECT(qlora_status_string(st) != nullptr);
  // the optimizer step and its clip scale
  for (int64_t n : {(int64_t)0, (int64_t)1, (int64_t)1000, (int64_t)524288, (int64_t)1 << 28}) {
    EXPECT(qlora_clip_scale_workspace(n, &ws) == QLORA_OK);
    use_ws(ws);
    EXPECT(qlora_clip_scale(n ? P(kBuf) : nullptr, n, 0.3f, (float*)P(kBuf + 0x100), P(kWs), ws, nullptr) ==
           QLORA_OK);
    EXPECT(qlora_adamw_step((float*)P(kBuf), nullptr, P(kBuf + 0x1000), (float*)P(kBuf + 0x2000),
                            (float*)P(kBuf + 0x3000), n, nullptr, 1e-4f, 0.9f, 0.999f, 1e-8f, 0.0f, 1, nullptr) ==
           QLORA_OK);
  }
  // the dropout mask generator
  EXPECT(qlora_dropout_mask(1, 2, 4096, 4096, 0.1f, P(kBuf), nullptr) == QLORA_OK);
  EXPECT(qlora_dropout_mask(~0ull, ~0ull, 3, 8, 0.999f, P(kBuf), nullptr) == QLORA_OK);
  EXPECT(qlora_dropout_mask(1, 2, 0, 64, 0.1f, nullptr, nullptr) == QLORA_OK);
  EXPECT(qlora_dropout_mask(1, 2, 4, 60, 0.1f, P(kBuf), nullptr) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_dropout_mask(1, 2, 4, 64, 1.0f, P(kBuf), nullptr) == QLORA_ERR_INVALID_ARG);
  EXPECT(qlora_dropout_mask(1, 2, (int64_t)1 << 40, 64, 0.1f, P(kBuf), nullptr) == QLORA_ERR_INVALID_ARG);
  // the paged optimizer step: staging sizes around the minimum
  for (int64_t sb : {(int64_t)4095, (int64_t)4096, (int64_t)16385, (int64_t)1 << 20, (int64_t)3 * 4096 + 7}) {
    use_ws(sb);
    const int want = sb >= 4096 ? QLORA_OK : QLORA_ERR_WORKSPACE_TOO_SMALL;
    EXPECT(qlora_adamw_step_paged((float*)P(kBuf), nullptr, P(kBuf + 0x1000), (float*)P(kBuf + 0x2000),
                                  (float*)P(kBuf + 0x3000), 100003, nullptr, 1e-4f, 0.9f, 0.999f, 1e-8f, 0.0f, 1,
                                  P(kWs), sb, nullptr, nullptr) == want);
  }
  EXPECT(stub::calls > 0);
  EXPECT(stub::bad == 0);
  if (fails) {
    fprintf(stderr, "%d expectation(s) failed\n", fails);
    return 1;
  }
  printf("ok %d launches\n", stub::calls);
  return 0;
}
