// Stand-ins for the kernel launchers of launch.h, for a CPU-only build of the
// C ABI and the host planning (no GPU, no device code).  Each stub checks
// that every buffer region the real kernel would write either lies wholly
// inside the workspace the caller passed or wholly outside it (a caller
// buffer), and counts its calls.
#include "launch_stubs.h"

#include <stdio.h>

namespace stub {
uintptr_t ws_lo = 0, ws_hi = 0;
int calls = 0, bad = 0;

void region(const void* p, int64_t bytes, const char* what) {
  if (!p || bytes <= 0) return;
  const uintptr_t a = (uintptr_t)p, b = a + (uintptr_t)bytes;
  const bool inside = a >= ws_lo && b <= ws_hi;
  const bool outside = b <= ws_lo || a >= ws_hi;
  if (!inside && !outside) {
    ++bad;
    fprintf(stderr, "region %s [%#lx, %#lx) straddles the workspace [%#lx, %#lx)\n", what, (unsigned long)a,
            (unsigned long)b, (unsigned long)ws_lo, (unsigned long)ws_hi);
  }
}
}  // namespace stub

namespace qlora {
using stub::region;

hipError_t launch_quantize(const void*, bool, int64_t numel, int code_type, uint8_t* codes, float* c2,
                           uint64_t* partials, hipStream_t) {
  ++stub::calls;
  region(codes, code_type == CODE_INT8 ? numel : (numel + 1) / 2, "codes");
  region(c2, 4 * ((numel + 63) / 64), "c2");
  region(partials, 8 * (int64_t)kMeanDigits * quantize_parts(numel), "mean partials");
  return hipSuccess;
}
hipError_t launch_quantize_batched(const QuantJob* jobs, int count, bool, int code_type, bool dq, hipStream_t) {
  ++stub::calls;
  for (int i = 0; i < count; ++i) {
    const QuantJob& j = jobs[i];
    region(j.codes, code_type == CODE_INT8 ? j.numel : (j.numel + 1) / 2, "batched codes");
    region(j.c2, 4 * ((j.numel + 63) / 64), "batched c2");
    if (dq) region(j.partials, 8 * (int64_t)kMeanDigits * quantize_parts(j.numel), "batched mean partials");
  }
  return hipSuccess;
}
hipError_t launch_double_quant(const float* c2, int64_t nb, const uint64_t* partials, int parts, uint8_t* absmax_q,
                               float* scale2, float* offset, hipStream_t) {
  ++stub::calls;
  region(c2, 4 * nb, "c2 read");
  region(partials, 8 * (int64_t)kMeanDigits * parts, "mean partials read");
  region(absmax_q, nb, "absmax_q");
  region(scale2, 4 * ((nb + 255) / 256), "scale2");
  region(offset, 4, "offset");
  return hipSuccess;
}
hipError_t launch_dequantize(const uint8_t*, int64_t numel, int, bool, const uint8_t*, const float*, const float*,
                             const float*, void* out, bool out_bf16, hipStream_t) {
  ++stub::calls;
  region(out, numel * (out_bf16 ? 2 : 4), "dequantised out");
  return hipSuccess;
}
hipError_t launch_skinny(const uint16_t*, const uint16_t*, bool, int64_t M, int64_t Q, int64_t, float* part,
                         int splits, uint16_t* out1, uint16_t* out2, int64_t QP, float, float, const uint8_t*,
                         hipStream_t) {
  ++stub::calls;
  region(part, 4 * (int64_t)splits * M * QP, "skinny partials");
  region(out1, 2 * M * Q, "skinny out1");
  region(out2, 2 * M * QP, "skinny out2");
  return hipSuccess;
}
hipError_t launch_fwd_main(const uint16_t*, int64_t M, int64_t K, const uint8_t*, const DQParams& dq, int64_t N,
                           const uint16_t* XAs, const uint16_t*, int64_t, int64_t rp, uint16_t* Y, float* split_ws,
                           hipStream_t) {
  ++stub::calls;
  region(XAs, 2 * M * rp, "s*XA read");
  region(Y, 2 * M * N, "Y");
  region(split_ws, main_split_bytes(M, N, K), "fwd split tiles");
  return hipSuccess;
}
hipError_t launch_gemv(const uint16_t*, int64_t M, int64_t K, const uint8_t*, const DQParams&, int64_t N, float* part,
                       int splits, const uint16_t*, int64_t, int64_t rp, const uint8_t*, float* xpart, hipStream_t) {
  ++stub::calls;
  region(part, 4 * (int64_t)splits * M * N, "gemv partials");
  region(xpart, 4 * (int64_t)xa_chunks(K) * M * rp, "xa chunk partials");
  return hipSuccess;
}
hipError_t launch_xa_chunks(const uint16_t*, int64_t M, int64_t K, const uint16_t*, int64_t, int64_t rp,
                            const uint8_t*, float* xpart, hipStream_t) {
  ++stub::calls;
  region(xpart, 4 * (int64_t)xa_chunks(K) * M * rp, "xa chunk partials (recompute)");
  return hipSuccess;
}
hipError_t launch_gemv_reduce(const float* part, int splits, int64_t M, int64_t N, const float* xpart, int xsplits,
                              int64_t rp, float, float, const uint16_t*, int64_t r, uint16_t* Y, uint16_t* XA,
                              hipStream_t) {
  ++stub::calls;
  region(part, 4 * (int64_t)splits * M * N, "gemv partials read");
  region(xpart, 4 * (int64_t)xsplits * M * rp, "xa partials read");
  region(Y, 2 * M * N, "Y");
  region(XA, 2 * M * r, "XA");
  return hipSuccess;
}
hipError_t launch_xa_reduce(const float* xpart, int xsplits, int64_t M, int64_t rp, float, int64_t r, uint16_t* XA,
                            hipStream_t) {
  ++stub::calls;
  region(xpart, 4 * (int64_t)xsplits * M * rp, "xa partials read");
  region(XA, 2 * M * r, "recomputed XA");
  return hipSuccess;
}
hipError_t launch_bwd_dx(const uint16_t*, int64_t M, int64_t N, const uint8_t*, const DQParams& dq, int64_t K,
                         const uint16_t* Ts, const uint16_t*, int64_t, int64_t rp, uint16_t* dX, float* split_ws,
                         const uint8_t*, float, hipStream_t) {
  ++stub::calls;
  region(Ts, 2 * M * rp, "s*T read");
  region(dX, 2 * M * K, "dX");
  region(split_ws, main_split_bytes(M, K, N), "bwd split tiles");
  return hipSuccess;
}
hipError_t launch_tn_pair(const uint16_t*, int64_t, int64_t Pa, const uint8_t*, const uint16_t*, int64_t, int64_t Qa,
                          float* part_a, int splits_a, uint16_t* out_a, float, const uint16_t*, int64_t, int64_t Pb,
                          const uint16_t*, int64_t, int64_t Qb, float* part_b, int splits_b, uint16_t* out_b, float,
                          int64_t, bool, hipStream_t) {
  ++stub::calls;
  region(part_a, 4 * (int64_t)splits_a * Pa * Qa, "dA partials");
  region(part_b, 4 * (int64_t)splits_b * Pb * Qb, "dB^T partials");
  region(out_a, 2 * Pa * Qa, "dA");
  region(out_b, 2 * Pb * Qb, "dB");
  return hipSuccess;
}
hipError_t launch_fill_zero_u16(uint16_t* dst, int64_t n, hipStream_t) {
  ++stub::calls;
  region(dst, 2 * n, "zero fill");
  return hipSuccess;
}
hipError_t launch_clip_scale(const uint16_t*, int64_t n, float, float* scale, double* partials, hipStream_t) {
  ++stub::calls;
  region(scale, 4, "clip scale");
  region(partials, 8 * (int64_t)clip_parts(n), "norm partials");
  return hipSuccess;
}
hipError_t launch_dropout_mask(uint8_t* mask, int64_t nbytes, uint64_t, uint64_t, uint32_t, hipStream_t) {
  ++stub::calls;
  region(mask, nbytes, "dropout mask");
  return hipSuccess;
}
hipError_t launch_adamw(float*, uint16_t*, const uint16_t*, float*, float*, int64_t, const float*, float, float, float,
                        float, float, int, hipStream_t) {
  ++stub::calls;
  return hipSuccess;
}
hipError_t launch_adamw_paged(float*, uint16_t*, const uint16_t*, float*, float*, int64_t, const float*, float, float,
                              float, float, float, int, float* staging, int64_t chunk, hipStream_t, hipStream_t) {
  ++stub::calls;
  region(staging, 16 * chunk, "paged optimizer staging");
  return chunk > 0 && chunk % 256 == 0 ? hipSuccess : hipErrorInvalidValue;
}
}  // namespace qlora
