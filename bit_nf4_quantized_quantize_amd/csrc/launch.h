// Internal host-side launchers shared between the kernel files and the C ABI.
// Every launcher only enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

// Quantisation lookup: the [-1, 1] range cut into 32 buckets of width 1/16.
// For x in bucket b, code(x) = base[b] + (x > thr[b]); thr[b] is the one
// decision threshold (midpoint of two adjacent NF4 values, rounded toward
// -inf to fp32) inside the bucket, or +inf when the bucket holds none.
struct QuantTable {
  float thr[32];
  uint32_t base[32];
};

struct NF4Values {
  float v[16];
};

// Library copies of the NF4 values and the derived quantisation table.
const NF4Values& nf4_values();
const QuantTable& quant_table();

// Number of partial sums the exact-mean reduction uses for nb constants.
int dq_mean_parts(int64_t nb);
constexpr int kMeanDigits = 10;  // 32-bit digits of the exact fixed-point sum

hipError_t launch_quantize(const void* w, bool w_bf16, int64_t numel, uint8_t* codes, float* c2,
                           hipStream_t stream);
hipError_t launch_double_quant(const float* c2, int64_t nb, uint64_t* partials, uint8_t* absmax_q,
                               float* scale2, float* offset, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* codes, int64_t numel, bool dq, const uint8_t* absmax_q,
                             const float* absmax, const float* scale2, const float* offset,
                             void* out, bool out_bf16, hipStream_t stream);

// Dequantisation parameters of a weight as the GEMM kernels take them.
struct DQParams {
  const uint8_t* absmax_q;  // double_quant: E4M3 bytes per block
  const float* absmax;      // !double_quant: fp32 absmax per block
  const float* scale2;      // double_quant: per 256 blocks
  const float* offset;      // double_quant: mean mu
  int double_quant;
};

// Linear-layer building blocks (all bf16 matrices row-major).
hipError_t launch_pad_copy(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst,
                           int64_t cols_pad, hipStream_t stream);
hipError_t launch_transpose_pad(const uint16_t* src, int64_t src_rows, int64_t src_cols,
                                uint16_t* dst, int64_t cols_pad, hipStream_t stream);
// C[M, Q] = U[M, L] * V[Q, L]^T; out1 (ld1 = Q, optional) = bf16(C),
// out2 (ld2) = bf16(alpha * C) with zeros in columns [Q, ld2).
hipError_t launch_gemm_nt(const uint16_t* U, const uint16_t* V, int64_t M, int64_t Q, int64_t L,
                          uint16_t* out1, uint16_t* out2, int64_t ld2, float alpha,
                          hipStream_t stream);
// Fused forward: Y = X * What^T + XAs * Bt^T (XAs [M, rp], Bt [N, rp]).
hipError_t launch_fwd_main(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes,
                           const DQParams& dq, int64_t N, const uint16_t* XAs, const uint16_t* Bt,
                           int64_t rp, uint16_t* Y, hipStream_t stream);
// Fused input gradient: dX = dY * What + Ts * Ap^T (Ts [M, rp], Ap [K, rp]).
hipError_t launch_bwd_dx(const uint16_t* dY, int64_t M, int64_t N, const uint8_t* codes,
                         const DQParams& dq, int64_t K, const uint16_t* Ts, const uint16_t* Ap,
                         int64_t rp, uint16_t* dX, hipStream_t stream);
// Split-M reduction C[P, Q] = U[M, P]^T * V[M, Q]: fp32 partials then
// out (bf16 [P, Q]) = bf16(alpha * sum of partials).
int tn_splits(int64_t M, int64_t P, int64_t Q);
// Only out[p][q] for p < Pout, q < Qout (ld Qout) is written.
hipError_t launch_gemm_tn(const uint16_t* U, const uint16_t* V, int64_t M, int64_t P, int64_t Q,
                          float* partials, int splits, uint16_t* out, int64_t Pout, int64_t Qout,
                          float alpha, hipStream_t stream);
hipError_t launch_fill_zero_u16(uint16_t* dst, int64_t n, hipStream_t stream);

}  // namespace qlora
