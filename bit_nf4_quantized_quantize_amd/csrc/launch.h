// Internal host-side launchers shared between the kernel files and the C ABI.
// Every launcher only enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "codebooks.h"

namespace qlora {

// Quantisation lookup: x in [-1, 1] goes to bucket b = round(16 x + 16)
// (0..32, ties to even), which covers [(b - 1/2)/16 - 1, (b + 1/2)/16 - 1].
// For x in bucket b, code(x) = base[b] + (x > thr[b]); thr[b] is the one
// decision threshold (midpoint of two adjacent NF4 values, rounded toward
// -inf to fp32) inside the bucket, or +inf when the bucket holds none.
constexpr int kBuckets = 33;
struct QuantTable {
  float thr[kBuckets];
  uint32_t base[kBuckets];
};

struct NF4Values {
  float v[16];
};

// The codebooks other than NF4 are quantised through a finer table built by
// each quantisation workgroup: kFineBuckets buckets of width 1/kFineScale,
// b = round(kFineScale x + kFineScale), each holding at most one decision
// point; an entry gives the threshold and the codes below and above it.
// CodeSpec carries what the kernel needs to build it: the exact midpoints
// between consecutive distinct values (fp64), the same rounded toward -inf to
// fp32, and the code of each distinct value in increasing order.
constexpr int kFineScale = 512;
constexpr int kFineBuckets = 2 * kFineScale + 1;
struct CodeSpec {
  double mid[15];
  float thr[15];
  uint32_t rank_code[16];
  int nmid;
};

// Int8 tables: value[c] of code byte c, and the 254 decision thresholds
// between the levels k and k + 1 (k = -127 .. 126) at thr[k + 127]: the
// exact midpoint of the two fp32 values rounded toward -inf, so that
// "x > thr" equals "x > midpoint" for every fp32 x.
struct Int8Tables {
  float value[256];
  float thr[254];
};
const Int8Tables& int8_tables();

// Library copies of the codebook values, the NF4 quantisation table and the
// spec of the finer table of another codebook.
const NF4Values& code_values(int code_type);
inline const NF4Values& nf4_values() { return code_values(CODE_NF4); }
const QuantTable& quant_table();
const CodeSpec& code_spec(int code_type);
// False when the quantisation table of `code_type` could not be built (a
// bucket would hold two decision points; never the case for the built-in
// codebooks).
bool quant_tables_ok(int code_type);

// Quantisation writes the codes and the fp32 block absmax c2; with
// `partials` it also writes, per workgroup, the exact sum of its c2 as
// kMeanDigits 32-bit digits in 64-bit counters (quantize_parts(numel)
// workgroups; digit k of workgroup p at partials[k * parts + p]).  Double
// quantisation then divides the total by nb for the mean
// and encodes the constants.
int quantize_parts(int64_t numel);
// A tensor's share of a batched launch: workgroups of at least
// kQuantBatchUnits grid units each (the batch fills the chip by itself, so
// every workgroup keeps a longer stream in flight); never more workgroups
// than quantize_parts, so the workspace of a single call holds its partials.
int quantize_parts_batched(int64_t numel);
constexpr int kMeanDigits = 10;  // 32-bit digits of the exact fixed-point sum
constexpr int kQuantMaxParts = 256;          // quantisation workgroups (and exact-sum partials) at most
constexpr int64_t kQuantGridUnit = 16384;    // weights per workgroup when sizing that grid
constexpr int64_t kQuantBatchUnits = 16;     // grid units per workgroup at least, in a batched launch

// Tiling constants the kernels and the host planning share.
constexpr int kCUs = 256;        // MI355X compute units
constexpr int SK_BK = 128;       // reduction indices per iteration of the skinny products
constexpr int TN_BK = 128;       // tokens per iteration of the token reductions
constexpr int G3_ROWS = 256;     // weight rows per workgroup of the small-token forward
constexpr int G3_CB = 4;         // 64-blocks per chunk of the small-token forward
constexpr int kOptThreads = 256; // threads per workgroup of the optimizer kernels
constexpr int kOptMaxParts = 256;// partial sums of the gradient norm at most

// Main-GEMM tile choice.  The 256 x 256 kernels run one workgroup per CU;
// their tiles go in rounds of kCUs, and when the last round would leave CUs
// idle its R tiles are cut along the reduction into `split` ranges
// (split * R <= kCUs) whose fp32 partial tiles a fixup pass adds.  The
// 128-wide generic tiles remain for shapes where even that leaves most of
// the chip idle.
struct SplitPlan {
  int tiles, full, split;  // split == 1: no split units
  int64_t units() const { return full + (int64_t)(tiles - full) * split; }
  int64_t part_floats() const { return split > 1 ? (int64_t)(tiles - full) * split * 65536 : 0; }
};
SplitPlan plan_256(int64_t M, int64_t ncols, int64_t L);
enum MainTile { T256x256 = 0, T256x128 = 1, T128x128 = 2 };
MainTile pick_tile(int64_t M, int64_t ncols, int64_t L);

hipError_t launch_quantize(const void* w, bool w_bf16, int64_t numel, int code_type, uint8_t* codes, float* c2,
                           uint64_t* partials, hipStream_t stream);
hipError_t launch_double_quant(const float* c2, int64_t nb, const uint64_t* partials, int parts,
                               uint8_t* absmax_q, float* scale2, float* offset, hipStream_t stream);
// Quantisation (and, with dq, double quantisation) of `count` tensors of
// one input dtype and code type: one quantise and one encode launch per
// kQuantBatch tensors, each tensor coded exactly as by its own launches.
// c2 and partials are the tensor's workspace regions (as for
// launch_quantize and launch_double_quant).
constexpr int kQuantBatch = 32;
struct QuantJob {
  const void* w;
  int64_t numel;
  uint8_t* codes;
  float* c2;
  uint64_t* partials;
  uint8_t* absmax_q;
  float* scale2;
  float* offset;
};
hipError_t launch_quantize_batched(const QuantJob* jobs, int count, bool w_bf16, int code_type, bool dq,
                                   hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* codes, int64_t numel, int code_type, bool dq, const uint8_t* absmax_q,
                             const float* absmax, const float* scale2, const float* offset,
                             void* out, bool out_bf16, hipStream_t stream);

// Dequantisation parameters of a weight as the GEMM kernels take them.
struct DQParams {
  const uint8_t* absmax_q;  // double_quant: E4M3 bytes per block
  const float* absmax;      // !double_quant: fp32 absmax per block
  const float* scale2;      // double_quant: per 256 blocks
  const float* offset;      // double_quant: mean mu
  int double_quant;
  int code_type;            // CodeType of the codes
};

// Linear-layer building blocks (all bf16 matrices row-major).
//
// Skinny product C[M, Q] = U[M, L] * V, V either [L, Q] (v_is_lq) or
// [Q, L]; the reduction is split into `splits` chunks of fp32 partials
// part[splits][M][QP], then out1 [M, Q] = bf16(scale1 * C) and out2 [M, QP]
// = bf16(alpha * C), zero in columns [Q, QP), each when given.  With out1
// and out2 both null only the partials are written.  With `keep` (a bit mask
// [M, L/8], bit j of byte (m, c) for U[m, 8c + j]; L % 8 == 0) the elements
// of U whose bit is clear count as zero (LoRA dropout).
int skinny_splits(int64_t M, int64_t Q, int64_t L);
hipError_t launch_skinny(const uint16_t* U, const uint16_t* V, bool v_is_lq, int64_t M, int64_t Q, int64_t L,
                         float* part, int splits, uint16_t* out1, uint16_t* out2, int64_t QP, float alpha,
                         float scale1, const uint8_t* keep, hipStream_t stream);
// Workspace bytes of the fp32 partial tiles a main product [M, ncols] with
// reduction length L uses (0 when no tile is split).
int64_t main_split_bytes(int64_t M, int64_t ncols, int64_t L);
// Fused forward: Y = X * W_bf16^T + XAs * B_pad (XAs [M, rp]; B [r, N], rows >= r as zero).
hipError_t launch_fwd_main(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes,
                           const DQParams& dq, int64_t N, const uint16_t* XAs, const uint16_t* B,
                           int64_t r, int64_t rp, uint16_t* Y, float* split_ws, hipStream_t stream);
// Small-token forward (1 <= M <= kGemvMaxM, N % 4 == 0): launch_gemv writes
// fp32 partials part[splits][M][N] of X * W_bf16^T over reduction splits
// and, per 256-wide reduction chunk, the partials xpart[xa_chunks(K)][M][rp]
// of C = X A (X keep-masked when `keep` is given; rp <= 256);
// launch_gemv_reduce adds both sets and writes Y = bf16(sum + bf16(alpha C)
// * B) and, when XA is given, XA = bf16(scale1 C) [M, r].  launch_xa_chunks
// writes the same X A partials alone (the backward's recomputation).
constexpr int kGemvMaxM = 16;
constexpr int kXaChunk = 256;  // reduction indices per X A partial slice
int gemv_splits(int64_t M, int64_t N, int64_t K);
int xa_chunks(int64_t K);      // ceil(K / kXaChunk)
hipError_t launch_gemv(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, const DQParams& dq, int64_t N,
                       float* part, int splits, const uint16_t* A, int64_t r, int64_t rp, const uint8_t* keep,
                       float* xpart, hipStream_t stream);
hipError_t launch_xa_chunks(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int64_t r, int64_t rp,
                            const uint8_t* keep, float* xpart, hipStream_t stream);
// XA [M, r] = bf16(scale1 C) from the skinny partials of C = X A exactly as
// launch_gemv_reduce forms it (the backward recomputes the small-token
// forward's XA with it, bit for bit).
hipError_t launch_xa_reduce(const float* xpart, int xsplits, int64_t M, int64_t rp, float scale1, int64_t r,
                            uint16_t* XA, hipStream_t stream);
hipError_t launch_gemv_reduce(const float* part, int splits, int64_t M, int64_t N, const float* xpart, int xsplits,
                              int64_t rp, float alpha, float scale1, const uint16_t* B, int64_t r, uint16_t* Y,
                              uint16_t* XA, hipStream_t stream);
// Fused input gradient: dX = dY * W_bf16 + Ts * A_pad^T (Ts [M, rp]; A [K, r]);
// with `keep` (bit mask [M, K/8] as for launch_skinny) the adapter term is
// multiplied by keep_scale where the bit is set and dropped where it is clear.
hipError_t launch_bwd_dx(const uint16_t* dY, int64_t M, int64_t N, const uint8_t* codes,
                         const DQParams& dq, int64_t K, const uint16_t* Ts, const uint16_t* A,
                         int64_t r, int64_t rp, uint16_t* dX, float* split_ws, const uint8_t* keep,
                         float keep_scale, hipStream_t stream);
// Two token reductions, one launch for both products and one for both
// epilogues: C_a [Pa, Qa] = U_a[M, Pa]^T * V_a[M, Qa] and C_b likewise
// (leading dimensions ld*), fp32 partials part_x [splits_x][P][Q], then
// out_a [Pa, Qa] = bf16(alpha_a * sum) and out_b = bf16(alpha_b * sum) written
// transposed, [Qb, Pb]; with `accumulate` the bf16 outputs are added to:
// out = bf16(out + alpha * sum).  keep_a (optional, bit mask [M, ldua/8])
// zeroes elements of U_a as for launch_skinny.
int tn_splits(int64_t M, int64_t P, int64_t Q);
hipError_t launch_tn_pair(const uint16_t* Ua, int64_t ldua, int64_t Pa, const uint8_t* keep_a, const uint16_t* Va,
                          int64_t ldva, int64_t Qa, float* part_a, int splits_a, uint16_t* out_a, float alpha_a,
                          const uint16_t* Ub,
                          int64_t ldub, int64_t Pb, const uint16_t* Vb, int64_t ldvb, int64_t Qb, float* part_b,
                          int splits_b, uint16_t* out_b, float alpha_b, int64_t M, bool accumulate,
                          hipStream_t stream);
hipError_t launch_fill_zero_u16(uint16_t* dst, int64_t n, hipStream_t stream);

// LoRA dropout keep mask [nbytes] (packed, bit j of byte b for element
// 8 b + j in row-major order) from Philox4x64-10: key (seed, 0), counter
// (b, offset, 0, 0), bit j set iff 32-bit word j of the output >= T.
hipError_t launch_dropout_mask(uint8_t* mask, int64_t nbytes, uint64_t seed, uint64_t offset, uint32_t T,
                               hipStream_t stream);

// Sets the calling thread's qlora_last_error() message and returns status.
int record_failure(int status, const char* msg);

// LoRA optimizer step.  launch_clip_scale writes scale = min(1, max_norm /
// (||g||_2 + 1e-6)) for the bf16 gradient g [n], using clip_parts(n) fp64
// partial sums; launch_adamw applies one AdamW step (bias corrections for
// `step` >= 1, gradient times *gscale when given) to fp32 parameters p and
// states m, v, and writes a bf16 copy of p when p_bf16 is given.
int clip_parts(int64_t n);
hipError_t launch_clip_scale(const uint16_t* g, int64_t n, float max_norm, float* scale, double* partials,
                             hipStream_t stream);
hipError_t launch_adamw(float* p, uint16_t* p_bf16, const uint16_t* g, float* m, float* v, int64_t n,
                        const float* gscale, float lr, float beta1, float beta2, float eps, float weight_decay,
                        int step, hipStream_t stream);
// The step with m, v in pinned host memory, paged through `staging`
// ([2][2][chunk] floats, chunk % 256 == 0) in chunks: copied in, updated by
// launch_adamw, copied back; copies on `copy` (if given and not `stream`),
// ordered against the updates by events.
hipError_t launch_adamw_paged(float* p, uint16_t* p_bf16, const uint16_t* g, float* m_host, float* v_host, int64_t n,
                              const float* gscale, float lr, float beta1, float beta2, float eps, float weight_decay,
                              int step, float* staging, int64_t chunk, hipStream_t stream, hipStream_t copy);

}  // namespace qlora
