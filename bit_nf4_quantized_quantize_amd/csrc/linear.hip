// QLoRA linear layer over a frozen NF4 weight, forward and backward, gfx950.
//
// QLoRA (Dettmers et al., arXiv 2305.14314):
//   section 2 "Low-rank Adapters", Eq. 3: Y = XW + s X L1 L2;
//   section 3 "QLoRA", Eq. 5 and 6: W is doubleDequant(c1, c2, W^NF4), used
//     in BF16 for every product, forward and backward;
//   section 3 "QLoRA", paragraph after Eq. 6: only the adapter gradients are
//     computed (no dE/dW); the input gradient goes through the BF16 weight.
//
// The weight is [N, K] = [out, in] with 64-element NF4 blocks along K.  The
// two large products (Y = X W^T and dX = dY W) dequantise W tile by tile into
// LDS and run bf16 MFMA 32x32x16 with fp32 accumulation; the rank-r adapter
// terms ride along as extra reduction steps over zero-padded bf16 operands:
//   Y  = [X | s XA] [W ; B^T]^T        (reduction K + r)
//   dX = [dY | s T] [W ; A^T]          (reduction N + r)
// The skinny adapter products (XA, T, dA, dB) use the same MFMA tile.
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int NT = 256;  // threads per workgroup for every GEMM kernel here

// NF4 value of a code times the block constant, in fp32 (Eq. 6 outer
// dequant); contraction is irrelevant here (one multiply).
__device__ __forceinline__ float block_scale(const DQParams& dq, int64_t blk, float mu) {
  if (dq.double_quant) {
    const float prod = __fmul_rn(e4m3_decode(dq.absmax_q[blk]), dq.scale2[blk >> 8]);
    return __fadd_rn(prod, mu);  // two roundings, never fused
  }
  return dq.absmax[blk];
}

// 16 bytes of bf16 from global (zero when out of range).
__device__ __forceinline__ uint4 ld16(const uint16_t* p, bool ok) {
  return ok ? *reinterpret_cast<const uint4*>(p) : make_uint4(0, 0, 0, 0);
}
__device__ __forceinline__ void st16(__bf16* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Stage a 128 x 64 bf16 tile of a row-major matrix (rows r0.., cols c0..)
// into LDS [128][LDK]; rows >= nrows read as zero.  Two threads per row.
__device__ __forceinline__ void stage_rows(__bf16* s, const uint16_t* g, int64_t ld, int64_t r0,
                                           int64_t nrows, int64_t c0, int tid) {
  const int row = tid >> 1, half = tid & 1;
  const bool ok = r0 + row < nrows;
  const uint16_t* src = g + (ok ? (r0 + row) * ld + c0 + half * 32 : 0);
#pragma unroll
  for (int i = 0; i < 4; ++i) st16(s + row * LDK + half * 32 + i * 8, ld16(src + i * 8, ok));
}

// Expand 8 NF4 codes (one 32-bit word, element 0 in the low nibble) into 8
// bf16 values of NF4[code] * c, rounded to nearest-even.
__device__ __forceinline__ uint4 dequant8(uint32_t w, float c, const float* nf4) {
  uint4 o;
  o.x = pack_bf2(nf4[w & 0xF] * c, nf4[(w >> 4) & 0xF] * c);
  o.y = pack_bf2(nf4[(w >> 8) & 0xF] * c, nf4[(w >> 12) & 0xF] * c);
  o.z = pack_bf2(nf4[(w >> 16) & 0xF] * c, nf4[(w >> 20) & 0xF] * c);
  o.w = pack_bf2(nf4[(w >> 24) & 0xF] * c, nf4[(w >> 28) & 0xF] * c);
  return o;
}

// ----------------------------------------------------- forward main GEMM
// Tile 128 (M) x 128 (N); per k-step of 64 the weight tile is 128 rows of one
// NF4 block each.  Two threads per weight row, 32 codes (16 bytes) each.
__global__ __launch_bounds__(NT) void fwd_main_kernel(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                                      const uint8_t* __restrict__ codes, DQParams dq, int64_t N,
                                                      const uint16_t* __restrict__ XAs,
                                                      const uint16_t* __restrict__ Bt, int64_t rp,
                                                      uint16_t* __restrict__ Y, NF4Values nf4v) {
  __shared__ __bf16 sA[TM * LDK];
  __shared__ __bf16 sB[TN * LDK];
  __shared__ float s_nf4[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  if (tid < 16) s_nf4[tid] = nf4v.v[tid];
  const float mu = dq.double_quant ? *dq.offset : 0.0f;
  __syncthreads();

  Acc22 acc;
  acc_zero(acc);
  const int wrow = tid >> 1, whalf = tid & 1;
  const int64_t n = n0 + wrow;
  const bool nok = n < N;
  const int64_t kblocks = K >> 6;

  for (int64_t kt = 0; kt < kblocks; ++kt) {
    stage_rows(sA, X, K, m0, M, kt * 64, tid);
    {
      uint4 cw = make_uint4(0, 0, 0, 0);
      float c = 0.0f;
      if (nok) {
        cw = *reinterpret_cast<const uint4*>(codes + ((n * K + kt * 64 + whalf * 32) >> 1));
        c = block_scale(dq, n * kblocks + kt, mu);
      }
      __bf16* dst = sB + wrow * LDK + whalf * 32;
      st16(dst + 0, dequant8(cw.x, c, s_nf4));
      st16(dst + 8, dequant8(cw.y, c, s_nf4));
      st16(dst + 16, dequant8(cw.z, c, s_nf4));
      st16(dst + 24, dequant8(cw.w, c, s_nf4));
    }
    __syncthreads();
    mma_128x128x64(sA, sB, acc, wm, wn, lane);
    __syncthreads();
  }
  for (int64_t jt = 0; jt < rp; jt += 64) {
    stage_rows(sA, XAs, rp, m0, M, jt, tid);
    stage_rows(sB, Bt, rp, n0, N, jt, tid);
    __syncthreads();
    mma_128x128x64(sA, sB, acc, wm, wn, lane);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + acc_col(wn, j, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + acc_row(wm, i, r, lane);
        if (row < M && col < N) Y[row * N + col] = f2bf(acc.c[i][j][r]);
      }
    }
}

// ------------------------------------------------- input-gradient GEMM
// dX[m, k] = sum_n dY[m, n] W[n, k].  Tile 128 (M) x 128 (K); per step of 64
// rows n the weight tile covers two NF4 blocks per row.  Four threads per
// row, 32 codes each, written transposed into LDS as [k][n].
__global__ __launch_bounds__(NT) void bwd_dx_kernel(const uint16_t* __restrict__ dY, int64_t M, int64_t N,
                                                    const uint8_t* __restrict__ codes, DQParams dq, int64_t K,
                                                    const uint16_t* __restrict__ Ts,
                                                    const uint16_t* __restrict__ Ap, int64_t rp,
                                                    uint16_t* __restrict__ dX, NF4Values nf4v) {
  __shared__ __bf16 sA[TM * LDK];
  __shared__ __bf16 sB[TN * LDK];
  __shared__ float s_nf4[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * TM, k0 = (int64_t)blockIdx.x * TN;
  if (tid < 16) s_nf4[tid] = nf4v.v[tid];
  const float mu = dq.double_quant ? *dq.offset : 0.0f;
  __syncthreads();

  Acc22 acc;
  acc_zero(acc);
  const int nrow = tid >> 2, quarter = tid & 3;
  const int64_t kcol = k0 + quarter * 32;
  const bool kok = kcol < K;
  const int64_t kblocks = K >> 6;

  for (int64_t nt = 0; nt < N; nt += 64) {
    stage_rows(sA, dY, N, m0, M, nt, tid);
    {
      const int64_t n = nt + nrow;
      uint4 cw = make_uint4(0, 0, 0, 0);
      float c = 0.0f;
      if (kok) {
        cw = *reinterpret_cast<const uint4*>(codes + ((n * K + kcol) >> 1));
        c = block_scale(dq, n * kblocks + (kcol >> 6), mu);
      }
      const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
#pragma unroll
      for (int wv = 0; wv < 4; ++wv)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = s_nf4[(words[wv] >> (4 * e)) & 0xF] * c;
          sB[(quarter * 32 + wv * 8 + e) * LDK + nrow] = (__bf16)v;
        }
    }
    __syncthreads();
    mma_128x128x64(sA, sB, acc, wm, wn, lane);
    __syncthreads();
  }
  for (int64_t jt = 0; jt < rp; jt += 64) {
    stage_rows(sA, Ts, rp, m0, M, jt, tid);
    stage_rows(sB, Ap, rp, k0, K, jt, tid);
    __syncthreads();
    mma_128x128x64(sA, sB, acc, wm, wn, lane);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = k0 + acc_col(wn, j, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + acc_row(wm, i, r, lane);
        if (row < M && col < K) dX[row * K + col] = f2bf(acc.c[i][j][r]);
      }
    }
}

// ------------------------------------------------------- NT small GEMM
// C[M, Q] = U[M, L] V[Q, L]^T, L % 64 == 0.  Used for XA = X (A^T)^T and
// T = dY B^T.  Epilogue: out1 = bf16(C) (ld Q), out2 = bf16(alpha C) (ld ld2,
// zero in columns [Q, ld2)).
__global__ __launch_bounds__(NT) void gemm_nt_kernel(const uint16_t* __restrict__ U, const uint16_t* __restrict__ V,
                                                     int64_t M, int64_t Q, int64_t L, uint16_t* __restrict__ out1,
                                                     uint16_t* __restrict__ out2, int64_t ld2, float alpha) {
  __shared__ __bf16 sA[TM * LDK];
  __shared__ __bf16 sB[TN * LDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * TM, q0 = (int64_t)blockIdx.x * TN;
  Acc22 acc;
  acc_zero(acc);
  for (int64_t lt = 0; lt < L; lt += 64) {
    stage_rows(sA, U, L, m0, M, lt, tid);
    stage_rows(sB, V, L, q0, Q, lt, tid);
    __syncthreads();
    mma_128x128x64(sA, sB, acc, wm, wn, lane);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = q0 + acc_col(wn, j, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + acc_row(wm, i, r, lane);
        if (row >= M) continue;
        const float v = acc.c[i][j][r];
        if (col < Q) {
          if (out1) out1[row * Q + col] = f2bf(v);
          if (out2) out2[row * ld2 + col] = f2bf(alpha * v);
        } else if (out2 && col < ld2) {
          out2[row * ld2 + col] = 0;
        }
      }
    }
}

// --------------------------------------------------- TN split-M GEMM
// partial[s][p][q] = sum_{m in chunk s} U[m, p] V[m, q]; U [M, P], V [M, Q]
// row-major with P % 64 == 0 and Q % 64 == 0 (callers pass padded operands).
// Tiles 128 (P) x 128 (Q); each step stages 64 rows m, transposed into LDS.
__global__ __launch_bounds__(NT) void gemm_tn_partial_kernel(const uint16_t* __restrict__ U,
                                                             const uint16_t* __restrict__ V, int64_t M,
                                                             int64_t P, int64_t Q, int64_t chunk,
                                                             float* __restrict__ partials) {
  __shared__ __bf16 sA[TM * LDK];
  __shared__ __bf16 sB[TN * LDK];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t p0 = (int64_t)blockIdx.x * TM, q0 = (int64_t)blockIdx.y * TN;
  const int64_t mbeg = (int64_t)blockIdx.z * chunk;
  const int64_t mend = mbeg + chunk < M ? mbeg + chunk : M;
  Acc22 acc;
  acc_zero(acc);
  const int mrow = tid >> 2, quarter = tid & 3;
  for (int64_t mt = mbeg; mt < mend; mt += 64) {
    const int64_t m = mt + mrow;
    const bool mok = m < mend;
    {
      const int64_t pc = p0 + quarter * 32;
      const bool ok = mok && pc < P;
      const uint16_t* src = U + (ok ? m * P + pc : 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = ld16(src + i * 8, ok);
        const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sA[(quarter * 32 + i * 8 + e) * LDK + mrow] = __builtin_bit_cast(__bf16, h[e]);
      }
    }
    {
      const int64_t qc = q0 + quarter * 32;
      const bool ok = mok && qc < Q;
      const uint16_t* src = V + (ok ? m * Q + qc : 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint4 v = ld16(src + i * 8, ok);
        const uint16_t* h = reinterpret_cast<const uint16_t*>(&v);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          sB[(quarter * 32 + i * 8 + e) * LDK + mrow] = __builtin_bit_cast(__bf16, h[e]);
      }
    }
    __syncthreads();
    mma_128x128x64(sA, sB, acc, wm, wn, lane);
    __syncthreads();
  }
  float* out = partials + (int64_t)blockIdx.z * P * Q;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = q0 + acc_col(wn, j, lane);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = p0 + acc_row(wm, i, r, lane);
        if (row < P && col < Q) out[row * Q + col] = acc.c[i][j][r];
      }
    }
}

// out[p][q] (p < Pout, q < Qout, ld Qout) = bf16(alpha * sum_s partial[s][p][q])
// with partials [splits][P][Q].
__global__ __launch_bounds__(256) void reduce_partials_kernel(const float* __restrict__ partials, int splits,
                                                              int64_t P, int64_t Q, int64_t Pout, int64_t Qout,
                                                              uint16_t* __restrict__ out, float alpha) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= Pout * Qout) return;
  const int64_t p = idx / Qout, q = idx - p * Qout;
  float s = 0.0f;
  for (int k = 0; k < splits; ++k) s += partials[(int64_t)k * P * Q + p * Q + q];
  out[idx] = f2bf(alpha * s);
}

// dst[i][j] = src[i][j] for j < cols, 0 for cols <= j < cols_pad.
__global__ __launch_bounds__(256) void pad_copy_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
                                                       uint16_t* __restrict__ dst, int64_t cols_pad) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * cols_pad) return;
  const int64_t i = idx / cols_pad, j = idx - i * cols_pad;
  dst[idx] = j < cols ? src[i * cols + j] : (uint16_t)0;
}

// dst[i][j] = src[j][i] for j < src_rows, 0 otherwise; dst is [src_cols, cols_pad].
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ src, int64_t src_rows,
                                                            int64_t src_cols, uint16_t* __restrict__ dst,
                                                            int64_t cols_pad) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= src_cols * cols_pad) return;
  const int64_t i = idx / cols_pad, j = idx - i * cols_pad;
  dst[idx] = j < src_rows ? src[j * src_cols + i] : (uint16_t)0;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint16_t* __restrict__ dst, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < n) dst[idx] = 0;
}

inline unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

}  // namespace

hipError_t launch_pad_copy(const uint16_t* src, int64_t rows, int64_t cols, uint16_t* dst, int64_t cols_pad,
                           hipStream_t stream) {
  if (rows * cols_pad == 0) return hipSuccess;
  hipLaunchKernelGGL(pad_copy_kernel, dim3(blocks_for(rows * cols_pad, 256)), dim3(256), 0, stream, src, rows, cols,
                     dst, cols_pad);
  return hipGetLastError();
}

hipError_t launch_transpose_pad(const uint16_t* src, int64_t src_rows, int64_t src_cols, uint16_t* dst,
                                int64_t cols_pad, hipStream_t stream) {
  if (src_cols * cols_pad == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_pad_kernel, dim3(blocks_for(src_cols * cols_pad, 256)), dim3(256), 0, stream, src,
                     src_rows, src_cols, dst, cols_pad);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(const uint16_t* U, const uint16_t* V, int64_t M, int64_t Q, int64_t L, uint16_t* out1,
                          uint16_t* out2, int64_t ld2, float alpha, hipStream_t stream) {
  const int64_t qcols = out2 && ld2 > Q ? ld2 : Q;
  const dim3 grid(blocks_for(qcols, TN), blocks_for(M, TM));
  hipLaunchKernelGGL(gemm_nt_kernel, grid, dim3(NT), 0, stream, U, V, M, Q, L, out1, out2, ld2, alpha);
  return hipGetLastError();
}

hipError_t launch_fwd_main(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, const DQParams& dq,
                           int64_t N, const uint16_t* XAs, const uint16_t* Bt, int64_t rp, uint16_t* Y,
                           hipStream_t stream) {
  const dim3 grid(blocks_for(N, TN), blocks_for(M, TM));
  hipLaunchKernelGGL(fwd_main_kernel, grid, dim3(NT), 0, stream, X, M, K, codes, dq, N, XAs, Bt, rp, Y, nf4_values());
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const uint16_t* dY, int64_t M, int64_t N, const uint8_t* codes, const DQParams& dq,
                         int64_t K, const uint16_t* Ts, const uint16_t* Ap, int64_t rp, uint16_t* dX,
                         hipStream_t stream) {
  const dim3 grid(blocks_for(K, TN), blocks_for(M, TM));
  hipLaunchKernelGGL(bwd_dx_kernel, grid, dim3(NT), 0, stream, dY, M, N, codes, dq, K, Ts, Ap, rp, dX, nf4_values());
  return hipGetLastError();
}

// Enough M-chunks that the grid has about 1024 workgroups, each chunk a
// multiple of 64 rows.
int tn_splits(int64_t M, int64_t P, int64_t Q) {
  const int64_t tiles = ((P + TM - 1) / TM) * ((Q + TN - 1) / TN);
  int64_t s = (1024 + tiles - 1) / tiles;
  const int64_t max_s = (M + 63) / 64;
  if (s > max_s) s = max_s;
  if (s < 1) s = 1;
  if (s > 64) s = 64;
  return (int)s;
}

hipError_t launch_gemm_tn(const uint16_t* U, const uint16_t* V, int64_t M, int64_t P, int64_t Q, float* partials,
                          int splits, uint16_t* out, int64_t Pout, int64_t Qout, float alpha, hipStream_t stream) {
  int64_t chunk = (M + splits - 1) / splits;
  chunk = (chunk + 63) / 64 * 64;
  const dim3 grid(blocks_for(P, TM), blocks_for(Q, TN), (unsigned)splits);
  hipLaunchKernelGGL(gemm_tn_partial_kernel, grid, dim3(NT), 0, stream, U, V, M, P, Q, chunk, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(reduce_partials_kernel, dim3(blocks_for(Pout * Qout, 256)), dim3(256), 0, stream, partials,
                     splits, P, Q, Pout, Qout, out, alpha);
  return hipGetLastError();
}

hipError_t launch_fill_zero_u16(uint16_t* dst, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks_for(n, 256)), dim3(256), 0, stream, dst, n);
  return hipGetLastError();
}

}  // namespace qlora
