// QLoRA linear layer over a frozen NF4 weight, forward and backward, gfx950.
//
// QLoRA (Dettmers et al., arXiv 2305.14314):
//   section 2 "Low-rank Adapters", Eq. 3: Y = XW + s X L1 L2;
//   section 3 "QLoRA", Eq. 5 and 6: W is doubleDequant(c1, c2, W^NF4), used
//     in BF16 for every product, forward and backward;
//   section 3 "QLoRA", paragraph after Eq. 6: only the adapter gradients are
//     computed (no dE/dW); the input gradient goes through the BF16 weight.
//
// The weight is [N, K] = [out, in] with 64-element NF4 blocks along K.
//
// Main products (bf16 MFMA 32x32x16, fp32 accumulation), 512 threads as a
// 2 x 4 grid of waves over a 256 x 256 output tile (128 x 64 per wave, two
// waves per SIMD), or 256 threads over 256 x 128 / 128 x 128 tiles for very
// short reductions; k-step 64, two LDS stages:
//   forward  Y [M, N]  = X [M, K] W^T     + (s XA) [M, rp] B [rp, N]
//   backward dX [M, K] = dY [M, N] W      + (s T) [M, rp] A^T
// Each k-step stages the activation tile (X or dY) and dequantises the
// weight tile: a thread expands NF4 blocks (a whole block in the narrow-tile
// kernel, half a block in the 256 x 256 kernel) through a per-block bf16
// lookup table (the exact bf16(NF4[code] * c2_hat) values) into LDS.  The
// forward tile is [n][k] (reduction contiguous); the backward tile is the
// same natural [n][k] layout, read through LDS transpose loads because there
// the reduction runs over n.  The rank-r adapter term is r_pad/64 extra
// reduction steps over bf16 operands (rows of B / A beyond r read as zero).
//
// With 1 <= M <= 16 tokens the forward instead streams the packed weight
// through a dedicated kernel (see the small-token section).
//
// Adapter products: XA = X A and T = dY B^T are skinny (r columns): split
// over the reduction into fp32 partials, then one pass writes bf16 XA and
// bf16(s XA) (zero-padded to r_pad).  dA = X^T (s T) and dB = s XA^T dY
// reduce over tokens: split over M into fp32 partials, then one reduction
// pass; both operands are read through LDS transpose loads.
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr int NT = 256;
constexpr int PK = 72;  // pitch (bf16) of a [rows][64] reduction-contiguous tile
// Padding (bf16) of a tile read through transpose loads ([red][cols], cols a
// multiple of 64).  Half a wave of frag_rc reads 4 reduction rows x 64
// bytes; with the row pitch = 32 or 96 mod 128 bf16 those rows start 16 or 48
// banks apart and cover all 64 banks once (with +16 they overlapped 2-way).
constexpr int kRcPad = 32;

// The codebooks (NF4 = QLoRA Appendix E, then the other 4-bit types of the
// section 3 comparison) in constant memory, read through a wave-uniform
// pointer for the lookup-table builds.
__constant__ float kCodeValues[CODE_TYPES][16] = QLORA_CODE_VALUES;

// c2_hat of one block (Eq. 6 inner dequant): two separately rounded fp32
// operations for double quantisation, or the stored absmax.
// `f` is the group's scale2 with double quantisation, else the block absmax.
__device__ __forceinline__ float block_scale(const DQParams& dq, uint32_t qbyte, float f, float mu) {
  if (dq.double_quant) return __fadd_rn(__fmul_rn(e4m3_decode(qbyte), f), mu);
  return f;
}

__device__ __forceinline__ BlockLUT lut_for(float c, const float* cv) {
  uint32_t p[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) p[j] = pack_bf2(cv[2 * j] * c, cv[2 * j + 1] * c);
  return make_lut(p);
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void sts16(__bf16* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// 8 bf16 of row `row` of a row-major [rows, cols] matrix starting at column
// c, zero where row >= rows or column >= cols.  Vector load when the whole
// chunk is inside and 16-byte aligned (cols % 8 == 0), else element-wise.
__device__ __forceinline__ uint4 load8_masked(const uint16_t* g, int64_t ld, int64_t row, int64_t rows, int64_t c,
                                              int64_t cols) {
  if (row >= rows || c >= cols) return make_uint4(0, 0, 0, 0);
  const uint16_t* p = g + row * ld + c;
  if ((ld & 7) == 0 && c + 8 <= cols) return ldg16(p);
  const int64_t n = cols - c;  // 1..7 valid elements, or an unaligned row
  auto h = [&](int e) -> uint32_t { return e < n ? (uint32_t)p[e] : 0u; };
  return make_uint4(h(0) | (h(1) << 16), h(2) | (h(3) << 16), h(4) | (h(5) << 16), h(6) | (h(7) << 16));
}

// ============================================================ main GEMM
struct MainArgs {
  const uint16_t* act;      // X [M, K] (fwd) or dY [M, N] (bwd)
  int64_t M, L;             // rows of act, reduction length (K fwd, N bwd)
  const uint8_t* codes;     // weight [Nw, Kw], packed NF4
  DQParams dq;
  int64_t Nw, Kw;
  const uint16_t* ext_act;  // s*XA or s*T  [M, rp]
  const uint16_t* ext_w;    // B [r, Nw] (fwd) or A [Kw, r] (bwd)
  int64_t r, rp;
  uint16_t* out;            // [M, ncols]
  int64_t ncols;            // Nw (fwd) or Kw (bwd)
  // split reduction of the last tiles (256 x 256 kernel only): tiles
  // [full_tiles, T) are each cut into `split` reduction ranges whose fp32
  // partial tiles go to part[unit][256][256]; a fixup pass adds them.
  int full_tiles, split;
  float* part;
  // LoRA dropout (backward only): bit mask [M, ncols/8] of the adapter term,
  // kept elements multiplied by keep_scale; null without dropout
  const uint8_t* keep;
  float keep_scale;
};

// Zeroes the bf16 elements of an 8-element chunk whose keep bit is clear
// (bit j of `keep` for element j).
__device__ __forceinline__ uint4 apply_keep8(uint4 v, uint32_t keep) {
  auto m2 = [&](int j) -> uint32_t {  // elements 2j (low half) and 2j + 1 (high half)
    return (((keep >> (2 * j)) & 1u) ? 0x0000FFFFu : 0u) | (((keep >> (2 * j + 1)) & 1u) ? 0xFFFF0000u : 0u);
  };
  return make_uint4(v.x & m2(0), v.y & m2(1), v.z & m2(2), v.w & m2(3));
}

// One 32 x 32 accumulator tile (MFMA layout) at rows r0.., columns c0..:
// element (row, col) times `scale` where bit col % 8 of keep[row * pitch +
// col / 8] is set, zero where it is clear (rows and columns clamped to the
// matrix, whose values outside are not stored).
__device__ __forceinline__ void mask_acc32(floatx16& acc, int lane, int64_t r0, int64_t c0, int64_t M, int64_t ncols,
                                           const uint8_t* __restrict__ keep, float scale) {
  const int64_t col = c0 + (lane & 31) < ncols ? c0 + (lane & 31) : ncols - 1;
  const int64_t pitch = ncols >> 3;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t row = r0 + acc_row32(e, lane) < M ? r0 + acc_row32(e, lane) : M - 1;
    const uint32_t b = keep[row * pitch + (col >> 3)];
    acc[e] = ((b >> (col & 7)) & 1u) ? acc[e] * scale : 0.0f;
  }
}

// The same for a block accumulated transposed (store_acc32t's layout: lane
// l holds row r0 + (l & 31), element 4 g + i column c0 + 8 g + 4 (l >> 5) + i,
// so each group's 4 columns share one mask byte).
__device__ __forceinline__ void mask_acc32t(floatx16& acc, int lane, int64_t r0, int64_t c0, int64_t M, int64_t ncols,
                                            const uint8_t* __restrict__ keep, float scale) {
  const int64_t row = r0 + (lane & 31) < M ? r0 + (lane & 31) : M - 1;
  const int64_t pitch = ncols >> 3;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int64_t col = c0 + 8 * g + 4 * (lane >> 5);
    const uint32_t b = keep[row * pitch + ((col < ncols ? col : 0) >> 3)] >> (col & 7);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[4 * g + i] = ((b >> i) & 1u) ? acc[4 * g + i] * scale : 0.0f;
  }
}

template <int BM, int BN, bool BWD>
struct MainCfg {
  static constexpr int WM = BM / 2, WN = BN / 2;       // wave tile
  static constexpr int TMW = WM / 32, TNW = WN / 32;   // 32x32 MFMA tiles per wave
  static constexpr int PRC = BN + kRcPad;              // pitch of a [64][BN] tile
  static constexpr int SA = BM * PK;
  static constexpr int SB = (BN * PK > 64 * PRC) ? BN * PK : 64 * PRC;
  static constexpr int XCH = BM * 8 / NT;              // 16-byte activation chunks per thread
  static constexpr int DQE = BN * 64 / NT;             // weights dequantised per thread per step
  static constexpr int DQW = DQE / 8;                  // 32-bit code words per thread
  static constexpr int ECH = BN * 8 / NT;              // 16-byte ext-weight chunks per thread
  static_assert(DQE == 32 || DQE == 64, "tile");
};

// I8: the weight holds one Int8 code byte per element (value k / 127,
// blockwise Eq. 1) instead of two 4-bit codes; each byte expands to
// bf16(fp32(k / 127) * c2_hat), the value the dequantiser writes.
// fp32(k / 127) for the Int8 code byte b (k its two's complement), without
// a division: q0 = k * fp32(1/127), then one correction step with the exact
// residual k - 127 q0.  Correctly rounded for all 256 codes (checked
// exhaustively in exact rational arithmetic).
__device__ __forceinline__ float i8_value(uint32_t b) {
  const float k = (float)(int)(int8_t)b;
  const float R = 0x1.020408p-7f;  // fp32(1 / 127)
  const float q0 = k * R;
  const float r = __builtin_fmaf(-q0, 127.0f, k);
  return __builtin_fmaf(r, R, q0);
}

template <int BM, int BN, bool BWD, bool I8 = false>
__global__ __launch_bounds__(NT, 1) void main_gemm_kernel(const MainArgs a) {
  using C = MainCfg<BM, BN, BWD>;
  __shared__ __attribute__((aligned(16))) __bf16 sA[2][C::SA];
  __shared__ __attribute__((aligned(16))) __bf16 sB[2][C::SB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * BM, c0 = (int64_t)blockIdx.x * BN;
  const float mu = a.dq.double_quant ? *a.dq.offset : 0.0f;
  const float* cv = kCodeValues[I8 ? 0 : a.dq.code_type];
  const int64_t kblocks = a.Kw >> 6;
  const int64_t nk = a.L >> 6;

  // --- dequantisation task of this thread (DQE consecutive weights of one block)
  int t_row, t_col;
  if (!BWD) {  // tile [BN rows n][64 k]
    constexpr int TPR = 64 / C::DQE;
    t_row = tid / TPR;
    t_col = (tid % TPR) * C::DQE;
  } else {     // tile [64 rows n][BN k]
    constexpr int TPR = BN / C::DQE;
    t_row = tid / TPR;
    t_col = (tid % TPR) * C::DQE;
  }
  const bool t_ok = BWD ? (c0 + t_col < a.Kw) : (c0 + t_row < a.Nw);

  floatx16 acc[C::TMW][C::TNW];
#pragma unroll
  for (int i = 0; i < C::TMW; ++i)
#pragma unroll
    for (int j = 0; j < C::TNW; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  uint4 xr[C::XCH];
  uint32_t cw[I8 ? 2 * C::DQW : C::DQW];  // 4-bit: 8 codes per word; Int8: 4
  uint32_t qb = 0;
  float sf = 0.0f;  // scale2 of the group (double quantisation) or the block absmax

  auto load_step = [&](int64_t kt) {
#pragma unroll
    for (int i = 0; i < C::XCH; ++i) {
      const int id = tid + NT * i, row = id >> 3, ch = id & 7;
      const int64_t m = m0 + row;
      xr[i] = (m < a.M) ? ldg16(a.act + m * a.L + kt * 64 + ch * 8) : make_uint4(0, 0, 0, 0);
    }
    const int64_t n = BWD ? kt * 64 + t_row : c0 + t_row;
    const int64_t k = BWD ? c0 + t_col : kt * 64 + t_col;
    constexpr int NW = I8 ? 2 * C::DQW : C::DQW;
    if (t_ok) {
      const uint8_t* src = a.codes + (I8 ? n * a.Kw + k : ((n * a.Kw + k) >> 1));
#pragma unroll
      for (int w = 0; w < NW; w += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(src + 4 * w);
        cw[w] = v.x; cw[w + 1] = v.y; cw[w + 2] = v.z; cw[w + 3] = v.w;
      }
      const int64_t blk = n * kblocks + (k >> 6);
      if (a.dq.double_quant) qb = a.dq.absmax_q[blk];
      sf = a.dq.double_quant ? a.dq.scale2[blk >> 8] : a.dq.absmax[blk];
    } else {
#pragma unroll
      for (int w = 0; w < NW; ++w) cw[w] = I8 ? 0u : 0x77777777u;  // the code of 0.0
      qb = 0; sf = 0.0f;
    }
  };

  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < C::XCH; ++i) {
      const int id = tid + NT * i, row = id >> 3, ch = id & 7;
      sts16(&sA[buf][row * PK + ch * 8], xr[i]);
    }
    const float c = t_ok ? block_scale(a.dq, qb, sf, mu) : 0.0f;
    __bf16* dst = BWD ? &sB[buf][t_row * C::PRC + t_col] : &sB[buf][t_row * PK + t_col];
    if (I8) {
#pragma unroll
      for (int w = 0; w < C::DQW; ++w) {  // 8 weights: code words 2w, 2w + 1
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t cwd = cw[2 * w + h];
          o[2 * h] = pack_bf2(i8_value(cwd & 0xFFu) * c, i8_value((cwd >> 8) & 0xFFu) * c);
          o[2 * h + 1] = pack_bf2(i8_value((cwd >> 16) & 0xFFu) * c, i8_value(cwd >> 24) * c);
        }
        sts16(dst + 8 * w, make_uint4(o[0], o[1], o[2], o[3]));
      }
    } else {
      const BlockLUT lut = lut_for(c, cv);
#pragma unroll
      for (int w = 0; w < C::DQW; ++w) {
        uint32_t o[4];
        lut_lookup8(lut, cw[w], o);
        sts16(dst + 8 * w, make_uint4(o[0], o[1], o[2], o[3]));
      }
    }
  };

  auto mma_step = [&](int buf, bool b_rc, int pitch_b) {
#pragma unroll
    for (int kk = 0; kk < 64; kk += 16) {
      bf16x8 af[C::TMW], bfr[C::TNW];
#pragma unroll
      for (int i = 0; i < C::TMW; ++i) af[i] = frag_kc(sA[buf], PK, wm * C::WM + 32 * i, kk, lane);
#pragma unroll
      for (int j = 0; j < C::TNW; ++j)
        bfr[j] = b_rc ? frag_rc(sB[buf], pitch_b, wn * C::WN + 32 * j, kk, lane)
                      : frag_kc(sB[buf], pitch_b, wn * C::WN + 32 * j, kk, lane);
#pragma unroll
      for (int i = 0; i < C::TMW; ++i)
#pragma unroll
        for (int j = 0; j < C::TNW; ++j) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    }
  };

  // ---- adapter term first: rp/64 reduction steps over bf16 operands (both
  // LDS stages are free), masked for LoRA dropout before the weight term
  for (int64_t jt = 0; jt < a.rp; jt += 64) {
#pragma unroll
    for (int i = 0; i < C::XCH; ++i) {
      const int id = tid + NT * i, row = id >> 3, ch = id & 7;
      const int64_t m = m0 + row;
      sts16(&sA[0][row * PK + ch * 8], (m < a.M) ? ldg16(a.ext_act + m * a.rp + jt + ch * 8) : make_uint4(0, 0, 0, 0));
    }
    if (!BWD) {  // B [r, Nw]: tile [64 j][BN n], read transposed
#pragma unroll
      for (int i = 0; i < C::ECH; ++i) {
        const int id = tid + NT * i, row = id / (BN / 8), ch = id % (BN / 8);
        sts16(&sB[0][row * C::PRC + ch * 8], load8_masked(a.ext_w, a.Nw, jt + row, a.r, c0 + ch * 8, a.Nw));
      }
    } else {     // A [Kw, r]: tile [BN k][64 j]
#pragma unroll
      for (int i = 0; i < C::ECH; ++i) {
        const int id = tid + NT * i, row = id >> 3, ch = id & 7;
        sts16(&sB[0][row * PK + ch * 8], load8_masked(a.ext_w, a.r, c0 + row, a.Kw, jt + ch * 8, a.r));
      }
    }
    __syncthreads();
    mma_step(0, !BWD, BWD ? PK : C::PRC);
    __syncthreads();
  }

  if (BWD && a.keep) {
#pragma unroll
    for (int i = 0; i < C::TMW; ++i)
#pragma unroll
      for (int j = 0; j < C::TNW; ++j)
        mask_acc32(acc[i][j], lane, m0 + wm * C::WM + 32 * i, c0 + wn * C::WN + 32 * j, a.M, a.ncols, a.keep,
                   a.keep_scale);
  }

  // ---- main reduction over the quantised weight, two LDS stages
  load_step(0);
  store_step(0);
  __syncthreads();
  for (int64_t kt = 0; kt < nk; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < nk) load_step(kt + 1);
    mma_step(cur, BWD, BWD ? C::PRC : PK);
    if (kt + 1 < nk) store_step(cur ^ 1);
    __syncthreads();
  }

  // ---- epilogue: bf16 output
#pragma unroll
  for (int i = 0; i < C::TMW; ++i)
#pragma unroll
    for (int j = 0; j < C::TNW; ++j) {
      const int64_t col = c0 + wn * C::WN + 32 * j + (lane & 31);
      if (col >= a.ncols) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + wm * C::WM + 32 * i + acc_row32(e, lane);
        if (row < a.M) a.out[row * a.ncols + col] = f2bf(acc[i][j][e]);
      }
    }
}

// Stores a 32 x 32 output block accumulated transposed, i.e. with the weight
// fragment as the MFMA's first operand and the activation fragment as its
// second: lane l then holds output row r0 + (l & 31), columns
// c0 + 8 g + 4 (l >> 5) + i of group g (i = 0..3), so each group is one
// 8-byte bf16 store with no exchange between lanes (rows >= M dropped).  The
// block's columns are inside the output (callers check the block's first
// column; widths are multiples of 32).
__device__ __forceinline__ void store_acc32t(const floatx16& acc, int lane, int64_t r0, int64_t c0, int64_t M,
                                             int64_t ncols, uint16_t* __restrict__ out) {
  const int64_t r = r0 + (lane & 31);
  if (r < M) {
    uint16_t* o = out + r * ncols + c0 + 4 * (lane >> 5);
#pragma unroll
    for (int g = 0; g < 4; ++g)
      *reinterpret_cast<uint2*>(o + 8 * g) =
          make_uint2(pack_bf2(acc[4 * g], acc[4 * g + 1]), pack_bf2(acc[4 * g + 2], acc[4 * g + 3]));
  }
  // one block at a time: keeps the compiler from reading every accumulator
  // out first (which spills)
  __builtin_amdgcn_sched_barrier(0);
}
// The same block into an fp32 partial tile (row pitch `pitch`): one 16-byte
// store per group.
__device__ __forceinline__ void store_acc32t_f32(const floatx16& acc, int lane, int r0, int c0, float* __restrict__ pt,
                                                 int pitch) {
  float* o = pt + (int64_t)(r0 + (lane & 31)) * pitch + c0 + 4 * (lane >> 5);
#pragma unroll
  for (int g = 0; g < 4; ++g)
    *reinterpret_cast<float4*>(o + 8 * g) = make_float4(acc[4 * g], acc[4 * g + 1], acc[4 * g + 2], acc[4 * g + 3]);
  __builtin_amdgcn_sched_barrier(0);
}

// ================================== main GEMM, 256 x 256, 4 waves, v5
// One wave per SIMD, each owning a 128 x 128 output tile (256 fp32
// accumulators), so every LDS fragment feeds four MFMAs.  The next k-step's
// weight tile is dequantised by the same waves, but its instructions are
// spread between the MFMAs by hand: after each MFMA one small item (a few
// VALU operations, one LDS store or one global load) is issued, and
// scheduling barriers keep that order, so the VALU work fills the MFMA
// shadow instead of running after it.  Fragment reads for sub-step kk+1 are
// issued while sub-step kk multiplies.
constexpr int V5_T = 256;

struct WordState {
  uint32_t e7, o7, me, mo, loE, hiE, loO, hiO;
};

// GW (forward, double quantisation, K / 64 a multiple of 4, aligned E4M3
// bytes): a thread's four E4M3 bytes of k-steps 4g .. 4g+3 are one aligned
// word, loaded once per four k-steps instead of one byte per k-step (each
// load instruction touches 64 rows); the k-loop is unrolled by four so the
// words rotate with fixed roles, and reduction ranges start on multiples of
// four k-steps.
template <bool BWD, bool DQ, bool GW = false>
__global__ __launch_bounds__(V5_T, 1) void main_v5_kernel(const MainArgs a) {
  static_assert(!GW || (!BWD && DQ), "grouped E4M3 words: forward, double quantisation");
  constexpr int BM = 256, BN = 256;
  constexpr int PRC = BN + kRcPad;
  constexpr int SA = BM * PK;
  constexpr int SB = (BN * PK > 64 * PRC) ? BN * PK : 64 * PRC;
  constexpr int XCH = BM * 8 / V5_T;  // 8 activation chunks per thread
  __shared__ __attribute__((aligned(16))) __bf16 sA[2][SA];
  __shared__ __attribute__((aligned(16))) __bf16 sB[2][SB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tn = (int)((a.ncols + BN - 1) / BN);
  const int nkt = (int)(a.L >> 6);  // k-steps of the whole reduction
  const int F = a.full_tiles, pid = blockIdx.x;
  // Work unit -> tile and reduction range.  Whole tiles first, in XCD-aware
  // order (consecutive workgroups go to different XCDs, so each XCD gets a
  // contiguous run of tiles); then the split units of the last tiles.
  int lid, ks = 0, ke = nkt, unit = -1;
  if (pid < F) {
    lid = (F % 8 == 0) ? (pid % 8) * (F / 8) + pid / 8 : pid;
  } else {
    unit = pid - F;
    const int sp = unit % a.split;
    lid = F + unit / a.split;
    ks = (int)((int64_t)sp * nkt / a.split);
    ke = (int)((int64_t)(sp + 1) * nkt / a.split);
    if constexpr (GW) {  // ranges of whole four-step groups (nkt % 4 == 0, at least four steps each)
      ks &= ~3;
      ke &= ~3;
    }
  }
  const bool last_range = ke == nkt;  // the range that also adds the adapter term
  const int64_t m0 = (int64_t)(lid / tn) * BM, c0 = (int64_t)(lid % tn) * BN;
  const int nk = ke;
  const int64_t kblocks = a.Kw >> 6;
  const float mu = DQ ? *a.dq.offset : 0.0f;
  const float* cv = kCodeValues[a.dq.code_type];

  // dequantisation task: one whole NF4 block (64 weights) per thread
  const int t_row = BWD ? (tid >> 2) : tid;
  const int t_col = BWD ? (tid & 3) * 64 : 0;
  const bool t_ok = BWD ? (c0 + t_col < a.Kw) : (c0 + t_row < a.Nw);
  const int64_t t_n = BWD ? 0 : (t_ok ? c0 + t_row : a.Nw - 1);
  const int64_t t_k = BWD ? (t_ok ? c0 + t_col : a.Kw - 64) : 0;

  floatx16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  uint4 xr[XCH];
  uint4 cwA[2], cwB[2];
  uint8_t qbA = 0, qbB = 0;
  float sfA = 0.0f, sfB = 0.0f;

  auto x_src = [&](int i, int kt) -> const uint16_t* {
    const int id = tid + V5_T * i, row = id >> 3, ch = id & 7;
    const int64_t m = m0 + row < a.M ? m0 + row : a.M - 1;
    return a.act + m * a.L + (int64_t)kt * 64 + ch * 8;
  };
  auto x_dst = [&](int i, int buf) -> __bf16* {
    const int id = tid + V5_T * i, row = id >> 3, ch = id & 7;
    return &sA[buf][row * PK + ch * 8];
  };
  auto load_codes = [&](int kt, uint4* c, uint8_t& q, float& f) {
    const int64_t n = BWD ? (int64_t)kt * 64 + t_row : t_n;
    const int64_t k = BWD ? t_k : (int64_t)kt * 64;
    const uint8_t* src = a.codes + ((n * a.Kw + k) >> 1);
    c[0] = *reinterpret_cast<const uint4*>(src);
    c[1] = *reinterpret_cast<const uint4*>(src + 16);
    const int64_t blk = n * kblocks + (k >> 6);
    if (DQ) {
      if constexpr (!GW) q = a.dq.absmax_q[blk];
      f = a.dq.scale2[blk >> 8];
    } else {
      f = a.dq.absmax[blk];
    }
  };
  auto wdst = [&](int buf, int w) -> __bf16* {
    return BWD ? &sB[buf][t_row * PRC + t_col + 8 * w] : &sB[buf][t_row * PK + t_col + 8 * w];
  };

  bf16x8 fa[2][4], fb[2][4];
  // The reads are issued in the order the sub-step's MFMAs consume them
  // (a0, b0..b3, a1..a3; scheduling barriers keep it), so the first MFMA of
  // a k-step waits for two reads instead of most of them.
  auto read_frags = [&](int buf, int kk, int slot, bool b_rc, int pitch_b) {
    fa[slot][0] = frag_kc(sA[buf], PK, wm * 128, kk, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      fb[slot][j] = b_rc ? frag_rc(sB[buf], pitch_b, wn * 128 + 32 * j, kk, lane)
                         : frag_kc(sB[buf], pitch_b, wn * 128 + 32 * j, kk, lane);
    }
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      fa[slot][i] = frag_kc(sA[buf], PK, wm * 128 + 32 * i, kk, lane);
    }
  };

  // ---- one k-step: multiply stage `cur` while producing stage `nxt`
  auto step = [&](int kt, const int cur, const uint4* cu, uint8_t qu, float fu, uint4* cl, uint8_t& ql, float& fl) {
    const int nxt = cur ^ 1;
    const int k2 = kt + 2 < nk ? kt + 2 : nk - 1;  // past the end: a harmless repeat
    const uint32_t words[8] = {cu[0].x, cu[0].y, cu[0].z, cu[0].w, cu[1].x, cu[1].y, cu[1].z, cu[1].w};
    float sc = 0.0f;
    uint32_t pw[8];
    BlockLUT lut;
    WordState ws[8];
    load_codes(k2, cl, ql, fl);
    read_frags(cur, 0, 0, BWD, BWD ? PRC : PK);
    __builtin_amdgcn_sched_barrier(0);
    // items interleaved with the 64 MFMAs, in order: 0-8 build the block's
    // lookup table, 9-48 expand the 8 code words (5 stages each, the last one
    // storing the word's 8 bf16 weights), 49-56 store the activation chunk of
    // step kt + 1 and load that of step kt + 2.  The three slots that issue
    // fragment reads take no item: a heavy item there delays the next MFMA.
    auto item = [&](int it) {
      if (it == 0) {
        const float bs = DQ ? __fadd_rn(__fmul_rn(e4m3_decode(qu), fu), mu) : fu;
        sc = t_ok ? bs : 0.0f;
        pw[0] = pack_bf2(cv[0] * sc, cv[1] * sc);
      } else if (it <= 7) {
        pw[it] = pack_bf2(cv[2 * it] * sc, cv[2 * it + 1] * sc);
      } else if (it == 8) {
        lut = make_lut(pw);
      } else if (it < 9 + 40) {
        const int w = (it - 9) / 5, stg = (it - 9) % 5;
        WordState& st = ws[w];
        const uint32_t wd = words[w];
        if (stg == 0) {
          st.e7 = wd & 0x07070707u;
          st.o7 = (wd >> 4) & 0x07070707u;
          const uint32_t t3 = wd >> 3;
          st.me = lut_half_sel(t3);
          st.mo = lut_half_sel(t3 >> 4);
        } else if (stg == 1) {
          st.loE = perm_b32(perm_b32(lut.lo[3], lut.lo[2], st.e7), perm_b32(lut.lo[1], lut.lo[0], st.e7), st.me);
          st.hiE = perm_b32(perm_b32(lut.hi[3], lut.hi[2], st.e7), perm_b32(lut.hi[1], lut.hi[0], st.e7), st.me);
        } else if (stg == 2) {
          st.loO = perm_b32(perm_b32(lut.lo[3], lut.lo[2], st.o7), perm_b32(lut.lo[1], lut.lo[0], st.o7), st.mo);
          st.hiO = perm_b32(perm_b32(lut.hi[3], lut.hi[2], st.o7), perm_b32(lut.hi[1], lut.hi[0], st.o7), st.mo);
        } else if (stg == 3) {
          const uint32_t e01 = perm_b32(st.hiE, st.loE, 0x05010400u);
          const uint32_t o01 = perm_b32(st.hiO, st.loO, 0x05010400u);
          const uint32_t e23 = perm_b32(st.hiE, st.loE, 0x07030602u);
          const uint32_t o23 = perm_b32(st.hiO, st.loO, 0x07030602u);
          st.loE = e01;  // the interleaved pairs, in the fields they came from
          st.hiE = o01;
          st.loO = e23;
          st.hiO = o23;
        } else {
          sts16(wdst(nxt, w), make_uint4(perm_b32(st.hiE, st.loE, 0x05040100u), perm_b32(st.hiE, st.loE, 0x07060302u),
                                         perm_b32(st.hiO, st.loO, 0x05040100u), perm_b32(st.hiO, st.loO, 0x07060302u)));
        }
      } else if (it < 49 + XCH) {
        const int i = it - 49;
        sts16(x_dst(i, nxt), xr[i]);
        xr[i] = ldg16(x_src(i, k2));
      }
    };
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int slot = kk & 1;
#pragma unroll
      for (int ij = 0; ij < 16; ++ij) {
        const int i = ij >> 2, j = ij & 3;
        acc[i][j] = mfma32(fb[slot][j], fa[slot][i], acc[i][j]);
        if (ij == 0 && kk < 3) {  // after the sub-step's first MFMA, whose reads come first
          __builtin_amdgcn_sched_barrier(0);
          read_frags(cur, 16 * (kk + 1), slot ^ 1, BWD, BWD ? PRC : PK);
        }
        {
          const int sl = kk * 16 + ij;  // slots 0, 16, 32 issue the fragment reads and take no item
          if (sl != 0 && sl != 16 && sl != 32) item(sl - 1 - (sl > 16) - (sl > 32));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  };

  // ---- prologue: stage 0 filled; X(ks+1) and codes(ks+1) in flight
  // GW: the E4M3 words of the thread's row, groups ks/4 and ks/4 + 1 first
  uint32_t wcur = 0, wnxt = 0, wnew = 0;
  const int lastg = (int)(kblocks >> 2) - 1;
  auto ldw = [&](int g) -> uint32_t {
    return *reinterpret_cast<const uint32_t*>(a.dq.absmax_q + t_n * kblocks + 4 * (int64_t)(g < lastg ? g : lastg));
  };
  if constexpr (GW) {
    wcur = ldw(ks >> 2);
    wnxt = ldw((ks >> 2) + 1);
  }
  load_codes(ks, cwB, qbB, sfB);
#pragma unroll
  for (int i = 0; i < XCH; ++i) xr[i] = ldg16(x_src(i, ks));
#pragma unroll
  for (int i = 0; i < XCH; ++i) sts16(x_dst(i, 0), xr[i]);
  {
    if constexpr (GW) qbB = (uint8_t)(wcur & 0xFFu);  // k-step ks = 4 (ks / 4)
    const float bs = DQ ? __fadd_rn(__fmul_rn(e4m3_decode(qbB), sfB), mu) : sfB;
    const BlockLUT lut = lut_for(t_ok ? bs : 0.0f, cv);
    const uint32_t words[8] = {cwB[0].x, cwB[0].y, cwB[0].z, cwB[0].w, cwB[1].x, cwB[1].y, cwB[1].z, cwB[1].w};
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      uint32_t o[4];
      lut_lookup8(lut, words[w], o);
      sts16(wdst(0, w), make_uint4(o[0], o[1], o[2], o[3]));
    }
  }
  load_codes(ks + 1 < nk ? ks + 1 : ks, cwA, qbA, sfA);
  // the codes and constants of ks + 1 go out before the activations, as in
  // the loop, so that the loop's load counts are the same on entry as after
  // a pass (the compiler waits for the stricter of the two)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < XCH; ++i) xr[i] = ldg16(x_src(i, ks + 1 < nk ? ks + 1 : ks));
  __syncthreads();

  if constexpr (GW) {
    // four k-steps per pass: step kt decodes the block of k-step kt + 1
    uint8_t qd = 0;  // the byte slot load_codes leaves alone
    for (int kt = ks; kt < nk; kt += 4) {
      wnew = ldw((kt >> 2) + 2);
      step(kt, 0, cwA, (uint8_t)(wcur >> 8), sfA, cwB, qd, sfB);
      step(kt + 1, 1, cwB, (uint8_t)(wcur >> 16), sfB, cwA, qd, sfA);
      step(kt + 2, 0, cwA, (uint8_t)(wcur >> 24), sfA, cwB, qd, sfB);
      step(kt + 3, 1, cwB, (uint8_t)wnxt, sfB, cwA, qd, sfA);
      wcur = wnxt;
      wnxt = wnew;
    }
  } else {
    for (int kt = ks; kt < nk; kt += 2) {
      step(kt, 0, cwA, qbA, sfA, cwB, qbB, sfB);
      if (kt + 1 < nk) step(kt + 1, 1, cwB, qbB, sfB, cwA, qbA, sfA);
    }
  }

  // ---- adapter term over bf16 operands (stage 0 is free)
  for (int64_t jt = 0; last_range && jt < a.rp; jt += 64) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int id = tid + V5_T * i, row = id >> 3, ch = id & 7;
      const int64_t m = m0 + row;
      sts16(&sA[0][row * PK + ch * 8], (m < a.M) ? ldg16(a.ext_act + m * a.rp + jt + ch * 8) : make_uint4(0, 0, 0, 0));
    }
    if (!BWD) {  // B [r, Nw]: tile [64 j][BN n], read transposed
#pragma unroll
      for (int i = 0; i < BN * 8 / V5_T; ++i) {
        const int id = tid + V5_T * i, row = id / (BN / 8), ch = id % (BN / 8);
        sts16(&sB[0][row * PRC + ch * 8], load8_masked(a.ext_w, a.Nw, jt + row, a.r, c0 + ch * 8, a.Nw));
      }
    } else {     // A [Kw, r]: tile [BN k][64 j]
#pragma unroll
      for (int i = 0; i < BN * 8 / V5_T; ++i) {
        const int id = tid + V5_T * i, row = id >> 3, ch = id & 7;
        sts16(&sB[0][row * PK + ch * 8], load8_masked(a.ext_w, a.r, c0 + row, a.Kw, jt + ch * 8, a.r));
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 64; kk += 16) {
      read_frags(0, kk, 0, !BWD, BWD ? PK : PRC);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma32(fb[0][j], fa[0][i], acc[i][j]);
    }
    __syncthreads();
  }

  // ---- epilogue: bf16 output, or the fp32 partial tile of a split unit
  __builtin_amdgcn_sched_barrier(0);
  if (unit >= 0) {
    float* pt = a.part + (int64_t)unit * (BM * BN);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) store_acc32t_f32(acc[i][j], lane, wm * 128 + 32 * i, wn * 128 + 32 * j, pt, BN);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c0 + wn * 128 + 32 * j < a.ncols)
          store_acc32t(acc[i][j], lane, m0 + wm * 128 + 32 * i, c0 + wn * 128 + 32 * j, a.M, a.ncols, a.out);
  }
}

// The backward kernel's dequantised weight tile [64 n][256 k] (row pitch
// 288 bf16) holds the 16-byte chunks of each 64-byte half-block permuted:
// chunk c of block b (b = k / 64) in tile row n sits at position
// c ^ ((b + 2 ((n >> 1) & 1)) & 3).  A dequantisation store instruction
// writes 4 rows x 4 blocks (16 lanes); with the plain layout the row pitch
// (16 banks mod 64) and the block stride (32 banks) put those 16 lanes on
// 4 bank offsets only (4-way conflicts), with the permutation on 16.  A
// transposed fragment read touches 8 bytes of one chunk per lane and 4 rows
// per 16 lanes, each inside its row's own 16-bank window, so the
// permutation leaves the reads conflict-free too.
__device__ __forceinline__ int bwd_tile_col(int n, int col) {
  const int s = (((col >> 6) & 3) + 2 * ((n >> 1) & 1)) & 3;
  return (col & ~31) | ((((col >> 3) & 3) ^ s) << 3) | (col & 7);
}

// frag_rc over the permuted backward tile (same lanes, same values).
__device__ __forceinline__ bf16x8 frag_rc_bwd(const __bf16* s, int pitch, int r0, int k0, int lane) {
  const int g = lane >> 4, q = lane & 15;
  const int col = r0 + 16 * (g & 1) + 4 * (q & 3);
  const int red = k0 + 8 * (g >> 1) + (q >> 2);
  const short4_t lo = ds_read_tr16(s + red * pitch + bwd_tile_col(red, col));
  const short4_t hi = ds_read_tr16(s + (red + 4) * pitch + bwd_tile_col(red + 4, col));
  const short8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// ================================== main GEMM, 256 x 256, 8 waves, v6
// Two waves per SIMD, each owning a 128 x 64 output tile (128 fp32
// accumulators), so that one wave's LDS reads and dequantisation VALU overlap
// the other wave's MFMAs.  Every thread dequantises half an NF4 block (32
// weights) of the next k-step; those instructions are spread between the
// MFMAs by hand as in the 4-wave kernel.  Fragment reads for sub-step kk+1
// are issued while sub-step kk multiplies.
constexpr int V6_T = 512;


template <bool BWD, bool DQ, bool I8 = false>
__global__ __launch_bounds__(V6_T, 1) void main_v6_kernel(const MainArgs a) {
  constexpr int CW = I8 ? 2 : 1;  // 16-byte code pieces per thread and step
  constexpr int BM = 256, BN = 256;
  constexpr int PRC = BN + kRcPad;
  constexpr int SA = BM * PK;
  constexpr int SB = (BN * PK > 64 * PRC) ? BN * PK : 64 * PRC;
  constexpr int XCH = BM * 8 / V6_T;  // 4 activation chunks per thread
  __shared__ __attribute__((aligned(16))) __bf16 sA[2][SA];
  __shared__ __attribute__((aligned(16))) __bf16 sB[2][SB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;  // rows wm * 128 .. +127, columns wn * 64 .. +63
  const int tn = (int)((a.ncols + BN - 1) / BN);
  const int nkt = (int)(a.L >> 6);
  const int F = a.full_tiles, pid = blockIdx.x;
  int lid, ks = 0, ke = nkt, unit = -1;
  if (pid < F) {
    lid = (F % 8 == 0) ? (pid % 8) * (F / 8) + pid / 8 : pid;
  } else {
    unit = pid - F;
    const int sp = unit % a.split;
    lid = F + unit / a.split;
    ks = (int)((int64_t)sp * nkt / a.split);
    ke = (int)((int64_t)(sp + 1) * nkt / a.split);
  }
  const bool last_range = ke == nkt;
  const int64_t m0 = (int64_t)(lid / tn) * BM, c0 = (int64_t)(lid % tn) * BN;
  const int nk = ke;
  const int64_t kblocks = a.Kw >> 6;
  const float mu = DQ ? *a.dq.offset : 0.0f;
  const float* cv = kCodeValues[I8 ? 0 : a.dq.code_type];

  // dequantisation task: half (t_half) of one block per thread; the 16
  // lanes of a store group take 16 different rows (fwd) or 4 rows x 4 blocks
  // (bwd)
  const int tq = tid & 255, t_half = tid >> 8;
  const int t_row = BWD ? (tq >> 2) : tq;
  const int t_col = BWD ? (tq & 3) * 64 : 0;
  const bool t_ok = BWD ? (c0 + t_col < a.Kw) : (c0 + t_row < a.Nw);
  const int64_t t_n = BWD ? 0 : (t_ok ? c0 + t_row : a.Nw - 1);
  const int64_t t_k = BWD ? (t_ok ? c0 + t_col : a.Kw - 64) : 0;

  floatx16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  uint4 xr[XCH];
  uint4 cwA[CW], cwB[CW];
  uint8_t qbA = 0, qbB = 0;
  float sfA = 0.0f, sfB = 0.0f;

  auto x_src = [&](int i, int kt) -> const uint16_t* {
    const int id = tid + V6_T * i, row = id >> 3, ch = id & 7;
    const int64_t m = m0 + row < a.M ? m0 + row : a.M - 1;
    return a.act + m * a.L + (int64_t)kt * 64 + ch * 8;
  };
  auto x_dst = [&](int i, int buf) -> __bf16* {
    const int id = tid + V6_T * i, row = id >> 3, ch = id & 7;
    return &sA[buf][row * PK + ch * 8];
  };
  auto load_codes = [&](int kt, uint4* c, uint8_t& q, float& f) {
    const int64_t n = BWD ? (int64_t)kt * 64 + t_row : t_n;
    const int64_t k = BWD ? t_k : (int64_t)kt * 64;
    if (I8) {  // one byte per weight
      const uint8_t* src = a.codes + n * a.Kw + k + 32 * t_half;
      c[0] = *reinterpret_cast<const uint4*>(src);
      c[CW - 1] = *reinterpret_cast<const uint4*>(src + 16);
    } else {
      c[0] = *reinterpret_cast<const uint4*>(a.codes + ((n * a.Kw + k) >> 1) + 16 * t_half);
    }
    const int64_t blk = n * kblocks + (k >> 6);
    if (DQ) {
      q = a.dq.absmax_q[blk];
      f = a.dq.scale2[blk >> 8];
    } else {
      f = a.dq.absmax[blk];
    }
  };
  // backward: chunk w of the thread's half-block goes to its permuted place
  // (see bwd_tile_col)
  const int t_swz = ((t_col >> 6) + 2 * ((t_row >> 1) & 1)) & 3;
  auto wdst = [&](int buf, int w) -> __bf16* {
    return BWD ? &sB[buf][t_row * PRC + t_col + 32 * t_half + 8 * (w ^ t_swz)]
               : &sB[buf][t_row * PK + t_col + 32 * t_half + 8 * w];
  };

  bf16x8 fa[2][4], fb[2][2];
  // reads in the order the MFMAs consume them (a0, b0, b1, a1..a3)
  auto read_frags = [&](int buf, int kk, int slot, bool b_rc, int pitch_b) {
    fa[slot][0] = frag_kc(sA[buf], PK, wm * 128, kk, lane);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      __builtin_amdgcn_sched_barrier(0);
      fb[slot][j] = b_rc ? (BWD ? frag_rc_bwd(sB[buf], pitch_b, wn * 64 + 32 * j, kk, lane)
                                : frag_rc(sB[buf], pitch_b, wn * 64 + 32 * j, kk, lane))
                         : frag_kc(sB[buf], pitch_b, wn * 64 + 32 * j, kk, lane);
    }
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      fa[slot][i] = frag_kc(sA[buf], PK, wm * 128 + 32 * i, kk, lane);
    }
  };

  // ---- one k-step: multiply stage `cur` while producing stage `nxt`
  auto step = [&](int kt, const int cur, const uint4* cu, uint8_t qu, float fu, uint4* cl, uint8_t& ql, float& fl) {
    const int nxt = cur ^ 1;
    const int k2 = kt + 2 < nk ? kt + 2 : nk - 1;  // past the end: a harmless repeat
    // 4-bit codes: 4 words of 8 codes; Int8: 8 words of 4 codes
    const uint32_t words[8] = {cu[0].x,      cu[0].y,      cu[0].z,      cu[0].w,
                               cu[CW - 1].x, cu[CW - 1].y, cu[CW - 1].z, cu[CW - 1].w};
    float sc = 0.0f;
    uint32_t pw[8];
    BlockLUT lut;
    WordState ws[4];
    load_codes(k2, cl, ql, fl);
    read_frags(cur, 0, 0, BWD, BWD ? PRC : PK);
    __builtin_amdgcn_sched_barrier(0);
    // items 0..32 interleaved with the 32 MFMAs, in order (slot 0 takes
    // items 0 and 1, slot s item s + 1).  Int8: item 0 forms the block's
    // constant, items 9..24 expand 2 code bytes each (the 8 weights of
    // 16-byte chunk w in items 9 + 4w .. 12 + 4w, the last one storing them)
    auto item = [&](int it) {
      if (I8 && it < 9) {
        if (it == 0) {
          const float bs = DQ ? __fadd_rn(__fmul_rn(e4m3_decode(qu), fu), mu) : fu;
          sc = t_ok ? bs : 0.0f;
        }
      } else if (I8 && it < 9 + 16) {
        const int w = (it - 9) >> 2, stg = (it - 9) & 3;
        const uint32_t wd = words[2 * w + (stg >> 1)] >> (16 * (stg & 1));
        pw[stg] = pack_bf2(i8_value(wd & 0xFFu) * sc, i8_value((wd >> 8) & 0xFFu) * sc);
        if (stg == 3) sts16(wdst(nxt, w), make_uint4(pw[0], pw[1], pw[2], pw[3]));
      } else if (it == 0) {
        const float bs = DQ ? __fadd_rn(__fmul_rn(e4m3_decode(qu), fu), mu) : fu;
        sc = t_ok ? bs : 0.0f;
        pw[0] = pack_bf2(cv[0] * sc, cv[1] * sc);
      } else if (it <= 7) {
        pw[it] = pack_bf2(cv[2 * it] * sc, cv[2 * it + 1] * sc);
      } else if (it == 8) {
        lut = make_lut(pw);
      } else if (it < 9 + 16) {
        const int w = (it - 9) >> 2, stg = (it - 9) & 3;
        WordState& st = ws[w];
        const uint32_t wd = words[w];
        if (stg == 0) {
          st.e7 = wd & 0x07070707u;
          st.o7 = (wd >> 4) & 0x07070707u;
          const uint32_t t3 = wd >> 3;
          st.me = lut_half_sel(t3);
          st.mo = lut_half_sel(t3 >> 4);
        } else if (stg == 1) {
          st.loE = perm_b32(perm_b32(lut.lo[3], lut.lo[2], st.e7), perm_b32(lut.lo[1], lut.lo[0], st.e7), st.me);
          st.hiE = perm_b32(perm_b32(lut.hi[3], lut.hi[2], st.e7), perm_b32(lut.hi[1], lut.hi[0], st.e7), st.me);
        } else if (stg == 2) {
          st.loO = perm_b32(perm_b32(lut.lo[3], lut.lo[2], st.o7), perm_b32(lut.lo[1], lut.lo[0], st.o7), st.mo);
          st.hiO = perm_b32(perm_b32(lut.hi[3], lut.hi[2], st.o7), perm_b32(lut.hi[1], lut.hi[0], st.o7), st.mo);
        } else {
          const uint32_t e01 = perm_b32(st.hiE, st.loE, 0x05010400u);
          const uint32_t o01 = perm_b32(st.hiO, st.loO, 0x05010400u);
          const uint32_t e23 = perm_b32(st.hiE, st.loE, 0x07030602u);
          const uint32_t o23 = perm_b32(st.hiO, st.loO, 0x07030602u);
          sts16(wdst(nxt, w), make_uint4(perm_b32(o01, e01, 0x05040100u), perm_b32(o01, e01, 0x07060302u),
                                         perm_b32(o23, e23, 0x05040100u), perm_b32(o23, e23, 0x07060302u)));
        }
      } else if (it < 25 + XCH) {
        const int i = it - 25;
        sts16(x_dst(i, nxt), xr[i]);
      } else if (it < 25 + 2 * XCH) {
        const int i = it - 25 - XCH;
        xr[i] = ldg16(x_src(i, k2));
      }
    };
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int slot = kk & 1;
#pragma unroll
      for (int ij = 0; ij < 8; ++ij) {
        const int i = ij >> 1, j = ij & 1;
        acc[i][j] = mfma32(fb[slot][j], fa[slot][i], acc[i][j]);
        if (ij == 0 && kk < 3) {  // after the sub-step's first MFMA, whose reads come first
          __builtin_amdgcn_sched_barrier(0);
          read_frags(cur, 16 * (kk + 1), slot ^ 1, BWD, BWD ? PRC : PK);
        }
        const int sl = kk * 8 + ij;
        if (sl == 0) {
          item(0);
          item(1);
        } else {
          item(sl + 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
  };

  // ---- adapter term first, over bf16 operands (both stages are free), masked
  // for LoRA dropout before the weight term is added
  for (int64_t jt = 0; last_range && jt < a.rp; jt += 64) {
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
      const int id = tid + V6_T * i, row = id >> 3, ch = id & 7;
      const int64_t m = m0 + row;
      sts16(&sA[0][row * PK + ch * 8], (m < a.M) ? ldg16(a.ext_act + m * a.rp + jt + ch * 8) : make_uint4(0, 0, 0, 0));
    }
    if (!BWD) {  // B [r, Nw]: tile [64 j][BN n], read transposed
#pragma unroll
      for (int i = 0; i < BN * 8 / V6_T; ++i) {
        const int id = tid + V6_T * i, row = id / (BN / 8), ch = id % (BN / 8);
        sts16(&sB[0][row * PRC + ch * 8], load8_masked(a.ext_w, a.Nw, jt + row, a.r, c0 + ch * 8, a.Nw));
      }
    } else {     // A [Kw, r]: tile [BN k][64 j]
#pragma unroll
      for (int i = 0; i < BN * 8 / V6_T; ++i) {
        const int id = tid + V6_T * i, row = id >> 3, ch = id & 7;
        sts16(&sB[0][row * PK + ch * 8], load8_masked(a.ext_w, a.r, c0 + row, a.Kw, jt + ch * 8, a.r));
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 64; kk += 16) {
      read_frags(0, kk, 0, !BWD, BWD ? PK : PRC);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mfma32(fb[0][j], fa[0][i], acc[i][j]);
    }
    __syncthreads();
  }

  if (BWD && a.keep && last_range) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        mask_acc32t(acc[i][j], lane, m0 + wm * 128 + 32 * i, c0 + wn * 64 + 32 * j, a.M, a.ncols, a.keep,
                    a.keep_scale);
  }

  // ---- prologue: stage 0 filled; X(ks+1) and codes(ks+1) in flight
  load_codes(ks, cwB, qbB, sfB);
#pragma unroll
  for (int i = 0; i < XCH; ++i) xr[i] = ldg16(x_src(i, ks));
#pragma unroll
  for (int i = 0; i < XCH; ++i) sts16(x_dst(i, 0), xr[i]);
  {
    const float bs = DQ ? __fadd_rn(__fmul_rn(e4m3_decode(qbB), sfB), mu) : sfB;
    const float c = t_ok ? bs : 0.0f;
    if (I8) {
      const uint32_t words[8] = {cwB[0].x, cwB[0].y, cwB[0].z, cwB[0].w,
                                 cwB[CW - 1].x, cwB[CW - 1].y, cwB[CW - 1].z, cwB[CW - 1].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t o[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t cwd = words[2 * w + h];
          o[2 * h] = pack_bf2(i8_value(cwd & 0xFFu) * c, i8_value((cwd >> 8) & 0xFFu) * c);
          o[2 * h + 1] = pack_bf2(i8_value((cwd >> 16) & 0xFFu) * c, i8_value(cwd >> 24) * c);
        }
        sts16(wdst(0, w), make_uint4(o[0], o[1], o[2], o[3]));
      }
    } else {
      const BlockLUT lut = lut_for(c, cv);
      const uint32_t words[4] = {cwB[0].x, cwB[0].y, cwB[0].z, cwB[0].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t o[4];
        lut_lookup8(lut, words[w], o);
        sts16(wdst(0, w), make_uint4(o[0], o[1], o[2], o[3]));
      }
    }
  }
  load_codes(ks + 1 < nk ? ks + 1 : ks, cwA, qbA, sfA);
#pragma unroll
  for (int i = 0; i < XCH; ++i) xr[i] = ldg16(x_src(i, ks + 1 < nk ? ks + 1 : ks));
  __syncthreads();

  for (int kt = ks; kt < nk; kt += 2) {
    step(kt, 0, cwA, qbA, sfA, cwB, qbB, sfB);
    if (kt + 1 < nk) step(kt + 1, 1, cwB, qbB, sfB, cwA, qbA, sfA);
  }

  // ---- epilogue: bf16 output, or the fp32 partial tile of a split unit
  __builtin_amdgcn_sched_barrier(0);
  if (unit >= 0) {
    float* pt = a.part + (int64_t)unit * (BM * BN);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) store_acc32t_f32(acc[i][j], lane, wm * 128 + 32 * i, wn * 64 + 32 * j, pt, BN);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (c0 + wn * 64 + 32 * j < a.ncols)
          store_acc32t(acc[i][j], lane, m0 + wm * 128 + 32 * i, c0 + wn * 64 + 32 * j, a.M, a.ncols, a.out);
  }
}

// Adds the `split` fp32 partial tiles of each split tile (fixed order) and
// writes the bf16 result.  Thread: 4 consecutive columns of one tile row.
__global__ __launch_bounds__(256) void main_fixup_kernel(const float* __restrict__ part, int split, int full_tiles,
                                                         int tn, int64_t M, int64_t ncols, uint16_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;  // over R * 256 * 64
  const int64_t t = idx >> 14, rem = idx & 16383;
  const int r = (int)(rem >> 6), c = (int)(rem & 63) * 4;
  const int lid = full_tiles + (int)t;
  const int64_t row = (int64_t)(lid / tn) * 256 + r, col0 = (int64_t)(lid % tn) * 256 + c;
  float4 sum = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int sp = 0; sp < split; ++sp) {
    const float4 v = *reinterpret_cast<const float4*>(part + ((t * split + sp) << 16) + r * 256 + c);
    sum.x += v.x; sum.y += v.y; sum.z += v.z; sum.w += v.w;
  }
  if (row >= M) return;
  const float sv[4] = {sum.x, sum.y, sum.z, sum.w};
  if (col0 + 4 <= ncols && (ncols & 3) == 0) {
    *reinterpret_cast<uint2*>(out + row * ncols + col0) = make_uint2(pack_bf2(sv[0], sv[1]), pack_bf2(sv[2], sv[3]));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col0 + e < ncols) out[row * ncols + col0 + e] = f2bf(sv[e]);
  }
}

// ====================================================== skinny products
// part[s][m][q] = sum over the s-th reduction chunk of U[m, l] * V(l, q),
// tile 64 (M) x 64 (Q), waves 2 x 2 of one 32x32 MFMA tile each, 128
// reduction indices per iteration with the next iteration's loads in flight.
//   NN: V(l, q) = V[l * Q + q]   (A [K, r] for XA)   -> tile [128 l][64 q], transposed reads
//   NT: V(l, q) = V[q * L + l]   (B [r, N] for dY B^T) -> tile [64 q][128 l]
constexpr int SK_PU = SK_BK + 8;   // [64][128] reduction-contiguous pitch
constexpr int SK_PV = 64 + kRcPad; // [128][64] transposed-read pitch

template <bool NN>
__global__ __launch_bounds__(NT) void skinny_kernel(const uint16_t* __restrict__ U, int64_t M, int64_t L,
                                                    const uint16_t* __restrict__ V, int64_t Q, int64_t chunk,
                                                    float* __restrict__ part, int64_t QP,
                                                    const uint8_t* __restrict__ keep) {
  constexpr int SV = NN ? SK_BK * SK_PV : 64 * SK_PU;
  __shared__ __attribute__((aligned(16))) __bf16 sU[64 * SK_PU];
  __shared__ __attribute__((aligned(16))) __bf16 sV[SV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t q0 = (int64_t)blockIdx.x * 64, m0 = (int64_t)blockIdx.y * 64;
  const int64_t lbeg = (int64_t)blockIdx.z * chunk;
  const int64_t lend = lbeg + chunk < L ? lbeg + chunk : L;
  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  uint4 ru[4], rv[4];
  uint32_t kb[4] = {0xFFu, 0xFFu, 0xFFu, 0xFFu};  // keep bits of the U chunks (dropout)
  const int64_t kpitch = L >> 3;
  // whole, aligned tiles (the usual case) load without per-element checks, so
  // that all loads of a tile are in flight together
  const bool inner = m0 + 64 <= M && q0 + 64 <= Q && (L & 7) == 0 && (Q & 7) == 0;
  auto load = [&](int64_t lt) {
    if (inner && lt + SK_BK <= lend) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int id = tid + NT * i;
        ru[i] = ldg16(U + (m0 + (id >> 4)) * L + lt + (id & 15) * 8);
        if (keep) kb[i] = keep[(m0 + (id >> 4)) * kpitch + ((lt >> 3) + (id & 15))];
        rv[i] = NN ? ldg16(V + (lt + (id >> 3)) * Q + q0 + (id & 7) * 8)
                   : ldg16(V + (q0 + (id >> 4)) * L + lt + (id & 15) * 8);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + NT * i;
      {  // U tile [64 m][128 l]
        const int row = id >> 4, ch = id & 15;
        const int64_t m = m0 + row, l = lt + ch * 8;
        ru[i] = (m < M && l < lend) ? ldg16(U + m * L + l) : make_uint4(0, 0, 0, 0);
        if (keep && m < M && l < lend) kb[i] = keep[m * kpitch + (l >> 3)];
      }
      if (NN) {  // V tile [128 l][64 q]
        const int row = id >> 3, ch = id & 7;
        rv[i] = (lt + row < lend) ? load8_masked(V, Q, lt + row, L, q0 + ch * 8, Q) : make_uint4(0, 0, 0, 0);
      } else {   // V tile [64 q][128 l]
        const int row = id >> 4, ch = id & 15;
        rv[i] = (lt + ch * 8 < lend) ? load8_masked(V, L, q0 + row, Q, lt + ch * 8, L) : make_uint4(0, 0, 0, 0);
      }
    }
  };
  if (lbeg < lend) load(lbeg);
  for (int64_t lt = lbeg; lt < lend; lt += SK_BK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int id = tid + NT * i;
      sts16(&sU[(id >> 4) * SK_PU + (id & 15) * 8], keep ? apply_keep8(ru[i], kb[i]) : ru[i]);
      if (NN) sts16(&sV[(id >> 3) * SK_PV + (id & 7) * 8], rv[i]);
      else sts16(&sV[(id >> 4) * SK_PU + (id & 15) * 8], rv[i]);
    }
    __syncthreads();
    if (lt + SK_BK < lend) load(lt + SK_BK);
#pragma unroll
    for (int kk = 0; kk < SK_BK; kk += 16) {
      const bf16x8 af = frag_kc(sU, SK_PU, wm * 32, kk, lane);
      const bf16x8 bv = NN ? frag_rc(sV, SK_PV, wn * 32, kk, lane) : frag_kc(sV, SK_PU, wn * 32, kk, lane);
      acc = mfma32(af, bv, acc);
    }
    __syncthreads();
  }
  float* out = part + (int64_t)blockIdx.z * M * QP;
  const int64_t col = q0 + wn * 32 + (lane & 31);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int64_t row = m0 + wm * 32 + acc_row32(e, lane);
    if (row < M) out[row * QP + col] = acc[e];
  }
}

// out1[m][q] = bf16(sum_s part) for q < Q (optional); out2[m][q] =
// bf16(alpha * sum_s part) for q < QP (columns >= Q are zero partials).
// ------------------------------------------------- split-sum reductions
// Both adapter reductions add S fp32 partial slices element by element.  A
// chunk is 4 consecutive elements; T threads share a chunk (thread t adds
// slices t, t + T, ...), and their T partial sums are then added in LDS in a
// fixed order, so the result does not depend on timing.  T grows when there
// are few chunks and many slices (few tokens), keeping the latency chain of
// one thread short.

// 4 elements of slice k at idx (elements beyond n read as 0).
__device__ __forceinline__ float4 slice4(const float* part, int64_t k, int64_t n, int64_t idx) {
  const float* p = part + k * n + idx;
  if ((n & 3) == 0) return *reinterpret_cast<const float4*>(p);
  float4 v;
  v.x = p[0];
  v.y = idx + 1 < n ? p[1] : 0.0f;
  v.z = idx + 2 < n ? p[2] : 0.0f;
  v.w = idx + 3 < n ? p[3] : 0.0f;
  return v;
}

// Sum over the S slices of the chunk at idx; the total is valid in t == 0.
template <int T>
__device__ __forceinline__ float4 split_sum4(const float* part, int S, int64_t n, int64_t idx, bool ok, int t,
                                             float4* red) {
  float4 s = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if (ok) {
#pragma unroll 4
    for (int k = t; k < S; k += T) {
      const float4 v = slice4(part, k, n, idx);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  }
  if (T == 1) return s;
  red[threadIdx.x] = s;
  __syncthreads();
  if (t == 0) {
    constexpr int CPW = 256 / T;
    for (int u = 1; u < T; ++u) {
      const float4 v = red[threadIdx.x + u * CPW];
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  }
  return s;
}

// XA-style epilogue: out2 [M, QP] = bf16(alpha * C) (C zero in columns
// >= Q) and out1 [M, Q] = bf16(scale1 * C), each when given.  part is
// [S][M][QP], QP % 64 == 0.
template <int T>
__global__ __launch_bounds__(256) void skinny_epilogue_kernel(const float* __restrict__ part, int S, int64_t M,
                                                              int64_t Q, int64_t QP, uint16_t* __restrict__ out1,
                                                              uint16_t* __restrict__ out2, float alpha,
                                                              float scale1) {
  __shared__ float4 red[T > 1 ? 256 : 1];
  constexpr int CPW = 256 / T;
  const int t = threadIdx.x / CPW;
  const int64_t idx = ((int64_t)blockIdx.x * CPW + threadIdx.x % CPW) * 4;
  const bool ok = idx < M * QP;
  const float4 s = split_sum4<T>(part, S, M * QP, idx, ok, t, red);
  if (!ok || t != 0) return;
  const int64_t m = idx / QP, q = idx - m * QP;
  const float sv[4] = {s.x, s.y, s.z, s.w};
  if (out2) {
    uint2 o;
    o.x = pack_bf2(alpha * sv[0], alpha * sv[1]);
    o.y = pack_bf2(alpha * sv[2], alpha * sv[3]);
    *reinterpret_cast<uint2*>(out2 + idx) = o;
  }
  if (out1) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (q + e < Q) out1[m * Q + q + e] = f2bf(scale1 * sv[e]);
  }
}

// ============================================== token-reduction products
// part[s][p][q] = sum over tokens m of chunk s of U[m, p] * V[m, q]
// (U [M, P] and V [M, Q] row-major, leading dimensions ldu, ldv).  Tile
// BP x BQ, waves 2 x 2; 128 tokens per iteration, next iteration's loads in
// flight; both tiles are staged as [128 m][cols] and read transposed.

struct TnProblem {
  const uint16_t* U;
  const uint16_t* V;
  int64_t ldu, ldv, P, Q, M, chunk;
  float* part;          // [splits][P][Q]
  const uint8_t* keep;  // dropout bit mask [M, ldu/8] of U, or null
};

template <int BP, int BQ>
__global__ __launch_bounds__(NT) void tn_kernel(const TnProblem pa, const TnProblem pb, int za) {
  // grid z below za: the splits of problem pa; from za on: those of pb
  const bool second = (int)blockIdx.z >= za;
  const TnProblem& pr = second ? pb : pa;
  const int64_t bz = second ? blockIdx.z - za : blockIdx.z;
  const uint16_t* __restrict__ U = pr.U;
  const uint16_t* __restrict__ V = pr.V;
  const int64_t ldu = pr.ldu, ldv = pr.ldv, P = pr.P, Q = pr.Q, M = pr.M, chunk = pr.chunk;
  float* __restrict__ part = pr.part;
  const uint8_t* __restrict__ keep = pr.keep;
  if ((int64_t)blockIdx.x * BP >= P || (int64_t)blockIdx.y * BQ >= Q) return;  // outside this problem's grid
  constexpr int PU = BP + kRcPad, PV = BQ + kRcPad;
  constexpr int TMW = BP / 64, TNW = BQ / 64;
  constexpr int CU_ = TN_BK * BP / 8 / NT, CV_ = TN_BK * BQ / 8 / NT;  // chunks per thread
  __shared__ __attribute__((aligned(16))) __bf16 sU[TN_BK * PU];
  __shared__ __attribute__((aligned(16))) __bf16 sV[TN_BK * PV];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t p0 = (int64_t)blockIdx.x * BP, q0 = (int64_t)blockIdx.y * BQ;
  const int64_t mbeg = bz * chunk;
  const int64_t mend = mbeg + chunk < M ? mbeg + chunk : M;
  floatx16 acc[TMW][TNW];
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  uint4 ru[CU_], rv[CV_];
  uint32_t kb[CU_];  // keep bits of the U chunks (dropout)
#pragma unroll
  for (int i = 0; i < CU_; ++i) kb[i] = 0xFFu;
  const int64_t kpitch = ldu >> 3;
  // whole, aligned tiles (the usual case) load without per-element checks, so
  // that all loads of a tile are in flight together
  const bool inner = p0 + BP <= P && q0 + BQ <= Q && (ldu & 7) == 0 && (ldv & 7) == 0;
  auto load = [&](int64_t mt) {
    if (inner && mt + TN_BK <= mend) {
#pragma unroll
      for (int i = 0; i < CU_; ++i) {
        const int id = tid + NT * i, row = id / (BP / 8), ch = id % (BP / 8);
        ru[i] = ldg16(U + (mt + row) * ldu + p0 + ch * 8);
        if (keep) kb[i] = keep[(mt + row) * kpitch + ((p0 >> 3) + ch)];
      }
#pragma unroll
      for (int i = 0; i < CV_; ++i) {
        const int id = tid + NT * i, row = id / (BQ / 8), ch = id % (BQ / 8);
        rv[i] = ldg16(V + (mt + row) * ldv + q0 + ch * 8);
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < CU_; ++i) {
      const int id = tid + NT * i, row = id / (BP / 8), ch = id % (BP / 8);
      ru[i] = load8_masked(U, ldu, mt + row, mend, p0 + ch * 8, P);
      if (keep && mt + row < mend && p0 + ch * 8 < P) kb[i] = keep[(mt + row) * kpitch + ((p0 >> 3) + ch)];
    }
#pragma unroll
    for (int i = 0; i < CV_; ++i) {
      const int id = tid + NT * i, row = id / (BQ / 8), ch = id % (BQ / 8);
      rv[i] = load8_masked(V, ldv, mt + row, mend, q0 + ch * 8, Q);
    }
  };
  if (mbeg < mend) load(mbeg);
  for (int64_t mt = mbeg; mt < mend; mt += TN_BK) {
#pragma unroll
    for (int i = 0; i < CU_; ++i) {
      const int id = tid + NT * i;
      sts16(&sU[(id / (BP / 8)) * PU + (id % (BP / 8)) * 8], keep ? apply_keep8(ru[i], kb[i]) : ru[i]);
    }
#pragma unroll
    for (int i = 0; i < CV_; ++i) {
      const int id = tid + NT * i;
      sts16(&sV[(id / (BQ / 8)) * PV + (id % (BQ / 8)) * 8], rv[i]);
    }
    __syncthreads();
    if (mt + TN_BK < mend) load(mt + TN_BK);
#pragma unroll
    for (int kk = 0; kk < TN_BK; kk += 16) {
      bf16x8 af[TMW], bv[TNW];
#pragma unroll
      for (int i = 0; i < TMW; ++i) af[i] = frag_rc(sU, PU, wm * (BP / 2) + 32 * i, kk, lane);
#pragma unroll
      for (int j = 0; j < TNW; ++j) bv[j] = frag_rc(sV, PV, wn * (BQ / 2) + 32 * j, kk, lane);
#pragma unroll
      for (int i = 0; i < TMW; ++i)
#pragma unroll
        for (int j = 0; j < TNW; ++j) acc[i][j] = mfma32(af[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  float* out = part + bz * P * Q;
#pragma unroll
  for (int i = 0; i < TMW; ++i)
#pragma unroll
    for (int j = 0; j < TNW; ++j) {
      const int64_t col = q0 + wn * (BQ / 2) + 32 * j + (lane & 31);
      if (col >= Q) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = p0 + wm * (BP / 2) + 32 * i + acc_row32(e, lane);
        if (row < P) out[row * Q + col] = acc[i][j][e];
      }
    }
}

// out[p][q] = bf16(alpha * sum_s part[s][p][q]), part [S][P][Q], out [P][Q].
// out [PQ] = bf16(alpha * sum of the S slices of part [S][PQ]).
// Token-reduction epilogue for up to two problems (blocks [0, nblk_a) take
// problem a): out = bf16(alpha * sum of the S partial slices [P][Q]), written
// as [P][Q], or as [Q][P] when `trans`.
struct TnOut {
  const float* part;
  int S;
  int64_t P, Q;
  uint16_t* out;
  float alpha;
  int trans;
  int accumulate;  // out = bf16(out + alpha * sum) instead of bf16(alpha * sum)
};

template <int T>
__global__ __launch_bounds__(256) void tn_reduce_kernel(const TnOut oa, const TnOut ob, int nblk_a) {
  __shared__ float4 red[T > 1 ? 256 : 1];
  constexpr int CPW = 256 / T;
  const bool second = (int)blockIdx.x >= nblk_a;
  const TnOut& o = second ? ob : oa;
  const int64_t bx = second ? blockIdx.x - nblk_a : blockIdx.x;
  const int64_t PQ = o.P * o.Q;
  const int t = threadIdx.x / CPW;
  const int64_t idx = (bx * CPW + threadIdx.x % CPW) * 4;
  const bool ok = idx < PQ;
  const float4 s = split_sum4<T>(o.part, o.S, PQ, idx, ok, t, red);
  if (!ok || t != 0) return;
  const float sv[4] = {s.x, s.y, s.z, s.w};
  // the bf16 value of element e: alpha * sum, plus the old value when accumulating
  auto val = [&](int e, int64_t at) -> uint16_t {
    const float v = o.alpha * sv[e];
    return f2bf(o.accumulate ? bf2f(o.out[at]) + v : v);
  };
  if (o.trans) {
    for (int e = 0; e < 4 && idx + e < PQ; ++e) {
      const int64_t p = (idx + e) / o.Q, q = (idx + e) - p * o.Q;
      o.out[q * o.P + p] = val(e, q * o.P + p);
    }
  } else if (idx + 4 <= PQ && (PQ & 3) == 0) {
    uint2 w;
    w.x = (uint32_t)val(0, idx) | ((uint32_t)val(1, idx + 1) << 16);
    w.y = (uint32_t)val(2, idx + 2) | ((uint32_t)val(3, idx + 3) << 16);
    *reinterpret_cast<uint2*>(o.out + idx) = w;
  } else {
    for (int e = 0; e < 4 && idx + e < PQ; ++e) o.out[idx + e] = val(e, idx + e);
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint16_t* __restrict__ dst, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < n) dst[idx] = 0;
}

// ================================ small-token forward (M <= kGemvMaxM)
// With a handful of tokens the forward is a stream over the packed weight
// (0.516 bytes per parameter), and the per-block scaled bf16 table of the
// large kernels (about 4 VALU operations per weight) would cost more than
// the weight's HBM time: the codes are looked up unscaled and each block's
// constant scales the fp32 MFMA result instead.
//
// Staged small-token forward.  The packed weight is read in full 128-byte
// lines: a workgroup owns 256 weight rows and walks its reduction split in
// chunks of 4 blocks (128 bytes of every row); each thread loads 16-byte
// pieces, so one load instruction covers 8 rows x 128 bytes.  The chunk goes
// to LDS with the 16-byte pieces of row r XOR-permuted by (r / 2) % 8, so the
// MFMA-layout reads below (16 rows x 8 bytes per half wave) hit 64 distinct
// banks.  The chunk's block constants travel with it (one row's four
// blocks per thread of the first four waves, decoded to fp32 as they are
// stored); with double quantisation and splits of at most G3_PREMAX
// chunks their E4M3 bytes come from an LDS copy of the whole split's bytes,
// loaded once at the start as contiguous runs of each row, instead of
// three scattered loads per chunk.  Three chunks are in
// flight in registers (a set's codes are reloaded as soon as they are in LDS,
// its activations once they have been used), LDS is double buffered, and one
// barrier per chunk orders the two.
//
// Code lookup: a byte (two codes) indexes a table of the two unscaled bf16
// codebook values.  The table is held once per LDS bank (entry e of copy l at
// word 64e + l) and lane l reads copy l % 64, so a lookup instruction never
// has a bank conflict; one v_perm_b32 builds its address from the code byte
// and the lane.
//
// Product (16x16x32 MFMA, tokens = the 16 rows of the A operand, rows >= M
// repeat token M-1 and are never stored): wave w takes block w % 4 of every
// chunk for rows 128 (w / 4) .. +127.  Lane (c, g) = (lane % 16, lane / 16)
// holds the codes 16g .. 16g+15 of its row's block (8 bytes); MFMA s of a
// block takes codes 16g + 8s .. +7 in reduction slots 8g .. 8g+7, so two MFMAs
// sum exactly that block's 64 products before its constant scales them.  The
// activation fragment of lane (t, g) is X[t][64b + 16g + 8s .. +7].  The
// codebook value, not its product with c2_hat, is rounded to bf16; the error
// is of the same size as rounding the product.  The partial tiles of the four
// waves that share rows are added in LDS at the end, giving fp32 partials
// part[S][M][N].
constexpr int G3_WAVES = 8;
constexpr int G3_T = G3_WAVES * 64;
constexpr int G3_RT = G3_ROWS * G3_CB / (16 * G3_WAVES);  // 16-row tiles per wave (8)
constexpr int G3_CHUNK16 = G3_ROWS * 2 * G3_CB;  // 16-byte pieces per chunk (2048)
constexpr int G3_LPT = G3_CHUNK16 / G3_T;        // piece loads per thread per chunk (4)
constexpr int G3_D = 3;                          // chunks in flight in registers
constexpr int G3_XA4 = 14;                       // an X A chunk's cost in code chunks, times 4 (measured)
constexpr int G3_PREMAX = 16;                    // longest split whose E4M3 bytes are preloaded
static_assert(G3_T == 2 * G3_ROWS && G3_CB == 4, "threads 0 .. G3_ROWS - 1 take a row's 4 block constants");
static_assert(G3_CB * kGemvMaxM * G3_ROWS * 4 <= 2 * G3_CHUNK16 * 16, "reduction buffer aliases the stages");

// Native 4 x u32 vectors (not HIP's uint4 struct), so that copies between
// global memory, registers and LDS stay plain vector loads and stores.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <bool DQ>
struct G3Set {
  u32x4 c[G3_LPT];  // this thread's code pieces of one chunk
  u32x4 x[2];       // the activations of this wave's block of the chunk
  // constants of this thread's row (threads < G3_ROWS): the fp32 absmax of
  // the chunk's 4 blocks, or (double quantisation) their E4M3 bytes in q4
  // and the second-level scales of the chunk's first and last block (4
  // consecutive blocks lie in at most two groups of 256)
  float f[DQ ? 2 : 4];
  uint32_t q4;
};

// The adapter input of the few-token forward, per reduction chunk: the
// partial X A over the 256 reduction indices of chunk c (fewer in the last
// chunk), xpart[c][m][j] for m < M, j < rp (columns past r are zero).  The
// whole 512-thread workgroup calls it.  The chunk of X (keep-masked for LoRA
// dropout when `keep` is given; rows 16..31 of the MFMA tile repeat row
// M - 1 and are not stored) goes to `lx` as [32][XA_PX] together with the
// first tile of A rows, which pass through `la` (64 KiB) in as few
// [rows][rp + kRcPad] tiles as fit; wave w multiplies column tile w (32
// columns) with 32x32x16 MFMAs in ascending reduction order.  The forward's
// weight-streaming kernel and the backward's recomputation of XA both take
// XA from these partials, so the two are bit-identical.
constexpr int XA_CHUNK = kXaChunk;
constexpr int XA_LDS_A = 65536;             // bytes of the A tiles
constexpr int XA_PX = XA_CHUNK + 8;          // pitch (bf16) of the X tile
constexpr int XA_LDS_X = 32 * XA_PX * 2;     // bytes of the X tile
__device__ __forceinline__ void xa_chunk_partial(const uint16_t* __restrict__ X, int M, int64_t K,
                                                 const uint16_t* __restrict__ A, int r, int rp,
                                                 const uint8_t* __restrict__ keep, int64_t c,
                                                 float* __restrict__ xpart, __bf16* la, __bf16* lx) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int pa = rp + kRcPad, ppr = rp >> 3;  // A tile pitch, 16-byte pieces per A row
  const int64_t kc = c * XA_CHUNK;
  const int rows = (int)(K - kc < XA_CHUNK ? K - kc : XA_CHUNK);  // a multiple of 64 (K % 64 == 0)
  const int rows_pass = 64 * (XA_LDS_A / (64 * pa * 2));           // 256 (rp = 64), 192, 128 or 64 (rp = 256)
  // X: piece q = 512 i + tid is row q / 32 (clamped), columns 8 (q % 32) ..
  uint4 xv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int q = 512 * i + tid, m = q >> 5, kk = 8 * (q & 31);
    const int64_t row = m < M ? m : M - 1;
    if (kk < rows) {
      xv[i] = ldg16(X + row * K + kc + kk);
      if (keep) xv[i] = apply_keep8(xv[i], keep[row * (K >> 3) + ((kc + kk) >> 3)]);
    }
  }
  const bool active = 32 * wave < rp;
  floatx16 acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
  for (int r0 = 0; r0 < rows; r0 += rows_pass) {
    const int nr = rows - r0 < rows_pass ? rows - r0 : rows_pass;
    // A: piece q = 512 i + tid of this tile is row q / ppr, columns 8 (q % ppr) ..
    uint4 av[6];  // rows_pass * ppr <= 6 * 512
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int q = 512 * i + tid;
      if (q < nr * ppr) av[i] = load8_masked(A, r, kc + r0 + q / ppr, K, 8 * (q % ppr), r);
    }
    if (r0) __syncthreads();  // the previous tile has been read
    if (r0 == 0) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int q = 512 * i + tid, kk = 8 * (q & 31);
        if (kk < rows) sts16(&lx[(q >> 5) * XA_PX + kk], xv[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      const int q = 512 * i + tid;
      if (q < nr * ppr) sts16(&la[(q / ppr) * pa + 8 * (q % ppr)], av[i]);
    }
    __syncthreads();
    if (active) {
      for (int kk = 0; kk < nr; kk += 16) {
        const bf16x8 xf = *reinterpret_cast<const bf16x8*>(&lx[(lane & 31) * XA_PX + r0 + kk + 8 * (lane >> 5)]);
        acc = mfma32(xf, frag_rc(la, pa, 32 * wave, kk, lane), acc);
      }
    }
  }
  if (active) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = acc_row32(e, lane);
      if (m < M) xpart[(c * M + m) * rp + 32 * wave + (lane & 31)] = acc[e];
    }
  }
}

// XA partials of every reduction chunk (one workgroup per chunk), for the
// backward's recomputation of the few-token forward's XA.
__global__ __launch_bounds__(512) void xa_chunks_kernel(const uint16_t* __restrict__ X, int M, int64_t K,
                                                        const uint16_t* __restrict__ A, int r, int rp,
                                                        const uint8_t* __restrict__ keep, float* __restrict__ xpart) {
  __shared__ __attribute__((aligned(16))) __bf16 la[XA_LDS_A / 2];
  __shared__ __attribute__((aligned(16))) __bf16 lx[XA_LDS_X / 2];
  xa_chunk_partial(X, M, K, A, r, rp, keep, blockIdx.x, xpart, la, lx);
}

// First chunk of reduction split y of row tile x (split_lo(S) = nchunks):
// the splits whose workgroup also computes an X A chunk (the first nxc
// workgroups, one chunk each when the grid has that many) are G3_XA4 / 4
// chunks shorter, the others longer, so that every workgroup of the tile
// streams for about as long.  T row tiles, S splits.
__host__ __device__ inline int gemv_split_lo(int y, int64_t x, int64_t T, int S, int nchunks, int64_t nxc) {
  const int nx = x < nxc ? (int)((int64_t)S < (nxc - x + T - 1) / T ? (int64_t)S : (nxc - x + T - 1) / T) : 0;
  int x4 = T * S >= nxc ? G3_XA4 : 0;
  if (4 * (int64_t)nchunks - 4 * (int64_t)S < (int64_t)x4 * (S - nx)) x4 = 0;  // every split keeps a chunk
  return (int)((4 * (int64_t)y * nchunks + (int64_t)x4 * ((int64_t)y * nx - (int64_t)S * (y < nx ? y : nx))) /
               (4 * (int64_t)S));
}

// PRE (double quantisation, whole-word constants, splits of at most
// G3_PREMAX chunks): the E4M3 bytes of the workgroup's whole split are
// loaded once at the start, as contiguous runs of each row, into LDS, and
// the row's one or two second-level scales into registers; a chunk step
// then reads its row's word from LDS instead of three scattered loads.
template <bool DQ, bool PRE = false>
__global__ __launch_bounds__(G3_T, 1) void gemv3_kernel(const uint16_t* __restrict__ X, int M, int64_t K,
                                                       const uint8_t* __restrict__ codes, const DQParams dq,
                                                       int64_t N, int S, float* __restrict__ part,
                                                       const uint16_t* __restrict__ lora_a, int rank, int rank_pad,
                                                       const uint8_t* __restrict__ keep, float* __restrict__ xpart) {
  __shared__ uint32_t tab[256 * 64];
  __shared__ u32x4 stage[2][G3_CHUNK16];  // code chunks; the partial tiles at the end
  __shared__ float4 cst[2][G3_ROWS];  // block constants cst[buf][row][block]
  __shared__ uint32_t qpre[PRE ? G3_PREMAX * G3_ROWS : 1];  // E4M3 words qpre[chunk - c_lo][row]
  static_assert(sizeof(stage) >= XA_LDS_A && sizeof(tab) >= XA_LDS_X, "the X A tiles fit in the stages and table");
  static_assert(!PRE || DQ, "preloaded constants are E4M3 bytes");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float* cv = kCodeValues[dq.code_type];

  const int64_t nbk = K >> 6, half_k = K >> 1;
  const int64_t n0 = (int64_t)blockIdx.x * G3_ROWS;
  const int nchunks = (int)((nbk + G3_CB - 1) / G3_CB);
  // the reduction split of this workgroup
  const int64_t nxc = (K + XA_CHUNK - 1) / XA_CHUNK;
  const int c_lo = gemv_split_lo(blockIdx.y, blockIdx.x, gridDim.x, S, nchunks, nxc);
  const int c_hi = gemv_split_lo(blockIdx.y + 1, blockIdx.x, gridDim.x, S, nchunks, nxc);  // c_hi > c_lo
  const float mu = DQ ? *dq.offset : 0.0f;

  // code pieces: load u of thread tid fills LDS slot P = u * G3_T + tid, i.e.
  // row P / 8, slot P % 8, with the row's piece (P % 8) ^ ((row / 2) % 8)
  const uint8_t* gsrc[G3_LPT];
  int gblk[G3_LPT];
#pragma unroll
  for (int u = 0; u < G3_LPT; ++u) {
    const int P = u * G3_T + tid, r = P >> 3;
    const int piece = (P & 7) ^ ((r >> 1) & 7);
    const int64_t row = n0 + r < N ? n0 + r : N - 1;  // rows past N: their constants are zero
    gblk[u] = piece >> 1;
    gsrc[u] = codes + row * half_k + 16 * (piece & 1);
  }
  // constants: threads 0..255 (waves 0..3) take row tid, the chunk's 4
  // blocks; with nbk % 4 == 0 those are one aligned 4-byte word (E4M3) or
  // 16 bytes (fp32) under one second-level scale
  const bool crow_ok = n0 + tid < N;
  const int64_t cbase = (crow_ok ? n0 + tid : N - 1) * nbk;
  const bool cwhole = (nbk & 3) == 0 && ((uintptr_t)(DQ ? (const void*)dq.absmax_q : (const void*)dq.absmax) &
                                            (DQ ? 3 : 15)) == 0;  // uniform
  float fpre[2] = {0.0f, 0.0f};  // PRE: second-level scales of the split's first and last block
  // activations: lane (t, g) of wave w, block w % 4 of the chunk
  const int t = lane & 15, g = lane >> 4, q = wave & 3, hrow = 128 * (wave >> 2);
  const uint16_t* xrow = X + (int64_t)(t < M ? t : M - 1) * K + 16 * g;

  // chunk kc >= c_hi (the pipeline's run-out) reloads chunk c_hi - 1, which
  // is still in L2; blocks past the weight's end reload its last block
  // (their constants are zero)
  auto blk = [&](int kc, int j) -> int64_t {
    const int64_t b = (int64_t)G3_CB * (kc < c_hi ? kc : c_hi - 1) + j;
    return b < nbk ? b : nbk - 1;
  };
  // loads of chunk kc into register set d: the code pieces and constants,
  // then (separately, once the set's activations have been used) the
  // activations
  auto issue_codes = [&](int kc, G3Set<DQ>& d) {
#pragma unroll
    for (int u = 0; u < G3_LPT; ++u) d.c[u] = *reinterpret_cast<const u32x4*>(gsrc[u] + blk(kc, gblk[u]) * 32);
    if (!PRE && tid < G3_ROWS) {
      if constexpr (DQ) {
        if (cwhole) {
          d.q4 = *reinterpret_cast<const uint32_t*>(dq.absmax_q + cbase + blk(kc, 0));
        } else {
          d.q4 = 0;
#pragma unroll
          for (int j = 0; j < 4; ++j) d.q4 |= (uint32_t)dq.absmax_q[cbase + blk(kc, j)] << (8 * j);
        }
        d.f[0] = dq.scale2[(cbase + blk(kc, 0)) >> 8];
        d.f[1] = dq.scale2[(cbase + blk(kc, 3)) >> 8];
      } else if (cwhole) {
        const float4 a = *reinterpret_cast<const float4*>(dq.absmax + cbase + blk(kc, 0));
        d.f[0] = a.x; d.f[1] = a.y; d.f[2] = a.z; d.f[3] = a.w;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) d.f[j] = dq.absmax[cbase + blk(kc, j)];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  auto issue_x = [&](int kc, G3Set<DQ>& d) {
    const uint16_t* xp = xrow + blk(kc, q) * 64;
    d.x[0] = *reinterpret_cast<const u32x4*>(xp);
    d.x[1] = *reinterpret_cast<const u32x4*>(xp + 8);
    __builtin_amdgcn_sched_barrier(0);
  };

  floatx4 acc[G3_RT];
#pragma unroll
  for (int rt = 0; rt < G3_RT; ++rt) acc[rt] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  const uint32_t lane4 = (uint32_t)lane << 2;

  // one chunk: codes and constants of register set d (chunk kc) to LDS
  // buffer kc & 1, the set refilled with the codes of chunk kc + G3_D,
  // barrier, then this wave's block of the chunk for its 128 rows, and the
  // set's activations refilled last
  auto step = [&](int kc, G3Set<DQ>& d) {
    const int sbuf = kc & 1;
#pragma unroll
    for (int u = 0; u < G3_LPT; ++u) stage[sbuf][u * G3_T + tid] = d.c[u];
    if (tid < G3_ROWS) {
      float c[4];
      const uint32_t qp = PRE ? qpre[(kc - c_lo) * G3_ROWS + tid] : 0u;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool ok = crow_ok && (int64_t)G3_CB * kc + j < nbk;
        float v;
        if constexpr (PRE) {
          // the split's blocks lie in at most two groups of 256
          const bool first = ((cbase + (int64_t)G3_CB * kc + j) >> 8) == ((cbase + (int64_t)G3_CB * c_lo) >> 8);
          v = __fadd_rn(__fmul_rn(e4m3_decode((qp >> (8 * j)) & 0xFFu), first ? fpre[0] : fpre[1]), mu);
        } else if constexpr (DQ) {
          const bool first = ((cbase + blk(kc, j)) >> 8) == ((cbase + blk(kc, 0)) >> 8);
          v = __fadd_rn(__fmul_rn(e4m3_decode((d.q4 >> (8 * j)) & 0xFFu), first ? d.f[0] : d.f[1]), mu);
        } else {
          v = d.f[j];
        }
        c[j] = ok ? v : 0.0f;
      }
      cst[sbuf][tid] = make_float4(c[0], c[1], c[2], c[3]);
    }
    issue_codes(kc + G3_D, d);
    __syncthreads();
    const bf16x8 x0 = __builtin_bit_cast(bf16x8, d.x[0]);
    const bf16x8 x1 = __builtin_bit_cast(bf16x8, d.x[1]);
    const int piece = 2 * q + (g >> 1);
    const uint8_t* sb = reinterpret_cast<const uint8_t*>(stage[sbuf]);
    const float* cs = reinterpret_cast<const float*>(cst[sbuf]);
    uint2 cw[G3_RT];
#pragma unroll
    for (int rt = 0; rt < G3_RT; ++rt) {
      const int r = hrow + 16 * rt + t;
      cw[rt] = *reinterpret_cast<const uint2*>(sb + r * 128 + 16 * (piece ^ ((r >> 1) & 7)) + 8 * (g & 1));
    }
    const char* tb = reinterpret_cast<const char*>(tab);
    auto look8 = [&](uint32_t w) -> bf16x8 {
      u32x4 v;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[k] = *reinterpret_cast<const uint32_t*>(tb + __builtin_amdgcn_perm(w, lane4, 0x0C0C0400u + (k << 8)));
      return __builtin_bit_cast(bf16x8, v);
    };
#pragma unroll
    for (int rt = 0; rt < G3_RT; ++rt) {
      const int r = hrow + 16 * rt + t;
      floatx4 p = {0.0f, 0.0f, 0.0f, 0.0f};
      p = mfma16(x0, look8(cw[rt].x), p);
      p = mfma16(x1, look8(cw[rt].y), p);
      const float c = cs[r * G3_CB + q];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[rt][i] = __builtin_fmaf(c, p[i], acc[rt][i]);
    }
    issue_x(kc + G3_D, d);
  };

  G3Set<DQ> A, B, C;  // G3_D register sets in rotation
  // PRE: the split's E4M3 words, loaded first (so that storing them waits
  // for nothing else) as runs of consecutive chunks of each row, and the
  // row's second-level scales of the split's first and last block
  constexpr int QPL = G3_PREMAX * G3_ROWS / G3_T;  // preload words per thread
  uint32_t qv[PRE ? QPL : 1];
  if constexpr (PRE) {
    const int nc = c_hi - c_lo;  // <= G3_PREMAX (the host checks)
#pragma unroll
    for (int k = 0; k < QPL; ++k) {
      const int i = k * G3_T + tid, row = i / nc, c = i - row * nc;
      const int64_t rr = n0 + row < N ? n0 + row : N - 1;
      if (i < G3_ROWS * nc)
        qv[k] = *reinterpret_cast<const uint32_t*>(dq.absmax_q + rr * nbk + (int64_t)G3_CB * (c_lo + c));
    }
    if (tid < G3_ROWS) {
      fpre[0] = dq.scale2[(cbase + (int64_t)G3_CB * c_lo) >> 8];
      fpre[1] = dq.scale2[(cbase + (int64_t)G3_CB * c_hi - 1) >> 8];
    }
  }
  issue_codes(c_lo, A);
  issue_x(c_lo, A);
  issue_codes(c_lo + 1, B);
  issue_x(c_lo + 1, B);
  issue_codes(c_lo + 2, C);
  issue_x(c_lo + 2, C);
  if constexpr (PRE) {
    const int nc = c_hi - c_lo;
#pragma unroll
    for (int k = 0; k < QPL; ++k) {
      const int i = k * G3_T + tid, row = i / nc, c = i - row * nc;
      if (i < G3_ROWS * nc) qpre[c * G3_ROWS + row] = qv[k];
    }
  }

  // while the first chunks are in flight, the first workgroups each take
  // one reduction chunk of X A (more when the grid is smaller than the
  // chunk count), in the space of the code stages and the table
  {
    const int64_t wid = (int64_t)blockIdx.y * gridDim.x + blockIdx.x;
    if (wid < nxc) {
      for (int64_t c = wid; c < nxc; c += (int64_t)gridDim.x * gridDim.y)
        xa_chunk_partial(X, M, K, lora_a, rank, rank_pad, keep, c, xpart, reinterpret_cast<__bf16*>(stage),
                         reinterpret_cast<__bf16*>(tab));
      __syncthreads();  // the tiles have been read before the table and stages are filled
    }
  }

  {
    // table: entry e (a code byte) = the bf16 pair (value[e % 16], value[e / 16]),
    // 64 copies side by side
    u32x4* tv = reinterpret_cast<u32x4*>(tab);
#pragma unroll
    for (int k = 0; k < 256 * 64 / 4 / G3_T; ++k) {
      const int i = k * G3_T + tid, e = i >> 4;
      const uint32_t v = pack_bf2(cv[e & 15], cv[e >> 4]);
      tv[i] = u32x4{v, v, v, v};
    }
  }
  if constexpr (PRE) __syncthreads();  // the preloaded words are in LDS (the first step reads them)

  int kc = c_lo;
  for (; kc + G3_D <= c_hi; kc += G3_D) {
    step(kc, A);
    step(kc + 1, B);
    step(kc + 2, C);
  }
  if (kc < c_hi) step(kc, A);  // the remaining 0..2 chunks (uniform branches)
  if (kc + 1 < c_hi) step(kc + 1, B);
  __syncthreads();  // the stages are free: they hold the partial tiles now

  float* red = reinterpret_cast<float*>(stage);  // [block q][m][G3_ROWS]
#pragma unroll
  for (int rt = 0; rt < G3_RT; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(q * kGemvMaxM + 4 * g + i) * G3_ROWS + hrow + 16 * rt + t] = acc[rt][i];
  __syncthreads();
  for (int o = tid; o < M * G3_ROWS; o += G3_T) {
    const int m = o / G3_ROWS, c = o % G3_ROWS;
    float v = 0.0f;
#pragma unroll
    for (int w = 0; w < G3_CB; ++w) v += red[(w * kGemvMaxM + m) * G3_ROWS + c];
    if (n0 + c < N) part[((int64_t)blockIdx.y * M + m) * N + n0 + c] = v;
  }
}

// Y[m, n] = bf16(sum_s part[s][m][n] + sum_j XAs[m, j] B[j, n]), with the
// adapter input formed here from the fp32 partials of X A, xpart[SX][M][rp]:
// C = sum of the slices, XAs = bf16(alpha C) (columns >= r are zero
// partials), and XA = bf16(scale1 C) [M, r] written by the blocks with
// blockIdx.x == 0 when XA is given.  One token row per blockIdx.y, 4 columns
// per thread (N % 4 == 0), rp <= 256.
// Row m of C = X A from the split partials xpart[SX][M][rp] (256 threads,
// rp <= 256): xas[j] = bf16(alpha C[m, j]) as fp32 for j < rp, and, when XA
// is given, XA[m, j] = bf16(scale1 C[m, j]) for j < r.  Thread (group u,
// column quad c4) adds the slices u, u + G, ... of 4 columns; the G group
// sums are then added in a fixed order.  The forward's small-token path and
// the backward's recomputation of XA both take XA from here, so the two are
// bit-identical.
__device__ __forceinline__ void xa_row(const float* __restrict__ xpart, int SX, int M, int m, int rp, float alpha,
                                       float scale1, int r, uint16_t* __restrict__ XA, float4* xsum, float* xas) {
  const int tid = threadIdx.x;
  const int nq = rp >> 2, G = 256 / nq, c4 = tid % nq, u = tid / nq;
  {
    float4 a = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
    for (int k = u; k < SX; k += G) {
      const float4 v = *reinterpret_cast<const float4*>(xpart + ((int64_t)k * M + m) * rp + 4 * c4);
      a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    }
    xsum[tid] = a;  // tid = u * nq + c4
  }
  __syncthreads();
  for (int j = tid; j < rp; j += 256) {
    const float* xs = reinterpret_cast<const float*>(xsum);
    float c = 0.0f;
    for (int w = 0; w < G; ++w) c += xs[w * rp + j];
    xas[j] = bf2f(f2bf(alpha * c));
    if (XA != nullptr && j < r) XA[(int64_t)m * r + j] = f2bf(scale1 * c);
  }
}

// XA [M, r] = bf16(scale1 * X A) from the split partials (one token row per
// workgroup).
__global__ __launch_bounds__(256) void xa_reduce_kernel(const float* __restrict__ xpart, int SX, int M, int rp,
                                                        float scale1, int r, uint16_t* __restrict__ XA) {
  __shared__ float4 xsum[256];
  __shared__ float xas[256];
  xa_row(xpart, SX, M, blockIdx.x, rp, 1.0f, scale1, r, XA, xsum, xas);
}

__global__ __launch_bounds__(256) void gemv_reduce_kernel(const float* __restrict__ part, int S, int M, int64_t N,
                                                          const float* __restrict__ xpart, int SX, int rp,
                                                          float alpha, float scale1, const uint16_t* __restrict__ B,
                                                          int r, uint16_t* __restrict__ Y,
                                                          uint16_t* __restrict__ XA) {
  __shared__ float4 xsum[256];  // [group][rp / 4]
  __shared__ float xas[256];
  const int tid = threadIdx.x, m = blockIdx.y;
  xa_row(xpart, SX, M, m, rp, alpha, scale1, r, blockIdx.x == 0 ? XA : nullptr, xsum, xas);
  // four groups of 64 threads share the workgroup's 256 columns: group q adds
  // the partial slices q, q + 4, ... and the adapter rows q, q + 4, ...; the
  // four group sums are then added in a fixed order
  const int q = tid >> 6, cq = tid & 63;
  const int64_t nc = ((int64_t)blockIdx.x * 64 + cq) * 4;
  float a0 = 0.0f, a1 = 0.0f, a2 = 0.0f, a3 = 0.0f;
  __syncthreads();
  if (nc < N) {
#pragma unroll 2
    for (int k = q; k < S; k += 4) {
      const float4 v = *reinterpret_cast<const float4*>(part + ((int64_t)k * M + m) * N + nc);
      a0 += v.x; a1 += v.y; a2 += v.z; a3 += v.w;
    }
#pragma unroll 4
    for (int j = q; j < r; j += 4) {
      const float x = xas[j];
      const uint2 bv = *reinterpret_cast<const uint2*>(B + (int64_t)j * N + nc);
      a0 = __builtin_fmaf(x, __uint_as_float(bv.x << 16), a0);
      a1 = __builtin_fmaf(x, __uint_as_float(bv.x & 0xFFFF0000u), a1);
      a2 = __builtin_fmaf(x, __uint_as_float(bv.y << 16), a2);
      a3 = __builtin_fmaf(x, __uint_as_float(bv.y & 0xFFFF0000u), a3);
    }
  }
  xsum[tid] = make_float4(a0, a1, a2, a3);
  __syncthreads();
  if (q != 0 || nc >= N) return;
  const float4 s1 = xsum[64 + cq], s2 = xsum[128 + cq], s3 = xsum[192 + cq];
  a0 = ((a0 + s1.x) + s2.x) + s3.x;
  a1 = ((a1 + s1.y) + s2.y) + s3.y;
  a2 = ((a2 + s1.z) + s2.z) + s3.z;
  a3 = ((a3 + s1.w) + s2.w) + s3.w;
  *reinterpret_cast<uint2*>(Y + (int64_t)m * N + nc) = make_uint2(pack_bf2(a0, a1), pack_bf2(a2, a3));
}

inline unsigned cdiv(int64_t n, int64_t d) { return (unsigned)((n + d - 1) / d); }

// Threads per chunk for the split-sum reductions: double while the grid has
// fewer than 64K threads and each thread would still add several slices.
int split_sum_threads(int64_t chunks, int S) {
  int T = 1;
  while (T < 64 && chunks * T < 65536 && 4 * T < S) T *= 2;
  return T;
}

template <int BM, int BN, bool BWD, bool I8 = false>
hipError_t launch_main(const MainArgs& a, hipStream_t stream) {
  const dim3 grid(cdiv(a.ncols, BN), cdiv(a.M, BM));
  hipLaunchKernelGGL((main_gemm_kernel<BM, BN, BWD, I8>), grid, dim3(NT), 0, stream, a);
  return hipGetLastError();
}

template <bool BWD>
hipError_t launch_main_any(MainArgs a, float* split_ws, hipStream_t stream) {
  // Int8 weights: the 8-wave 256 x 256 kernel with 8-bit code loads in both
  // directions on that tile (few-token forwards included), else the generic
  // kernel's 8-bit variant
  const bool i8 = a.dq.code_type == CODE_INT8;
  const MainTile tk = pick_tile(a.M, a.ncols, a.L);
  if (i8 && tk != T256x256) return launch_main<256, 256, BWD, true>(a, stream);
  switch (tk) {
    case T256x256: {
      const SplitPlan p = plan_256(a.M, a.ncols, a.L);
      a.full_tiles = p.full;
      a.split = p.split;
      a.part = split_ws;
      if (p.split > 1 && !split_ws) return hipErrorInvalidValue;
      const dim3 grid1((unsigned)p.units());
      // forward: one wave per SIMD (128 x 128 wave tiles); backward: two
      // waves per SIMD (128 x 64), whose transpose-load fragment reads and
      // dequantisation gain more from a second wave to hide them
      if (i8) {
        if (a.dq.double_quant)
          hipLaunchKernelGGL((main_v6_kernel<BWD, true, true>), grid1, dim3(V6_T), 0, stream, a);
        else
          hipLaunchKernelGGL((main_v6_kernel<BWD, false, true>), grid1, dim3(V6_T), 0, stream, a);
      } else if (BWD) {
        if (a.dq.double_quant)
          hipLaunchKernelGGL((main_v6_kernel<true, true>), grid1, dim3(V6_T), 0, stream, a);
        else
          hipLaunchKernelGGL((main_v6_kernel<true, false>), grid1, dim3(V6_T), 0, stream, a);
      } else {
        const bool gw = a.dq.double_quant && (a.Kw >> 6) % 4 == 0 && ((uintptr_t)a.dq.absmax_q & 3) == 0;
        if (gw)
          hipLaunchKernelGGL((main_v5_kernel<false, true, true>), grid1, dim3(V5_T), 0, stream, a);
        else if (a.dq.double_quant)
          hipLaunchKernelGGL((main_v5_kernel<false, true>), grid1, dim3(V5_T), 0, stream, a);
        else
          hipLaunchKernelGGL((main_v5_kernel<false, false>), grid1, dim3(V5_T), 0, stream, a);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || p.split == 1) return e;
      const int tn = (int)cdiv(a.ncols, 256);
      const int64_t threads = (int64_t)(p.tiles - p.full) * 256 * 64;
      hipLaunchKernelGGL(main_fixup_kernel, dim3(cdiv(threads, 256)), dim3(256), 0, stream, split_ws, p.split,
                         p.full, tn, a.M, a.ncols, a.out);
      return hipGetLastError();
    }
    case T256x128: return launch_main<256, 128, BWD>(a, stream);
    default: return launch_main<128, 128, BWD>(a, stream);
  }
}

}  // namespace

// ------------------------------------------------------------ launchers


hipError_t launch_skinny(const uint16_t* U, const uint16_t* V, bool v_is_lq, int64_t M, int64_t Q, int64_t L,
                         float* part, int splits, uint16_t* out1, uint16_t* out2, int64_t QP, float alpha,
                         float scale1, const uint8_t* keep, hipStream_t stream) {
  if (keep && (L & 7)) return hipErrorInvalidValue;
  int64_t chunk = (L + splits - 1) / splits;
  chunk = (chunk + SK_BK - 1) / SK_BK * SK_BK;
  const dim3 grid(cdiv(QP, 64), cdiv(M, 64), (unsigned)splits);
  if (v_is_lq)
    hipLaunchKernelGGL(skinny_kernel<true>, grid, dim3(NT), 0, stream, U, M, L, V, Q, chunk, part, QP, keep);
  else
    hipLaunchKernelGGL(skinny_kernel<false>, grid, dim3(NT), 0, stream, U, M, L, V, Q, chunk, part, QP, keep);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (out1 == nullptr && out2 == nullptr)) return e;  // partials only
  const int T = split_sum_threads(cdiv(M * QP, 4), splits);
#define QLORA_EPI(TT)                                                                                        \
  case TT:                                                                                                   \
    hipLaunchKernelGGL(skinny_epilogue_kernel<TT>, dim3(cdiv(cdiv(M * QP, 4), 256 / TT)), dim3(256), 0, stream, \
                       part, splits, M, Q, QP, out1, out2, alpha, scale1);                                   \
    break;
  switch (T) { QLORA_EPI(1) QLORA_EPI(2) QLORA_EPI(4) QLORA_EPI(8) QLORA_EPI(16) QLORA_EPI(32) default: QLORA_EPI(64) }
#undef QLORA_EPI
  return hipGetLastError();
}


hipError_t launch_tn_pair(const uint16_t* Ua, int64_t ldua, int64_t Pa, const uint8_t* keep_a, const uint16_t* Va,
                          int64_t ldva, int64_t Qa, float* part_a, int splits_a, uint16_t* out_a, float alpha_a,
                          const uint16_t* Ub, int64_t ldub, int64_t Pb, const uint16_t* Vb, int64_t ldvb, int64_t Qb,
                          float* part_b, int splits_b, uint16_t* out_b, float alpha_b, int64_t M, bool accumulate,
                          hipStream_t stream) {
  if (keep_a && (ldua & 7)) return hipErrorInvalidValue;
  auto chunk_of = [&](int splits) {
    const int64_t c = (M + splits - 1) / splits;
    return (c + TN_BK - 1) / TN_BK * TN_BK;
  };
  const TnProblem pa{Ua, Va, ldua, ldva, Pa, Qa, M, chunk_of(splits_a), part_a, keep_a};
  const TnProblem pb{Ub, Vb, ldub, ldvb, Pb, Qb, M, chunk_of(splits_b), part_b, nullptr};
  const dim3 grid(cdiv(Pa > Pb ? Pa : Pb, 128), cdiv(Qa > Qb ? Qa : Qb, 64), (unsigned)(splits_a + splits_b));
  hipLaunchKernelGGL((tn_kernel<128, 64>), grid, dim3(NT), 0, stream, pa, pb, splits_a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t ca = cdiv(Pa * Qa, 4), cb = cdiv(Pb * Qb, 4);
  const int T = split_sum_threads(ca < cb ? ca : cb, splits_a > splits_b ? splits_a : splits_b);
  const TnOut oa{part_a, splits_a, Pa, Qa, out_a, alpha_a, 0, accumulate ? 1 : 0};
  const TnOut ob{part_b, splits_b, Pb, Qb, out_b, alpha_b, 1, accumulate ? 1 : 0};
#define QLORA_RED(TT)                                                                                       \
  case TT: {                                                                                                \
    const int na = (int)cdiv(ca, 256 / TT), nb = (int)cdiv(cb, 256 / TT);                                  \
    hipLaunchKernelGGL(tn_reduce_kernel<TT>, dim3((unsigned)(na + nb)), dim3(256), 0, stream, oa, ob, na);  \
    break;                                                                                                  \
  }
  switch (T) { QLORA_RED(1) QLORA_RED(2) QLORA_RED(4) QLORA_RED(8) QLORA_RED(16) QLORA_RED(32) default: QLORA_RED(64) }
#undef QLORA_RED
  return hipGetLastError();
}

hipError_t launch_fill_zero_u16(uint16_t* dst, int64_t n, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(cdiv(n, 256)), dim3(256), 0, stream, dst, n);
  return hipGetLastError();
}


hipError_t launch_fwd_main(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, const DQParams& dq,
                           int64_t N, const uint16_t* XAs, const uint16_t* B, int64_t r, int64_t rp, uint16_t* Y,
                           float* split_ws, hipStream_t stream) {
  MainArgs a;
  a.act = X; a.M = M; a.L = K;
  a.codes = codes; a.dq = dq; a.Nw = N; a.Kw = K;
  a.ext_act = XAs; a.ext_w = B; a.r = r; a.rp = rp;
  a.out = Y; a.ncols = N;
  a.full_tiles = 0; a.split = 1; a.part = nullptr;
  a.keep = nullptr; a.keep_scale = 1.0f;
  return launch_main_any<false>(a, split_ws, stream);
}


hipError_t launch_gemv(const uint16_t* X, int64_t M, int64_t K, const uint8_t* codes, const DQParams& dq, int64_t N,
                       float* part, int splits, const uint16_t* A, int64_t r, int64_t rp, const uint8_t* keep,
                       float* xpart, hipStream_t stream) {
  if (M < 1 || M > kGemvMaxM || splits < 1 || K < 64 || N < 1) return hipErrorInvalidValue;
  if (splits > ((K >> 6) + G3_CB - 1) / G3_CB) return hipErrorInvalidValue;  // an empty split
  if (K % 64 || rp % 64 || rp > 256 || r > rp) return hipErrorInvalidValue;
  static_assert(G3_T == 512, "the X A chunks are computed by 512-thread workgroups");
  const dim3 grid(cdiv(N, G3_ROWS), (unsigned)splits);
  // the split lengths of this grid (they depend on the row tile through the
  // X A chunks): preload the E4M3 bytes when every split fits G3_PREMAX
  const int64_t nbk = K >> 6, T = grid.x, nxc = (K + XA_CHUNK - 1) / XA_CHUNK;
  const int nchunks = (int)((nbk + G3_CB - 1) / G3_CB);
  bool pre = dq.double_quant && nbk % G3_CB == 0 && ((uintptr_t)dq.absmax_q & 3) == 0;
  for (int64_t x = 0; pre && x < T && x < nxc + 1; ++x)  // tiles x >= nxc split alike
    for (int y = 0; pre && y < splits; ++y)
      pre = gemv_split_lo(y + 1, x, T, splits, nchunks, nxc) - gemv_split_lo(y, x, T, splits, nchunks, nxc) <=
            G3_PREMAX;
  if (pre)
    hipLaunchKernelGGL((gemv3_kernel<true, true>), grid, dim3(G3_T), 0, stream, X, (int)M, K, codes, dq, N, splits,
                       part, A, (int)r, (int)rp, keep, xpart);
  else if (dq.double_quant)
    hipLaunchKernelGGL((gemv3_kernel<true>), grid, dim3(G3_T), 0, stream, X, (int)M, K, codes, dq, N, splits, part,
                       A, (int)r, (int)rp, keep, xpart);
  else
    hipLaunchKernelGGL((gemv3_kernel<false>), grid, dim3(G3_T), 0, stream, X, (int)M, K, codes, dq, N, splits, part,
                       A, (int)r, (int)rp, keep, xpart);
  return hipGetLastError();
}

hipError_t launch_xa_chunks(const uint16_t* X, int64_t M, int64_t K, const uint16_t* A, int64_t r, int64_t rp,
                            const uint8_t* keep, float* xpart, hipStream_t stream) {
  if (M < 1 || M > kGemvMaxM || rp % 64 || rp > 256 || r > rp || K < 64 || K % 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(xa_chunks_kernel, dim3((unsigned)xa_chunks(K)), dim3(512), 0, stream, X, (int)M, K, A, (int)r,
                     (int)rp, keep, xpart);
  return hipGetLastError();
}

hipError_t launch_gemv_reduce(const float* part, int splits, int64_t M, int64_t N, const float* xpart, int xsplits,
                              int64_t rp, float alpha, float scale1, const uint16_t* B, int64_t r, uint16_t* Y,
                              uint16_t* XA, hipStream_t stream) {
  if (N % 4 || rp % 64 || rp > 256 || r > rp || xsplits < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(gemv_reduce_kernel, dim3(cdiv(N, 256), (unsigned)M), dim3(256), 0, stream, part, splits, (int)M,
                     N, xpart, xsplits, (int)rp, alpha, scale1, B, (int)r, Y, XA);
  return hipGetLastError();
}

hipError_t launch_xa_reduce(const float* xpart, int xsplits, int64_t M, int64_t rp, float scale1, int64_t r,
                            uint16_t* XA, hipStream_t stream) {
  if (rp % 64 || rp > 256 || r > rp || xsplits < 1 || M < 1) return hipErrorInvalidValue;
  hipLaunchKernelGGL(xa_reduce_kernel, dim3((unsigned)M), dim3(256), 0, stream, xpart, xsplits, (int)M, (int)rp,
                     scale1, (int)r, XA);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const uint16_t* dY, int64_t M, int64_t N, const uint8_t* codes, const DQParams& dq,
                         int64_t K, const uint16_t* Ts, const uint16_t* A, int64_t r, int64_t rp, uint16_t* dX,
                         float* split_ws, const uint8_t* keep, float keep_scale, hipStream_t stream) {
  if (keep && (K & 7)) return hipErrorInvalidValue;
  MainArgs a;
  a.act = dY; a.M = M; a.L = N;
  a.codes = codes; a.dq = dq; a.Nw = N; a.Kw = K;
  a.ext_act = Ts; a.ext_w = A; a.r = r; a.rp = rp;
  a.out = dX; a.ncols = K;
  a.full_tiles = 0; a.split = 1; a.part = nullptr;
  a.keep = keep; a.keep_scale = keep_scale;
  return launch_main_any<true>(a, split_ws, stream);
}

}  // namespace qlora
