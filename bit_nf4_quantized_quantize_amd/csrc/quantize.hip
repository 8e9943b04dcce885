// NF4 blockwise quantisation, double quantisation of the block constants and
// dequantisation for gfx950.
//
// QLoRA (Dettmers et al., arXiv 2305.14314):
//   section 2 "Block-wise k-bit Quantization": absmax scaling (Eq. 1), its
//     inverse (Eq. 2, read as multiplying by the absmax), and chunking the
//     flattened tensor into contiguous blocks with one constant each;
//   section 3 "4-bit NormalFloat Quantization": normalise each block by its
//     absmax to [-1, 1], then take the nearest NF4 value; Appendix E gives
//     the 16 values;
//   section 3 "Double Quantization": the fp32 block constants c2 are
//     mean-centred and quantised to 8-bit floats in blocks of 256, giving
//     c2^FP8 and one fp32 second-level constant c1 per 256 blocks;
//   section 3 "QLoRA", Eq. 6: doubleDequant = dequant(dequant(c1, c2), W).
//
// All kernels are bandwidth-bound streams over the weight; see the design
// notes for their byte counts.
#include <math.h>
#include <string.h>

#include "device.h"
#include "launch.h"

// Stored codes and constants are decided by fp32 arithmetic with one rounding
// per operation; nothing in this file may be contracted into an FMA.
#pragma clang fp contract(off)

namespace qlora {

// A block (or a group of constants) whose absmax is an fp32 subnormal is
// first scaled by 2^32, exactly, so that the reciprocal of Eq. 1's constant
// stays finite; normal blocks are unaffected.  The second-level constant
// divides 448 rather than 1, so its threshold is 2^-118 (448 * 2^118 is
// still below the largest fp32).
constexpr float kTiny = 0x1p-126f;
constexpr float kTinyDQ = 0x1p-118f;
constexpr float kPrescale = 0x1p32f;

// ----------------------------------------------------------------- tables

// QLoRA Appendix E, code 0 .. 15 (each value exact in fp32).
static const float kNF4[16] = {
    -1.0f,
    -0.6961928009986877f,
    -0.5250730514526367f,
    -0.39491748809814453f,
    -0.28444138169288635f,
    -0.18477343022823334f,
    -0.09105003625154495f,
    0.0f,
    0.07958029955625534f,
    0.16093020141124725f,
    0.24611230194568634f,
    0.33791524171829224f,
    0.44070982933044434f,
    0.5626170039176941f,
    0.7229568362236023f,
    1.0f,
};

const NF4Values& nf4_values() {
  static const NF4Values v = [] {
    NF4Values t;
    memcpy(t.v, kNF4, sizeof(kNF4));
    return t;
  }();
  return v;
}

// Decision thresholds between codes i and i+1 are the exact midpoints
// (NF4[i] + NF4[i+1]) / 2 (exact in double), rounded toward -inf to fp32 so
// that "x > thr" equals "x > midpoint" for every fp32 x; a tie (x equal to a
// midpoint) keeps the lower code.  Buckets [b/16 - 1, (b+1)/16 - 1) each
// hold at most one midpoint, and none lies within 2^-20 of a bucket edge, so
// a bucket index computed with one fp32 rounding is off by at most one only
// where that cannot change the code.
const QuantTable& quant_table() {
  static const QuantTable t = [] {
    QuantTable q;
    double mid[15];
    float thr[15];
    for (int i = 0; i < 15; ++i) {
      mid[i] = 0.5 * ((double)kNF4[i] + (double)kNF4[i + 1]);
      float f = (float)mid[i];
      if ((double)f > mid[i]) f = nextafterf(f, -INFINITY);
      thr[i] = f;
    }
    for (int b = 0; b < 32; ++b) {
      const double lo = b / 16.0 - 1.0, hi = (b + 1) / 16.0 - 1.0;
      uint32_t base = 0;
      float t_in = INFINITY;
      int inside = 0;
      for (int i = 0; i < 15; ++i) {
        if (mid[i] < lo) ++base;
        else if (mid[i] < hi) { t_in = thr[i]; ++inside; }
      }
      if (inside > 1) abort();  // cannot happen for the Appendix E values
      q.thr[b] = t_in;
      q.base[b] = base;
    }
    return q;
  }();
  return t;
}

// --------------------------------------------------- exact mean of c2
// The mean mu is the exact sum of all c2 divided by their count, rounded
// once to fp32.  Every non-negative fp32 value is an integer multiple of
// 2^-149, so the sum is accumulated as an integer in units of 2^-149 split
// into 32-bit digits held in 64-bit counters (no carries are needed while
// summing: each addend is below 2^32 and there are fewer than 2^31 of them
// per counter).  The result is order-independent and bit-reproducible.
// The quantisation kernel adds the constants it produces into per-workgroup
// counters; one small kernel then adds the workgroups' counters and divides.

// Digit index and the two 32-bit digit addends of c (|c| finite or not).
__device__ __forceinline__ void c2_digits(float c, uint32_t& d, uint32_t& lo, uint32_t& hi) {
  const uint32_t bits = __float_as_uint(c) & 0x7FFFFFFFu;
  uint32_t e = bits >> 23, m = bits & 0x7FFFFFu;
  if (e == 0xFF) { e = 0xFE; m = 0x7FFFFFu; }  // non-finite input: result undefined, stay in range
  const uint32_t shift = e ? e - 1 : 0;
  m |= e ? 0x800000u : 0u;
  const uint64_t v = (uint64_t)m << (shift & 31);
  d = shift >> 5;  // 0..7
  lo = (uint32_t)v;
  hi = (uint32_t)(v >> 32);
}

// ------------------------------------------------------- quantise kernel
// A workgroup of 512 threads = 8 waves handles chunks of 8192 consecutive
// weights (128 blocks), striding over the tensor by the grid size (at most
// one workgroup per CU).  In each of 4 steps of a chunk a wave covers 256
// weights = 4 blocks; a lane holds 4
// consecutive weights, so a block is one row of 16 lanes and its absmax is a
// 16-lane DPP reduction.  Each lane writes its 4 codes as one 16-bit store;
// lane 0 of each row writes the block's absmax and, with double
// quantisation, adds it to the workgroup's exact-sum counters in LDS.  The
// next chunk's weights are loaded before the current one is coded (two
// register sets; a chunk past the end re-reads the current one).  A final
// partial chunk is coded by the workgroup that owns it, with bounds checks.

constexpr int QZ_THREADS = 512;
constexpr int QZ_WAVES = QZ_THREADS / 64;
constexpr int QZ_STEPS = 4;
constexpr int QZ_PER_WG = QZ_THREADS * 4 * QZ_STEPS;  // 8192 weights
constexpr int QZ_MAX_WG = 256;                        // also the number of exact-sum partials

int quantize_parts(int64_t numel) {
  const int64_t chunks = (numel + QZ_PER_WG - 1) / QZ_PER_WG;
  return (int)(chunks < 1 ? 1 : (chunks > QZ_MAX_WG ? QZ_MAX_WG : chunks));
}

template <bool BF16_IN>
__device__ __forceinline__ void load4(const void* w, int64_t e0, int64_t numel, float v[4]) {
  if (e0 + 3 < numel) {
    if (BF16_IN) {
      const uint2 p = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(w) + e0);
      v[0] = __uint_as_float(p.x << 16);
      v[1] = __uint_as_float(p.x & 0xFFFF0000u);
      v[2] = __uint_as_float(p.y << 16);
      v[3] = __uint_as_float(p.y & 0xFFFF0000u);
    } else {
      const float4 p = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(w) + e0);
      v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t e = e0 + i;
      if (e < numel)
        v[i] = BF16_IN ? bf2f(reinterpret_cast<const uint16_t*>(w)[e]) : reinterpret_cast<const float*>(w)[e];
      else
        v[i] = 0.0f;
    }
  }
}

// 4 weights of a full chunk (no bounds checks).
template <bool BF16_IN>
__device__ __forceinline__ void load4_full(const void* w, int64_t e0, float v[4]) {
  if (BF16_IN) {
    const uint2 p = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(w) + e0);
    v[0] = __uint_as_float(p.x << 16);
    v[1] = __uint_as_float(p.x & 0xFFFF0000u);
    v[2] = __uint_as_float(p.y << 16);
    v[3] = __uint_as_float(p.y & 0xFFFF0000u);
  } else {
    const float4 p = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(w) + e0);
    v[0] = p.x; v[1] = p.y; v[2] = p.z; v[3] = p.w;
  }
}

// The quantisation of one workgroup's chunks (grid-stride over 8192-weight
// chunks); with `partials` it ends by storing the workgroup's exact-sum
// counters at partials[blockIdx.x].
template <bool BF16_IN>
__device__ __forceinline__ void quantize_chunks(const void* __restrict__ w, int64_t numel,
                                                uint8_t* __restrict__ codes, float* __restrict__ c2out,
                                                uint64_t* __restrict__ partials, const QuantTable& tab) {
  __shared__ uint2 s_tab[32];  // {threshold bits, base code}
  __shared__ unsigned long long s_acc[kMeanDigits];
  const int tid = threadIdx.x;
  if (tid < 32) s_tab[tid] = make_uint2(__float_as_uint(tab.thr[tid]), tab.base[tid]);
  if (tid < kMeanDigits) s_acc[tid] = 0;
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int64_t nb = (numel + 63) >> 6;
  const int64_t nfull = numel / QZ_PER_WG;
  const int64_t G = gridDim.x;
  const bool sums = partials != nullptr;

  // code one step (4 weights per lane) starting at element e0
  auto code_step = [&](int64_t e0, float v[4], bool full) {
    float m = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    const float c2 = row16_max(m);
    float cs = c2;
    const bool tiny = c2 > 0.0f && c2 < kTiny;
    if (__builtin_amdgcn_ballot_w64(tiny)) {  // rare, wave-uniform branch
      const float sc = tiny ? kPrescale : 1.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] *= sc;
      cs = c2 * sc;
    }
    const float inv = cs > 0.0f ? 1.0f / cs : 0.0f;  // correctly rounded division
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = v[i] * inv;                     // in [-1, 1]
      int b = (int)__builtin_fmaf(x, 16.0f, 16.0f);   // bucket 0..32 (x*16 is exact)
      b = b < 0 ? 0 : (b > 31 ? 31 : b);
      const uint2 t = s_tab[b];
      const uint32_t code = t.y + (x > __uint_as_float(t.x) ? 1u : 0u);
      packed |= code << (4 * i);
    }
    if (full) {
      *reinterpret_cast<uint16_t*>(codes + (e0 >> 1)) = (uint16_t)packed;
    } else {
      // past the end: the nibble of a missing element is 0
      const int64_t have = numel - e0;  // may be <= 0
      if (have < 4) packed &= have <= 0 ? 0u : (0xFFFFu >> (4 * (4 - have)));
      if (e0 < numel) codes[e0 >> 1] = (uint8_t)(packed & 0xFF);
      if (e0 + 2 < numel) codes[(e0 >> 1) + 1] = (uint8_t)(packed >> 8);
    }
    const int64_t blk = e0 >> 6;
    if ((lane & 15) == 0 && blk < nb) {
      c2out[blk] = c2;
      if (sums && c2 > 0.0f) {
        uint32_t d, lo, hi;
        c2_digits(c2, d, lo, hi);
        atomicAdd(&s_acc[d], (unsigned long long)lo);
        if (hi) atomicAdd(&s_acc[d + 1], (unsigned long long)hi);
      }
    }
  };
  auto elem = [&](int64_t c, int s) { return c * QZ_PER_WG + (int64_t)(s * QZ_WAVES + wave) * 256 + lane * 4; };

  float va[QZ_STEPS][4], vb[QZ_STEPS][4];
  int64_t c = blockIdx.x;
  if (c < nfull) {
#pragma unroll
    for (int s = 0; s < QZ_STEPS; ++s) load4_full<BF16_IN>(w, elem(c, s), va[s]);
  }
  while (c < nfull) {
    const int64_t c1 = c + G;
    const int64_t l1 = c1 < nfull ? c1 : c;  // past the end: re-read the current chunk (cached)
#pragma unroll
    for (int s = 0; s < QZ_STEPS; ++s) load4_full<BF16_IN>(w, elem(l1, s), vb[s]);
#pragma unroll
    for (int s = 0; s < QZ_STEPS; ++s) code_step(elem(c, s), va[s], true);
    if (c1 >= nfull) break;
    const int64_t c2i = c1 + G;
    const int64_t l2 = c2i < nfull ? c2i : c1;
#pragma unroll
    for (int s = 0; s < QZ_STEPS; ++s) load4_full<BF16_IN>(w, elem(l2, s), va[s]);
#pragma unroll
    for (int s = 0; s < QZ_STEPS; ++s) code_step(elem(c1, s), vb[s], true);
    c = c2i;
  }
  // the partial last chunk, if any
  if (nfull * QZ_PER_WG < numel && (nfull % G) == blockIdx.x) {
#pragma unroll
    for (int s = 0; s < QZ_STEPS; ++s) load4<BF16_IN>(w, elem(nfull, s), numel, va[s]);
#pragma unroll
    for (int s = 0; s < QZ_STEPS; ++s) code_step(elem(nfull, s), va[s], elem(nfull, s) + 3 < numel);
  }
  if (sums) {
    __syncthreads();
    if (tid < kMeanDigits) partials[(int64_t)blockIdx.x * kMeanDigits + tid] = s_acc[tid];
  }
}

template <bool BF16_IN>
__global__ __launch_bounds__(QZ_THREADS) void nf4_quantize_kernel(const void* __restrict__ w, int64_t numel,
                                                                  uint8_t* __restrict__ codes,
                                                                  float* __restrict__ c2out,
                                                                  uint64_t* __restrict__ partials, QuantTable tab) {
  quantize_chunks<BF16_IN>(w, numel, codes, c2out, partials, tab);
}

hipError_t launch_quantize(const void* w, bool w_bf16, int64_t numel, uint8_t* codes, float* c2, uint64_t* partials,
                           hipStream_t stream) {
  const int grid = quantize_parts(numel);
  if (w_bf16)
    hipLaunchKernelGGL(nf4_quantize_kernel<true>, dim3((unsigned)grid), dim3(QZ_THREADS), 0, stream, w,
                       numel, codes, c2, partials, quant_table());
  else
    hipLaunchKernelGGL(nf4_quantize_kernel<false>, dim3((unsigned)grid), dim3(QZ_THREADS), 0, stream, w,
                       numel, codes, c2, partials, quant_table());
  return hipGetLastError();
}

// Round the rational (sum / nb) in units of 2^-149 to the nearest fp32
// (ties to even).  The fp32 bit pattern of a value v < 2^-125 is v / 2^-149
// itself; above that the pattern is (shift << 23) + mantissa for a 24-bit
// mantissa scaled by 2^shift, which also absorbs a rounding carry.
// s_sum[k] are the summed 64-bit digit counters.
__device__ float exact_mean(const uint64_t* s_sum, int64_t nb) {
  // carry-propagate into 32-bit digits: S = sum_k dig[k] 2^(32k)
  constexpr int ND = kMeanDigits + 1;
  uint32_t dig[ND];
  uint64_t carry = 0;
#pragma unroll
  for (int k = 0; k < kMeanDigits; ++k) {
    const uint64_t t = (s_sum[k] & 0xFFFFFFFFull) + carry;
    dig[k] = (uint32_t)t;
    carry = (t >> 32) + (s_sum[k] >> 32);
  }
  dig[kMeanDigits] = (uint32_t)carry;
  int h = -1;  // highest nonzero digit
#pragma unroll
  for (int k = ND - 1; k >= 0; --k)
    if (h < 0 && dig[k]) h = k;
  const uint64_t den = (uint64_t)nb;
  // S / nb = q * 2^E + f with 0 <= f < 2^E; `rest` is set when f's exact
  // value is nonzero beyond what the remainder r of q shows (bits of S below
  // 2^E).  With S < 2^64, E = 0 and q, r are exact; otherwise q = floor(T /
  // nb) for the top 64 bits T of S, which has at least 31 significant bits,
  // so the bits of the result that fp32 rounding looks at all lie in q.
  uint64_t q, r;
  int E = 0;
  bool rest = false;
  if (h <= 1) {
    const uint64_t S = ((uint64_t)dig[1] << 32) | dig[0];
    q = S / den;
    r = S - q * den;
  } else {
    uint32_t a = 0, b = 0, c = 0;
    bool below = false;  // any nonzero digit under the top three
#pragma unroll
    for (int k = 0; k < ND; ++k) {
      if (k == h) a = dig[k];
      if (k == h - 1) b = dig[k];
      if (k == h - 2) c = dig[k];
      if (k < h - 2) below = below || dig[k] != 0;
    }
    const int lz = __builtin_clz(a);
    const uint64_t ab = ((uint64_t)a << 32) | b;
    const uint64_t T = lz ? (ab << lz) | (c >> (32 - lz)) : ab;
    const uint32_t cmask = lz ? (1u << (32 - lz)) - 1u : 0xFFFFFFFFu;  // bits of c under 2^E
    rest = below || (c & cmask) != 0;
    E = 32 * (h - 1) - lz;
    q = T / den;
    r = T - q * den;
  }
  uint32_t result;
  const int t = q ? 63 - __builtin_clzll(q) : -1;  // highest set bit of q
  if (E == 0 && t < 24) {
    // value below 2^24 units: the integer part is the bit pattern already
    const uint64_t twice = 2 * r;
    const bool up = twice > den || (twice == den && (q & 1u));
    result = (uint32_t)q + (up ? 1u : 0u);
  } else {
    const int sh = t - 23;  // >= 1 (E > 0 implies t >= 31)
    const uint32_t mant = (uint32_t)(q >> sh);
    const uint32_t rbit = (uint32_t)(q >> (sh - 1)) & 1u;
    const bool sticky = (q & ((1ull << (sh - 1)) - 1ull)) != 0 || r != 0 || rest;
    const bool up = rbit && (sticky || (mant & 1u));
    result = ((uint32_t)(sh + E) << 23) + mant + (up ? 1u : 0u);
  }
  return __uint_as_float(result);
}

// ------------------------------------------------ second-level encode
// One wave per group of 256 constants, 4 per lane: d = c2 - mu, c1 = max |d|,
// byte = E4M3(clamp(d * fp32(448 / c1))), scale2 = c1 / 448.

// Every workgroup first adds the quantisation workgroups' exact-sum
// counters (at most 256, one per thread) and divides for mu; workgroup 0
// stores mu.  This costs each workgroup one 20 KB read from L2 instead of a
// separate single-workgroup launch.
// mu from the exact-sum counters of `parts` workgroups (at most WAVES * 64,
// one per thread), reduced across this workgroup; every thread gets it.
template <int WAVES>
__device__ __forceinline__ float mean_from_partials(const uint64_t* __restrict__ partials, int parts, int64_t nb) {
  __shared__ uint64_t s_part[WAVES][kMeanDigits];
  __shared__ uint64_t s_sum[kMeanDigits];
  __shared__ float s_mu;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint64_t v[kMeanDigits];
  const int p = threadIdx.x;
#pragma unroll
  for (int k = 0; k < kMeanDigits; ++k) v[k] = p < parts ? partials[(int64_t)p * kMeanDigits + k] : 0;
#pragma unroll
  for (int k = 0; k < kMeanDigits; ++k) {
    const uint64_t t = wave_sum_u64(v[k]);
    if (lane == 0) s_part[wave][k] = t;
  }
  __syncthreads();
  if (threadIdx.x < kMeanDigits) {
    uint64_t t = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) t += s_part[w][threadIdx.x];
    s_sum[threadIdx.x] = t;
  }
  __syncthreads();
  if (threadIdx.x == 0) s_mu = exact_mean(s_sum, nb);
  __syncthreads();
  return s_mu;
}

// The constants c2[256 g .. +255] of 256-group g, four per lane (zero past nb).
__device__ __forceinline__ void load_group(const float* __restrict__ c2, int64_t g, int64_t nb, int lane,
                                           float cv[4]) {
  const int64_t i0 = g * 256 + lane * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) cv[i] = i0 + i < nb ? c2[i0 + i] : 0.0f;
}

// Double quantisation of 256-group g by one wave (Sec. 3 of the QLoRA paper,
// reading G4 for mu): d = c2 - mu, c1 = max |d| over the group, byte =
// E4M3(clamp(d * fp32(448 / c1), +-448)) nearest-even, scale2 = c1 / 448; a
// group with c1 < 2^-118 is first scaled by 2^32 (reading G13).
__device__ __forceinline__ void encode_group(const float cv[4], int64_t g, int64_t nb, float mu,
                                             uint8_t* __restrict__ absmax_q, float* __restrict__ scale2,
                                             int lane) {
  const int64_t i0 = g * 256 + lane * 4;
  float d[4];
  float m = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t idx = i0 + i;
    d[i] = idx < nb ? cv[i] - mu : 0.0f;
    if (idx < nb) m = fmaxf(m, fabsf(d[i]));
  }
  const float c1 = wave_max(m);
  const bool tiny = c1 > 0.0f && c1 < kTinyDQ;   // same for the whole wave
  const float sc = tiny ? kPrescale : 1.0f;
  const float c1s = c1 * sc;
  const float f = c1s > 0.0f ? 448.0f / c1s : 0.0f;
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float y = (d[i] * sc) * f;
    y = fminf(fmaxf(y, -448.0f), 448.0f);
    const uint32_t byte = c1 > 0.0f ? e4m3_encode(y) : 0u;
    word |= byte << (8 * i);
  }
  if (i0 + 3 < nb) {
    *reinterpret_cast<uint32_t*>(absmax_q + i0) = word;
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (i0 + i < nb) absmax_q[i0 + i] = (uint8_t)(word >> (8 * i));
  }
  if (lane == 0) scale2[g] = c1 / 448.0f;
}

// Second kernel of the two-launch double quantisation: one wave per 256-group;
// every workgroup first forms mu from the exact-sum counters (workgroup 0
// stores it).
__global__ __launch_bounds__(256) void dq_encode_kernel(const float* __restrict__ c2, int64_t nb,
                                                        const uint64_t* __restrict__ partials, int parts,
                                                        float* __restrict__ mu_out,
                                                        uint8_t* __restrict__ absmax_q,
                                                        float* __restrict__ scale2) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t g = (int64_t)blockIdx.x * 4 + wave;
  float cv[4];
  load_group(c2, g, nb, lane, cv);  // independent of mu: these loads go out first
  const float mu = mean_from_partials<4>(partials, parts, nb);
  if (blockIdx.x == 0 && threadIdx.x == 0) *mu_out = mu;
  if (g * 256 >= nb) return;  // whole wave exits together
  encode_group(cv, g, nb, mu, absmax_q, scale2, lane);
}

hipError_t launch_double_quant(const float* c2, int64_t nb, const uint64_t* partials, int parts, uint8_t* absmax_q,
                               float* scale2, float* offset, hipStream_t stream) {
  if (parts < 1 || parts > QZ_MAX_WG || QZ_MAX_WG > 256) return hipErrorInvalidValue;
  const int64_t ng = (nb + 255) / 256;
  hipLaunchKernelGGL(dq_encode_kernel, dim3((unsigned)((ng + 3) / 4)), dim3(256), 0, stream, c2, nb, partials, parts,
                     offset, absmax_q, scale2);
  return hipGetLastError();
}

// --------------------------------------------------------- dequantise
// Each thread expands 8 codes (one 32-bit word) of one block; a workgroup of
// 256 threads covers 4 x 2048 weights.  c2_hat is computed as two separately
// rounded fp32 operations (this file is built without contraction).

constexpr int DQZ_THREADS = 256;
constexpr int DQZ_STEPS = 4;
constexpr int DQZ_PER_WG = DQZ_THREADS * 8 * DQZ_STEPS;

template <bool DQ, bool BF16_OUT>
__global__ __launch_bounds__(DQZ_THREADS) void nf4_dequant_kernel(const uint8_t* __restrict__ codes, int64_t numel,
                                                                  const uint8_t* __restrict__ absmax_q,
                                                                  const float* __restrict__ absmax,
                                                                  const float* __restrict__ scale2,
                                                                  const float* __restrict__ offset,
                                                                  void* __restrict__ out, NF4Values nf4) {
  __shared__ float s_nf4[16];
  if (threadIdx.x < 16) s_nf4[threadIdx.x] = nf4.v[threadIdx.x];
  __syncthreads();
  const float mu = DQ ? *offset : 0.0f;
  const int64_t wg0 = (int64_t)blockIdx.x * DQZ_PER_WG;
  if (wg0 + DQZ_PER_WG <= numel) {
    // a whole chunk: every load goes out before the first is used
    uint32_t word[DQZ_STEPS], qb[DQZ_STEPS];
    float f[DQZ_STEPS];
#pragma unroll
    for (int s = 0; s < DQZ_STEPS; ++s) {
      const int64_t e0 = wg0 + ((int64_t)s * DQZ_THREADS + threadIdx.x) * 8;
      const int64_t blk = e0 >> 6;
      word[s] = *reinterpret_cast<const uint32_t*>(codes + (e0 >> 1));
      if (DQ) {
        qb[s] = absmax_q[blk];
        f[s] = scale2[blk >> 8];
      } else {
        qb[s] = 0;
        f[s] = absmax[blk];
      }
    }
#pragma unroll
    for (int s = 0; s < DQZ_STEPS; ++s) {
      const int64_t e0 = wg0 + ((int64_t)s * DQZ_THREADS + threadIdx.x) * 8;
      const float c = DQ ? e4m3_decode(qb[s]) * f[s] + mu : f[s];
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = s_nf4[(word[s] >> (4 * i)) & 0xF] * c;
      if (BF16_OUT) {
        uint4 o;
        o.x = pack_bf2(v[0], v[1]);
        o.y = pack_bf2(v[2], v[3]);
        o.z = pack_bf2(v[4], v[5]);
        o.w = pack_bf2(v[6], v[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + e0) = o;
      } else {
        float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + e0);
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    }
    return;
  }
#pragma unroll
  for (int s = 0; s < DQZ_STEPS; ++s) {
    const int64_t e0 = wg0 + ((int64_t)s * DQZ_THREADS + threadIdx.x) * 8;
    if (e0 >= numel) break;
    const int64_t blk = e0 >> 6;
    float c;
    if (DQ) {
      const float prod = e4m3_decode(absmax_q[blk]) * scale2[blk >> 8];
      c = prod + mu;
    } else {
      c = absmax[blk];
    }
    uint32_t word;
    if (e0 + 7 < numel) {
      word = *reinterpret_cast<const uint32_t*>(codes + (e0 >> 1));
    } else {
      word = 0;
      for (int i = 0; i < 4; ++i)
        if (e0 + 2 * i < numel) word |= (uint32_t)codes[(e0 >> 1) + i] << (8 * i);
    }
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = s_nf4[(word >> (4 * i)) & 0xF] * c;
    if (e0 + 7 < numel) {
      if (BF16_OUT) {
        uint4 o;
        o.x = pack_bf2(v[0], v[1]);
        o.y = pack_bf2(v[2], v[3]);
        o.z = pack_bf2(v[4], v[5]);
        o.w = pack_bf2(v[6], v[7]);
        *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(out) + e0) = o;
      } else {
        float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + e0);
        o[0] = make_float4(v[0], v[1], v[2], v[3]);
        o[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    } else {
      for (int i = 0; i < 8; ++i) {
        if (e0 + i >= numel) break;
        if (BF16_OUT) reinterpret_cast<uint16_t*>(out)[e0 + i] = f2bf(v[i]);
        else reinterpret_cast<float*>(out)[e0 + i] = v[i];
      }
    }
  }
}

hipError_t launch_dequantize(const uint8_t* codes, int64_t numel, bool dq, const uint8_t* absmax_q,
                             const float* absmax, const float* scale2, const float* offset, void* out,
                             bool out_bf16, hipStream_t stream) {
  const dim3 grid((unsigned)((numel + DQZ_PER_WG - 1) / DQZ_PER_WG)), block(DQZ_THREADS);
  const NF4Values& t = nf4_values();
  if (dq) {
    if (out_bf16)
      hipLaunchKernelGGL((nf4_dequant_kernel<true, true>), grid, block, 0, stream, codes, numel, absmax_q, absmax,
                         scale2, offset, out, t);
    else
      hipLaunchKernelGGL((nf4_dequant_kernel<true, false>), grid, block, 0, stream, codes, numel, absmax_q, absmax,
                         scale2, offset, out, t);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((nf4_dequant_kernel<false, true>), grid, block, 0, stream, codes, numel, absmax_q, absmax,
                         scale2, offset, out, t);
    else
      hipLaunchKernelGGL((nf4_dequant_kernel<false, false>), grid, block, 0, stream, codes, numel, absmax_q, absmax,
                         scale2, offset, out, t);
  }
  return hipGetLastError();
}

}  // namespace qlora
