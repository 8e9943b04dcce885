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
// A lane codes 8 consecutive weights, so a block of 64 is one group of 8
// lanes (an octet) and its absmax is a 3-step DPP reduction.  A workgroup of
// 512 threads = 8 waves takes chunks of STEPS * 8 * 512 weights (STEPS = 8
// for bf16 input, 4 for fp32), striding over the tensor by the grid size;
// step s of a wave is the 512 weights at chunk + (8 s + wave) * 512.  A chunk
// is coded in three phases:
//   A. the absmax of every step; lane 8j+k keeps that of block j of step k,
//      so the wave's blocks end up one per lane;
//   B. per lane, one block: store c2, add it to the exact-sum counters and
//      take the correctly rounded reciprocal (one division per lane for up
//      to 8 blocks, instead of one per block and step);
//   C. per step, every lane fetches its block's reciprocal from lane 8j+s
//      (ds_bpermute) and codes its 8 weights into one 32-bit store.
// The next chunk is loaded while the current one is coded.  A chunk holding
// a subnormal or non-finite absmax takes a generic per-step path instead
// (prescaling, clamped bucket index), and so does the final partial chunk,
// which is spread over the workgroups as 512-weight wave steps with bounds
// checks.  Each wave has its own exact-sum counters in LDS.

constexpr int QZ_THREADS = 512;
constexpr int QZ_WAVES = QZ_THREADS / 64;
constexpr int QZ_MAX_WG = kQuantMaxParts;  // also the number of exact-sum partials

typedef uint32_t qz_u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short qz_u16x2 __attribute__((ext_vector_type(2)));

template <bool BF16>
struct QzGeo {
  static constexpr int STEPS = BF16 ? 8 : 4;   // steps per chunk and wave
  static constexpr int NV = BF16 ? 1 : 2;      // 16-byte loads per lane and step
  static constexpr int64_t CH = (int64_t)STEPS * QZ_WAVES * 512;
};

// Max over the 8 lanes of each octet (every lane gets its octet's max).
__device__ __forceinline__ uint32_t octet_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));  // row_half_mirror
  return v;
}

// fp32 bit pattern of max |w| over a lane's 8 weights.  For values that are
// not NaN the order of |w| is the unsigned order of its bit pattern.
template <bool BF16>
__device__ __forceinline__ uint32_t absmax_bits(const qz_u32x4* r) {
  if (BF16) {
    const qz_u16x2 a0 = __builtin_bit_cast(qz_u16x2, r[0].x & 0x7FFF7FFFu);
    const qz_u16x2 a1 = __builtin_bit_cast(qz_u16x2, r[0].y & 0x7FFF7FFFu);
    const qz_u16x2 a2 = __builtin_bit_cast(qz_u16x2, r[0].z & 0x7FFF7FFFu);
    const qz_u16x2 a3 = __builtin_bit_cast(qz_u16x2, r[0].w & 0x7FFF7FFFu);
    const uint32_t m = __builtin_bit_cast(
        uint32_t, __builtin_elementwise_max(__builtin_elementwise_max(a0, a1), __builtin_elementwise_max(a2, a3)));
    return max(m << 16, m & 0xFFFF0000u);
  } else {
    uint32_t m = 0;
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = max(m, r[v][i] & 0x7FFFFFFFu);
    return m;
  }
}

// Weight i (0..7) of a lane's 8 as fp32.
template <bool BF16>
__device__ __forceinline__ float weight_of(const qz_u32x4* r, int i) {
  if (BF16) {
    const uint32_t wd = r[0][i >> 1];
    return __uint_as_float((i & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
  }
  return __uint_as_float(r[i >> 2][i & 3]);
}

// Bucket of x: b = round-to-nearest-even(16 x + 16), 0..32 for x in [-1, 1].
// One fma lands 16 x + 16 + 1.5 * 2^23 in [2^23, 2^24), where fp32 spacing is
// 1, so b is the low mantissa field; shifting the bit pattern left by 3 and
// removing the shifted exponent bits (mod 2^32) gives the table entry's byte
// offset 8 b.
// With MAPPED (a codebook other than NF4) the same holds for the finer table:
// scale 512 instead of 16, and the entry's second word holds the codes below
// and above the threshold (low and high 16 bits) instead of a base code.
constexpr uint32_t kBucketBits = 0x4B400000u; // bit pattern of 1.5 * 2^23
constexpr uint32_t kBucketBias = 0u - (kBucketBits << 3);

template <bool MAPPED>
struct QzBuckets {
  static constexpr float S = MAPPED ? (float)kFineScale : 16.0f;      // buckets per unit of x
  static constexpr float MAGIC = 12582912.0f + S;                    // 1.5 * 2^23 + S
  static constexpr int N = MAPPED ? kFineBuckets : kBuckets;
};

template <bool MAPPED>
__device__ __forceinline__ uint32_t code_of(float x, uint2 t) {
  const bool above = x > __uint_as_float(t.x);
  if (MAPPED) return above ? (t.y >> 16) : (t.y & 0xFFFFu);
  return t.y + (above ? 1u : 0u);
}

// Codes of a lane's 8 weights (normalised by inv, |x| <= 1), packed
// low nibble first.
template <bool BF16, bool MAPPED>
__device__ __forceinline__ uint32_t code8_fast(const qz_u32x4* r, float inv, const uint2* s_tab) {
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = weight_of<BF16>(r, i) * inv;
    const float y = __builtin_fmaf(x, QzBuckets<MAPPED>::S, QzBuckets<MAPPED>::MAGIC);
    const uint32_t off = (__float_as_uint(y) << 3) + kBucketBias;
    const uint2 t = *reinterpret_cast<const uint2*>(reinterpret_cast<const char*>(s_tab) + off);
    packed |= code_of<MAPPED>(x, t) << (4 * i);
  }
  return packed;
}

// As code8_fast with the weights first scaled by sc (exact) and the bucket
// index clamped, so that any input (NaN included) reads inside the table.
template <bool BF16, bool MAPPED>
__device__ __forceinline__ uint32_t code8_generic(const qz_u32x4* r, float sc, float inv, const uint2* s_tab) {
  uint32_t packed = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = (weight_of<BF16>(r, i) * sc) * inv;
    const float y = __builtin_fmaf(x, QzBuckets<MAPPED>::S, QzBuckets<MAPPED>::MAGIC);
    int b = (int)(__float_as_uint(y) - kBucketBits);
    b = b < 0 ? 0 : (b > QzBuckets<MAPPED>::N - 1 ? QzBuckets<MAPPED>::N - 1 : b);
    const uint2 t = s_tab[b];
    packed |= code_of<MAPPED>(x, t) << (4 * i);
  }
  return packed;
}

// Entry b of the finer table of a codebook: bucket [(b - 1/2)/S - 1,
// (b + 1/2)/S - 1] holds at most one midpoint; below it lie `base` of them.
__device__ __forceinline__ uint2 fine_entry(const CodeSpec& sp, int b) {
  const double lo = (b - 0.5) / kFineScale - 1.0, hi = (b + 0.5) / kFineScale - 1.0;
  int base = 0, in = -1;
  for (int i = 0; i < sp.nmid; ++i) {
    base += sp.mid[i] < lo;
    if (sp.mid[i] >= lo && sp.mid[i] < hi) in = i;
  }
  const uint32_t below = sp.rank_code[base];
  const uint32_t above = in >= 0 ? sp.rank_code[base + 1] : below;
  return make_uint2(in >= 0 ? __float_as_uint(sp.thr[in]) : 0x7F800000u, below | (above << 16));
}

__device__ __forceinline__ void add_c2(unsigned long long* acc, float c2) {
  uint32_t d, lo, hi;
  c2_digits(c2, d, lo, hi);
  atomicAdd(&acc[d], (unsigned long long)lo);
  if (hi) atomicAdd(&acc[d + 1], (unsigned long long)hi);
}

// One wave step of 512 weights with every check: the lane's 8 weights start
// at e0 (zeros past numel); block constants of blocks past nb are not
// stored, and the nibble of a missing element is 0.
template <bool BF16, bool MAPPED>
__device__ __forceinline__ void generic_step(const qz_u32x4* r, int64_t e0, int64_t numel, int64_t nb,
                                             uint8_t* __restrict__ codes, float* __restrict__ c2out,
                                             unsigned long long* acc, const uint2* s_tab, int lane) {
  const float c2 = __uint_as_float(octet_max(absmax_bits<BF16>(r)));
  const bool tiny = c2 > 0.0f && c2 < kTiny;
  const float sc = tiny ? kPrescale : 1.0f;
  const float cs = c2 * sc;
  const float inv = cs > 0.0f ? 1.0f / cs : 0.0f;  // correctly rounded division
  uint32_t packed = code8_generic<BF16, MAPPED>(r, sc, inv, s_tab);
  if (e0 + 7 < numel) {
    *reinterpret_cast<uint32_t*>(codes + (e0 >> 1)) = packed;
  } else if (e0 < numel) {
    const int have = (int)(numel - e0);  // 1..7
    packed &= (1u << (4 * have)) - 1u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (2 * j < have) codes[(e0 >> 1) + j] = (uint8_t)(packed >> (8 * j));
  }
  const int64_t blk = e0 >> 6;
  if ((lane & 7) == 0 && blk < nb) {
    c2out[blk] = c2;
    if (acc && c2 > 0.0f) add_c2(acc, c2);
  }
}

// A lane's 8 weights from e0 with bounds checks (zeros past numel).
template <bool BF16>
__device__ __forceinline__ void load_partial(const void* __restrict__ w, int64_t e0, int64_t numel, qz_u32x4* r) {
  if (e0 + 7 < numel) {
    const qz_u32x4* p = reinterpret_cast<const qz_u32x4*>(BF16 ? (const char*)w + e0 * 2 : (const char*)w + e0 * 4);
#pragma unroll
    for (int v = 0; v < QzGeo<BF16>::NV; ++v) r[v] = p[v];
    return;
  }
#pragma unroll
  for (int v = 0; v < QzGeo<BF16>::NV; ++v) r[v] = qz_u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t e = e0 + i;
    if (e < numel) {
      if (BF16) {
        const uint32_t h = reinterpret_cast<const uint16_t*>(w)[e];
        r[0][i >> 1] |= (i & 1) ? (h << 16) : h;
      } else {
        r[i >> 2][i & 3] = reinterpret_cast<const uint32_t*>(w)[e];
      }
    }
  }
}

// The work of workgroup `bid` of `G` quantising one tensor (the grid of a
// single-tensor launch, or this tensor's share of a batched launch).
template <bool BF16, bool MAPPED>
__device__ __forceinline__ void nf4_quantize_wg(const void* __restrict__ w, int64_t numel, uint8_t* __restrict__ codes,
                                                float* __restrict__ c2out, uint64_t* __restrict__ partials,
                                                const QuantTable& tab, const CodeSpec& spec, int64_t G, int64_t bid) {
  using Geo = QzGeo<BF16>;
  constexpr int STEPS = Geo::STEPS, NV = Geo::NV;
  constexpr int64_t CH = Geo::CH;
  constexpr int ES = BF16 ? 2 : 4;  // bytes per input weight
  __shared__ uint2 s_tab[QzBuckets<MAPPED>::N];  // {threshold bits, base code | codes below/above}
  __shared__ unsigned long long s_acc[QZ_WAVES][kMeanDigits];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (MAPPED) {
    for (int b = tid; b < QzBuckets<MAPPED>::N; b += QZ_THREADS) s_tab[b] = fine_entry(spec, b);
  } else if (tid < kBuckets) {
    s_tab[tid] = make_uint2(__float_as_uint(tab.thr[tid]), tab.base[tid]);
  }
  if (tid < QZ_WAVES * kMeanDigits) (&s_acc[0][0])[tid] = 0;
  __syncthreads();

  const int64_t nb = (numel + 63) >> 6;
  const int64_t nfull = numel / CH;
  unsigned long long* acc = partials ? s_acc[wave] : nullptr;
  const uint32_t lane_off = (uint32_t)(wave * 512 + lane * 8);  // weights, within a step row
  const int k = lane & 7;

  auto load_chunk = [&](int64_t c, qz_u32x4 (&r)[STEPS][NV]) {
    const char* base = (const char*)w + c * CH * ES;
#pragma unroll
    for (int s = 0; s < STEPS; ++s)
#pragma unroll
      for (int v = 0; v < NV; ++v)
        r[s][v] = *reinterpret_cast<const qz_u32x4*>(base + ((uint32_t)(s * QZ_WAVES * 512) + lane_off) * ES + 16 * v);
  };

  auto process = [&](int64_t c, qz_u32x4 (&r)[STEPS][NV]) {
    // A: every step's block absmax; lane 8j+k keeps block j of step k
    uint32_t comb = 0;
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const uint32_t m = octet_max(absmax_bits<BF16>(r[s]));
      comb = k == s ? m : comb;
    }
    const bool mine = k < STEPS;
    const bool normal = comb == 0u || comb - 0x00800000u < 0x7F000000u;  // zero, or a finite normal
    if (__builtin_amdgcn_ballot_w64(mine && !normal)) {  // rare, wave-uniform
#pragma unroll
      for (int s = 0; s < STEPS; ++s)
        generic_step<BF16, MAPPED>(r[s], c * CH + s * QZ_WAVES * 512 + lane_off, numel, nb, codes, c2out, acc,
                                   s_tab, lane);
      return;
    }
    // B: one block per lane
    const float c2 = __uint_as_float(comb);
    if (mine) {
      c2out[c * (CH / 64) + (k * QZ_WAVES + wave) * 8 + (lane >> 3)] = c2;
      if (acc && comb) add_c2(acc, c2);
    }
    const float inv = comb ? 1.0f / c2 : 0.0f;  // correctly rounded division
    // C: code each step with its block's reciprocal
    const int src = (lane & ~7) << 2;
    uint8_t* cb = codes + c * (CH / 2);
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      const float inv_s = __int_as_float(__builtin_amdgcn_ds_bpermute(src + 4 * s, __float_as_int(inv)));
      *reinterpret_cast<uint32_t*>(cb + (((uint32_t)(s * QZ_WAVES * 512) + lane_off) >> 1)) =
          code8_fast<BF16, MAPPED>(r[s], inv_s, s_tab);
    }
  };

  qz_u32x4 ra[STEPS][NV], rb[STEPS][NV];
  int64_t c = bid;
  if (c < nfull) load_chunk(c, ra);
  while (c < nfull) {
    const int64_t c1 = c + G;
    if (c1 < nfull) load_chunk(c1, rb);
    process(c, ra);
    if (c1 >= nfull) break;
    const int64_t c2i = c1 + G;
    if (c2i < nfull) load_chunk(c2i, ra);
    process(c1, rb);
    c = c2i;
  }

  // the final partial chunk, as 512-weight wave steps over all workgroups
  const int64_t tail0 = nfull * CH;
  if (tail0 < numel) {
    const int64_t T = (numel - tail0 + 511) >> 9;
    const int64_t rot = (bid + G - nfull % G) % G;  // workgroups with fewer full chunks first
    for (int64_t t = rot * QZ_WAVES + wave; t < T; t += G * QZ_WAVES) {
      const int64_t e0 = tail0 + t * 512 + lane * 8;
      qz_u32x4 r[NV];
      load_partial<BF16>(w, e0, numel, r);
      generic_step<BF16, MAPPED>(r, e0, numel, nb, codes, c2out, acc, s_tab, lane);
    }
  }
  if (partials) {
    __syncthreads();
    if (tid < kMeanDigits) {
      unsigned long long t = 0;
#pragma unroll
      for (int v = 0; v < QZ_WAVES; ++v) t += s_acc[v][tid];
      partials[(int64_t)tid * G + bid] = t;  // digit-major
    }
  }
}

template <bool BF16, bool MAPPED>
__global__ __launch_bounds__(QZ_THREADS) void nf4_quantize_kernel(const void* __restrict__ w, int64_t numel,
                                                                  uint8_t* __restrict__ codes,
                                                                  float* __restrict__ c2out,
                                                                  uint64_t* __restrict__ partials, QuantTable tab,
                                                                  CodeSpec spec) {
  nf4_quantize_wg<BF16, MAPPED>(w, numel, codes, c2out, partials, tab, spec, gridDim.x, blockIdx.x);
}

// ------------------------------------------------- Int8 quantise kernel
// Blockwise Eq. 1 with 127 levels per side.  A lane codes 8 consecutive
// weights (one 8-byte store), an octet of lanes one 64-block, a wave 512
// weights per step.  Waves stride over the steps of the tensor, U steps per
// iteration so that U loads are in flight (the last, partial step with
// bounds checks); every lane takes its octet's
// absmax (DPP) and the correctly rounded reciprocal itself.  The level of x:
// p0 = rint(127 x) is within one of it, the side of 127 x from p0 names the
// pair (p, p + 1) it lies between, and one threshold of that pair decides
// (ties keep p, the smaller value).  NaN and out-of-range x clamp into
// [-127, 127].  Away from the decision points p0 itself is the level, so the
// threshold lookup runs only for lanes holding a weight near one.  Exact-sum counters and the c2 layout are those of the 4-bit
// kernel, so double quantisation is shared.

// 16 waves per workgroup (the grid is capped at QZ_MAX_WG workgroups, one
// exact-sum partial each, so occupancy comes from the workgroup size).
constexpr int Q8_THREADS = 1024;
constexpr int Q8_WAVES = Q8_THREADS / 64;

template <bool BF16>
struct Q8Geo {
  static constexpr int U = BF16 ? 4 : 1;   // steps in flight per wave
  static constexpr int NV = BF16 ? 1 : 2;  // 16-byte loads per lane and step
};

__device__ __forceinline__ uint32_t int8_code_exact(float x, const float* s_thr) {
  const float t = x * 127.0f;
  const float p0 = __builtin_rintf(t);
  float p = t >= p0 ? p0 : p0 - 1.0f;
  p = fminf(fmaxf(p, -127.0f), 126.0f);  // NaN becomes -127
  const int pi = (int)p;
  return (uint32_t)(pi + (x > s_thr[pi + 127] ? 1 : 0)) & 0xFFu;
}

// Fast path: rint(127 x) is the level unless 127 x lies within 5e-4 of a
// half-integer (the fp32 roundings of 127 x and of the levels k / 127 move
// the comparison by under 1e-5).  Such an x, or NaN, sets `near`, and the
// caller codes the lane again through the thresholds.
__device__ __forceinline__ uint32_t int8_code_fast(float x, bool& near) {
  const float t = x * 127.0f;
  const float p0 = __builtin_rintf(t);
  near = near || !(fabsf(t - p0) <= 0.4995f);
  return (uint32_t)(int)p0 & 0xFFu;
}

template <bool BF16>
__device__ __forceinline__ void int8_quantize_wg(const void* __restrict__ w, int64_t numel,
                                                 uint8_t* __restrict__ codes, float* __restrict__ c2out,
                                                 uint64_t* __restrict__ partials, const Int8Tables& tab, int64_t G,
                                                 int64_t bid) {
  constexpr int U = Q8Geo<BF16>::U, NV = Q8Geo<BF16>::NV;
  constexpr int ES = BF16 ? 2 : 4;
  __shared__ float s_thr[254];
  __shared__ unsigned long long s_acc[Q8_WAVES][kMeanDigits];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  if (tid < 254) s_thr[tid] = tab.thr[tid];
  if (tid < Q8_WAVES * kMeanDigits) (&s_acc[0][0])[tid] = 0;
  __syncthreads();
  unsigned long long* acc = partials ? s_acc[wave] : nullptr;
  const int64_t nb = (numel + 63) >> 6;
  const int64_t nsteps = (numel + 511) >> 9, GW = G * Q8_WAVES;

  // One step of a lane: 8 codes and, from lane 8j of each octet, the
  // block's constant.  `full`: all 512 weights of the step exist.
  auto code_step = [&](const qz_u32x4* r, int64_t e0, bool full) {
    const float c2 = __uint_as_float(octet_max(absmax_bits<BF16>(r)));
    const bool tiny = c2 > 0.0f && c2 < kTiny;
    const float sc = tiny ? kPrescale : 1.0f;
    const float cs = c2 * sc;
    const float inv = cs > 0.0f ? 1.0f / cs : 0.0f;  // correctly rounded division
    float x[8];
    if (__builtin_amdgcn_ballot_w64(tiny)) {  // rare, wave-uniform
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = (weight_of<BF16>(r, i) * sc) * inv;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = weight_of<BF16>(r, i) * inv;
    }
    bool near = false;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t b = int8_code_fast(x[i], near);
      if (i < 4) lo |= b << (8 * i);
      else hi |= b << (8 * (i - 4));
    }
    if (near) {
      lo = hi = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t b = int8_code_exact(x[i], s_thr);
        if (i < 4) lo |= b << (8 * i);
        else hi |= b << (8 * (i - 4));
      }
    }
    if (full || e0 + 7 < numel) {
      *reinterpret_cast<uint2*>(codes + e0) = make_uint2(lo, hi);
    } else if (e0 < numel) {
      for (int i = 0; i < 8 && e0 + i < numel; ++i) codes[e0 + i] = (uint8_t)((i < 4 ? lo : hi) >> (8 * (i & 3)));
    }
    const int64_t blk = e0 >> 6;
    if ((lane & 7) == 0 && (full || blk < nb)) {
      c2out[blk] = c2;
      if (acc && c2 > 0.0f) add_c2(acc, c2);
    }
  };

  const int64_t nfull = numel >> 9;  // steps with all 512 weights present
  for (int64_t t = bid * Q8_WAVES + wave; t < nsteps; t += U * GW) {  // wave-uniform
    qz_u32x4 r[U][NV];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tu = t + u * GW, e0 = (tu << 9) + lane * 8;
      if (tu < nfull) {
#pragma unroll
        for (int v = 0; v < NV; ++v) r[u][v] = *reinterpret_cast<const qz_u32x4*>((const char*)w + e0 * ES + 16 * v);
      } else if (tu < nsteps) {
        load_partial<BF16>(w, e0, numel, r[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t tu = t + u * GW;
      if (tu < nfull) code_step(r[u], (tu << 9) + lane * 8, true);
      else if (tu < nsteps) code_step(r[u], (tu << 9) + lane * 8, false);
    }
  }
  if (partials) {
    __syncthreads();
    if (tid < kMeanDigits) {
      unsigned long long s = 0;
#pragma unroll
      for (int v = 0; v < Q8_WAVES; ++v) s += s_acc[v][tid];
      partials[(int64_t)tid * G + bid] = s;  // digit-major
    }
  }
}

template <bool BF16>
__global__ __launch_bounds__(Q8_THREADS) void int8_quantize_kernel(const void* __restrict__ w, int64_t numel,
                                                                   uint8_t* __restrict__ codes,
                                                                   float* __restrict__ c2out,
                                                                   uint64_t* __restrict__ partials, Int8Tables tab) {
  int8_quantize_wg<BF16>(w, numel, codes, c2out, partials, tab, gridDim.x, blockIdx.x);
}

// ------------------------------------------------ batched quantisation
// Up to kQuantBatch tensors per launch: tensor i takes workgroups
// [begin[i], begin[i + 1]) of the grid, quantize_parts_batched of them
// (fewer than its own launch for small tensors: the batch fills the chip,
// so each workgroup streams longer).  Codes and c2 are per element and the
// exact-sum partials add to the same total in any split, so every tensor is
// coded exactly as by its own call.  The tensor of a workgroup is found
// with an unrolled scan over constant indices (no dynamic indexing of the
// kernel argument, which would go through scratch).
struct QuantBatchArgs {
  const void* w[kQuantBatch];
  int64_t numel[kQuantBatch];
  uint8_t* codes[kQuantBatch];
  float* c2[kQuantBatch];
  uint64_t* partials[kQuantBatch];
  int parts[kQuantBatch];
  int begin[kQuantBatch];
  int count;
};

struct QuantBatchPick {
  const void* w;
  int64_t numel;
  uint8_t* codes;
  float* c2;
  uint64_t* partials;
  int parts, begin;
};

__device__ __forceinline__ QuantBatchPick pick_tensor(const QuantBatchArgs& b) {
  QuantBatchPick t{b.w[0], b.numel[0], b.codes[0], b.c2[0], b.partials[0], b.parts[0], b.begin[0]};
  const int bid = blockIdx.x;
#pragma unroll
  for (int j = 1; j < kQuantBatch; ++j) {
    if (j < b.count && bid >= b.begin[j]) {
      t = QuantBatchPick{b.w[j], b.numel[j], b.codes[j], b.c2[j], b.partials[j], b.parts[j], b.begin[j]};
    }
  }
  return t;
}

template <bool BF16, bool MAPPED>
__global__ __launch_bounds__(QZ_THREADS) void nf4_quantize_batched_kernel(const QuantBatchArgs b, QuantTable tab,
                                                                          CodeSpec spec) {
  const QuantBatchPick t = pick_tensor(b);
  nf4_quantize_wg<BF16, MAPPED>(t.w, t.numel, t.codes, t.c2, t.partials, tab, spec, t.parts,
                                (int64_t)blockIdx.x - t.begin);
}

template <bool BF16>
__global__ __launch_bounds__(Q8_THREADS) void int8_quantize_batched_kernel(const QuantBatchArgs b, Int8Tables tab) {
  const QuantBatchPick t = pick_tensor(b);
  int8_quantize_wg<BF16>(t.w, t.numel, t.codes, t.c2, t.partials, tab, t.parts, (int64_t)blockIdx.x - t.begin);
}

hipError_t launch_quantize(const void* w, bool w_bf16, int64_t numel, int code_type, uint8_t* codes, float* c2,
                           uint64_t* partials, hipStream_t stream) {
  if (code_type < 0 || code_type > CODE_INT8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)quantize_parts(numel)), block(QZ_THREADS);
  if (code_type == CODE_INT8) {
    const Int8Tables& t8 = int8_tables();
    if (w_bf16)
      hipLaunchKernelGGL((int8_quantize_kernel<true>), grid, dim3(Q8_THREADS), 0, stream, w, numel, codes, c2,
                         partials, t8);
    else
      hipLaunchKernelGGL((int8_quantize_kernel<false>), grid, dim3(Q8_THREADS), 0, stream, w, numel, codes, c2,
                         partials, t8);
    return hipGetLastError();
  }
  const QuantTable& tab = quant_table();
  const CodeSpec& spec = code_spec(code_type);
  if (code_type == CODE_NF4) {
    if (w_bf16)
      hipLaunchKernelGGL((nf4_quantize_kernel<true, false>), grid, block, 0, stream, w, numel, codes, c2, partials,
                         tab, spec);
    else
      hipLaunchKernelGGL((nf4_quantize_kernel<false, false>), grid, block, 0, stream, w, numel, codes, c2, partials,
                         tab, spec);
  } else {
    if (w_bf16)
      hipLaunchKernelGGL((nf4_quantize_kernel<true, true>), grid, block, 0, stream, w, numel, codes, c2, partials,
                         tab, spec);
    else
      hipLaunchKernelGGL((nf4_quantize_kernel<false, true>), grid, block, 0, stream, w, numel, codes, c2, partials,
                         tab, spec);
  }
  return hipGetLastError();
}

namespace {

// Workgroups of the encode kernel for nb constants.
int encode_wgs(int64_t nb);

}  // namespace

// Encode workgroups of tensor i: [begin[i], begin[i + 1]) of the grid.
struct EncodeBatchArgs {
  const float* c2[kQuantBatch];
  int64_t nb[kQuantBatch];
  const uint64_t* partials[kQuantBatch];
  int parts[kQuantBatch];
  uint8_t* absmax_q[kQuantBatch];
  float* scale2[kQuantBatch];
  float* offset[kQuantBatch];
  int wgs[kQuantBatch];
  int begin[kQuantBatch];
  int count;
};

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
  for (int k = 0; k < kMeanDigits; ++k) v[k] = p < parts ? partials[(int64_t)k * parts + p] : 0;
  wave_sum_u64<kMeanDigits>(v);
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < kMeanDigits; ++k) s_part[wave][k] = v[k];
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

// Second kernel of the double quantisation: every workgroup first forms mu
// from the exact-sum counters (workgroup 0 stores it), then its waves encode
// 256-groups in a grid-stride loop (one group per wave at a time, the next
// group's constants loading while the current one is encoded).  The grid is
// capped, so mu is formed at most DQE_MAX_WG times.
constexpr int DQE_MAX_WG = 512;

// The work of encode workgroup `bid` of `G` for one tensor.
__device__ __forceinline__ void dq_encode_wg(const float* __restrict__ c2, int64_t nb,
                                             const uint64_t* __restrict__ partials, int parts,
                                             float* __restrict__ mu_out, uint8_t* __restrict__ absmax_q,
                                             float* __restrict__ scale2, int64_t G, int64_t bid) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t ng = (nb + 255) >> 8, gstep = G * 4;
  int64_t g = bid * 4 + wave;
  float cv[4];
  load_group(c2, g < ng ? g : 0, nb, lane, cv);  // independent of mu: these loads go out first
  const float mu = mean_from_partials<4>(partials, parts, nb);
  if (bid == 0 && threadIdx.x == 0) *mu_out = mu;
  for (; g < ng; g += gstep) {  // wave-uniform
    float cn[4];
    if (g + gstep < ng) load_group(c2, g + gstep, nb, lane, cn);
    encode_group(cv, g, nb, mu, absmax_q, scale2, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) cv[i] = cn[i];
  }
}

__global__ __launch_bounds__(256) void dq_encode_kernel(const float* __restrict__ c2, int64_t nb,
                                                        const uint64_t* __restrict__ partials, int parts,
                                                        float* __restrict__ mu_out,
                                                        uint8_t* __restrict__ absmax_q,
                                                        float* __restrict__ scale2) {
  dq_encode_wg(c2, nb, partials, parts, mu_out, absmax_q, scale2, gridDim.x, blockIdx.x);
}

__global__ __launch_bounds__(256) void dq_encode_batched_kernel(const EncodeBatchArgs b) {
  const float* c2 = b.c2[0];
  int64_t nb = b.nb[0];
  const uint64_t* partials = b.partials[0];
  int parts = b.parts[0], wgs = b.wgs[0], begin = b.begin[0];
  uint8_t* absmax_q = b.absmax_q[0];
  float* scale2 = b.scale2[0];
  float* offset = b.offset[0];
  const int bid = blockIdx.x;
#pragma unroll
  for (int j = 1; j < kQuantBatch; ++j) {
    if (j < b.count && bid >= b.begin[j]) {
      c2 = b.c2[j]; nb = b.nb[j]; partials = b.partials[j]; parts = b.parts[j]; wgs = b.wgs[j];
      begin = b.begin[j]; absmax_q = b.absmax_q[j]; scale2 = b.scale2[j]; offset = b.offset[j];
    }
  }
  dq_encode_wg(c2, nb, partials, parts, offset, absmax_q, scale2, wgs, bid - begin);
}

namespace {
int encode_wgs(int64_t nb) {
  const int64_t ng = (nb + 255) / 256;
  return (int)((ng + 3) / 4 < DQE_MAX_WG ? (ng + 3) / 4 : DQE_MAX_WG);
}
}  // namespace

hipError_t launch_double_quant(const float* c2, int64_t nb, const uint64_t* partials, int parts, uint8_t* absmax_q,
                               float* scale2, float* offset, hipStream_t stream) {
  if (parts < 1 || parts > QZ_MAX_WG || QZ_MAX_WG > 256) return hipErrorInvalidValue;
  const int64_t wgs = encode_wgs(nb);
  hipLaunchKernelGGL(dq_encode_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, c2, nb, partials, parts, offset,
                     absmax_q, scale2);
  return hipGetLastError();
}

hipError_t launch_quantize_batched(const QuantJob* jobs, int count, bool w_bf16, int code_type, bool dq,
                                   hipStream_t stream) {
  if (code_type < 0 || code_type > CODE_INT8 || count < 0) return hipErrorInvalidValue;
  for (int j0 = 0; j0 < count; j0 += kQuantBatch) {
    const int n = count - j0 < kQuantBatch ? count - j0 : kQuantBatch;
    QuantBatchArgs qa;
    memset(&qa, 0, sizeof(qa));
    int total = 0;
    for (int i = 0; i < n; ++i) {
      const QuantJob& jb = jobs[j0 + i];
      qa.w[i] = jb.w; qa.numel[i] = jb.numel; qa.codes[i] = jb.codes; qa.c2[i] = jb.c2;
      qa.partials[i] = dq ? jb.partials : nullptr;
      qa.parts[i] = quantize_parts_batched(jb.numel);
      qa.begin[i] = total;
      total += qa.parts[i];
    }
    qa.count = n;
    const dim3 grid((unsigned)total);
    if (code_type == CODE_INT8) {
      const Int8Tables& t8 = int8_tables();
      if (w_bf16)
        hipLaunchKernelGGL((int8_quantize_batched_kernel<true>), grid, dim3(Q8_THREADS), 0, stream, qa, t8);
      else
        hipLaunchKernelGGL((int8_quantize_batched_kernel<false>), grid, dim3(Q8_THREADS), 0, stream, qa, t8);
    } else {
      const QuantTable& tab = quant_table();
      const CodeSpec& spec = code_spec(code_type);
      if (code_type == CODE_NF4) {
        if (w_bf16)
          hipLaunchKernelGGL((nf4_quantize_batched_kernel<true, false>), grid, dim3(QZ_THREADS), 0, stream, qa, tab,
                             spec);
        else
          hipLaunchKernelGGL((nf4_quantize_batched_kernel<false, false>), grid, dim3(QZ_THREADS), 0, stream, qa,
                             tab, spec);
      } else {
        if (w_bf16)
          hipLaunchKernelGGL((nf4_quantize_batched_kernel<true, true>), grid, dim3(QZ_THREADS), 0, stream, qa, tab,
                             spec);
        else
          hipLaunchKernelGGL((nf4_quantize_batched_kernel<false, true>), grid, dim3(QZ_THREADS), 0, stream, qa, tab,
                             spec);
      }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !dq) {
      if (e != hipSuccess) return e;
      continue;
    }
    EncodeBatchArgs ea;
    memset(&ea, 0, sizeof(ea));
    total = 0;
    for (int i = 0; i < n; ++i) {
      const QuantJob& jb = jobs[j0 + i];
      const int64_t nb = (jb.numel + 63) / 64;
      ea.c2[i] = jb.c2; ea.nb[i] = nb; ea.partials[i] = jb.partials; ea.parts[i] = qa.parts[i];
      ea.absmax_q[i] = jb.absmax_q; ea.scale2[i] = jb.scale2; ea.offset[i] = jb.offset;
      ea.wgs[i] = encode_wgs(nb);
      ea.begin[i] = total;
      total += ea.wgs[i];
    }
    ea.count = n;
    hipLaunchKernelGGL(dq_encode_batched_kernel, dim3((unsigned)total), dim3(256), 0, stream, ea);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

// --------------------------------------------------------- dequantise
// Each thread expands 8 codes (one 32-bit word of 4-bit codes, or 8 Int8
// bytes) of one block; a workgroup of 256 threads covers 4 x 2048 weights.
// c2_hat is computed as two separately rounded fp32 operations (this file is
// built without contraction).

constexpr int DQZ_THREADS = 256;
constexpr int DQZ_STEPS = 4;
constexpr int DQZ_PER_WG = DQZ_THREADS * 8 * DQZ_STEPS;

// Value of every code: 16 entries used for the 4-bit types, 256 for Int8.
struct DequantTable {
  float v[256];
};

// Codes e0 .. e0 + 7 as 8 table indices packed in 4 bits (uint2.x) or 8 bits
// (uint2.y:x) each.
template <bool INT8>
__device__ __forceinline__ uint2 load_codes8(const uint8_t* __restrict__ codes, int64_t e0) {
  if (INT8) return *reinterpret_cast<const uint2*>(codes + e0);
  return make_uint2(*reinterpret_cast<const uint32_t*>(codes + (e0 >> 1)), 0u);
}

template <bool INT8>
__device__ __forceinline__ uint2 load_codes8_partial(const uint8_t* __restrict__ codes, int64_t e0, int64_t numel) {
  uint32_t lo = 0, hi = 0;
  if (INT8) {
    for (int i = 0; i < 8 && e0 + i < numel; ++i) {
      const uint32_t b = codes[e0 + i];
      if (i < 4) lo |= b << (8 * i);
      else hi |= b << (8 * (i - 4));
    }
  } else {
    for (int i = 0; i < 4; ++i)
      if (e0 + 2 * i < numel) lo |= (uint32_t)codes[(e0 >> 1) + i] << (8 * i);
  }
  return make_uint2(lo, hi);
}

template <bool INT8>
__device__ __forceinline__ uint32_t code_at(uint2 c, int i) {
  if (INT8) return ((i < 4 ? c.x : c.y) >> (8 * (i & 3))) & 0xFFu;
  return (c.x >> (4 * i)) & 0xFu;
}

template <bool BF16_OUT>
__device__ __forceinline__ void store8(void* __restrict__ out, int64_t e0, const float v[8]) {
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

template <bool DQ, bool BF16_OUT, bool INT8>
__global__ __launch_bounds__(DQZ_THREADS) void nf4_dequant_kernel(const uint8_t* __restrict__ codes, int64_t numel,
                                                                  const uint8_t* __restrict__ absmax_q,
                                                                  const float* __restrict__ absmax,
                                                                  const float* __restrict__ scale2,
                                                                  const float* __restrict__ offset,
                                                                  void* __restrict__ out, DequantTable tab) {
  constexpr int NT = INT8 ? 256 : 16;
  __shared__ float s_val[NT];
  if (threadIdx.x < NT) s_val[threadIdx.x] = tab.v[threadIdx.x];
  __syncthreads();
  const float mu = DQ ? *offset : 0.0f;
  const int64_t wg0 = (int64_t)blockIdx.x * DQZ_PER_WG;
  if (wg0 + DQZ_PER_WG <= numel) {
    // a whole chunk: every load goes out before the first is used
    uint2 word[DQZ_STEPS];
    uint32_t qb[DQZ_STEPS];
    float f[DQZ_STEPS];
#pragma unroll
    for (int s = 0; s < DQZ_STEPS; ++s) {
      const int64_t e0 = wg0 + ((int64_t)s * DQZ_THREADS + threadIdx.x) * 8;
      const int64_t blk = e0 >> 6;
      word[s] = load_codes8<INT8>(codes, e0);
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
      for (int i = 0; i < 8; ++i) v[i] = s_val[code_at<INT8>(word[s], i)] * c;
      store8<BF16_OUT>(out, e0, v);
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
    const uint2 word = e0 + 7 < numel ? load_codes8<INT8>(codes, e0) : load_codes8_partial<INT8>(codes, e0, numel);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = s_val[code_at<INT8>(word, i)] * c;
    if (e0 + 7 < numel) {
      store8<BF16_OUT>(out, e0, v);
    } else {
      for (int i = 0; i < 8; ++i) {
        if (e0 + i >= numel) break;
        if (BF16_OUT) reinterpret_cast<uint16_t*>(out)[e0 + i] = f2bf(v[i]);
        else reinterpret_cast<float*>(out)[e0 + i] = v[i];
      }
    }
  }
}

template <bool INT8>
hipError_t launch_dequant_t(const uint8_t* codes, int64_t numel, bool dq, const uint8_t* absmax_q,
                            const float* absmax, const float* scale2, const float* offset, void* out, bool out_bf16,
                            const DequantTable& t, hipStream_t stream) {
  const dim3 grid((unsigned)((numel + DQZ_PER_WG - 1) / DQZ_PER_WG)), block(DQZ_THREADS);
  if (dq) {
    if (out_bf16)
      hipLaunchKernelGGL((nf4_dequant_kernel<true, true, INT8>), grid, block, 0, stream, codes, numel, absmax_q,
                         absmax, scale2, offset, out, t);
    else
      hipLaunchKernelGGL((nf4_dequant_kernel<true, false, INT8>), grid, block, 0, stream, codes, numel, absmax_q,
                         absmax, scale2, offset, out, t);
  } else {
    if (out_bf16)
      hipLaunchKernelGGL((nf4_dequant_kernel<false, true, INT8>), grid, block, 0, stream, codes, numel, absmax_q,
                         absmax, scale2, offset, out, t);
    else
      hipLaunchKernelGGL((nf4_dequant_kernel<false, false, INT8>), grid, block, 0, stream, codes, numel, absmax_q,
                         absmax, scale2, offset, out, t);
  }
  return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, int64_t numel, int code_type, bool dq, const uint8_t* absmax_q,
                             const float* absmax, const float* scale2, const float* offset, void* out,
                             bool out_bf16, hipStream_t stream) {
  if (code_type < 0 || code_type > CODE_INT8) return hipErrorInvalidValue;
  DequantTable t;
  memset(&t, 0, sizeof(t));
  if (code_type == CODE_INT8) {
    memcpy(t.v, int8_tables().value, sizeof(t.v));
    return launch_dequant_t<true>(codes, numel, dq, absmax_q, absmax, scale2, offset, out, out_bf16, t, stream);
  }
  memcpy(t.v, code_values(code_type).v, 16 * sizeof(float));
  return launch_dequant_t<false>(codes, numel, dq, absmax_q, absmax, scale2, offset, out, out_bf16, t, stream);
}

}  // namespace qlora
