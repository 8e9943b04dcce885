// The keep mask of LoRA dropout drawn on the device from a counter-based
// generator, gfx950.
//
// QLoRA (Dettmers et al., arXiv 2305.14314), Appendix B.2: LoRA dropout 0.1
// (up to 13B) or 0.05 (33B, 65B), read as a Bernoulli(1 - p) mask on the
// adapter input.  The draw is Philox4x64-10 (Salmon, Moraes, Dror, Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011): mask byte b of the
// packed [M, K/8] mask takes key (seed, 0) and counter (b, offset, 0, 0); its
// four 64-bit outputs are eight 32-bit words u_j, and bit j (element 8c + j
// of the row) is 1 (kept) iff u_j >= T = floor(p * 2^32).  Every byte is
// independent, so a thread draws four bytes and writes one 32-bit word.
#include "device.h"
#include "launch.h"

namespace qlora {

namespace {

constexpr uint64_t kPhiloxM0 = 0xD2E7470EE14C6C93ull;  // the 4x64 round multipliers
constexpr uint64_t kPhiloxM1 = 0xCA5A826395121157ull;
constexpr uint64_t kPhiloxW0 = 0x9E3779B97F4A7C15ull;  // the key's Weyl increments
constexpr uint64_t kPhiloxW1 = 0xBB67AE8584CAA73Bull;

// One mask byte: the keep bits of the eight words of Philox4x64-10(counter
// (b, offset, 0, 0), key (seed, 0)).
__device__ __forceinline__ uint32_t mask_byte(uint64_t b, uint64_t offset, uint64_t seed, uint32_t T) {
  uint64_t c0 = b, c1 = offset, c2 = 0, c3 = 0, k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += kPhiloxW0;
      k1 += kPhiloxW1;
    }
    const uint64_t lo0 = kPhiloxM0 * c0, hi0 = __umul64hi(kPhiloxM0, c0);
    const uint64_t lo1 = kPhiloxM1 * c2, hi1 = __umul64hi(kPhiloxM1, c2);
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  const uint64_t o[4] = {c0, c1, c2, c3};
  uint32_t byte = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) byte |= (uint32_t)((uint32_t)(o[j >> 1] >> (32 * (j & 1))) >= T) << j;
  return byte;
}

__global__ __launch_bounds__(256) void dropout_mask_kernel(uint8_t* __restrict__ mask, int64_t nbytes, uint64_t seed,
                                                           uint64_t offset, uint32_t T) {
  const int64_t stride = (int64_t)gridDim.x * 256 * 4;
  for (int64_t b0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4; b0 < nbytes; b0 += stride) {
    if (b0 + 4 <= nbytes) {
      uint32_t w = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) w |= mask_byte((uint64_t)(b0 + i), offset, seed, T) << (8 * i);
      *reinterpret_cast<uint32_t*>(mask + b0) = w;
    } else {
      for (int64_t b = b0; b < nbytes; ++b) mask[b] = (uint8_t)mask_byte((uint64_t)b, offset, seed, T);
    }
  }
}

}  // namespace

hipError_t launch_dropout_mask(uint8_t* mask, int64_t nbytes, uint64_t seed, uint64_t offset, uint32_t T,
                               hipStream_t stream) {
  if (nbytes <= 0) return hipSuccess;
  int64_t wgs = (nbytes + 1023) / 1024;
  if (wgs > 8 * kCUs) wgs = 8 * kCUs;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)wgs), dim3(256), 0, stream, mask, nbytes, seed, offset, T);
  return hipGetLastError();
}

}  // namespace qlora
