// Device helpers for the gfx950 QLoRA NF4 kernels: vector types, bf16 and
// FP8 (OCP E4M3FN) conversions, wave-level reductions and the MFMA tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlora {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------ bf16 helpers

// Nearest-even fp32 -> bf16 bit pattern (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return (uint32_t)f2bf(lo) | ((uint32_t)f2bf(hi) << 16);
}
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// ------------------------------------------------------- FP8 E4M3FN codec
// OCP E4M3FN: sign, 4-bit exponent with bias 7, 3-bit mantissa; exponent
// field 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN; largest finite 448.

__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  const uint32_t e = (b >> 3) & 0xF, m = b & 0x7;
  float v;
  if (e == 0) {
    v = (float)m * 0x1p-9f;  // exact
  } else if (e == 0xF && m == 0x7) {
    v = __uint_as_float(0x7FC00000u);
  } else {
    v = __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) * 2^(e-7)
  }
  return (b & 0x80) ? -v : v;
}

// Nearest-even encode of y with |y| <= 448 (callers clamp first); the sign
// is kept, so a negative value that rounds to zero gives 0x80.
__device__ __forceinline__ uint32_t e4m3_encode(float y) {
  const uint32_t bits = __float_as_uint(y);
  const uint32_t sign = (bits >> 24) & 0x80;
  const uint32_t a = bits & 0x7FFFFFFFu;
  uint32_t code;
  if (a < 0x3C800000u) {                 // |y| < 2^-6: subnormal grid m * 2^-9
    const float q = __uint_as_float(a) * 512.0f;  // exact power-of-two scaling
    code = (uint32_t)__builtin_rintf(q);          // nearest-even, 0..8 (8 = 2^-6)
  } else {
    const uint32_t e = (a >> 23) - 120u;          // E4M3 exponent field, >= 1
    const uint32_t mant = a & 0x7FFFFFu;
    uint32_t q = mant >> 20;
    const uint32_t rem = mant & 0xFFFFFu;
    const uint32_t up = (rem > 0x80000u) | ((rem == 0x80000u) & (q & 1u));
    code = ((e << 3) | q) + up;                   // a mantissa carry bumps the exponent
  }
  return sign | code;
}

// --------------------------------------------------------- wave reductions

// Max over each row of 16 lanes (every lane of the row gets the result).
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x121, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x122, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x124, 0xF, 0xF, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false)));
  return v;
}

// Max over the whole 64-lane wave (every lane gets the result).
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = __shfl_xor((uint32_t)v, o, 64);
    const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, 64);
    v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

// ------------------------------------------------------------- MFMA tile
// Block tile 128 x 128, k-step 64, 256 threads = 4 waves in a 2 x 2 grid,
// each wave 64 x 64 = 2 x 2 MFMA 32x32x16 bf16 tiles.
//
// v_mfma_f32_32x32x16_bf16 operand layout (lane l of 64):
//   A (32 x 16): row l % 32, k = 8 * (l / 32) .. +7
//   B (16 x 32): col l % 32, k = 8 * (l / 32) .. +7
//   D (32 x 32): col l % 32, register j -> row 8*(j/4) + 4*(l/32) + j%4
// Both LDS tiles hold 8 consecutive k per row segment ("k-contiguous"), so
// an operand fragment is one 16-byte LDS read.
constexpr int TM = 128, TN = 128, TK = 64;
constexpr int LDK = TK + 8;  // row pitch in bf16: 144 B keeps 8-lane groups conflict-free

struct Acc22 {
  floatx16 c[2][2];
};

__device__ __forceinline__ void acc_zero(Acc22& a) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) a.c[i][j][r] = 0.0f;
}

__device__ __forceinline__ void mma_128x128x64(const __bf16* sA, const __bf16* sB, Acc22& acc,
                                               int wm, int wn, int lane) {
  const int lr = lane & 31, lk = 8 * (lane >> 5);
#pragma unroll
  for (int kk = 0; kk < TK; kk += 16) {
    bf16x8 a[2], b[2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(sA + (wm * 64 + i * 32 + lr) * LDK + kk + lk);
#pragma unroll
    for (int j = 0; j < 2; ++j)
      b[j] = *reinterpret_cast<const bf16x8*>(sB + (wn * 64 + j * 32 + lr) * LDK + kk + lk);
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc.c[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc.c[i][j], 0, 0, 0);
  }
}

// Row / column of accumulator element (i, j, reg) for a lane.
__device__ __forceinline__ int acc_row(int wm, int i, int reg, int lane) {
  return wm * 64 + i * 32 + 8 * (reg >> 2) + 4 * (lane >> 5) + (reg & 3);
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) {
  return wn * 64 + j * 32 + (lane & 31);
}

}  // namespace qlora
