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
// Two of them packed (lo in bits 0..15): one v_cvt_pk_bf16_f32 on both
// operands, where two scalar conversions would need a shift and an or more.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ float bf2f(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// ------------------------------------------------------- FP8 E4M3FN codec
// OCP E4M3FN: sign, 4-bit exponent with bias 7, 3-bit mantissa; exponent
// field 0 is subnormal (m * 2^-9); 0x7F / 0xFF are NaN; largest finite 448.

// Exact decode of the low byte of b with gfx950's native conversion
// (v_cvt_f32_fp8 reads the OCP E4M3FN format on this target).  One
// instruction and no branches, which matters where it sits between MFMAs.
__device__ __forceinline__ float e4m3_decode(uint32_t b) {
  return __builtin_amdgcn_cvt_f32_fp8((int)b, 0);
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

// ------------------------------------------------- byte permute (v_perm_b32)
// Result byte i = byte sel_i of the 64-bit value {s0:s1} (s1 = bytes 0..3);
// selector 12 gives 0x00 and 13..15 give 0xFF (8..11, sign replication, are
// not used here).  The host version exists so the lookup below can be
// checked on the CPU.
__host__ __device__ __forceinline__ uint32_t perm_b32(uint32_t s0, uint32_t s1, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_perm(s0, s1, sel);
#else
  const uint64_t v = ((uint64_t)s0 << 32) | s1;
  uint32_t out = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t sb = (sel >> (8 * i)) & 0xFF;
    uint32_t b;
    if (sb < 8) b = (uint32_t)(v >> (8 * sb)) & 0xFF;
    else if (sb == 12) b = 0;
    else b = 0xFF;
    out |= b << (8 * i);
  }
  return out;
#endif
}

// ------------------------------------------- per-block bf16 lookup table
// One NF4 block shares one constant c, so its 16 possible bf16 values
// bf16(NF4[i] * c) form a table.  The table is kept as two 16-byte planes
// (low and high bytes of each bf16), four registers each; v_perm_b32 then
// looks up four codes per instruction from one half-plane, and a third
// v_perm_b32, with a selector made from code bit 3, picks the half.  Values are exactly those of the
// dequantisation kernel: fp32 product, nearest-even bf16.
struct BlockLUT {
  uint32_t lo[4], hi[4];
};

// p[j] = bf16(v[2j]) | bf16(v[2j+1]) << 16 for the 16 table values v.
__host__ __device__ __forceinline__ BlockLUT make_lut(const uint32_t p[8]) {
  BlockLUT t;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    t.lo[q] = perm_b32(p[2 * q + 1], p[2 * q], 0x06040200u);
    t.hi[q] = perm_b32(p[2 * q + 1], p[2 * q], 0x07050301u);
  }
  return t;
}

// Selector that picks, per byte, byte i of the second v_perm_b32 operand
// (the table half for codes 0..7) when bit 0 of byte i of t is 0 and byte i
// of the first operand (codes 8..15) when it is 1.
__host__ __device__ __forceinline__ uint32_t lut_half_sel(uint32_t t) {
  return ((t & 0x01010101u) << 2) + 0x03020100u;
}

// Eight codes of one 32-bit word (element 0 in the low nibble) -> eight bf16
// in element order, as four 32-bit words.
__host__ __device__ __forceinline__ void lut_lookup8(const BlockLUT& t, uint32_t w, uint32_t out[4]) {
  const uint32_t e7 = w & 0x07070707u;                 // even elements, code & 7
  const uint32_t o7 = (w >> 4) & 0x07070707u;          // odd elements
  const uint32_t t3 = w >> 3;
  const uint32_t me = lut_half_sel(t3);                 // code bit 3 of the even elements
  const uint32_t mo = lut_half_sel(t3 >> 4);            // of the odd elements
  const uint32_t loE = perm_b32(perm_b32(t.lo[3], t.lo[2], e7), perm_b32(t.lo[1], t.lo[0], e7), me);
  const uint32_t hiE = perm_b32(perm_b32(t.hi[3], t.hi[2], e7), perm_b32(t.hi[1], t.hi[0], e7), me);
  const uint32_t loO = perm_b32(perm_b32(t.lo[3], t.lo[2], o7), perm_b32(t.lo[1], t.lo[0], o7), mo);
  const uint32_t hiO = perm_b32(perm_b32(t.hi[3], t.hi[2], o7), perm_b32(t.hi[1], t.hi[0], o7), mo);
  const uint32_t e01 = perm_b32(hiE, loE, 0x05010400u);  // bf16 of elements 0, 2
  const uint32_t o01 = perm_b32(hiO, loO, 0x05010400u);  // elements 1, 3
  const uint32_t e23 = perm_b32(hiE, loE, 0x07030602u);  // elements 4, 6
  const uint32_t o23 = perm_b32(hiO, loO, 0x07030602u);  // elements 5, 7
  out[0] = perm_b32(o01, e01, 0x05040100u);
  out[1] = perm_b32(o01, e01, 0x07060302u);
  out[2] = perm_b32(o23, e23, 0x05040100u);
  out[3] = perm_b32(o23, e23, 0x07060302u);
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

// Sums over the whole 64-lane wave of N values at once (every lane gets the
// sums); the N exchanges of each butterfly step are in flight together.
template <int N>
__device__ __forceinline__ void wave_sum_u64(uint64_t (&v)[N]) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    uint32_t lo[N], hi[N];
#pragma unroll
    for (int k = 0; k < N; ++k) {
      lo[k] = __shfl_xor((uint32_t)v[k], o, 64);
      hi[k] = __shfl_xor((uint32_t)(v[k] >> 32), o, 64);
    }
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] += ((uint64_t)hi[k] << 32) | lo[k];
  }
}

// ------------------------------------------------------- MFMA fragments
// v_mfma_f32_32x32x16_bf16 operand layout (lane l of 64):
//   A (32 x 16): row l % 32, k = 8 * (l / 32) .. +7
//   B (16 x 32): col l % 32, k = 8 * (l / 32) .. +7
//   D (32 x 32): col l % 32, register j -> row 8*(j/4) + 4*(l/32) + j%4
// Both operands want 8 consecutive reduction indices per lane.  Tiles in LDS
// come in two orders:
//   KC  [rows][red]  reduction contiguous: a fragment is one 16-byte read;
//   RC  [red][rows]  rows contiguous: a fragment is two ds_read_b64_tr_b16.
// ds_read_b64_tr_b16 works on groups of 16 lanes: lane i of a group receives
// element (i & 3) of the 8-byte chunk read by lane 4j + (i >> 2), for
// j = 0..3.  Pointing lane q of the group at reduction row base + q/4,
// column c0 + 4*(q%4) therefore hands lane q the four reduction values
// base..base+3 of column c0 + q.

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

__device__ __forceinline__ bf16x8 frag_kc(const __bf16* s, int pitch, int r0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8*>(s + (r0 + (lane & 31)) * pitch + k0 + 8 * (lane >> 5));
}

__device__ __forceinline__ short4_t ds_read_tr16(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)((__attribute__((address_space(3))) __bf16*)p));
}

__device__ __forceinline__ bf16x8 frag_rc(const __bf16* s, int pitch, int r0, int k0, int lane) {
  const int g = lane >> 4, q = lane & 15;
  const int col = r0 + 16 * (g & 1) + 4 * (q & 3);
  const int red = k0 + 8 * (g >> 1) + (q >> 2);
  const short4_t lo = ds_read_tr16(s + red * pitch + col);
  const short4_t hi = ds_read_tr16(s + (red + 4) * pitch + col);
  const short8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ floatx16 mfma32(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16 (lane l of 64): A (16 x 32) row l % 16 and B
// (32 x 16) column l % 16, each with reduction slots 8 * (l / 16) .. +7;
// D (16 x 16) column l % 16, register j -> row 4 * (l / 16) + j.
__device__ __forceinline__ floatx4 mfma16(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Row of accumulator register j of a 32x32 tile for a lane (column: lane % 32).
__device__ __forceinline__ int acc_row32(int j, int lane) {
  return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3);
}

}  // namespace qlora
