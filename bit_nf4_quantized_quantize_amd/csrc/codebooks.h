// The 4-bit codebooks the library quantises against, in code order.
//
// NF4 is QLoRA Appendix E.  The other three are the types of the data-type
// comparison in QLoRA section 3 (Table 2: Int4, Float4 (E2M1), Float4
// (E3M0)), which the page names without values; each is taken from its
// bit-field definition with the largest magnitude normalised to 1, so that
// x = w / absmax in [-1, 1] is quantised against it exactly like NF4:
//   FP4 E2M1  code s e1 e0 m: magnitude m/2 (e = 0) or 2^(e-1) (1 + m/2),
//             divided by the largest, 6 (the OCP microscaling 4-bit float);
//   FP4 E3M0  code s e2 e1 e0: magnitude 0 (e = 0) or 2^(e-7);
//   INT4      code = two's-complement integer k, value k / 7 (Eq. 1's
//             absmax scaling with 7 levels per side; -8/7 is never produced).
// Every entry is an fp32 value (ratios rounded to nearest).
#pragma once

namespace qlora {

enum CodeType { CODE_NF4 = 0, CODE_FP4_E2M1 = 1, CODE_FP4_E3M0 = 2, CODE_INT4 = 3, CODE_TYPES = 4 };

// The 8-bit storage type (QLoRA section 2, Eq. 1, read blockwise like the
// 4-bit types): one byte per weight, the two's complement of k, value k / 127
// rounded to fp32 (256 entries; k = -128 is never produced).  The 4-bit
// tables above do not cover it; the generic GEMM kernel has an 8-bit
// variant, the 256 x 256 and weight-streaming kernels take 4-bit codes.
constexpr int CODE_INT8 = CODE_TYPES;

#define QLORA_CODE_VALUES                                                                                      \
  {                                                                                                            \
    {-1.0f, -0.6961928009986877f, -0.5250730514526367f, -0.39491748809814453f, -0.28444138169288635f,         \
     -0.18477343022823334f, -0.09105003625154495f, 0.0f, 0.07958029955625534f, 0.16093020141124725f,          \
     0.24611230194568634f, 0.33791524171829224f, 0.44070982933044434f, 0.5626170039176941f,                   \
     0.7229568362236023f, 1.0f},                                                                               \
    {0.0f, 0.5f / 6.0f, 1.0f / 6.0f, 1.5f / 6.0f, 2.0f / 6.0f, 3.0f / 6.0f, 4.0f / 6.0f, 1.0f,                \
     -0.0f, -0.5f / 6.0f, -1.0f / 6.0f, -1.5f / 6.0f, -2.0f / 6.0f, -3.0f / 6.0f, -4.0f / 6.0f, -1.0f},       \
    {0.0f, 0x1p-6f, 0x1p-5f, 0x1p-4f, 0x1p-3f, 0x1p-2f, 0x1p-1f, 1.0f,                                        \
     -0.0f, -0x1p-6f, -0x1p-5f, -0x1p-4f, -0x1p-3f, -0x1p-2f, -0x1p-1f, -1.0f},                               \
    {0.0f, 1.0f / 7.0f, 2.0f / 7.0f, 3.0f / 7.0f, 4.0f / 7.0f, 5.0f / 7.0f, 6.0f / 7.0f, 1.0f,                \
     -8.0f / 7.0f, -1.0f, -6.0f / 7.0f, -5.0f / 7.0f, -4.0f / 7.0f, -3.0f / 7.0f, -2.0f / 7.0f, -1.0f / 7.0f} \
  }

constexpr float kCodeValuesHost[CODE_TYPES][16] = QLORA_CODE_VALUES;

}  // namespace qlora
