// Host driver for the per-block bf16 lookup of the GEMM kernels (BlockLUT,
// make_lut, lut_lookup8 in device.h, whose perm_b32 has a host branch).
// Reads lines of 9 + n hex words from stdin: the 8 packed table words
// p[j] = bf16(v[2j]) | bf16(v[2j+1]) << 16, the count n, then n 32-bit code
// words (8 codes each, element 0 in the low nibble); prints, per code word,
// the 4 output words (bf16 pairs in element order) in hex.
#include <stdio.h>

#include "device.h"

int main() {
  unsigned p[8], n;
  while (scanf("%x %x %x %x %x %x %x %x %x", &p[0], &p[1], &p[2], &p[3], &p[4], &p[5], &p[6], &p[7], &n) == 9) {
    uint32_t pw[8];
    for (int j = 0; j < 8; ++j) pw[j] = p[j];
    const qlora::BlockLUT t = qlora::make_lut(pw);
    for (unsigned i = 0; i < n; ++i) {
      unsigned w;
      if (scanf("%x", &w) != 1) return 2;
      uint32_t o[4];
      qlora::lut_lookup8(t, w, o);
      printf("%08x %08x %08x %08x\n", o[0], o[1], o[2], o[3]);
    }
  }
  return 0;
}
