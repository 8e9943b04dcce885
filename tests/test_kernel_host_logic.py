"""CPU checks of the arithmetic the GEMM kernels use to expand codes, against
the oracle (no GPU):

  * the per-block bf16 lookup (device.h: make_lut / lut_lookup8 over
    perm_b32, whose host branch models v_perm_b32) gives, for all 16 codes in
    every nibble position, the oracle's dequantised bf16 value
    bf16(value[code] * c) of QLoRA Eq. 6, for every 4-bit codebook and
    several block constants c;
  * the 8-bit expansion fp32(k / 127) = fma(r, R, q0) with q0 = k * R,
    R = fp32(1/127), r = k - 127 q0 (exact), is the correctly rounded
    k / 127 for all 256 code bytes, in exact rational arithmetic.
"""

import os
import shutil
import subprocess
from fractions import Fraction

import numpy as np
import pytest

from oracle import blockwise, codebook

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "bit_nf4_quantized_quantize_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.fixture(scope="module")
def lut_driver(tmp_path_factory):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    out = str(tmp_path_factory.mktemp("lut") / "lut_lookup_check")
    src = os.path.join(ROOT, "tests", "host", "lut_lookup_check.cpp")
    r = subprocess.run([HIPCC, "-O1", "-std=c++17", "-I", CSRC, src, "-o", out], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    return out


def _bf16_bits(x32):
    """bf16 bit patterns of fp32 values x32 (nearest-even, the oracle's rounding)."""
    return (blockwise.bf16_round(np.asarray(x32, np.float32)).view(np.uint32) >> 16).astype(np.uint32)


def test_block_lookup_matches_oracle_values(lut_driver):
    rng = np.random.default_rng(7)
    scales = [np.float32(1.0), np.float32(0.0123), np.float32(3.7e-5), np.float32(0.57), np.float32(2.0 ** -120),
              np.float32(1.5e3), np.float32(0.0)]
    # code words: code (i + j) % 16 in nibble j for every i (all 16 codes in
    # every position), then random words
    words = [sum(((i + j) % 16) << (4 * j) for j in range(8)) for i in range(16)]
    words += [int(w) for w in rng.integers(0, 2 ** 32, 48, dtype=np.uint64)]
    lines, expect = [], []
    for ct, values in codebook.CODEBOOKS.items():
        for c in scales:
            # the values the table holds: bf16 of the fp32 products (Eq. 6 with
            # the block constant c), as the oracle's dequantiser writes them
            tv = _bf16_bits(blockwise.dequantize(np.arange(16), np.full(1, c, np.float32), codebook=values))
            p = [int(tv[2 * j]) | (int(tv[2 * j + 1]) << 16) for j in range(8)]
            lines.append(" ".join(f"{x:x}" for x in p + [len(words)] + words))
            for w in words:
                codes = [(w >> (4 * j)) & 15 for j in range(8)]
                expect.append([int(tv[codes[2 * k]]) | (int(tv[codes[2 * k + 1]]) << 16) for k in range(4)])
    r = subprocess.run([lut_driver], input="\n".join(lines) + "\n", capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stderr
    got = [[int(x, 16) for x in ln.split()] for ln in r.stdout.strip().splitlines()]
    assert len(got) == len(expect)
    bad = [(i, g, e) for i, (g, e) in enumerate(zip(got, expect)) if g != e]
    assert not bad, f"{len(bad)} lookups differ, first {bad[:3]}"


def _round_f32(q):
    """The fp32 nearest to the rational q, ties to even (|q| in the normal
    range or zero)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * ulp


def test_round_f32_model_matches_numpy():
    """The rational rounding model agrees with numpy's fp64 -> fp32 cast where
    the fp64 value is exact (a pin of the model itself)."""
    rng = np.random.default_rng(3)
    for x in rng.standard_normal(200):
        q = Fraction(float(x))
        assert float(_round_f32(q)) == float(np.float32(x))


def test_int8_expansion_correctly_rounded():
    R = _round_f32(Fraction(1, 127))
    assert float(R) == float(np.float32(1.0 / 127.0))
    for b in range(256):
        k = b - 256 if b >= 128 else b
        q0 = _round_f32(k * R)
        resid = k - 127 * q0
        assert _round_f32(resid) == resid, f"residual of k={k} is not exact in fp32"
        got = _round_f32(resid * R + q0)
        want = _round_f32(Fraction(k, 127))
        assert got == want, f"k={k}: {float(got)!r} != {float(want)!r}"
        assert float(want) == float(codebook.INT8[b])
