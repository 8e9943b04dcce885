"""NF4 codebook (oracle side).  Test infrastructure only.

QLoRA, section 3 "4-bit NormalFloat Quantization" and Appendix E
"NormalFloat 4-bit data type".

Reading G1: Eq. (4) cannot be used as printed (its first value is the mean of
Q(0) = -inf and Q(1/17)), and the page does not state the probabilities of the
two asymmetric halves.  Appendix E prints the exact 16 values; they are
normative here.  `derive_from_quantiles` rebuilds them from N(0,1) quantiles
(7 negative and 8 positive quantiles plus one exact zero, normalised to
[-1, 1]) so that a test can check the printed table against the construction
the section describes.
"""

import numpy as np

# Appendix E, in order from code 0 to code 15.  All sixteen are exactly
# representable in fp32.
APPENDIX_E = (
    -1.0,
    -0.6961928009986877,
    -0.5250730514526367,
    -0.39491748809814453,
    -0.28444138169288635,
    -0.18477343022823334,
    -0.09105003625154495,
    0.0,
    0.07958029955625534,
    0.16093020141124725,
    0.24611230194568634,
    0.33791524171829224,
    0.44070982933044434,
    0.5626170039176941,
    0.7229568362236023,
    1.0,
)

NF4 = np.array(APPENDIX_E, dtype=np.float32)

# Index of the exact zero: the code an all-zero block gets.
ZERO_CODE = 7


def derive_from_quantiles():
    """Rebuild the NF4 values from N(0,1) quantiles (section 3, Eq. 4 and the
    asymmetric construction that follows it).

    The positive half takes 8 quantiles at probabilities evenly spaced from
    p_max down to (excluding) 1/2, the negative half 7 such quantiles, plus a
    single exact zero; everything is divided by the largest value so the range
    is [-1, 1].  The page gives no p_max; the value used,
    1 - (1/32 + 1/30)/2, centres the outermost quantile between the 2^k+1
    and 2^k-1 spacings of Eq. 4 on each side.  Returns fp64.
    """
    from scipy.stats import norm

    p_max = 1.0 - 0.5 * (1.0 / 32.0 + 1.0 / 30.0)
    pos = norm.ppf(np.linspace(p_max, 0.5, 9)[:-1])
    neg = -norm.ppf(np.linspace(p_max, 0.5, 8)[:-1])
    vals = np.sort(np.concatenate([neg, [0.0], pos]))
    return vals / vals.max()


# ------------------------------------------- the other 4-bit storage types
# QLoRA section 3 compares NF4 with Int4 and two 4-bit floats, Float4 (E2M1)
# and Float4 (E3M0) (Table 2, mean perplexity per data type), but prints no
# values for them.  Readings (G14): each type is taken from its bit-field
# definition, its largest magnitude normalised to 1 so that x = w / absmax in
# [-1, 1] is quantised against it exactly as for NF4:
#   FP4 E2M1  code = s e1 e0 m (the OCP microscaling 4-bit float): magnitude
#             m / 2 for e = 0 (subnormal), 2^(e-1) * (1 + m/2) otherwise;
#             the largest, 6, is divided out.
#   FP4 E3M0  code = s e2 e1 e0: magnitude 0 for e = 0, 2^(e-7) otherwise
#             (exponent only; the largest, 2^0, is already 1).
#   INT4      code = two's-complement 4-bit integer k, value k / 7 (Eq. 1's
#             absmax scaling with 2^(4-1) - 1 = 7 levels per side; k = -8 is
#             never produced by quantisation).
# Values are fp32 (m / 6 and k / 7 rounded to nearest).

CODE_NF4, CODE_FP4_E2M1, CODE_FP4_E3M0, CODE_INT4 = 0, 1, 2, 3
CODE_NAMES = {CODE_NF4: "nf4", CODE_FP4_E2M1: "fp4_e2m1", CODE_FP4_E3M0: "fp4_e3m0", CODE_INT4: "int4"}


def _e2m1_magnitude(e, m):
    return m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)


def _fp4_e2m1():
    out = []
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        out.append((-1.0 if s else 1.0) * _e2m1_magnitude(e, m) / _e2m1_magnitude(3, 1))
    return np.array(out, dtype=np.float32)


def _fp4_e3m0():
    out = []
    for c in range(16):
        s, e = c >> 3, c & 7
        mag = 0.0 if e == 0 else 2.0 ** (e - 7)
        out.append((-1.0 if s else 1.0) * mag)
    return np.array(out, dtype=np.float32)


def _int4():
    return np.array([(c - 16 if c >= 8 else c) / 7.0 for c in range(16)], dtype=np.float32)


FP4_E2M1 = _fp4_e2m1()
FP4_E3M0 = _fp4_e3m0()
INT4 = _int4()

CODEBOOKS = {CODE_NF4: NF4, CODE_FP4_E2M1: FP4_E2M1, CODE_FP4_E3M0: FP4_E3M0, CODE_INT4: INT4}


# ---------------------------------------------------- the 8-bit storage type
# Section 2, Eq. 1 quantises to Int8 by absmax scaling into [-127, 127], and
# section 3's Table 3 compares QLoRA with Int8 against NF4.  Read
# blockwise (same 64-blocks and double quantisation as NF4) and exactly like
# Int4 above with 2^7 - 1 = 127 levels per side: code = the two's-complement
# byte of k, value k / 127 rounded to fp32; the byte 0x80 (k = -128) is never
# produced by quantisation.  Not in CODEBOOKS, which holds the 4-bit types.
CODE_INT8 = 4


def _int8():
    return np.array([(c - 256 if c >= 128 else c) / 127.0 for c in range(256)], dtype=np.float32)


INT8 = _int8()


def codebook_of(code_type):
    """Value table of a code type: 16 entries for the 4-bit types, 256 for Int8."""
    return INT8 if code_type == CODE_INT8 else CODEBOOKS[code_type]


def sorted_levels(codebook):
    """The distinct values of a codebook (16 or 256 entries) in increasing
    order, each with the code that stands for it (the smallest such code, so
    +0 rather than -0 for the float types).  Nearest-value search runs over
    this list, ties to the smaller value (G6 read per value: for NF4 the
    smaller value is the lower index)."""
    cb = np.asarray(codebook, dtype=np.float32)
    first = {}
    for i, x in enumerate(cb):
        first.setdefault(float(x), i)
    vals, codes = [], []
    for v in sorted(first):
        vals.append(v)
        codes.append(first[v])
    return np.array(vals, dtype=np.float32), np.array(codes, dtype=np.uint8)


def zero_code(codebook):
    """The code an all-zero block gets: the one standing for 0.0."""
    vals, codes = sorted_levels(codebook)
    return int(codes[list(vals).index(0.0)])
