"""Blockwise NF4 quantisation, double quantisation and dequantisation (oracle
side).  Test infrastructure only; see the package docstring.

Sources on the page "QLoRA: Efficient Finetuning of Quantized LLMs":
  section 2 "Block-wise k-bit Quantization", Eq. (1) and (2), and the
      paragraph on chunking a flattened tensor into n = (b*h)/B contiguous
      blocks, each with its own constant;
  section 3 "4-bit NormalFloat Quantization", steps (1)-(3);
  section 3 "Double Quantization";
  section 3 "QLoRA", Eq. (5) and (6), and the sentence fixing NF4 for W,
      FP8 for c2, block size 64 for W and 256 for c2.

Readings where the page is silent or garbled (tags match the design notes):
  G2  Eq. (2) as printed multiplies by c = 127/absmax, which does not invert
      Eq. (1); dequantisation here multiplies by the absmax (divides by c).
      Eq. (1)'s "multiply by a precomputed constant" is why quantisation is
      reciprocal-then-multiply: x = fp32(w * fp32(1/absmax)).
  G4  one mean of c2 per tensor, stored as one fp32, equal to the exact mean
      rounded once to nearest-even.  A mean per 256-group would add bits the
      page's 0.127 bits/param figure does not contain.
  G5  an all-zero block has absmax 0 and every code is the exact zero (7).
  G6  nearest-code ties go to the lower index.
  G7  NF4 codes are taken against the exact fp32 absmax, so they do not depend
      on the double quantisation of that absmax.
  G8  packing: byte j holds element 2j in its low nibble and element 2j+1 in
      its high nibble; an odd tail leaves the high nibble 0.
  G9  a tail block (or 256-group) shorter than the block size takes its
      constant over the elements that exist.
  G11 the weight is flattened in its [out, in] row-major order.
  G13 Eq. (1)'s constant must be finite: for a block whose absmax is an fp32
      subnormal (0 < absmax < 2^-126) the reciprocal would overflow, so the
      block and its absmax are first multiplied by 2^32 (exact for such
      values) before the reciprocal and the product are taken.  The
      second-level constant takes the same rule with its own numerator:
      fp32(448 / c1) overflows already for c1 below about 1.3e-36, so a
      256-group whose c1 lies below 2^-118 is scaled by 2^32 first.
      Codes of normal blocks are unaffected, and the rule keeps the codes
      invariant under power-of-two scaling of a block.
"""

from fractions import Fraction

import numpy as np

from .codebook import NF4, ZERO_CODE, CODEBOOKS, CODE_NF4, CODE_INT8, INT8, codebook_of, sorted_levels, zero_code
from . import fp8_e4m3

BLOCKSIZE = 64      # first-level block (elements of W per constant)
BLOCKSIZE2 = 256    # second-level block (first-level constants per FP8 scale)
FP8_MAX = np.float32(448.0)
TINY = np.float32(2.0 ** -126)     # smallest normal fp32
PRESCALE = np.float32(2.0 ** 32)   # G13
TINY_DQ = np.float32(2.0 ** -118)  # G13, second level: 448 * 2^118 < FLT_MAX

_F32 = np.float32


# ---------------------------------------------------------------- helpers

def _num_blocks(n, bs):
    return (n + bs - 1) // bs


def block_absmax(flat, blocksize=BLOCKSIZE):
    """c2: absmax over each contiguous block of the flattened tensor (G9 for a
    short tail).  Exact in fp32."""
    flat = np.asarray(flat, dtype=_F32).reshape(-1)
    n = flat.size
    nb = _num_blocks(n, blocksize)
    padded = np.zeros(nb * blocksize, dtype=_F32)
    padded[:n] = np.abs(flat)
    return padded.reshape(nb, blocksize).max(axis=1)


def nearest_code(x, codebook=NF4):
    """Index of the nearest codebook value for each fp32 x, ties to the lower
    index (G6).  Brute force over the codebook in fp64: the difference of two
    fp32 numbers of similar magnitude is exact in fp64, so ties are seen
    exactly where they can occur."""
    x = np.asarray(x, dtype=_F32).reshape(-1).astype(np.float64)
    q = np.asarray(codebook, dtype=np.float64)
    out = np.empty(x.size, dtype=np.int64)
    step = max(1024, (1 << 22) // q.size)  # rows per slice of the distance matrix
    for s in range(0, x.size, step):
        d = np.abs(x[s:s + step, None] - q[None, :])
        out[s:s + step] = np.argmin(d, axis=1)  # first occurrence = lower index
    return out


def nearest_level(x, codebook):
    """Code of the nearest value of a codebook (16 or 256 entries) for each
    fp32 x, ties to the smaller value (G6, G14).  Brute force over the codebook's sorted
    distinct values in fp64, as nearest_code; for NF4, whose codes are in
    increasing order, the two agree."""
    vals, codes = sorted_levels(codebook)
    return codes[nearest_code(x, vals)]


def bf16_round(x):
    """Round fp32 values to bfloat16 (nearest-even), returned as fp32 values.
    The 16 dropped bits decide the rounding; NaN stays NaN."""
    x = np.ascontiguousarray(x, dtype=_F32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    out = rounded.view(_F32).copy()
    nan = np.isnan(x)
    out[nan] = x[nan]
    return out


def bf16_bits(x):
    """bfloat16 bit patterns (uint16) of fp32 values after nearest-even rounding."""
    return (bf16_round(x).view(np.uint32) >> 16).astype(np.uint16)


# ------------------------------------------------- first level: NF4 codes

def quantize_4bit(w, codebook, blocksize=BLOCKSIZE):
    """quantize_nf4 against any of the 4-bit codebooks of section 3's data
    type comparison (G14), or the 256-entry Int8 table (Eq. 1 read
    blockwise): the same absmax scaling and reciprocal, then the nearest
    codebook value, ties to the smaller value; an all-zero block gets the
    code of 0.0.  For NF4 the result equals quantize_nf4's."""
    flat = np.asarray(w, dtype=_F32).reshape(-1)
    n = flat.size
    c2 = block_absmax(flat, blocksize)
    if not np.all(np.isfinite(c2)):
        raise ValueError("non-finite input: codes are undefined")
    blk = np.arange(n) // blocksize
    tiny = (c2 > 0) & (c2 < TINY)                       # G13
    sc = np.where(tiny, PRESCALE, _F32(1.0)).astype(_F32)
    cs = (c2 * sc).astype(_F32)
    ws = (flat * sc[blk]).astype(_F32)
    inv = np.where(cs > 0, _F32(1.0) / np.where(cs > 0, cs, _F32(1.0)), _F32(0.0)).astype(_F32)
    x = (ws * inv[blk]).astype(_F32)
    codes = nearest_level(x, codebook).astype(np.uint8)
    codes[c2[blk] == 0] = zero_code(codebook)
    return codes, c2


def quantize_nf4(w, blocksize=BLOCKSIZE, codebook=NF4):
    """NF4-quantise a tensor blockwise (section 3 steps (1)-(3), Eq. (1)).

    Returns (codes, c2): codes is uint8 with one code (0..15) per element of
    the flattened tensor; c2 is the fp32 absmax per block.  Per block:
      c2  = max |w|                         (exact)
      inv = fp32(1 / c2)                    (correctly rounded)
      x   = fp32(w * inv)                   (lies in [-1, 1])
      code = nearest codebook index of x    (G6)
    and an all-zero block gets code 7 everywhere (G5).
    """
    flat = np.asarray(w, dtype=_F32).reshape(-1)
    n = flat.size
    c2 = block_absmax(flat, blocksize)
    if not np.all(np.isfinite(c2)):
        raise ValueError("non-finite input: NF4 codes are undefined")
    blk = np.arange(n) // blocksize
    tiny = (c2 > 0) & (c2 < TINY)                       # G13
    sc = np.where(tiny, PRESCALE, _F32(1.0)).astype(_F32)
    cs = (c2 * sc).astype(_F32)
    ws = (flat * sc[blk]).astype(_F32)
    inv = np.where(cs > 0, _F32(1.0) / np.where(cs > 0, cs, _F32(1.0)), _F32(0.0)).astype(_F32)
    x = (ws * inv[blk]).astype(_F32)
    codes = nearest_code(x, codebook).astype(np.uint8)
    codes[c2[blk] == 0] = ZERO_CODE
    return codes, c2


def pack_nibbles(codes):
    """Two codes per byte: element 2j in the low nibble, 2j+1 in the high (G8)."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1)
    if codes.size % 2:
        codes = np.concatenate([codes, np.zeros(1, np.uint8)])
    return (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed, n):
    packed = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed & 0xF
    out[1::2] = packed >> 4
    return out[:n]


# ---------------------------------------- second level: double quantisation

def f32_scaled_int(v):
    """Each non-negative finite fp32 value times 2^149, as exact integers
    (fp32's smallest subnormal is 2^-149, so every fp32 is an integer
    multiple of it).  Returns (mantissa int64 array, shift int64 array) with
    value * 2^149 = mantissa << shift."""
    bits = np.ascontiguousarray(v, dtype=_F32).view(np.uint32).astype(np.int64)
    if np.any(bits >> 31):
        raise ValueError("expects non-negative values")
    e = (bits >> 23) & 0xFF
    if np.any(e == 0xFF):
        raise ValueError("non-finite value")
    m = bits & 0x7FFFFF
    mant = np.where(e > 0, m | 0x800000, m)
    shift = np.where(e > 0, e - 1, 0)
    return mant, shift


def round_rational_to_f32(num, den):
    """Nearest fp32 to the positive rational num/den, ties to even mantissa.
    Exact: candidates are compared as fractions."""
    q = Fraction(int(num), int(den))
    if q == 0:
        return _F32(0.0)
    c = _F32(float(q))  # float() of a Fraction is correctly rounded to fp64
    cands = [np.nextafter(c, _F32(-np.inf)), c, np.nextafter(c, _F32(np.inf))]
    best = None
    for cand in cands:
        if not np.isfinite(cand) or cand < 0:
            continue
        err = abs(Fraction(float(cand)) - q)
        key = (err, int(np.asarray(cand, _F32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return _F32(best[1])


def exact_mean_f32(c2):
    """Mean of the fp32 values c2, computed exactly and rounded once to fp32
    (reading G4: section 3 "Double Quantization" subtracts "the mean" of c2
    before quantising it)."""
    c2 = np.asarray(c2, dtype=_F32).reshape(-1)
    if c2.size == 0:
        raise ValueError("empty")
    mant, shift = f32_scaled_int(c2)
    total = 0
    for s in np.unique(shift):
        total += int(mant[shift == s].sum()) << int(s)
    return round_rational_to_f32(total, c2.size * (1 << 149))


def double_quantize(c2, blocksize2=BLOCKSIZE2):
    """Quantise the first-level constants (section 3 "Double Quantization").

    Returns (absmax_q, scale2, mu):
      mu          = exact mean of c2 rounded to fp32              (G4)
      d_b         = fp32(c2_b - mu)
      c1_g        = max |d_b| over group g of 256 constants        (G9 tail)
      absmax_q_b  = E4M3 byte of clamp(fp32(d_b * fp32(448 / c1_g)), +-448),
                    nearest-even; all bytes 0 and scale 0 when c1_g == 0;
                    when c1_g < 2^-118, d_b and c1_g are first
                    multiplied by 2^32 (G13)
      scale2_g    = fp32(c1_g / 448)   (the page's second-level constant c1,
                    stored in the multiplicative form dequantisation uses)
    """
    c2 = np.asarray(c2, dtype=_F32).reshape(-1)
    nb = c2.size
    mu = exact_mean_f32(c2)
    d = (c2 - mu).astype(_F32)
    ng = _num_blocks(nb, blocksize2)
    grp = np.arange(nb) // blocksize2
    c1 = np.zeros(ng, dtype=_F32)
    np.maximum.at(c1, grp, np.abs(d))
    tiny = (c1 > 0) & (c1 < TINY_DQ)                    # G13
    sc = np.where(tiny, PRESCALE, _F32(1.0)).astype(_F32)
    c1s = (c1 * sc).astype(_F32)
    ds = (d * sc[grp]).astype(_F32)
    f = np.where(c1s > 0, FP8_MAX / np.where(c1s > 0, c1s, _F32(1.0)), _F32(0.0)).astype(_F32)
    y = (ds * f[grp]).astype(_F32)
    y = np.clip(y, -FP8_MAX, FP8_MAX).astype(_F32)
    q = fp8_e4m3.encode(y)
    q[c1[grp] == 0] = 0
    scale2 = (c1 / FP8_MAX).astype(_F32)
    return q, scale2, mu


def dq_reconstruct(absmax_q, scale2, mu, blocksize2=BLOCKSIZE2):
    """Eq. (6) inner dequant: c2_hat_b = fp32(fp32(fp8(q_b) * scale2_g) + mu),
    two separately rounded operations."""
    absmax_q = np.asarray(absmax_q, dtype=np.uint8).reshape(-1)
    grp = np.arange(absmax_q.size) // blocksize2
    prod = (fp8_e4m3.decode(absmax_q) * np.asarray(scale2, _F32)[grp]).astype(_F32)
    return (prod + _F32(mu)).astype(_F32)


# --------------------------------------------------------- dequantisation

def dequantize(codes, c2_hat, blocksize=BLOCKSIZE, codebook=NF4):
    """Eq. (6) outer dequant: w_hat = fp32(NF4[code] * c2_hat_block) (G2).
    codes: one code per element (unpacked).  Returns fp32 flat array."""
    codes = np.asarray(codes, dtype=np.uint8).reshape(-1)
    blk = np.arange(codes.size) // blocksize
    return (np.asarray(codebook, _F32)[codes] * np.asarray(c2_hat, _F32)[blk]).astype(_F32)


# ------------------------------------------------------- whole-tensor API

class QuantState:
    """Everything the oracle's quantiser produces for one tensor."""

    def __init__(self, shape, codes, c2, double_quant, absmax_q=None, scale2=None, mu=None, code_type=CODE_NF4):
        self.shape = tuple(shape)
        self.code_type = code_type  # which codebook the codes index (4-bit types, Int8)
        self.codes = codes          # uint8 per element
        self.c2 = c2                # fp32 per block (exact first-level constant)
        self.double_quant = double_quant
        self.absmax_q = absmax_q    # uint8 per block (double_quant)
        self.scale2 = scale2        # fp32 per 256-group (double_quant)
        self.mu = mu                # fp32 scalar (double_quant)

    @property
    def packed(self):
        """The stored code bytes: two 4-bit codes per byte (G8); Int8 codes
        one per byte."""
        if self.code_type == CODE_INT8:
            return np.asarray(self.codes, dtype=np.uint8).copy()
        return pack_nibbles(self.codes)

    def c2_hat(self):
        if self.double_quant:
            return dq_reconstruct(self.absmax_q, self.scale2, self.mu)
        return self.c2

    def dequantize(self):
        return dequantize(self.codes, self.c2_hat(), codebook=codebook_of(self.code_type)).reshape(self.shape)


def quantize(w, double_quant=True, code_type=CODE_NF4):
    """NF4 (or another 4-bit type of section 3's comparison, G14, or
    blockwise Int8, Eq. 1) + optional double quantisation of a tensor, as
    QLoRA section 3 defines its storage type."""
    w = np.asarray(w, dtype=_F32)
    if code_type == CODE_NF4:
        codes, c2 = quantize_nf4(w)
    else:
        codes, c2 = quantize_4bit(w, codebook_of(code_type))
    if not double_quant:
        return QuantState(w.shape, codes, c2, False, code_type=code_type)
    q, s2, mu = double_quantize(c2)
    return QuantState(w.shape, codes, c2, True, q, s2, mu, code_type=code_type)


def storage_bytes(numel, double_quant=True, code_type=CODE_NF4):
    """Bytes of each stored buffer for a tensor of `numel` elements (Int8
    codes take a byte each, the 4-bit types half a byte)."""
    nb = _num_blocks(numel, BLOCKSIZE)
    out = {"codes": numel if code_type == CODE_INT8 else (numel + 1) // 2}
    if double_quant:
        out["absmax_q"] = nb
        out["scale2"] = 4 * _num_blocks(nb, BLOCKSIZE2)
        out["offset"] = 4
    else:
        out["absmax"] = 4 * nb
    return out


def bits_per_param(numel, double_quant=True):
    """Storage bits per weight from the buffer sizes (section 3 "Double
    Quantization" accounts 32/64 = 0.5 bits of constants without it and
    8/64 + 32/(64*256) with it)."""
    return 8.0 * sum(storage_bytes(numel, double_quant).values()) / numel
