"""8-bit float used for the quantised quantisation constants (oracle side).
Test infrastructure only.

QLoRA, section 3 "Double Quantization" and the definition after Eq. (5)/(6):
the first-level constants are quantised to 8-bit floats ("FP8") in blocks of
256.  Reading G3': the page does not name the FP8 variant; the variant used is
OCP E4M3FN (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, no
infinities, a single NaN mantissa pattern, largest finite value 448).  Three
mantissa bits is the most precise 8-bit float, and 448 plays the role 127
plays in Eq. (1).

Encoding is done here by brute force: the nearest of the 127 non-negative
finite magnitudes, ties to the code with an even mantissa (i.e. an even
code), sign copied from the input (so a negative value that rounds to zero
encodes as 0x80).  Inputs are clamped to [-448, 448] first, which is the
saturating behaviour the double quantisation relies on.
"""

import numpy as np


def decode_byte(b):
    """Value of one E4M3FN byte as a Python float (NaN for 0x7F/0xFF)."""
    b = int(b) & 0xFF
    sign = -1.0 if (b & 0x80) else 1.0
    e = (b >> 3) & 0xF
    m = b & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * m * 2.0 ** -9  # subnormal: m/8 * 2^(1-7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


# Decode table over all 256 bytes, fp32 (every finite E4M3 value is exact in fp32).
DECODE = np.array([decode_byte(b) for b in range(256)], dtype=np.float32)

# Non-negative finite magnitudes, indexed by code 0x00..0x7E; strictly increasing.
_MAGS = DECODE[:0x7F].astype(np.float64)

MAX_FINITE = 448.0


def encode(y):
    """Round fp32 values to E4M3FN bytes, nearest-even, saturating at 448.

    y: array-like of fp32.  Returns uint8 array of the same shape.
    """
    y = np.asarray(y, dtype=np.float32)
    flat = y.reshape(-1).astype(np.float64)
    neg = np.signbit(flat)
    mag = np.minimum(np.abs(flat), MAX_FINITE)
    out = np.empty(flat.shape, dtype=np.uint8)
    # Brute force over the 127 magnitudes in chunks to bound memory.
    step = 1 << 16
    for s in range(0, flat.size, step):
        m = mag[s:s + step]
        dist = np.abs(m[:, None] - _MAGS[None, :])  # exact: both sides are fp32 values
        best = dist.min(axis=1, keepdims=True)
        ties = dist == best
        # Among equidistant codes (at most two adjacent ones) take the even code.
        even_tie = ties & ((np.arange(_MAGS.size) % 2) == 0)[None, :]
        has_even = even_tie.any(axis=1)
        code = np.where(has_even, np.argmax(even_tie, axis=1), np.argmax(ties, axis=1))
        out[s:s + step] = code.astype(np.uint8)
    out = np.where(neg, out | 0x80, out).astype(np.uint8)
    return out.reshape(y.shape)


def decode(b):
    """Decode an array of E4M3FN bytes to fp32."""
    return DECODE[np.asarray(b, dtype=np.uint8)]
