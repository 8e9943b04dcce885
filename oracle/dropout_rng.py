"""Counter-based draws of the LoRA dropout keep mask (oracle side).  Test
infrastructure only; see the package docstring.

The page "QLoRA: Efficient Finetuning of Quantized LLMs", Appendix B.2,
trains with LoRA dropout 0.1 (models up to 13B) or 0.05 (33B, 65B); reading
G15 takes it as a Bernoulli(1 - p) keep mask on the adapter input.  The page
does not say how the mask is drawn.  Reading G19: it is drawn from
Philox4x64-10, the counter-based generator of Salmon, Moraes, Dror and Shaw
("Parallel random numbers: as easy as 1, 2, 3", SC 2011), so that the
device can draw any part of the mask independently and the oracle can
reproduce it bit for bit:

  * key = (seed, 0), counter = (b, offset, 0, 0) for mask byte b of the
    row-major [M, K/8] packed mask (b = m * K/8 + c);
  * the generator's four 64-bit outputs o_0..o_3 are read as eight 32-bit
    words u_j = (o_{j // 2} >> (32 (j % 2))) mod 2^32;
  * element 8c + j of row m is kept iff u_j >= T with T = floor(p * 2^32),
    so an element is kept with probability 1 - T / 2^32 (within 2^-32 of
    1 - p); bit j of the mask byte is the keep flag of element 8c + j.

Philox4x64-10: ten rounds of
    (lo0, hi0) = M0 * c0,  (lo1, hi1) = M1 * c2       (128-bit products)
    c = (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0)
with the key bumped by (W0, W1) (mod 2^64) before every round but the
first.  M0, M1 are the paper's 4x64 multipliers and W0, W1 its Weyl
increments (the golden ratio and sqrt(3) - 1 scaled to 2^64).
"""

import numpy as np

MASK64 = (1 << 64) - 1
PHILOX_M0 = 0xD2E7470EE14C6C93
PHILOX_M1 = 0xCA5A826395121157
PHILOX_W0 = 0x9E3779B97F4A7C15
PHILOX_W1 = 0xBB67AE8584CAA73B


def philox4x64_10(ctr, key):
    """Philox4x64-10 of one counter (4 ints) and key (2 ints), in plain
    Python integers; returns the 4 output words."""
    c0, c1, c2, c3 = (int(x) & MASK64 for x in ctr)
    k0, k1 = (int(x) & MASK64 for x in key)
    for r in range(10):
        if r:
            k0 = (k0 + PHILOX_W0) & MASK64
            k1 = (k1 + PHILOX_W1) & MASK64
        p0 = PHILOX_M0 * c0
        p1 = PHILOX_M1 * c2
        lo0, hi0 = p0 & MASK64, p0 >> 64
        lo1, hi1 = p1 & MASK64, p1 >> 64
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return c0, c1, c2, c3


def _mulhilo64(a, b):
    """Low and high 64 bits of the 128-bit products of uint64 arrays a and a
    uint64 scalar b, from 32-bit halves."""
    m32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    b = np.uint64(b)
    a0, a1 = a & m32, a >> s32
    b0, b1 = b & m32, b >> s32
    p00, p01, p10, p11 = a0 * b0, a0 * b1, a1 * b0, a1 * b1
    mid = (p00 >> s32) + (p01 & m32) + (p10 & m32)
    hi = p11 + (p01 >> s32) + (p10 >> s32) + (mid >> s32)
    lo = a * b  # wraps mod 2^64
    return lo, hi


def philox4x64_10_array(ctr, key):
    """Philox4x64-10 over arrays: ctr is a (4, n) uint64 array of counters,
    key a pair of ints; returns a (4, n) uint64 array of outputs."""
    c0, c1, c2, c3 = (np.array(ctr[i], dtype=np.uint64) for i in range(4))
    k0, k1 = int(key[0]) & MASK64, int(key[1]) & MASK64
    with np.errstate(over="ignore"):
        for r in range(10):
            if r:
                k0 = (k0 + PHILOX_W0) & MASK64
                k1 = (k1 + PHILOX_W1) & MASK64
            lo0, hi0 = _mulhilo64(c0, PHILOX_M0)
            lo1, hi1 = _mulhilo64(c2, PHILOX_M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ np.uint64(k0), lo1, hi0 ^ c3 ^ np.uint64(k1), lo0
    return np.stack([c0, c1, c2, c3])


def keep_threshold(p):
    """T = floor(p * 2^32) for the fp32 drop probability p in [0, 1)."""
    p = float(np.float32(p))
    if not 0.0 <= p < 1.0:
        raise ValueError("p must be in [0, 1)")
    return int(np.floor(p * 4294967296.0))  # exact: p has 24 significant bits


def keep_mask_packed(seed, offset, M, K, p):
    """The packed keep mask u8 [M, K/8] (K % 8 == 0) of reading G19."""
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    nbytes = M * (K // 8)
    b = np.arange(nbytes, dtype=np.uint64)
    ctr = np.stack([b, np.full(nbytes, int(offset) & MASK64, np.uint64), np.zeros(nbytes, np.uint64),
                    np.zeros(nbytes, np.uint64)])
    out = philox4x64_10_array(ctr, (int(seed) & MASK64, 0))
    words = np.stack([out[j // 2] >> np.uint64(32 * (j % 2)) & np.uint64(0xFFFFFFFF) for j in range(8)])
    keep = words >= np.uint64(keep_threshold(p))                      # [8, nbytes]
    byte = np.zeros(nbytes, np.uint8)
    for j in range(8):
        byte |= keep[j].astype(np.uint8) << np.uint8(j)
    return byte.reshape(M, K // 8)


def keep_mask(seed, offset, M, K, p):
    """The keep mask as bool [M, K]: element 8c + j of row m is bit j of byte
    (m, c)."""
    packed = keep_mask_packed(seed, offset, M, K, p)
    bits = (packed[:, :, None] >> np.arange(8, dtype=np.uint8)[None, None, :]) & 1
    return bits.reshape(M, K).astype(bool)
