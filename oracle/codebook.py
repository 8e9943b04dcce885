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
