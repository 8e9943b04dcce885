"""Pins of the oracle's dropout-mask generator (reading G19: Philox4x64-10
of Salmon et al., SC 2011, drawing the Bernoulli(1 - p) keep mask of QLoRA
Appendix B.2's LoRA dropout) against what does not come from the oracle:

  * numpy's own Philox bit generator (numpy.random.Philox is Philox4x64-10;
    it increments its counter before each draw, so its first four outputs
    for counter c are Philox(c + 1));
  * the vectorised oracle against the plain-integer oracle on random
    counters and keys;
  * the mask layout against a direct per-element evaluation of the
    definition, the threshold against exact arithmetic, and the keep rate
    against its binomial bound.
"""

import numpy as np
import pytest

from oracle import dropout_rng as D

MASK64 = (1 << 64) - 1


@pytest.mark.parametrize("key", [(0, 0), (1, 0), (0xDEADBEEF, 7), (MASK64, MASK64), (2 ** 63 + 12345, 99)])
@pytest.mark.parametrize("counter", [0, 1, 41, 2 ** 64 - 1, (5 << 64) | 3, (1 << 200) + 17])
def test_philox_matches_numpy_bit_generator(key, counter):
    bg = np.random.Philox(counter=counter, key=np.array(key, dtype=np.uint64))
    raw = [int(x) for x in bg.random_raw(8)]
    c = counter + 1
    want0 = D.philox4x64_10([(c >> (64 * i)) & MASK64 for i in range(4)], key)
    c += 1
    want1 = D.philox4x64_10([(c >> (64 * i)) & MASK64 for i in range(4)], key)
    assert raw == list(want0) + list(want1)


def test_array_version_equals_integer_version():
    rng = np.random.default_rng(8)
    ctr = rng.integers(0, 2 ** 63, size=(4, 64), dtype=np.uint64) * np.uint64(2) + rng.integers(0, 2, size=(4, 64),
                                                                                                 dtype=np.uint64)
    for key in [(0, 0), (int(rng.integers(0, 2 ** 63)) * 2 + 1, int(rng.integers(0, 2 ** 63)))]:
        out = D.philox4x64_10_array(ctr, key)
        for i in range(ctr.shape[1]):
            assert [int(v) for v in out[:, i]] == list(D.philox4x64_10([int(v) for v in ctr[:, i]], key))


def test_threshold_exact():
    for p in (0.0, 0.05, 0.1, 0.5, 0.9999999):
        T = D.keep_threshold(p)
        q = float(np.float32(p))
        assert T <= q * 2 ** 32 < T + 1
    with pytest.raises(ValueError):
        D.keep_threshold(1.0)


def test_mask_layout_matches_definition():
    seed, offset, M, K, p = 0x1234ABCD, 5, 3, 40, 0.3
    packed = D.keep_mask_packed(seed, offset, M, K, p)
    T = D.keep_threshold(p)
    for m in range(M):
        for c in range(K // 8):
            b = m * (K // 8) + c
            o = D.philox4x64_10((b, offset, 0, 0), (seed, 0))
            for j in range(8):
                u = (o[j // 2] >> (32 * (j % 2))) & 0xFFFFFFFF
                assert ((int(packed[m, c]) >> j) & 1) == int(u >= T), (m, c, j)
    keep = D.keep_mask(seed, offset, M, K, p)
    assert keep.shape == (M, K)
    assert np.array_equal(np.packbits(keep.reshape(M, K // 8, 8), axis=-1, bitorder="little")[..., 0], packed)


def test_keep_rate_and_streams():
    M, K, p = 256, 4096, 0.1
    keep = D.keep_mask(7, 0, M, K, p)
    n = keep.size
    rate = 1.0 - D.keep_threshold(p) / 2 ** 32
    sigma = np.sqrt(n * rate * (1 - rate))
    assert abs(keep.sum() - n * rate) < 6 * sigma
    assert D.keep_mask(7, 0, 4, 64, 0.0).all()
    # other offsets and seeds draw other masks
    assert not np.array_equal(keep, D.keep_mask(7, 1, M, K, p))
    assert not np.array_equal(keep, D.keep_mask(8, 0, M, K, p))
