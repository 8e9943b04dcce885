"""Pins for the CPU oracle against what the page and the mathematics fix.

Each test checks the oracle against something other than itself: values the
page prints (golden fixtures), closed forms, exact rational arithmetic, brute
force on tiny inputs, special cases that reduce to a textbook formula, and an
independent library (torch's float8 and bfloat16 casts, torch.autograd).
"""

import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import blockwise, codebook, fp8_e4m3, linear

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _read_golden(name):
    vals = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                vals.append(line)
    return vals


# ------------------------------------------------------------------ codebook

def test_codebook_equals_appendix_e_bit_exact():
    printed = np.array([float(v) for v in _read_golden("nf4_appendix_e.txt")], dtype=np.float64)
    assert printed.size == 16
    # every printed value is exactly an fp32 value
    assert np.all(printed.astype(F32).astype(np.float64) == printed)
    assert np.array_equal(codebook.NF4.view(np.uint32), printed.astype(F32).view(np.uint32))


def test_codebook_invariants():
    q = codebook.NF4.astype(np.float64)
    assert np.all(np.diff(q) > 0)
    assert q[0] == -1.0 and q[15] == 1.0
    assert q[codebook.ZERO_CODE] == 0.0 and not np.signbit(codebook.NF4[7])
    # 2^(k-1) = 8 non-positive-side quantiles incl. the shared zero, 2^(k-1)+1 = 9 on the
    # positive side; one duplicate zero removed -> 7 negative, 1 zero, 8 positive values
    assert (q < 0).sum() == 7 and (q > 0).sum() == 8


def test_codebook_matches_normal_quantile_construction():
    derived = codebook.derive_from_quantiles()
    q = codebook.NF4.astype(np.float64)
    assert np.max(np.abs(derived - q)) <= 2.5e-7
    assert derived[0] == -1.0 and derived[15] == 1.0 and derived[7] == 0.0


# -------------------------------------------------------------- nearest code

def _exact_midpoints():
    q = [Fraction(float(v)) for v in codebook.NF4]
    return [(q[i] + q[i + 1]) / 2 for i in range(15)]


def test_nearest_code_equals_exact_threshold_count():
    """code = #{i : x > m_i} with exact rational midpoints; a tie (x == m_i)
    is not counted, i.e. goes to the lower index."""
    mids = _exact_midpoints()
    rng = np.random.default_rng(1)
    xs = list(rng.uniform(-1, 1, 3000).astype(F32))
    # every fp32 at and next to each midpoint
    for m in mids:
        c = F32(float(m))
        for v in (np.nextafter(c, F32(-2)), c, np.nextafter(c, F32(2))):
            xs.append(F32(v))
    xs += [F32(-1), F32(1), F32(0), F32(-0.0), F32(1e-30), F32(-1e-30)]
    xs = np.array(xs, dtype=F32)
    got = blockwise.nearest_code(xs)
    for x, g in zip(xs, got):
        fx = Fraction(float(x))
        assert g == sum(1 for m in mids if fx > m), float(x)


def test_exact_midpoint_ties_go_to_lower_code():
    mids = _exact_midpoints()
    exact = [i for i, m in enumerate(mids) if Fraction(float(F32(float(m)))) == m]
    assert exact == [2, 6, 7, 9, 11, 13]
    xs = np.array([float(mids[i]) for i in exact], dtype=F32)
    assert list(blockwise.nearest_code(xs)) == exact


def test_nearest_code_minimises_reconstruction_error_bruteforce():
    """Per element, the chosen code minimises |w - NF4[c] * absmax| in exact
    arithmetic over all 16 codes, except inside a 1e-6 band around a decision
    boundary where the fp32 rounding of w/absmax may decide."""
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((4, 128)) * 0.02).astype(F32)
    codes, c2 = blockwise.quantize_nf4(w)
    q = [Fraction(float(v)) for v in codebook.NF4]
    flat = w.reshape(-1)
    ambiguous = 0
    for i, (x, c) in enumerate(zip(flat, codes)):
        a = Fraction(float(c2[i // 64]))
        errs = [abs(Fraction(float(x)) - qq * a) for qq in q]
        best = min(errs)
        if errs[c] != best:
            ambiguous += 1
            assert (errs[c] - best) <= Fraction(1, 10 ** 6) * a
    assert ambiguous <= 2


def test_eq1_int8_special_case():
    """With the uniform table {k/127}, the blockwise absmax quantiser is Eq. (1):
    round(127 / absmax(X) * X) per block."""
    table = (np.arange(-127, 128) / 127.0).astype(F32)
    rng = np.random.default_rng(3)
    w = (rng.standard_normal(64 * 50) * 3.0).astype(F32)
    codes, c2 = blockwise.quantize_nf4(w, codebook=table)
    got = codes.astype(np.int64) - 127
    blk = np.arange(w.size) // 64
    t = 127.0 * w.astype(np.float64) / c2[blk].astype(np.float64)
    ref = np.rint(t).astype(np.int64)
    near_half = np.abs(np.abs(t - np.floor(t)) - 0.5) < 1e-5
    assert np.array_equal(got[~near_half], ref[~near_half])
    assert near_half.sum() <= 3
    # the block's absmax element maps to +-127 exactly
    for b in range(50):
        j = np.argmax(np.abs(w[b * 64:(b + 1) * 64]))
        assert abs(got[b * 64 + j]) == 127


# -------------------------------------------------------- round trips, zeros

def test_codebook_block_round_trip_exact():
    vals = np.tile(codebook.NF4, 4)                       # 64 values, absmax 1
    for scale in (1.0, 2.0 ** -7, 2.0 ** 5):
        w = (vals * F32(scale)).astype(F32)
        codes, c2 = blockwise.quantize_nf4(w)
        assert list(codes) == list(range(16)) * 4
        assert c2[0] == F32(scale)
        st = blockwise.quantize(w, double_quant=False)
        assert np.array_equal(st.dequantize(), w)


def test_double_quant_round_trip_exact_when_absmax_shared():
    """All blocks share one absmax: c2 - mu = 0, so c1 = 0 and c2_hat = mu = c2."""
    block = np.tile(codebook.NF4, 4).astype(F32)
    w = np.concatenate([block * F32(0.125)] * 300).astype(F32)   # 300 blocks, 2 groups
    rng = np.random.default_rng(4)
    for b in range(300):   # permute within blocks: codes differ, absmax does not
        w[b * 64:(b + 1) * 64] = rng.permutation(w[b * 64:(b + 1) * 64])
    st = blockwise.quantize(w, double_quant=True)
    assert st.mu == F32(0.125)
    assert np.all(st.scale2 == 0) and np.all(st.absmax_q == 0)
    assert np.array_equal(st.dequantize(), w)


def test_codes_invariant_under_power_of_two_block_scaling():
    """Codes depend only on w / absmax, so scaling a block by 2^e keeps them,
    down to blocks of fp32 subnormals (reading G13 keeps the reciprocal finite)."""
    rng = np.random.default_rng(9)
    w = (rng.standard_normal(64 * 8)).astype(F32)
    ref, _ = blockwise.quantize_nf4(w)
    for e in (-20, -100, -126, -130, -140, 60):
        ws = (w.astype(np.float64) * 2.0 ** e)
        if e <= -126:
            # keep only values whose scaled copy is exact in fp32 (subnormals drop low bits)
            w2 = (np.round(w * 2.0 ** 6) / 2.0 ** 6).astype(F32)
            ref2, _ = blockwise.quantize_nf4(w2)
            ws = (w2.astype(np.float64) * 2.0 ** e)
            assert np.all(ws.astype(F32).astype(np.float64) == ws)
            codes, c2 = blockwise.quantize_nf4(ws.astype(F32))
            assert np.array_equal(codes, ref2), e
        else:
            codes, c2 = blockwise.quantize_nf4(ws.astype(F32))
            assert np.array_equal(codes, ref), e
    # double quantisation of tiny, nearly equal constants stays finite and ordered
    c2 = (np.float32(2.0 ** -140) * np.arange(1, 300)).astype(F32)
    q, s2, mu = blockwise.double_quantize(c2)
    rec = blockwise.dq_reconstruct(q, s2, mu)
    assert np.all(np.isfinite(rec)) and np.all(np.diff(rec[:256]) >= 0)


def test_all_zero_block():
    w = np.zeros(128, F32)
    w[64:] = np.linspace(-1, 1, 64, dtype=F32)
    codes, c2 = blockwise.quantize_nf4(w)
    assert c2[0] == 0 and np.all(codes[:64] == codebook.ZERO_CODE)
    st = blockwise.quantize(w, double_quant=False)
    assert np.all(st.dequantize()[:64] == 0)


def test_tail_block_and_packing():
    w = np.array([0.5, -1.0, 0.25], dtype=F32)       # one short block, odd length
    codes, c2 = blockwise.quantize_nf4(w)
    assert c2.size == 1 and c2[0] == 1.0
    assert codes[1] == 0
    packed = blockwise.pack_nibbles(codes)
    assert packed.size == 2 and (packed[1] >> 4) == 0
    assert packed[0] == (codes[0] | (codes[1] << 4))
    assert np.array_equal(blockwise.unpack_nibbles(packed, 3), codes)
    assert list(blockwise.pack_nibbles(np.array([1, 2, 3, 4], np.uint8))) == [0x21, 0x43]


# ------------------------------------------------------------------ E4M3

def test_e4m3_decode_matches_torch():
    b = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    ours = fp8_e4m3.DECODE
    nan = np.isnan(b)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(b[~nan].view(np.uint32), ours[~nan].view(np.uint32))
    assert fp8_e4m3.DECODE[0x7E] == 448.0 and fp8_e4m3.DECODE[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(5)
    y = np.concatenate([
        rng.uniform(-448, 448, 20000),
        rng.standard_normal(20000) * 0.01,
        rng.standard_normal(20000) * 2.0 ** -8,
        (fp8_e4m3.DECODE[:0x7E].astype(np.float64)[:-1] + fp8_e4m3.DECODE[1:0x7F].astype(np.float64)[:-1]) / 2,
    ]).astype(F32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp8_e4m3.encode(y), ref)


def test_e4m3_encode_ties_saturation_and_identity():
    enc = lambda v: int(fp8_e4m3.encode(np.array([v], F32))[0])  # noqa: E731
    assert fp8_e4m3.DECODE[enc(1.0625)] == 1.0
    assert fp8_e4m3.DECODE[enc(1.1875)] == 1.25
    assert fp8_e4m3.DECODE[enc(3 * 2.0 ** -10)] == 2.0 ** -8
    assert enc(2.0 ** -10) == 0x00 and enc(-(2.0 ** -10)) == 0x80
    assert enc(448.0) == 0x7E and enc(1e9) == 0x7E and enc(-1e9) == 0xFE
    assert enc(-0.0) == 0x80
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(fp8_e4m3.encode(fp8_e4m3.decode(codes)), codes)


# ------------------------------------------------------------- exact mean

def test_exact_mean_against_fractions():
    rng = np.random.default_rng(6)
    cases = [
        rng.uniform(0, 0.1, 1000).astype(F32),
        np.concatenate([rng.uniform(0, 1, 50) * 1e30, rng.uniform(0, 1, 50) * 1e-30]).astype(F32),
        np.array([1e-45, 3e-45, 1e-44], F32),                     # subnormals
        np.array([3.4e38, 3.4e38], F32),
        (2.0 ** rng.integers(-140, 120, 500) * rng.uniform(1, 2, 500)).astype(F32),
    ]
    for c in cases:
        exact = sum(Fraction(float(v)) for v in c) / len(c)
        mu = blockwise.exact_mean_f32(c)
        lo, hi = np.nextafter(mu, F32(-np.inf)), np.nextafter(mu, F32(np.inf))
        e0 = abs(Fraction(float(mu)) - exact)
        assert e0 <= abs(Fraction(float(lo)) - exact)
        assert e0 <= abs(Fraction(float(hi)) - exact)


def test_exact_mean_closed_forms():
    assert blockwise.exact_mean_f32(np.full(777, 0.3, F32)) == F32(0.3)
    assert blockwise.exact_mean_f32(np.array([1.0, 2.0], F32)) == F32(1.5)
    # mean exactly halfway between two fp32 values -> even mantissa
    a = F32(1.0)
    b = np.nextafter(a, F32(2))                # 1 + 2^-23, odd mantissa
    assert blockwise.exact_mean_f32(np.array([a, b], F32)) == a
    c = np.nextafter(b, F32(2))                # 1 + 2^-22
    assert blockwise.exact_mean_f32(np.array([b, c], F32)) == c


# ----------------------------------------------- double quantisation, sizes

def test_bits_per_param_closed_form_against_page():
    g = dict(line.split() for line in _read_golden("dq_bits_per_param.txt"))
    numel = 4096 * 4096
    no_dq = blockwise.bits_per_param(numel, False)
    dq = blockwise.bits_per_param(numel, True)
    assert no_dq == 4.5 and no_dq - 4 == float(g["no_dq_constant_bits"])
    assert dq - 4 == 8 / 64 + 32 / (64 * 256) + 32 / numel
    assert round(dq - 4, 3) == float(g["dq_constant_bits"])
    saving = no_dq - dq
    assert round(saving, 3) == float(g["saving_bits"])
    assert round(65e9 * saving / 8 / 1e9) == int(g["saving_65b_gigabytes"])


def test_double_quant_error_bound_and_monotonicity():
    rng = np.random.default_rng(7)
    w = (rng.standard_t(5, 64 * 700) * 0.0155).astype(F32)
    st = blockwise.quantize(w, double_quant=True)
    c2, c2h = st.c2.astype(np.float64), st.c2_hat().astype(np.float64)
    grp = np.arange(c2.size) // 256
    c1 = st.scale2.astype(np.float64) * 448.0
    # E4M3 keeps 3 mantissa bits: relative half-ulp 2^-4 of |c2 - mu|, plus
    # the fp32 roundings of the scale and of the final sum.
    d = np.abs(c2 - float(st.mu))
    bound = d * 2.0 ** -4 + c1[grp] * 2.0 ** -9 * 2 ** -4 + 4 * np.spacing(c2.astype(F32)).astype(np.float64)
    assert np.all(np.abs(c2h - c2) <= bound)
    mu_f = float(np.mean(c2))
    assert abs(float(st.mu) - mu_f) <= 1e-6 * mu_f
    for g in range(grp.max() + 1):
        sel = grp == g
        order = np.argsort(c2[sel], kind="stable")
        assert np.all(np.diff(c2h[sel][order]) >= 0)


def test_double_quant_power_of_two_invariance():
    # Scaling every first-level constant by 2^-k scales the mean, the
    # differences and c1 exactly (the values stay normal fp32 and their
    # differences are exact), so the FP8 bytes must not change: this holds
    # through the range where 448 / c1 alone would overflow fp32 (G13).
    rng = np.random.default_rng(17)
    base = rng.uniform(0.5, 1.0, 700).astype(F32)
    q0, s0, mu0 = blockwise.double_quantize(base)
    for k in (40, 100, 117, 119, 121, 123, 125):
        sc = F32(2.0 ** -k)
        with np.errstate(over="raise", divide="raise", invalid="raise", under="ignore"):
            q, s, mu = blockwise.double_quantize((base * sc).astype(F32))
        assert np.array_equal(q, q0), k
        assert float(mu) == float(mu0) * 2.0 ** -k
        assert np.all(np.isfinite(s)) and np.all(s > 0)


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal(10000), rng.standard_normal(1000) * 1e-39,
                        [0.0, -0.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8]]).astype(F32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(blockwise.bf16_round(x).view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------- linear layer

def _tiny_linear(seed, M=3, K=8, N=5, r=2):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((M, K)), rng.standard_normal((N, K)),
            rng.standard_normal((K, r)), rng.standard_normal((r, N)), rng.standard_normal((M, N)))


def test_forward_brute_force_loops():
    X, W, A, B, _ = _tiny_linear(10)
    s = 0.75
    Y, XA = linear.forward(X, W, A, B, s)
    M, K = X.shape
    N, r = W.shape[0], A.shape[1]
    for m, n in itertools.product(range(M), range(N)):
        base = sum(X[m, k] * W[n, k] for k in range(K))
        lora = sum(sum(X[m, k] * A[k, j] for k in range(K)) * B[j, n] for j in range(r))
        assert math.isclose(Y[m, n], base + s * lora, rel_tol=1e-12, abs_tol=1e-12)


def test_forward_special_cases_and_torch_linear():
    X, W, A, B, _ = _tiny_linear(11)
    s = 2.0
    Y, _ = linear.forward(X, W, A, B, s)
    Yt = torch.nn.functional.linear(torch.from_numpy(X), torch.from_numpy(W)) + \
        s * (torch.from_numpy(X) @ torch.from_numpy(A)) @ torch.from_numpy(B)
    assert np.allclose(Y, Yt.numpy(), rtol=1e-12, atol=1e-12)
    Y0, _ = linear.forward(X, W, A, np.zeros_like(B), s)          # B = 0: base linear
    assert np.allclose(Y0, X @ W.T, rtol=1e-13, atol=1e-13)
    Yw, _ = linear.forward(X, np.zeros_like(W), A, B, s)          # W = 0: pure adapter
    assert np.allclose(Yw, s * X @ A @ B, rtol=1e-13, atol=1e-13)
    Ys, _ = linear.forward(X, W, A, B, 0.0)                       # s = 0
    assert np.allclose(Ys, X @ W.T, rtol=1e-13, atol=1e-13)


def test_backward_finite_differences():
    X, W, A, B, dY = _tiny_linear(12)
    s = 0.5
    dX, dA, dB = linear.backward(dY, X, W, A, B, s)

    def loss(X_, A_, B_):
        return float(np.sum(dY * linear.forward(X_, W, A_, B_, s)[0]))

    h = 1e-6
    for name, arr, grad in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            p, m = arr.copy(), arr.copy()
            p[idx] += h
            m[idx] -= h
            args = {"X": X, "A": A, "B": B}
            args[name] = p
            lp = loss(args["X"], args["A"], args["B"])
            args[name] = m
            lm = loss(args["X"], args["A"], args["B"])
            num[idx] = (lp - lm) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-7), name


def test_backward_matches_torch_autograd_fp64():
    X, W, A, B, dY = _tiny_linear(13, M=4, K=16, N=8, r=3)
    s = 0.25
    tX, tA, tB = (torch.tensor(v, requires_grad=True) for v in (X, A, B))
    Y = tX @ torch.from_numpy(W).T + s * (tX @ tA) @ tB
    Y.backward(torch.from_numpy(dY))
    dX, dA, dB = linear.backward(dY, X, W, A, B, s)
    assert np.allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dA, tA.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dB, tB.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_flops_formula():
    assert linear.flops(4096, 4096, 4096, 64) == 4 * 4096 ** 3 + 6 * 4096 * 64 * 8192


# ------------------------------------------- pins catch planted oracle mistakes

def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle and check that a pin fails."""
    X, W, A, B, dY = _tiny_linear(14)
    s = 0.5
    good = linear.backward(dY, X, W, A, B, s)

    def bad_backward(dY_, X_, W_, A_, B_, s_):
        dX, dA, dB = good
        return dX, dA, dB / s_          # dropped scale on dB
    h = 1e-6
    num = np.zeros_like(B)
    for idx in np.ndindex(B.shape):
        p, m = B.copy(), B.copy()
        p[idx] += h
        m[idx] -= h
        num[idx] = (np.sum(dY * linear.forward(X, W, A, p, s)[0]) -
                    np.sum(dY * linear.forward(X, W, A, m, s)[0])) / (2 * h)
    assert not np.allclose(bad_backward(dY, X, W, A, B, s)[2], num, rtol=1e-6, atol=1e-7)
    # a tie rule to the upper index breaks the exact-midpoint pin
    mids = _exact_midpoints()
    x = F32(float(mids[7]))
    upper = int(np.argmin(np.abs(x - codebook.NF4[::-1].astype(np.float64))))
    assert 15 - upper != 7


# ------------------------------------------- other 4-bit storage types (G14)

def _golden_fp4(fmt):
    for line in _read_golden("fp4_formats.txt"):
        parts = line.split()
        if parts[0] == fmt:
            return np.array([float(v) for v in parts[1:]], dtype=np.float64)
    raise KeyError(fmt)


def test_fp4_codebooks_equal_format_tables():
    """Codes 0..7 are the format's magnitudes (largest normalised to 1), codes
    8..15 their negatives; every value is the fp32 rounding of that ratio."""
    for fmt, cb in (("e2m1", codebook.FP4_E2M1), ("e3m0", codebook.FP4_E3M0)):
        mags = _golden_fp4(fmt)
        want = np.concatenate([mags, -mags]) / mags.max()
        assert np.array_equal(cb, want.astype(F32)), fmt
        assert cb[7] == 1.0 and cb[15] == -1.0


def test_int4_codebook_is_twos_complement_over_7():
    for c in range(16):
        k = c - 16 if c & 8 else c
        assert float(codebook.INT4[c]) == float(F32(k / 7.0))
        assert round(float(codebook.INT4[c]) * 7) == k


def _nearest_bruteforce(x, cb):
    """Smallest-value code among those at minimal |x - v| (exact in fp64)."""
    d = [abs(float(x) - float(v)) for v in cb]
    best = min(d)
    cands = [c for c in range(len(cb)) if d[c] == best]
    vmin = min(float(cb[c]) for c in cands)
    return min(c for c in cands if float(cb[c]) == vmin)


def test_nearest_level_bruteforce_all_types():
    rng = np.random.default_rng(21)
    for ct, cb in list(codebook.CODEBOOKS.items()) + [(codebook.CODE_INT8, codebook.INT8)]:
        vals, _ = codebook.sorted_levels(cb)
        mids = [(float(a) + float(b)) / 2 for a, b in zip(vals[:-1], vals[1:])]
        xs = list(rng.uniform(-1, 1, 300).astype(F32))
        for m in mids:  # at, just below and just above every decision point
            f = F32(m)
            xs += [f, np.nextafter(f, F32(-2)), np.nextafter(f, F32(2))]
        xs += [F32(0.0), F32(-0.0), F32(1.0), F32(-1.0)]
        xs = np.array(xs, dtype=F32)
        got = blockwise.nearest_level(xs, cb)
        want = np.array([_nearest_bruteforce(x, cb) for x in xs])
        assert np.array_equal(got, want), ct
    # NF4 codes are in increasing order: the per-value rule is the per-index one
    x = rng.uniform(-1, 1, 2000).astype(F32)
    assert np.array_equal(blockwise.nearest_level(x, codebook.NF4), blockwise.nearest_code(x))


def test_int4_is_eq1_rounding_to_seven_levels():
    """For Int4 the nearest level is Eq. 1's absmax rounding with 2^3 - 1 = 7
    levels per side (ties to the smaller value): k = ceil(7x - 1/2)."""
    rng = np.random.default_rng(22)
    x = np.concatenate([rng.uniform(-1, 1, 5000), (np.arange(-7, 7) + 0.5) / 7.0]).astype(F32)
    k = np.ceil(7.0 * x.astype(np.float64) - 0.5)
    # the fp32 levels are k/7 rounded, which moves each decision point by
    # under 1e-7: compare away from the points (the brute-force pin covers
    # them)
    t = 7.0 * x.astype(np.float64)
    clear = np.abs(np.abs(t - np.floor(t)) - 0.5) > 1e-5
    codes = blockwise.nearest_level(x, codebook.INT4)
    got_k = np.array([int(c) - 16 if c & 8 else int(c) for c in codes])
    assert np.array_equal(got_k[clear], k[clear].astype(int))


# ------------------------------------------- blockwise Int8 (section 2, Eq. 1)

def _nearest_f32(q):
    """The fp32 value nearest to the rational q (ties to the even pattern),
    by exact comparison of the candidates."""
    c = F32(float(q))
    cands = [np.nextafter(c, F32(-np.inf)), c, np.nextafter(c, F32(np.inf))]
    return min(cands, key=lambda v: (abs(Fraction(float(v)) - q), int(np.asarray(v, F32).view(np.uint32)) & 1))


def _int8_k(codes):
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c >= 128, c - 256, c)


def test_int8_table_is_k_over_127():
    """Byte c stands for k / 127 rounded to fp32, k its two's-complement value."""
    assert codebook.INT8.shape == (256,) and codebook.INT8.dtype == np.float32
    for c in range(256):
        k = c - 256 if c & 0x80 else c
        assert float(codebook.INT8[c]) == float(_nearest_f32(Fraction(k, 127))), c
    assert codebook.INT8[0] == 0.0 and codebook.INT8[127] == 1.0 and codebook.INT8[0x81] == -1.0
    assert codebook.zero_code(codebook.INT8) == 0


def test_int8_is_eq1_rounding_per_block():
    """Blockwise Int8 is Eq. 1 on every 64-block: k = round(127 w / absmax),
    ties to the smaller value, stored as its two's-complement byte (one per
    weight); an all-zero block is all zeros and each block's absmax element
    maps to +-127."""
    rng = np.random.default_rng(41)
    w = (rng.standard_normal(64 * 300) * 0.02).astype(F32)
    w[64 * 7:64 * 8] = 0.0
    q = blockwise.quantize(w, double_quant=False, code_type=codebook.CODE_INT8)
    got = _int8_k(q.codes)
    blk = np.arange(w.size) // 64
    c2 = np.abs(w).reshape(-1, 64).max(axis=1)
    assert np.array_equal(q.c2, c2)
    t = 127.0 * w.astype(np.float64) / np.where(c2 > 0, c2, 1.0)[blk]
    k = np.ceil(t - 0.5)
    # x = w * fp32(1/absmax) is rounded to fp32 first, which moves t by under
    # 2e-5: compare away from the decision points (the brute-force pin covers them)
    clear = np.abs(np.abs(t - np.floor(t)) - 0.5) > 5e-5
    assert clear.sum() > w.size - 10
    assert np.array_equal(got[clear], k[clear].astype(np.int64))
    assert np.all(got[64 * 7:64 * 8] == 0)
    for b in range(300):
        if b != 7:
            assert abs(got[b * 64 + int(np.argmax(np.abs(w[b * 64:(b + 1) * 64])))]) == 127
    assert q.packed.dtype == np.uint8 and np.array_equal(q.packed, q.codes.astype(np.uint8))
    assert blockwise.storage_bytes(w.size, False, codebook.CODE_INT8)["codes"] == w.size


def test_int8_round_trip_and_error_bound():
    """Every level k / 127 survives quantise -> dequantise exactly when the
    block's absmax is 1, and on normal weights the error is at most half a
    step (absmax / 254) plus the fp32 roundings."""
    vals = codebook.INT8[[c for c in range(256) if c != 0x80]]
    blocks = []
    for i in range(0, vals.size, 63):
        b = np.zeros(64, dtype=F32)
        part = vals[i:i + 63]
        b[:part.size] = part
        b[63] = F32(1.0)
        blocks.append(b)
    w = np.concatenate(blocks)
    q = blockwise.quantize(w, double_quant=False, code_type=codebook.CODE_INT8)
    assert np.array_equal(q.dequantize(), w)
    w = (np.random.default_rng(42).standard_normal(64 * 500) * 0.02).astype(F32)
    q = blockwise.quantize(w, double_quant=False, code_type=codebook.CODE_INT8)
    c2 = q.c2[np.arange(w.size) // 64].astype(np.float64)
    err = np.abs(q.dequantize().astype(np.float64) - w)
    assert np.all(err <= c2 * (0.5 / 127 + 4e-7))
    # Int8 reconstructs normal weights far better than any 4-bit type
    e8 = np.sqrt(np.mean(err ** 2))
    e4 = np.sqrt(np.mean((blockwise.quantize(w, False, codebook.CODE_NF4).dequantize() - w).astype(np.float64) ** 2))
    assert e8 < e4 / 8


def test_pins_catch_planted_int8_ties_to_even():
    """Rounding 127 x half-to-even (np.rint) instead of to the smaller value
    disagrees with the brute-force pin at an exact decision point."""
    vals, codes = codebook.sorted_levels(codebook.INT8)
    hits = 0
    for i in range(1, vals.size - 1):
        m = (float(vals[i]) + float(vals[i + 1])) / 2
        if float(F32(m)) != m:
            continue
        x = F32(m)
        right = _nearest_bruteforce(x, codebook.INT8)
        assert int(blockwise.nearest_level(np.array([x]), codebook.INT8)[0]) == right
        planted = int(np.rint(127.0 * float(x))) & 0xFF
        hits += planted != right
    assert hits > 0


def test_other_types_round_trip_and_zero_block():
    for ct, cb in codebook.CODEBOOKS.items():
        vals, codes = codebook.sorted_levels(cb)
        inside = np.abs(vals) <= 1.0
        block = np.zeros(64, dtype=F32)
        block[:inside.sum()] = vals[inside]
        block[-1] = F32(1.0)  # absmax 1: x = w exactly
        got, c2 = blockwise.quantize_4bit(block, cb)
        assert c2[0] == 1.0
        assert np.array_equal(cb[got], block), ct
        z, _ = blockwise.quantize_4bit(np.zeros(64, F32), cb)
        assert np.all(cb[z] == 0.0) and np.all(z == codebook.zero_code(cb))
    # NF4 through the generic path equals the NF4 quantiser
    w = (np.random.default_rng(23).standard_normal(64 * 50) * 0.02).astype(F32)
    assert np.array_equal(blockwise.quantize_4bit(w, codebook.NF4)[0], blockwise.quantize_nf4(w)[0])


def test_nf4_has_the_lowest_error_on_normal_weights():
    """Section 3 motivates NF4 as the information-theoretically optimal 4-bit
    type for normally distributed weights: on N(0, 0.02^2) blocks its
    reconstruction error is the smallest of the four types."""
    w = (np.random.default_rng(24).standard_normal(64 * 4000) * 0.02).astype(F32)
    err = {}
    for ct in codebook.CODEBOOKS:
        q = blockwise.quantize(w, double_quant=False, code_type=ct)
        err[ct] = float(np.sqrt(np.mean((q.dequantize().astype(np.float64) - w) ** 2)))
    assert min(err, key=err.get) == codebook.CODE_NF4
    assert all(err[ct] > 1.1 * err[codebook.CODE_NF4] for ct in err if ct != codebook.CODE_NF4)


def test_pins_catch_planted_code_order_tie_rule():
    """Searching the FP4 codebook in code order (ties to the lower code, not
    the smaller value) is caught by the brute-force pin at a midpoint."""
    cb = codebook.FP4_E2M1
    x = F32((float(cb[9]) + 0.0) / 2)  # between -1/12 (code 9) and 0 (codes 0, 8)
    wrong = int(np.argmin(np.abs(float(x) - cb.astype(np.float64))))
    assert wrong != _nearest_bruteforce(x, cb)
    assert int(blockwise.nearest_level(np.array([x]), cb)[0]) == _nearest_bruteforce(x, cb)


# --------------------------------------------------- LoRA dropout (G15)

def _keep_mask(seed, shape, p):
    return np.random.default_rng(seed).random(shape) >= p


def test_dropout_reduces_to_plain_layer():
    """An all-ones mask with p = 0 is the plain layer (forward and backward)."""
    X, W, A, B, dY = _tiny_linear(30)
    keep = np.ones(X.shape, dtype=bool)
    for a, b in zip(linear.forward_dropout(X, W, A, B, 0.5, keep, 0.0), linear.forward(X, W, A, B, 0.5)):
        assert np.array_equal(a, b)
    for a, b in zip(linear.backward_dropout(dY, X, W, A, B, 0.5, keep, 0.0), linear.backward(dY, X, W, A, B, 0.5)):
        assert np.allclose(a, b, rtol=1e-15, atol=0)


def test_dropout_forward_brute_force_loops():
    X, W, A, B, _ = _tiny_linear(31)
    s, p = 0.75, 0.25
    keep = _keep_mask(1, X.shape, p)
    Y, XA = linear.forward_dropout(X, W, A, B, s, keep, p)
    M, K = X.shape
    N, r = W.shape[0], A.shape[1]
    for m, n in itertools.product(range(M), range(N)):
        base = sum(X[m, k] * W[n, k] for k in range(K))
        xa = [sum(X[m, k] * (1.0 if keep[m, k] else 0.0) / (1 - p) * A[k, j] for k in range(K)) for j in range(r)]
        assert math.isclose(Y[m, n], base + s * sum(xa[j] * B[j, n] for j in range(r)), rel_tol=1e-12, abs_tol=1e-12)
        for j in range(r):
            assert math.isclose(XA[m, j], xa[j], rel_tol=1e-12, abs_tol=1e-12)


def test_dropout_backward_finite_differences():
    """With the mask fixed the layer is linear in X, A and B: central
    differences of L = sum(dY * Y) match the analytic gradients."""
    X, W, A, B, dY = _tiny_linear(32)
    s, p = 0.5, 0.1
    keep = _keep_mask(2, X.shape, p)
    dX, dA, dB = linear.backward_dropout(dY, X, W, A, B, s, keep, p)

    def loss(X_, A_, B_):
        return float(np.sum(dY * linear.forward_dropout(X_, W, A_, B_, s, keep, p)[0]))

    h = 1e-6
    for name, arr, grad in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            pl, mi = arr.copy(), arr.copy()
            pl[idx] += h
            mi[idx] -= h
            args = {"X": X, "A": A, "B": B}
            args[name] = pl
            lp = loss(args["X"], args["A"], args["B"])
            args[name] = mi
            lm = loss(args["X"], args["A"], args["B"])
            num[idx] = (lp - lm) / (2 * h)
        assert np.allclose(grad, num, rtol=1e-6, atol=1e-7), name


def test_dropout_backward_matches_torch_autograd_fp64():
    X, W, A, B, dY = _tiny_linear(33, M=6, K=16, N=7, r=3)
    s, p = 0.25, 0.05
    keep = _keep_mask(3, X.shape, p)
    tX, tA, tB = (torch.tensor(v, dtype=torch.float64, requires_grad=True) for v in (X, A, B))
    tW, tk = torch.tensor(W, dtype=torch.float64), torch.tensor(keep, dtype=torch.float64)
    Y = tX @ tW.T + s * ((tX * tk / (1 - p)) @ tA) @ tB
    (Y * torch.tensor(dY)).sum().backward()
    dX, dA, dB = linear.backward_dropout(dY, X, W, A, B, s, keep, p)
    assert np.allclose(dX, tX.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dA, tA.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(dB, tB.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_pins_catch_planted_dropout_mistake(monkeypatch):
    """A dX that forgets to mask the adapter term fails the finite-difference pin."""
    X, W, A, B, dY = _tiny_linear(34)
    s, p = 0.5, 0.2
    keep = _keep_mask(4, X.shape, p)
    good = linear.backward_dropout(dY, X, W, A, B, s, keep, p)
    T = dY @ B.T
    bad_dX = dY @ W + s * (T @ A.T) / (1 - p)
    assert not np.allclose(bad_dX, good[0], rtol=1e-6, atol=1e-7)


# --------------------------------------------- LoRA optimizer step (G16)

from oracle import optim  # noqa: E402


def test_adamw_matches_torch_adamw_fp64():
    """Five steps of the oracle equal torch.optim.AdamW in fp64, with global
    gradient-norm clipping as torch.nn.utils.clip_grad_norm_ does it."""
    rng = np.random.default_rng(40)
    shapes = [(16, 4), (4, 24)]
    params = [rng.standard_normal(s) * 0.01 for s in shapes]
    tp = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in params]
    opt = torch.optim.AdamW(tp, lr=2e-4, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.01)
    ps = [a.copy() for a in params]
    ms = [np.zeros(s) for s in shapes]
    vs = [np.zeros(s) for s in shapes]
    for t in range(1, 6):
        grads = [rng.standard_normal(s) * (3.0 if t % 2 else 0.01) for s in shapes]
        for x, gr in zip(tp, grads):
            x.grad = torch.tensor(gr, dtype=torch.float64)
        torch.nn.utils.clip_grad_norm_(tp, 0.3)
        opt.step()
        sc = optim.clip_scale(grads, 0.3)
        for i in range(len(shapes)):
            ps[i], ms[i], vs[i] = optim.adamw_step(ps[i], grads[i], ms[i], vs[i], t, 2e-4, 0.9, 0.999, 1e-8, 0.01, sc)
        for a, x in zip(ps, tp):
            assert np.allclose(a, x.detach().numpy(), rtol=1e-12, atol=1e-15)


def test_adamw_first_step_closed_form():
    """At step 1 the bias-corrected moments are g and g^2, so without weight
    decay the update is lr * g / (|g| + eps): about lr * sign(g)."""
    g = np.array([1e-3, -2.0, 0.5, -1e-7])
    p, m, v = optim.adamw_step(np.zeros(4), g, np.zeros(4), np.zeros(4), 1, 0.1, 0.9, 0.999, 1e-8, 0.0)
    assert np.allclose(p, -0.1 * g / (np.abs(g) + 1e-8), rtol=1e-12)
    assert np.allclose(m, 0.1 * g) and np.allclose(v, 0.001 * g * g)


def test_clip_scale_closed_forms():
    assert optim.clip_scale([np.array([3.0, 4.0])], 0.3) == 0.3 / (5.0 + 1e-6)
    assert optim.clip_scale([np.array([0.1]), np.array([0.1])], 0.3) == 1.0
    assert optim.clip_scale([np.zeros(3)], 0.3) == 1.0


# ------------------------------------ QLoRA decoder block (reading G18)

from oracle import block  # noqa: E402


def _tiny_block(seed, hidden=16, mlp=24, r=3, b=2, t=5):
    rng = np.random.default_rng(seed)
    W = {n: rng.standard_normal(sh) * 0.2 for n, sh in block.shapes(hidden, mlp).items()}
    A = {n: rng.standard_normal((W[n].shape[1], r)) * 0.3 for n in block.LINEARS}
    B = {n: rng.standard_normal((r, W[n].shape[0])) * 0.3 for n in block.LINEARS}
    x = rng.standard_normal((b, t, hidden))
    g1, g2 = 1 + 0.1 * rng.standard_normal(hidden), 1 + 0.1 * rng.standard_normal(hidden)
    dy = rng.standard_normal((b, t, hidden))
    return x, W, A, B, g1, g2, dy


def _tt(a):
    return torch.tensor(np.asarray(a, dtype=np.float64))


def test_block_attention_is_sdpa_and_causal():
    """The attention core equals torch's causal scaled-dot-product attention
    (fp64), and position t ignores every later position."""
    rng = np.random.default_rng(50)
    q, k, v = (_tt(rng.standard_normal((2, 6, 8))) for _ in range(3))
    got = block.causal_attention(q, k, v, heads=2)
    split = lambda z: z.reshape(2, 6, 2, 4).permute(0, 2, 1, 3)  # noqa: E731
    ref = torch.nn.functional.scaled_dot_product_attention(split(q), split(k), split(v), is_causal=True)
    assert torch.allclose(got, ref.permute(0, 2, 1, 3).reshape(2, 6, 8), rtol=1e-12, atol=1e-12)
    k2, v2 = k.clone(), v.clone()
    k2[:, 4:] += 5.0
    v2[:, 4:] -= 3.0
    got2 = block.causal_attention(q, k2, v2, heads=2)
    assert torch.equal(got[:, :4], got2[:, :4]) and not torch.allclose(got[:, 4:], got2[:, 4:])


def test_block_rms_norm_and_identity():
    """rmsnorm is invariant to scaling its input (up to eps); with every W and
    every B zero the block is the identity (both residual branches vanish)."""
    rng = np.random.default_rng(51)
    z, g = _tt(rng.standard_normal((3, 16))), _tt(rng.standard_normal(16))
    assert torch.allclose(block.rms_norm(z * 1e3, g), block.rms_norm(z, g), rtol=1e-6, atol=0)  # eps = 1e-6
    one = torch.ones(16, dtype=torch.float64)
    assert torch.allclose(torch.mean(block.rms_norm(z, one) ** 2, dim=-1), torch.ones(3, dtype=torch.float64), rtol=1e-5)
    x, W, A, B, g1, g2, dy = _tiny_block(52)
    W0 = {n: np.zeros_like(W[n]) for n in W}
    B0 = {n: np.zeros_like(B[n]) for n in B}
    y, dx, dA, dB = block.forward_backward(x, W0, A, B0, g1, g2, 0.5, 2, dy)
    assert np.array_equal(y, x) and np.array_equal(dx, dy)
    assert all(np.all(dA[n] == 0) for n in block.LINEARS)


def test_block_linear_is_eq5():
    """Each block linear is the oracle's Eq. 5 layer."""
    x, W, A, B, *_ = _tiny_block(53)
    X = x.reshape(-1, 16)
    Y, _ = linear.forward(X, W["q"], A["q"], B["q"], 0.75)
    got = block.qlora_linear(_tt(X), _tt(W["q"]), _tt(A["q"]), _tt(B["q"]), 0.75).numpy()
    assert np.allclose(got, Y, rtol=1e-13, atol=1e-13)


def test_block_gradients_finite_differences():
    """Central differences of L = sum(dy * y) against the block's dx, dA, dB
    on a sample of entries of every linear."""
    x, W, A, B, g1, g2, dy = _tiny_block(54)
    s, heads = 0.5, 2
    y, dx, dA, dB = block.forward_backward(x, W, A, B, g1, g2, s, heads, dy)

    def loss(x_, A_, B_):
        with torch.no_grad():
            out = block.forward(_tt(x_), {n: _tt(W[n]) for n in W}, {n: _tt(A_[n]) for n in A},
                                {n: _tt(B_[n]) for n in B}, _tt(g1), _tt(g2), s, heads)
        return float((out * _tt(dy)).sum())

    h = 1e-6
    rng = np.random.default_rng(55)
    checks = [("x", None, dx)] + [("A", n, dA[n]) for n in block.LINEARS] + [("B", n, dB[n]) for n in block.LINEARS]
    for kind, name, grad in checks:
        for _ in range(3):
            idx = tuple(int(rng.integers(0, d)) for d in grad.shape)
            args = {"x": x.copy(), "A": {n: A[n].copy() for n in A}, "B": {n: B[n].copy() for n in B}}
            tgt = args["x"] if kind == "x" else args[kind][name]
            tgt[idx] += h
            lp = loss(args["x"], args["A"], args["B"])
            tgt[idx] -= 2 * h
            lm = loss(args["x"], args["A"], args["B"])
            num = (lp - lm) / (2 * h)
            assert math.isclose(num, grad[idx], rel_tol=1e-5, abs_tol=1e-7), (kind, name, idx, num, grad[idx])


def test_pins_catch_planted_non_causal_attention(monkeypatch):
    """Attention without the causal mask fails the SDPA/causality pin."""
    def no_mask(q, k, v, heads):
        b, t, hd = q.shape
        d = hd // heads
        split = lambda z: z.reshape(b, t, heads, d).permute(0, 2, 1, 3)  # noqa: E731
        p = torch.softmax(split(q) @ split(k).transpose(-1, -2) / math.sqrt(d), dim=-1)
        return (p @ split(v)).permute(0, 2, 1, 3).reshape(b, t, hd)
    monkeypatch.setattr(block, "causal_attention", no_mask)
    with pytest.raises(AssertionError):
        test_block_attention_is_sdpa_and_causal()
