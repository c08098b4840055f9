"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every test here runs on the CPU. The oracle is checked against hand-worked
fixtures (tests/golden), exact rational arithmetic, closed forms of the
quantizers on Gaussian inputs, brute force on tiny shapes and special cases
(identity weights, keep = K, keep = 0), never against a retyped copy of itself.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.stats import norm

import oracle as O
from synth import activations_bf16, bf16_bits_to_f32, latent_weights, normal
from tests.golden_io import arr, read_cases, scalar

F32 = np.float32


# ----------------------------------------------------------------------------- constants and sums
def test_sqrt7_is_nearest_float32():
    """The INT4 scale constant is the float32 nearest to sqrt(7) (exact rational bracket)."""
    c = O.SQRT7_F32
    lo = np.nextafter(c, F32(0))
    hi = np.nextafter(c, F32(10))
    mid_lo = (Fraction(float(lo)) + Fraction(float(c))) / 2
    mid_hi = (Fraction(float(c)) + Fraction(float(hi))) / 2
    assert mid_lo * mid_lo < 7 < mid_hi * mid_hi


def test_exact_abs_sum_matches_rational_sum():
    """exact_abs_sum is the correctly rounded double of the exact rational sum."""
    rng = np.random.default_rng(5)
    for trial in range(20):
        n = int(rng.integers(1, 400))
        # mantissas times wildly different powers of two: naive summation would lose bits
        v = rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n).astype(np.float64))
        v = v.astype(np.float32)
        exact = sum((Fraction(float(abs(t))) for t in v), Fraction(0))
        assert O.exact_abs_sum(v) == float(exact)      # float(Fraction) rounds correctly


def test_roundclip_half_even_and_clip():
    x = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 9.7, -9.7, 0.49999997])
    assert O.roundclip(x, -8, 7).tolist() == [0, 2, 2, 0, -2, -2, 7, -8, 0]


# ----------------------------------------------------------------------------- ternary weights
@pytest.mark.parametrize("case", read_cases("ternary_hand.txt"))
def test_ternary_hand_cases(case):
    eps, w, alpha, codes = case
    got_codes, got_alpha = O.ternarize(arr(w, np.float32), eps=scalar(eps))
    assert got_alpha == F32(scalar(alpha))
    np.testing.assert_array_equal(got_codes, arr(codes).astype(np.int8))


def test_ternary_gaussian_closed_forms():
    """For N(0, s^2) latents: alpha -> s*sqrt(2/pi) and P(code = 0) -> 2*Phi(0.5*sqrt(2/pi)) - 1 = 0.3101.

    (The write-up's "roughly half become +-1" is loose; the threshold is alpha/2, which gives 69% nonzero.)
    """
    sigma = 0.02
    w = latent_weights(77, 1024, 2048, sigma)
    codes, alpha = O.ternarize(w)
    assert abs(alpha - sigma * math.sqrt(2 / math.pi)) < 2e-5
    p0 = 2 * norm.cdf(0.5 * math.sqrt(2 / math.pi)) - 1
    n = codes.size
    assert abs((codes == 0).mean() - p0) < 5 * math.sqrt(p0 * (1 - p0) / n)
    assert set(np.unique(codes).tolist()) == {-1, 0, 1}
    # sign symmetry
    assert abs((codes == 1).mean() - (codes == -1).mean()) < 0.005


def test_ternary_codes_bruteforce_against_fraction_threshold():
    """Brute force: code = 0 iff |RN32(w/(alpha+eps))| <= 1/2, sign otherwise; alpha from exact rationals."""
    rng = np.random.default_rng(11)
    w = (rng.standard_normal((6, 10)) * 0.05).astype(np.float32)
    codes, alpha = O.ternarize(w, 1e-5)
    exact_mean = sum((Fraction(float(abs(t))) for t in w.ravel()), Fraction(0)) / w.size
    assert alpha == F32(float(exact_mean)) or abs(float(alpha) - float(exact_mean)) <= 2 ** -24 * float(exact_mean)
    den = F32(alpha + F32(1e-5))
    for i in range(6):
        for j in range(10):
            q = float(F32(w[i, j]) / den)
            want = 0 if abs(q) <= 0.5 else (1 if q > 0 else -1)
            assert codes[i, j] == want


# ----------------------------------------------------------------------------- INT4
@pytest.mark.parametrize("case", read_cases("int4_hand.txt"))
def test_int4_hand_cases(case):
    eps, x, beta, codes, dscale = case
    c, d, b = O.quant_int4(arr(x, np.float32), eps=scalar(eps))
    assert b[0] == F32(scalar(beta))
    np.testing.assert_array_equal(c, arr(codes).astype(np.int8))
    assert abs(float(d[0]) - scalar(dscale)) <= 1e-7 * max(1.0, scalar(dscale))


def test_int4_gaussian_closed_forms():
    """N(0,1) rows: beta -> sqrt(2/pi); P(c=0) = 2*Phi(t0)-1, P(c=7) = 1-Phi(6.5 b/sqrt7), P(c=-8) = Phi(-7.5 b/sqrt7).

    Also the write-up's range statement: 8*beta/sqrt7 = 3.02 beta ~ 2.4 sigma covers ~98% of a Gaussian.
    """
    x = bf16_bits_to_f32(activations_bf16(123, 128, 4096))
    c, d, beta = O.quant_int4(x)
    b = math.sqrt(2 / math.pi)
    assert abs(beta.mean() - b) < 0.005
    step = b / math.sqrt(7)                      # one code step in units of sigma
    n = c.size
    p0 = 2 * norm.cdf(0.5 * step) - 1
    p7 = 1 - norm.cdf(6.5 * step)
    pm8 = norm.cdf(-7.5 * step)
    for got, p in (((c == 0).mean(), p0), ((c == 7).mean(), p7), ((c == -8).mean(), pm8)):
        assert abs(got - p) < 5 * math.sqrt(p * (1 - p) / n) + 0.002   # +bf16 discretisation slack
    assert sorted(np.unique(c).tolist()) == list(range(-8, 8))          # exactly the 16 INT4 values
    assert abs(8 / math.sqrt(7) - 3.02) < 0.01
    assert abs((2 * norm.cdf(8 * step) - 1) - 0.98) < 0.01


def test_int4_zero_row_and_scaling_invariance():
    x = bf16_bits_to_f32(activations_bf16(9, 4, 256))
    c1, d1, _ = O.quant_int4(x, eps=1e-30)
    c2, d2, _ = O.quant_int4(x * F32(4.0), eps=1e-30)       # power-of-two scaling is exact
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(d2, d1 * F32(4.0))


# ----------------------------------------------------------------------------- FP4
@pytest.mark.parametrize("case", read_cases("fp4_hand.txt"))
def test_fp4_hand_cases(case):
    eps, x, nib, dbl = case
    n, d2, ds, g = O.quant_fp4(arr(x, np.float32), eps=scalar(eps))
    np.testing.assert_array_equal(n, arr(nib).astype(np.uint8))
    np.testing.assert_array_equal(d2, arr(dbl).astype(np.int8))


def test_e2m1_round_bruteforce():
    """Nearest-value rounding against an exhaustive argmin over the 8 magnitudes (ties -> even code)."""
    rng = np.random.default_rng(3)
    mags = np.concatenate([rng.uniform(0, 7, 5000), np.arange(0, 6.5, 0.125)])
    got = O.e2m1_round(mags)
    g = O.E2M1_GRID
    for m, i in zip(mags, got):
        d = np.abs(g - m)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert i == want, (m, i, want)


def test_fp4_row_max_maps_to_six():
    x = bf16_bits_to_f32(activations_bf16(31, 16, 512))
    n, d2, ds, g = O.quant_fp4(x)
    amax = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(d2[np.arange(16), amax]) == 12)
    assert set(np.unique(np.abs(d2)).tolist()) <= {0, 1, 2, 3, 4, 6, 8, 12}


# ----------------------------------------------------------------------------- Top-K + INT8
def test_fp4_pow2_exponent_bruteforce():
    """p is the smallest integer with 6 * 2^p >= gamma (exact rationals), clamped at -126."""
    rng = np.random.default_rng(9)
    gam = np.concatenate([np.float32([1.5, 1.5000001, 3.0, 6.0, 6.0000005, 12.0, 0.75, 1e-38, 2.0 ** -140]),
                          (rng.standard_normal(300) * np.exp2(rng.integers(-60, 60, 300))).astype(np.float32)])
    gam = np.abs(gam).astype(np.float32)
    p = O.fp4_pow2_exponent(gam)
    for g, q in zip(gam.tolist(), p.tolist()):
        fg = Fraction(g)
        if q > -126:
            assert 6 * Fraction(2) ** q >= fg > 6 * Fraction(2) ** (q - 1)
        else:
            assert 6 * Fraction(2) ** -126 >= fg


def test_fp4_pow2_codes_are_exact_scalings():
    x = bf16_bits_to_f32(activations_bf16(31, 6, 256))
    x[2] = 0.0
    nib, doubled, d, g = O.quant_fp4(x, pow2=True)
    assert d[2] == 0 and np.all(doubled[2] == 0)
    for r in (0, 1, 3, 4, 5):
        p = O.fp4_pow2_exponent(g[r:r + 1])[0]
        assert d[r] == np.float32(2.0 ** p)
        v = x[r].astype(np.float64) * 2.0 ** -p          # exact in float64
        assert np.abs(v).max() <= 6.0 and np.abs(v).max() > 3.0
        idx = O.e2m1_round(np.abs(v))
        np.testing.assert_array_equal(np.abs(doubled[r]), 2 * O.E2M1_GRID[idx])


def test_per_tensor_hand_example():
    """One scale for the tensor [[1, -1], [3, -3]]: beta = 2, gamma = 3 (hand-computed codes)."""
    x = np.float32([[1, -1], [3, -3]])
    c, d, b = O.quant_int4(x, eps=1e-5, per_tensor=True)
    assert np.all(b == np.float32(2.0))
    np.testing.assert_array_equal(c, [[1, -1], [4, -4]])        # round(x * sqrt7 / 2)
    c8, _, d8, g8 = O.quant_int8(x, eps=1e-5, per_tensor=True)
    assert np.all(g8 == 3)
    np.testing.assert_array_equal(c8, [[42, -42], [127, -127]])  # round(x * 127 / 3)
    _, doubled, _, g4 = O.quant_fp4(x, eps=1e-5, per_tensor=True)
    np.testing.assert_array_equal(doubled, [[4, -4], [12, -12]])  # x * 2 -> E2M1 2 and 6
    _, doubled2, dp, _ = O.quant_fp4(x, per_tensor=True, pow2=True)
    assert np.all(dp == 0.5)                                     # 6 * 2^-1 = 3 >= 3 > 1.5
    np.testing.assert_array_equal(doubled2, [[4, -4], [12, -12]])
    # per token the same rows give other codes
    assert not np.array_equal(O.quant_int4(x, eps=1e-5)[0], c)


@pytest.mark.parametrize("fmt", ["int4", "fp4", "fp4_pow2", "int8"])
def test_per_tensor_is_per_token_of_one_long_row(fmt):
    """per-tensor(X) == per-token(X.reshape(1, M*K)) with the scale repeated on every row."""
    x = bf16_bits_to_f32(activations_bf16(77, 5, 512))
    flat = x.reshape(1, -1)
    if fmt == "int4":
        (c, d, _), (cf, df, _) = O.quant_int4(x, per_tensor=True), O.quant_int4(flat)
    elif fmt == "int8":
        (c, _, d, _), (cf, _, df, _) = O.quant_int8(x, per_tensor=True), O.quant_int8(flat)
    else:
        pw = fmt == "fp4_pow2"
        (_, c, d, _), (_, cf, df, _) = O.quant_fp4(x, per_tensor=True, pow2=pw), O.quant_fp4(flat, pow2=pw)
    np.testing.assert_array_equal(c.reshape(1, -1), cf)
    np.testing.assert_array_equal(d, np.full(5, df[0], np.float32))


@pytest.mark.parametrize("case", read_cases("int8_hand.txt"))
def test_int8_hand_cases(case):
    eps, keep, x, codes, dscale = case
    k = int(scalar(keep))
    c, m, d, g = O.quant_int8(arr(x, np.float32), eps=scalar(eps), keep=None if k < 0 else k)
    np.testing.assert_array_equal(c, arr(codes).astype(np.int8))
    assert abs(float(d[0]) - scalar(dscale)) <= 1e-7 * max(1e-3, scalar(dscale))


def test_topk_bruteforce_pairs():
    """Exactly keep survivors; every survivor beats every non-survivor by (|x| desc, index asc)."""
    rng = np.random.default_rng(8)
    # few distinct magnitudes -> many ties at the boundary
    x = (rng.integers(-4, 5, (12, 40)) * 0.5).astype(np.float32)
    for keep in (0, 1, 7, 20, 39, 40):
        m = O.topk_mask(x, keep)
        for r in range(x.shape[0]):
            assert m[r].sum() == keep
            a = np.abs(x[r])
            s = np.flatnonzero(m[r])
            ns = np.flatnonzero(~m[r])
            for i in s:
                for j in ns:
                    assert a[i] > a[j] or (a[i] == a[j] and i < j)


def test_int8_invariants_and_special_keeps():
    x = bf16_bits_to_f32(activations_bf16(41, 32, 1024, outlier_scale=20.0, outlier_kind="t3"))
    c, m, d, g = O.quant_int8(x)
    assert c.min() >= -127 and c.max() <= 127                      # absmax never reaches -128
    amax = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(c[np.arange(32), amax]) == 127)
    cK, mK, _, _ = O.quant_int8(x, keep=1024)                      # keep = K is plain INT8 absmax
    np.testing.assert_array_equal(cK, c)
    c0, m0, _, _ = O.quant_int8(x, keep=0)
    assert not c0.any() and not m0.any()
    ch, mh, _, _ = O.quant_int8(x, keep=512)
    assert np.all(mh.sum(axis=1) == 512)
    np.testing.assert_array_equal(ch, np.where(mh, c, 0))          # mask-then-quantize == quantize-then-mask


# ----------------------------------------------------------------------------- GEMM + epilogues
def test_gemm_int_bruteforce():
    rng = np.random.default_rng(2)
    a = rng.integers(-128, 128, (5, 33)).astype(np.int8)
    t = rng.integers(-1, 2, (7, 33)).astype(np.int8)
    acc = O.gemm_int(a, t)
    for i in range(5):
        for j in range(7):
            assert acc[i, j] == sum(int(a[i, k]) * int(t[j, k]) for k in range(33))


def test_dequant_matches_float_matmul_of_dequantized_operands():
    """y equals float64 matmul of Q_INT4(X) (dequantized) times Q_w(W)^T (dequantized)."""
    x = bf16_bits_to_f32(activations_bf16(5, 6, 64))
    w = latent_weights(6, 10, 64)
    t, alpha = O.ternarize(w)
    r = O.bitlinear_a4(x, t, alpha)
    xq = r["codes"].astype(np.float64) * r["dscale"].astype(np.float64)[:, None]
    wq = t.astype(np.float64) * float(alpha)
    np.testing.assert_allclose(r["y"], xq @ wq.T, rtol=1e-12, atol=1e-300)


def test_identity_weights_pin_layout():
    """W = c*I ternarizes to I; then y[m, n] = dscale[m] * alpha * code[m, n] (pins transpose/layout)."""
    K = 48
    w = (np.eye(K) * 0.75).astype(np.float32)
    t, alpha = O.ternarize(w)
    np.testing.assert_array_equal(t, np.eye(K, dtype=np.int8))
    x = bf16_bits_to_f32(activations_bf16(12, 5, K))
    r = O.bitlinear_a4(x, t, alpha)
    np.testing.assert_allclose(r["y"], r["codes"] * (r["dscale"][:, None].astype(np.float64) * float(alpha)),
                               rtol=1e-15)
    r8 = O.bitlinear_a8(x, t, alpha, keep=K // 2)
    np.testing.assert_allclose(r8["y"], r8["codes"] * (r8["dscale"][:, None].astype(np.float64) * float(alpha)),
                               rtol=1e-15)


def test_fp4_gemm_counts_half_units():
    x = bf16_bits_to_f32(activations_bf16(15, 4, 64))
    w = latent_weights(16, 8, 64)
    t, alpha = O.ternarize(w)
    r = O.bitlinear_a4(x, t, alpha, fmt="fp4")
    vals = O.E2M1_GRID[r["nibbles"] & 7] * np.where(r["nibbles"] & 8, -1.0, 1.0)
    ref = (vals * r["dscale"].astype(np.float64)[:, None]) @ (t.astype(np.float64) * float(alpha)).T
    np.testing.assert_allclose(r["y"], ref, rtol=1e-12, atol=1e-300)


# ----------------------------------------------------------------------------- fixed-order fp32 epilogue
def rn32(q: Fraction) -> Fraction:
    """IEEE binary32 round-to-nearest-even of an exact rational, in integer arithmetic (subnormals
    included; the values used here never overflow)."""
    if q == 0:
        return Fraction(0)
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()       # 2^e <= a < 2^(e+1) after the fix-up
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum = Fraction(2) ** (max(e, -126) - 23)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    assert r < Fraction(2) ** 128
    return r if q > 0 else -r


def epilogue_exact(acc, d, alpha, unit):
    """RN32(RN32(acc * unit) * RN32(d * alpha)), every step rounded from the exact rational."""
    a = rn32(Fraction(int(acc)) * Fraction(unit))
    sc = rn32(Fraction(float(d)) * Fraction(float(alpha)))
    return rn32(a * sc)


@pytest.mark.parametrize("case", read_cases("epilogue_hand.txt"))
def test_dequant_f32_hand_cases(case):
    acc, d, alpha, unit, y = case
    got = O.dequant_f32(np.array([[int(scalar(acc))]]), np.float32([scalar(d)]), F32(scalar(alpha)), scalar(unit))
    assert got.dtype == np.float32 and float(got[0, 0]) == scalar(y)


def test_rn32_helper_against_float32_conversion():
    """The rational rounding helper agrees with numpy's float64 -> float32 conversion (a single IEEE
    rounding of an exact double) on doubles of every range, ties and subnormals included."""
    rng = np.random.default_rng(31)
    v = rng.standard_normal(3000) * np.exp2(rng.integers(-150, 120, 3000).astype(np.float64))
    ties = (np.float32(rng.standard_normal(500)).astype(np.float64) * (1 + 2.0 ** -24))   # halfway cases
    for x in np.concatenate([v, ties, [2.0 ** -149 * 1.5, 2.0 ** -149 * 0.5, 2.0 ** -149 * 2.5]]):
        assert float(rn32(Fraction(float(x)))) == float(np.float32(x)), x


def test_dequant_f32_is_the_fixed_order_rounding():
    """dequant_f32 rounds exactly three times, in the stated order, on accumulators of every size
    the matmuls produce (beyond 2^24 for INT8 at long K, where RN32(acc) itself rounds), for both
    accumulator units; plausible mistakes (scales multiplied in another order, one rounding,
    alpha or the unit dropped) disagree with it on this set."""
    rng = np.random.default_rng(17)
    n = 600
    mags = np.concatenate([rng.integers(0, 64, n // 4), rng.integers(0, 1 << 14, n // 4),
                           rng.integers((1 << 24) - 64, (1 << 24) + 64, n // 4),
                           rng.integers(1 << 24, 127 * 261888 + 1, n - 3 * (n // 4))])
    acc = mags * rng.choice([-1, 1], n)
    d = (rng.random(n) * np.exp2(rng.integers(-20, 4, n).astype(np.float64))).astype(np.float32)
    alpha = (rng.random(n) * np.exp2(rng.integers(-8, 2, n).astype(np.float64))).astype(np.float32)
    other = {"order": 0, "once": 0, "no_alpha": 0, "no_unit": 0}
    for unit in (1.0, 0.5):
        for i in range(n):
            got = O.dequant_f32(np.array([[int(acc[i])]]), d[i:i + 1], alpha[i], unit)[0, 0]
            want = epilogue_exact(acc[i], d[i], alpha[i], unit)
            assert Fraction(float(got)) == want, (int(acc[i]), float(d[i]), float(alpha[i]), unit)
            A, D, Al, U = Fraction(int(acc[i])), Fraction(float(d[i])), Fraction(float(alpha[i])), Fraction(unit)
            other["order"] += rn32(rn32(rn32(A * U) * D) * Al) != want
            other["once"] += rn32(A * U * D * Al) != want
            other["no_alpha"] += rn32(rn32(A * U) * rn32(D)) != want
            other["no_unit"] += unit != 1.0 and rn32(rn32(A) * rn32(D * Al)) != want
    assert all(v > 0 for v in other.values()), other


def test_dequant_f32_agrees_with_float64_dequant():
    """Three roundings of 2^-24 each: |dequant_f32 - dequant| <= 2^-22 |dequant| in the normal range."""
    rng = np.random.default_rng(19)
    acc = rng.integers(-127 * 261888, 127 * 261888 + 1, (64, 48))
    d = (rng.random(64) * 0.05 + 1e-3).astype(np.float32)
    alpha = F32(0.0159576)
    for unit in (1.0, 0.5):
        y32 = O.dequant_f32(acc, d, alpha, unit).astype(np.float64)
        y64 = O.dequant(acc, d, alpha, unit)
        assert np.all(np.abs(y32 - y64) <= 2.0 ** -22 * np.abs(y64))


@pytest.mark.parametrize("case", read_cases("relu2_hand.txt"))
def test_relu2_hand_cases(case):
    g, u, h = case
    got = O.relu2_glu(arr(g, np.float32)[0], arr(u, np.float32)[0])
    np.testing.assert_array_equal(got, arr(h, np.float32)[0])


def test_ffn_composition_and_sparsity():
    """FFN: h zero wherever the gate is <= 0 (about half for i.i.d. data); down input INT8 without Top-K."""
    x = bf16_bits_to_f32(activations_bf16(21, 8, 256))
    tg, ag = O.ternarize(latent_weights(22, 384, 256))
    tu, au = O.ternarize(latent_weights(23, 384, 256))
    td, ad = O.ternarize(latent_weights(24, 256, 384))
    r = O.ffn_ref(x, tg, ag, tu, au, td, ad)
    g = O.dequant_f32(r["acc_g"], r["dscale"], ag)
    assert np.all(r["h"][g <= 0] == 0)
    assert 0.4 < (r["h"] == 0).mean() < 0.6
    np.testing.assert_array_equal(r["h_absmax"], np.abs(r["h"]).max(axis=1))
    assert np.all(np.abs(r["h_codes"]).max(axis=1) == 127)
    # down output against float64 matmul of the dequantized operands
    hq = r["h_codes"].astype(np.float64) * r["h_dscale"].astype(np.float64)[:, None]
    wq = td.astype(np.float64) * float(ad)
    bound = 1e-12 * (np.abs(hq) @ np.abs(wq).T)          # cancellation-aware float64 bound
    assert np.all(np.abs(r["y"] - hq @ wq.T) <= bound)


def test_relu2_glu_conditional_skips_dead_channels_and_matches_full_glu():
    """Conditional up projection: u is requested only for live channels; h equals the full ReLU^2
    GLU as numbers and is +0 (bit pattern 0) wherever the gate is <= 0."""
    rng = np.random.default_rng(5)
    g = rng.standard_normal((3, 40)).astype(np.float32)
    g[:, :6] = -np.abs(g[:, :6])                     # six channels dead in every row
    g[0, 6] = 0.0
    u = rng.standard_normal((3, 40)).astype(np.float32)
    seen = []

    def u_fn(cols):
        seen.append(np.asarray(cols))
        return u[:, cols]

    h, live = O.relu2_glu_conditional(g, u_fn)
    full = O.relu2_glu(g, u)
    np.testing.assert_array_equal(h, full)          # -0 == +0 as numbers
    assert np.all(h.view(np.uint32)[g <= 0] == 0)
    np.testing.assert_array_equal(live, np.flatnonzero((g > 0).any(axis=0)))
    assert len(seen) == 1 and not set(range(6)) & set(seen[0].tolist())
    mask = g > 0
    np.testing.assert_array_equal(h.view(np.uint32)[mask], full.view(np.uint32)[mask])


def test_ffn_gate_up_conditional_matches_ffn_ref():
    x = bf16_bits_to_f32(activations_bf16(25, 3, 256))
    tg, ag = O.ternarize(latent_weights(26, 96, 256))
    tu, au = O.ternarize(latent_weights(27, 96, 256))
    td, ad = O.ternarize(latent_weights(28, 256, 96))
    full = O.ffn_ref(x, tg, ag, tu, au, td, ad)
    r = O.ffn_gate_up_conditional_ref(x, tg, ag, tu, au)
    np.testing.assert_array_equal(r["h"], full["h"])
    np.testing.assert_array_equal(r["g"], O.dequant_f32(full["acc_g"], full["dscale"], ag))
    np.testing.assert_array_equal(r["h_absmax"], full["h_absmax"])
    assert 0 < r["live"].size < 96


def test_oproj_residual():
    x = bf16_bits_to_f32(activations_bf16(51, 4, 128, outlier_scale=20.0, outlier_kind="t3"))
    t, a = O.ternarize(latent_weights(52, 64, 128))
    res = normal(53, 4 * 64).reshape(4, 64).astype(np.float32)
    r = O.oproj_ref(x, t, a, res, keep=64)
    assert np.all(r["mask"].sum(axis=1) == 64)
    # against a float64 matmul of the dequantized, masked INT8 codes plus the residual
    xq = r["codes"].astype(np.float64) * r["dscale"].astype(np.float64)[:, None]
    wq = t.astype(np.float64) * float(a)
    ref = xq @ wq.T + res.astype(np.float64)
    bound = 1e-12 * (np.abs(xq) @ np.abs(wq).T + np.abs(res))        # cancellation-aware
    assert np.all(np.abs(r["y"] - ref) <= bound)
    # the residual really enters: an all-zero input row returns the residual row exactly
    x0 = x.copy()
    x0[1] = 0
    r0 = O.oproj_ref(x0, t, a, res, keep=64)
    np.testing.assert_array_equal(r0["y"][1], res[1].astype(np.float64))


def test_generators_are_deterministic_and_gaussian():
    a = normal(7, 200000)
    assert np.array_equal(a, normal(7, 200000))
    assert abs(a.mean()) < 0.01 and abs(a.std() - 1) < 0.01
    bits = activations_bf16(3, 2, 16)
    f = bf16_bits_to_f32(bits)
    assert np.all((f.view(np.uint32) & 0xFFFF) == 0)


# ----------------------------------------------------------------------------- KV cache (R17)
def test_kv_quant_hand_example():
    """gamma = 3: 3 bits scale by 3/(3+eps), 4 bits by 7/(3+eps); offsets 4 and 8 (hand-computed)."""
    x = np.float32([[[1, -1, 0.5, -3]]])
    u3, d3, g = O.kv_quant(x, 3)
    np.testing.assert_array_equal(u3[0, 0], [5, 3, 4, 1])      # c = 1, -1, 0 (0.49999 rounds down), -3
    assert d3[0, 0] == np.float32(1.0) and g[0, 0] == 3
    u4, d4, _ = O.kv_quant(x, 4)
    np.testing.assert_array_equal(u4[0, 0], [10, 6, 9, 1])     # c = 2, -2, 1, -7
    assert d4[0, 0] == np.float32(3.0) / np.float32(7.0)


@pytest.mark.parametrize("bits", [3, 4])
def test_kv_quant_range_and_error_bound(bits):
    """Codes lie in [1, 2^b - 1], the head max maps to an end code, and the dequantized value is
    within (gamma + eps) / (2 Qp) + eps of x (round-to-nearest on the absmax grid)."""
    rng = np.random.default_rng(bits)
    x = (rng.standard_normal((9, 4, 64)) * np.exp2(rng.integers(-8, 8, (9, 4, 1)))).astype(np.float32)
    x[3, 2] = 0.0
    eps = 1e-5
    u, d, g = O.kv_quant(x, bits, eps)
    off, qp = 2 ** (bits - 1), 2 ** (bits - 1) - 1
    assert u.min() >= 1 and u.max() <= 2 ** bits - 1
    assert np.all(u[3, 2] == off) and d[3, 2] == 0
    am = np.abs(x).argmax(axis=2)
    top = np.take_along_axis(u, am[..., None], axis=2)[..., 0].astype(int)
    assert np.all((top == 2 * qp + 1) | (top == 1) | (g == 0))
    deq = (u.astype(np.float64) - off) * g[..., None].astype(np.float64) / qp
    bound = (g[..., None].astype(np.float64) + eps) / (2 * qp) * (1 + 1e-6) + eps
    assert np.all(np.abs(deq - x) <= bound)
    # a wrong level count (2^b - 1 in place of Qp) breaks the bound somewhere
    wrong = (u.astype(np.float64) - off) * g[..., None] / (2 ** bits - 1)
    assert np.any(np.abs(wrong - x) > bound)


def test_rope_special_angles_and_complex_product():
    rng = np.random.default_rng(5)
    T, H, D = 6, 3, 16
    x = rng.standard_normal((T, H, D)).astype(np.float32)
    pos = np.array([0, 1, 2, 3, 0, 2])
    ang = rng.uniform(-3, 3, (4, D // 2))
    cos, sin = np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
    cos[0], sin[0] = 1, 0                     # position 0: identity
    cos[1], sin[1] = 0, 1                     # position 1: quarter turn, (a, b) -> (-b, a)
    r = O.rope_rotate_half(x, pos, cos, sin)
    np.testing.assert_array_equal(r[0], x[0])
    np.testing.assert_array_equal(r[4], x[4])
    np.testing.assert_array_equal(r[1], np.concatenate([-x[1, :, D // 2:], x[1, :, :D // 2]], axis=1))
    # the pair turns as the complex product (a + ib)(c + is), to a few fp32 ulps
    z = (x[..., :D // 2].astype(np.float64) + 1j * x[..., D // 2:]) * \
        (cos[pos][:, None].astype(np.float64) + 1j * sin[pos][:, None])
    ref = np.concatenate([z.real, z.imag], axis=2)
    scale = np.abs(x[..., :D // 2]).astype(np.float64) + np.abs(x[..., D // 2:])
    assert np.all(np.abs(r - ref) <= 4 * 2.0 ** -24 * np.concatenate([scale, scale], axis=2))
    # swapping the halves' roles (a wrong pairing) is caught
    assert not np.allclose(r[2:4], O.rope_rotate_half(x[2:4, :, ::-1].copy(), pos[2:4], cos, sin)[:, :, ::-1])


def test_kv_cache_quant_bos_records():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((5, 2, 32)).astype(np.float32)
    bos = np.array([True, False, False, True, False])
    out = O.kv_cache_quant(x, 3, bos=bos)
    u4, d4, _ = O.kv_quant(x, 4)
    np.testing.assert_array_equal(out["bos_u"][bos], u4[bos])
    np.testing.assert_array_equal(out["bos_dscale"][bos], d4[bos])
    np.testing.assert_array_equal(out["u"], O.kv_quant(x, 3)[0])
    assert O.kv_cache_quant(x, 4, bos=bos)["bos_u"] is None
