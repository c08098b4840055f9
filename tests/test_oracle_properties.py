"""Property tests of the CPU oracle over random small shapes and values (hypothesis).

Each property follows from the definitions of the quantizers and of BitLinear in "BitNet a4.8:
4-bit Activations for 1-bit LLMs" (section 3, Eq. 1-9) and of ternary absmean weights in "The Era
of 1-bit LLMs" (BitNet b1.58, section 2), not from the oracle's code: ranges, signs, monotonicity,
order independence of the exact sums, exact invariance under power-of-two scaling (with eps = 0,
where every rounding step scales exactly), error bounds of round-to-nearest, the Top-K tie rule,
row and column independence, and exact rational checks of the float32 steps. The examples are
derandomized, so every run draws the same cases.
"""
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle as O
from tests.test_oracle_pins import rn32

F32 = np.float32
PROPS = settings(max_examples=60, deadline=None, derandomize=True, database=None,
                 suppress_health_check=[HealthCheck.too_slow])

seeds = st.integers(min_value=0, max_value=2 ** 32 - 1)
rows = st.integers(min_value=1, max_value=6)
cols = st.integers(min_value=1, max_value=96)


def draw_values(seed, shape, kind):
    """Finite float32 test values: Gaussian, heavy-tailed (Student-t, df 3), few distinct magnitudes
    (many ties), or a wide exponent spread; a seeded share of exact zeros in each."""
    rng = np.random.default_rng(seed)
    if kind == "normal":
        v = rng.standard_normal(shape)
    elif kind == "heavy":
        v = rng.standard_t(3, shape)
    elif kind == "ties":
        v = rng.choice([-3.0, -1.5, -0.25, 0.25, 1.5, 3.0], size=shape)
    else:
        v = rng.standard_normal(shape) * np.exp2(rng.integers(-12, 12, shape).astype(np.float64))
    v = np.where(rng.random(shape) < 0.1, 0.0, v)
    return v.astype(np.float32)


kinds = st.sampled_from(["normal", "heavy", "ties", "spread"])


def rows_with_mass(x, floor=1e-2):
    """Rows whose mean |x| is at least floor (there eps / beta is at most 1e-3)."""
    return np.abs(x.astype(np.float64)).mean(axis=1) >= floor


# ----------------------------------------------------------------------------- ternary weights
@PROPS
@given(seeds, rows, cols, st.integers(-20, 20))
def test_ternarize_properties(seed, n, k, e):
    w = (np.random.default_rng(seed).standard_normal((n, k)) * 0.02).astype(np.float32)
    t, alpha = O.ternarize(w)
    assert set(np.unique(t)) <= {-1, 0, 1}
    assert np.all((t == 0) | (np.sign(t) == np.sign(w)))
    # alpha is mean |W|: within one float32 rounding (and one double rounding) of the exact mean
    exact = sum(Fraction(float(abs(v))) for v in w.ravel()) / w.size
    assert abs(Fraction(float(alpha)) - exact) <= exact * Fraction(1, 2 ** 23)
    # the rounding threshold of |W / (alpha + eps)| is 1/2: codes away from it are fixed
    den = float(alpha) + 1e-5
    r = np.abs(w.astype(np.float64)) / den
    assert np.all(t[r > 0.5 * (1 + 2 ** -20)] != 0)
    assert np.all(t[r < 0.5 * (1 - 2 ** -20)] == 0)
    # order independence (alpha is an exact sum) and exact power-of-two scaling with eps = 0
    p = np.random.default_rng(seed + 1).permutation(w.size)
    tp, ap = O.ternarize(w.ravel()[p].reshape(n, k))
    assert ap == alpha and np.array_equal(tp.ravel(), t.ravel()[p])
    t0, a0 = O.ternarize(w, eps=0.0)
    ts, as_ = O.ternarize((w * F32(2.0 ** e)).astype(np.float32), eps=0.0)
    assert np.array_equal(ts, t0) and float(as_) == float(a0) * 2.0 ** e


# ----------------------------------------------------------------------------- INT4 absmean
@PROPS
@given(seeds, rows, cols, kinds)
def test_int4_properties(seed, m, k, kind):
    x = draw_values(seed, (m, k), kind)
    codes, dscale, beta = O.quant_int4(x)
    assert codes.dtype == np.int8 and codes.min(initial=0) >= -8 and codes.max(initial=0) <= 7
    assert np.all((codes == 0) | (np.sign(codes) == np.sign(x)))
    for r in range(m):
        exact = sum(Fraction(float(abs(v))) for v in x[r]) / k
        assert abs(Fraction(float(beta[r])) - exact) <= exact * Fraction(1, 2 ** 23)
        # monotone in x: sorting the row sorts its codes
        o = np.argsort(x[r], kind="stable")
        assert np.all(np.diff(codes[r][o].astype(np.int32)) >= 0)
        # a row alone gives the same codes (per-token quantizer)
        c1, d1, _ = O.quant_int4(x[r:r + 1])
        assert np.array_equal(c1[0], codes[r]) and d1[0] == dscale[r]
    # round-to-nearest of x * sqrt7 / beta: within 1/2 of the code unless clipped
    ok = rows_with_mass(x)
    z = x[ok].astype(np.float64) / dscale[ok, None].astype(np.float64)
    c = codes[ok].astype(np.float64)
    tol = 1e-3 * (1 + np.abs(z))
    inner = (c > -8) & (c < 7)
    assert np.all(np.abs(z - c)[inner] <= 0.5 + tol[inner])
    assert np.all(z[c == 7] >= 6.5 - tol[c == 7]) and np.all(z[c == -8] <= -7.5 + tol[c == -8])


@PROPS
@given(seeds, rows, cols, kinds, st.integers(-20, 20))
def test_int4_permutation_and_pow2_scaling(seed, m, k, kind, e):
    x = draw_values(seed, (m, k), kind)
    codes, dscale, beta = O.quant_int4(x)
    p = np.random.default_rng(seed + 7).permutation(k)
    cp, dp, bp = O.quant_int4(x[:, p])
    assert np.array_equal(cp, codes[:, p]) and np.array_equal(bp, beta) and np.array_equal(dp, dscale)
    with np.errstate(divide="ignore", invalid="ignore"):       # all-zero rows divide by zero at eps = 0
        c0, d0, _ = O.quant_int4(x, eps=0.0)
        cs, ds, _ = O.quant_int4((x * F32(2.0 ** e)).astype(np.float32), eps=0.0)
    live = np.abs(x).sum(axis=1) > 0
    assert np.array_equal(cs[live], c0[live])
    assert np.array_equal(ds[live].astype(np.float64), d0[live].astype(np.float64) * 2.0 ** e)


# ----------------------------------------------------------------------------- FP4 E2M1 MinMax
@PROPS
@given(seeds, rows, cols, kinds, st.booleans())
def test_fp4_properties(seed, m, k, kind, pow2):
    x = draw_values(seed, (m, k), kind)
    nib, doubled, dscale, gamma = O.quant_fp4(x, pow2=pow2)
    idx = (nib & 7).astype(np.int64)
    neg = (nib & 8) != 0
    assert np.all(nib < 16)
    assert np.array_equal(np.abs(doubled.astype(np.int64)), (2 * O.E2M1_GRID[idx]).astype(np.int64))
    assert np.all(neg == (doubled < 0)) and np.all(~neg | (x < 0))      # no -0, signs follow x
    assert np.array_equal(gamma, np.max(np.abs(x), axis=1))
    for r in range(m):
        o = np.argsort(np.abs(x[r]), kind="stable")
        assert np.all(np.diff(idx[r][o]) >= 0)                        # monotone in |x|
        live = gamma[r] >= 1e-2
        if live:
            j = int(np.argmax(np.abs(x[r])))
            # the row maximum is coded 6 (eps only: 6 gamma / (gamma + eps) > 5); with a
            # power-of-two scale it lands in [3, 6]
            assert O.E2M1_GRID[idx[r, j]] == 6.0 if not pow2 else 3.0 <= O.E2M1_GRID[idx[r, j]] <= 6.0


@PROPS
@given(seeds, rows, cols, kinds, st.integers(-20, 20), st.booleans())
def test_fp4_pow2_scaling(seed, m, k, kind, e, pow2):
    x = draw_values(seed, (m, k), kind)
    with np.errstate(divide="ignore", invalid="ignore"):       # all-zero rows divide by zero at eps = 0
        n0, _, d0, _ = O.quant_fp4(x, eps=0.0, pow2=pow2)
        ns, _, ds, _ = O.quant_fp4((x * F32(2.0 ** e)).astype(np.float32), eps=0.0, pow2=pow2)
    live = np.abs(x).max(axis=1) > 0
    assert np.array_equal(ns[live], n0[live])
    assert np.array_equal(ds[live].astype(np.float64), d0[live].astype(np.float64) * 2.0 ** e)


# ----------------------------------------------------------------------------- Top-K + INT8 absmax
@PROPS
@given(seeds, rows, cols, kinds, st.floats(0.0, 1.0))
def test_topk_mask_properties(seed, m, k, kind, frac):
    x = draw_values(seed, (m, k), kind)
    keep = int(round(frac * k))
    mask = O.topk_mask(x, keep)
    a = np.abs(x)
    assert np.all(mask.sum(axis=1) == keep)
    for r in range(m):
        kept, dropped = a[r][mask[r]], a[r][~mask[r]]
        if kept.size and dropped.size:
            assert kept.min() >= dropped.max()
        # ties: among equal magnitudes, a kept index is never after a dropped one
        for v in np.unique(a[r]):
            same = np.flatnonzero(a[r] == v)
            flags = mask[r][same]
            assert np.all(np.diff(flags.astype(np.int8)) <= 0)


@PROPS
@given(seeds, rows, cols, kinds, st.floats(0.0, 1.0))
def test_int8_properties(seed, m, k, kind, frac):
    x = draw_values(seed, (m, k), kind)
    keep = int(round(frac * k))
    codes, mask, dscale, gamma = O.quant_int8(x, keep=keep)
    full, fmask, fd, fg = O.quant_int8(x)
    assert np.all(fmask)
    # the mask only zeroes codes: the scale comes from the whole row
    assert np.array_equal(codes, np.where(mask, full, 0)) and np.array_equal(dscale, fd)
    assert np.array_equal(gamma, np.max(np.abs(x), axis=1))
    assert full.min(initial=0) >= -127 and full.max(initial=0) <= 127     # the -128 clip never acts
    assert np.all((full == 0) | (np.sign(full) == np.sign(x)))
    ok = gamma >= 1e-2
    z = x[ok].astype(np.float64) / dscale[ok, None].astype(np.float64)
    assert np.all(np.abs(z - full[ok]) <= 0.5 + 1e-3 * (1 + np.abs(z)))
    for r in np.flatnonzero(ok):
        j = int(np.argmax(np.abs(x[r])))
        assert abs(int(full[r, j])) == 127


# ----------------------------------------------------------------------------- matmul and epilogues
@PROPS
@given(seeds, st.integers(1, 5), st.integers(1, 7), st.integers(1, 300))
def test_gemm_int_is_the_integer_sum(seed, m, n, k):
    rng = np.random.default_rng(seed)
    a = rng.integers(-127, 128, (m, k)).astype(np.int8)
    t = rng.integers(-1, 2, (n, k)).astype(np.int8)
    acc = O.gemm_int(a, t)
    for i in range(m):
        for j in range(n):
            assert int(acc[i, j]) == sum(int(p) * int(q) for p, q in zip(a[i], t[j]))


@PROPS
@given(seeds, st.integers(1, 5), st.integers(1, 6), st.sampled_from([128, 256, 384]),
       st.sampled_from(["int4", "fp4", "fp4_pow2"]))
def test_bitlinear_rows_and_columns_are_independent(seed, m, n, k, fmt):
    """Per-token activation scales and a weight scale given as input: every output row depends on
    its own token only, and splitting the weight rows splits the output columns."""
    x = draw_values(seed, (m, k), "heavy")
    w = (np.random.default_rng(seed + 3).standard_normal((n, k)) * 0.02).astype(np.float32)
    t, alpha = O.ternarize(w)
    r = O.bitlinear_a4(x, t, alpha, fmt=fmt)
    for i in range(m):
        ri = O.bitlinear_a4(x[i:i + 1], t, alpha, fmt=fmt)
        assert np.array_equal(ri["acc"][0], r["acc"][i]) and np.array_equal(ri["y"][0], r["y"][i])
    c = n // 2
    ra = O.bitlinear_a4(x, t[:c], alpha, fmt=fmt)
    rb = O.bitlinear_a4(x, t[c:], alpha, fmt=fmt)
    assert np.array_equal(np.concatenate([ra["y"], rb["y"]], axis=1), r["y"])


@PROPS
@given(seeds, st.integers(1, 4), st.integers(1, 8))
def test_relu2_glu_is_exactly_rounded(seed, m, n):
    rng = np.random.default_rng(seed)
    g = (rng.standard_normal((m, n)) * np.exp2(rng.integers(-8, 8, (m, n)))).astype(np.float32)
    u = (rng.standard_normal((m, n)) * np.exp2(rng.integers(-8, 8, (m, n)))).astype(np.float32)
    g[rng.random((m, n)) < 0.3] = 0.0
    h = O.relu2_glu(g, u)
    for i in range(m):
        for j in range(n):
            gp = Fraction(float(g[i, j])) if g[i, j] > 0 else Fraction(0)
            want = rn32(rn32(gp * gp) * Fraction(float(u[i, j])))
            assert Fraction(float(h[i, j])) == want
            if g[i, j] <= 0:                                      # +0 times u: a zero with u's sign
                assert h[i, j] == 0 and np.signbit(h[i, j]) == (u[i, j] < 0)


@PROPS
@given(seeds, st.integers(1, 3), st.integers(1, 6))
def test_dequant_f32_monotone_in_the_accumulator(seed, m, n):
    """A larger integer sum never gives a smaller float32 output (every rounding step is monotone)."""
    rng = np.random.default_rng(seed)
    acc = np.sort(rng.integers(-2 ** 26, 2 ** 26, (m, n)), axis=1)
    d = (rng.random(m) + 0.01).astype(np.float32)
    y = O.dequant_f32(acc, d, F32(0.0173))
    assert np.all(np.diff(y.astype(np.float64), axis=1) >= 0)


# ----------------------------------------------------------------------------- KV cache
@PROPS
@given(seeds, st.integers(1, 4), st.integers(1, 3), st.sampled_from([2, 8, 16, 128]), st.sampled_from([3, 4]),
       kinds)
def test_kv_quant_properties(seed, t, h, d, bits, kind):
    x = draw_values(seed, (t, h, d), kind)
    u, dscale, gamma = O.kv_quant(x, bits)
    qp = 2 ** (bits - 1) - 1
    assert u.max(initial=0) <= 2 ** bits - 1
    c = u.astype(np.int64) - 2 ** (bits - 1)
    assert c.min(initial=0) >= -qp                               # the -Qp-1 clip never acts
    assert np.array_equal(gamma, np.max(np.abs(x), axis=2))
    ok = gamma >= 1e-2
    z = x[ok].astype(np.float64) / dscale[ok][:, None].astype(np.float64)
    assert np.all(np.abs(z - c[ok]) <= 0.5 + 1e-3 * (1 + np.abs(z)))
    p = np.random.default_rng(seed + 5).permutation(d)
    up, dp, _ = O.kv_quant(x[..., p], bits)
    assert np.array_equal(up, u[..., p]) and np.array_equal(dp, dscale)


@PROPS
@given(seeds, st.integers(1, 5), st.integers(1, 3), st.sampled_from([4, 16, 128]))
def test_rope_special_rotations_and_norm(seed, t, h, d):
    x = draw_values(seed, (t, h, d), "normal")
    half = d // 2
    rng = np.random.default_rng(seed + 11)
    ang = rng.random((4, half)) * 2 * np.pi
    cos = np.concatenate([np.ones((1, half)), np.zeros((1, half)), np.cos(ang)]).astype(np.float32)
    sin = np.concatenate([np.zeros((1, half)), np.ones((1, half)), np.sin(ang)]).astype(np.float32)
    pos = rng.integers(0, cos.shape[0], t)
    out = O.rope_rotate_half(x, pos, cos, sin)
    for i in range(t):
        a, b = x[i, :, :half], x[i, :, half:]
        if pos[i] == 0:                                          # angle 0: identity
            assert np.array_equal(out[i], x[i])
        elif pos[i] == 1:                                        # quarter turn: (a, b) -> (-b, a)
            assert np.array_equal(out[i, :, :half], -b) and np.array_equal(out[i, :, half:], a)
        n0 = a.astype(np.float64) ** 2 + b.astype(np.float64) ** 2
        n1 = out[i, :, :half].astype(np.float64) ** 2 + out[i, :, half:].astype(np.float64) ** 2
        assert np.all(np.abs(n1 - n0) <= 1e-5 * (n0 + 1e-30))      # a rotation keeps each pair's norm


@PROPS
@given(seeds, st.integers(1, 6), st.integers(1, 3))
def test_kv_cache_bos_records_are_the_4bit_quantizer(seed, t, h):
    x = draw_values(seed, (t, h, 128), "heavy")
    bos = np.random.default_rng(seed + 2).random(t) < 0.5
    o = O.kv_cache_quant(x, 3, bos=bos)
    u3, d3, _ = O.kv_quant(x, 3)
    u4, d4, _ = O.kv_quant(x, 4)
    assert np.array_equal(o["u"], u3) and np.array_equal(o["dscale"], d3)
    assert np.array_equal(o["bos_u"][bos], u4[bos]) and np.array_equal(o["bos_dscale"][bos], d4[bos])
    assert not o["bos_u"][~bos].any() and not o["bos_dscale"][~bos].any()


if __name__ == "__main__":
    raise SystemExit(pytest.main([__file__, "-q"]))
