"""GPU parity: every entry point of libbitlinear (through the C ABI) against the CPU oracle.

Codes, masks, scales and ternary weights must match bit for bit; float32 outputs must equal the
oracle's fixed-order float32 dequantization of its exact integer accumulators bit for bit, and lie
within 1e-5 relative of the float64 value. Shapes span several tiles with ragged M and N tails.
"""
import numpy as np
import pytest

import oracle as O
import ternary_weight_quantized_amd as tw
from synth import activations_bf16, latent_weights, normal, to_bf16_bits
from tests.gpu_util import (assert_y_close, dev_bf16, dev_f32, e3m2_values, host, int4_values, int8_values,
                            mask_bits, nibbles, torch_cuda, x_f32)
from tests.packed_layout import unpack_ternary, unpack_ternary_rows

pytestmark = pytest.mark.gpu

EPS = 1e-5


# ----------------------------------------------------------------------------- inputs
def special_rows(K, rng, f32=False):
    """Degenerate rows: all zero, huge exponent spread (forces the exact-sum fallback),
    subnormals, few distinct magnitudes (Top-K ties), one nonzero."""
    rows = []
    rows.append(np.zeros(K))
    wide = rng.standard_normal(K) * np.exp2(rng.integers(-70, 70, K).astype(np.float64))
    rows.append(wide)
    sub = rng.standard_normal(K) * 2.0 ** -130
    rows.append(sub)
    rows.append(rng.integers(-3, 4, K) * 0.5)
    one = np.zeros(K)
    one[K // 3] = -3.25
    rows.append(one)
    a = np.array(rows)
    return a.astype(np.float32) if f32 else to_bf16_bits(a)


def make_x(seed, M, K, f32=False, special=True):
    rng = np.random.default_rng(seed)
    if f32:
        x = normal(seed, M * K).reshape(M, K).astype(np.float32)
        if special and M >= 6:
            x[1:6] = special_rows(K, rng, True)
        return x
    x = activations_bf16(seed, M, K)
    if special and M >= 6:
        x[1:6] = special_rows(K, rng)
    return x


def to_dev(x):
    return dev_f32(x) if x.dtype == np.float32 else dev_bf16(x)


def packed_weights(seed, N, K, sigma=0.02, a8=False):
    """Latent weights, the oracle's ternary codes and alpha, and the library's packed weights: the
    standard layout, or with a8 the layout of the matmuls with INT8 activations."""
    w = latent_weights(seed, N, K, sigma)
    codes, alpha = O.ternarize(w, EPS)
    packed, a = (tw.bitlinear_pack_ternary_a8 if a8 else tw.bitlinear_pack_ternary)(dev_f32(w), EPS)
    return w, codes, alpha, packed, a


# ----------------------------------------------------------------------------- pack
@pytest.mark.parametrize("N,K", [(16, 256), (32, 384), (48, 768), (160, 4096), (2048, 2048)])
def test_pack_ternary(N, K):
    torch_cuda()
    w, codes, alpha, packed, a = packed_weights(100 + N, N, K)
    assert host(a)[0] == alpha, (host(a)[0], alpha)
    np.testing.assert_array_equal(unpack_ternary(host(packed), N, K), codes)


@pytest.mark.parametrize("N,K", [(16, 256), (32, 384), (48, 768), (160, 4096), (2048, 2048)])
def test_pack_ternary_a8(N, K):
    """The A8 tile layout holds the oracle's codes (decoded from the header's description) and the
    same alpha as the standard layout."""
    torch_cuda()
    w, codes, alpha, packed, a = packed_weights(150 + N, N, K, a8=True)
    assert host(a)[0] == alpha
    np.testing.assert_array_equal(unpack_ternary(host(packed), N, K, a8=True), codes)
    _, _, _, p_std, a_std = packed_weights(150 + N, N, K)
    assert host(a_std)[0] == alpha
    if N * K >= 16 * 256:
        assert not np.array_equal(host(packed), host(p_std))       # the two layouts differ


@pytest.mark.parametrize("N,K", [(16, 256), (32, 384), (48, 768), (160, 4096)])
def test_pack_ternary_rows(N, K):
    torch_cuda()
    w = latent_weights(150 + N, N, K)
    codes, alpha = O.ternarize(w, EPS)
    packed, a = tw.bitlinear_pack_ternary_rows(dev_f32(w), EPS)
    assert host(a)[0] == alpha
    np.testing.assert_array_equal(unpack_ternary_rows(host(packed), N, K), codes)


def test_pack_ternary_wide_exponents_and_zero():
    torch_cuda()
    rng = np.random.default_rng(4)
    N, K = 32, 512
    w = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-60, 60, (N, K)))).astype(np.float32)
    w[3] = 0.0
    codes, alpha = O.ternarize(w, EPS)
    packed, a = tw.bitlinear_pack_ternary(dev_f32(w), EPS)
    assert host(a)[0] == alpha
    np.testing.assert_array_equal(unpack_ternary(host(packed), N, K), codes)
    z = np.zeros((16, 256), np.float32)
    packed, a = tw.bitlinear_pack_ternary(dev_f32(z), EPS)
    assert host(a)[0] == 0.0 and not host(packed).any()


# ----------------------------------------------------------------------------- quantizers
# K = 384 and 16512 are odd multiples of 128 (a half 256-group at the end); 16512 and 32768 take the
# streaming kernels (rows longer than 16384)
QSHAPES = [(1, 256), (6, 384), (7, 768), (64, 2048), (33, 4096), (9, 4352), (6, 11008), (6, 16512), (2, 32768)]


@pytest.mark.parametrize("fmt", ["int4", "int4_e3m2"])
@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("M,K", QSHAPES)
def test_quantize_int4(M, K, f32, fmt):
    torch_cuda()
    x = make_x(1000 + M + K, M, K, f32)
    codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), fmt, eps=EPS)
    c, d, _ = O.quant_int4(x_f32(x), EPS)
    got = int4_values(host(codes)) if fmt == "int4" else e3m2_values(host(codes), M)
    np.testing.assert_array_equal(got, c)
    np.testing.assert_array_equal(host(scale), d)


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("M,K", QSHAPES)
def test_quantize_fp4_pow2(M, K, f32):
    torch_cuda()
    x = make_x(3500 + M + K, M, K, f32)
    codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), "fp4_pow2", eps=EPS)
    nib, _, d, _ = O.quant_fp4(x_f32(x), EPS, pow2=True)
    np.testing.assert_array_equal(nibbles(host(codes)), nib)
    np.testing.assert_array_equal(host(scale), d)


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("M,K", [(2049, 640), (2100, 8192)])
def test_quantize_many_rows(M, K, f32):
    """More rows than the part holds blocks at once (two rounds of blocks), at an odd multiple of 128
    and at 8192: every plain format (INT4 nibbles and E3M2 tiles, FP4, FP4 power of two, INT8 with
    and without the row-max hint) bit-exact over the whole tensor, special rows included."""
    torch_cuda()
    x = make_x(4500 + M + K, M, K, f32)
    xf = x_f32(x)
    c, d, _ = O.quant_int4(xf, EPS)
    for fmt in ("int4", "int4_e3m2"):
        codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), fmt, eps=EPS)
        got = int4_values(host(codes)) if fmt == "int4" else e3m2_values(host(codes), M)
        np.testing.assert_array_equal(got, c)
        np.testing.assert_array_equal(host(scale), d)
    for pow2 in (False, True):
        codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), "fp4_pow2" if pow2 else "fp4", eps=EPS)
        nib, _, d4, _ = O.quant_fp4(xf, EPS, pow2=pow2)
        np.testing.assert_array_equal(nibbles(host(codes)), nib)
        np.testing.assert_array_equal(host(scale), d4)
    c8, _, d8, g8 = O.quant_int8(xf, EPS)
    for hint in (None, dev_f32(g8)):
        codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), "int8", eps=EPS, row_absmax_hint=hint)
        np.testing.assert_array_equal(int8_values(host(codes)), c8)
        np.testing.assert_array_equal(host(scale), d8)


FP4_TIES = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6), (6.0, 7)]


def fp4_boundary_row(K, f32):
    """A row whose largest magnitude is 6, so that the power-of-two FP4 scale is exactly 1 and every
    element reaches the E2M1 rounding unchanged: the grid midpoints (ties) and the maximum, their
    neighbours one unit in the last place away, the negatives of all of them, negative values that
    round to zero, -0 and subnormals. Returns the row and the positions of the ties and of their
    negatives."""
    vals, pos = [], []
    for t, _ in FP4_TIES:
        pos.append(len(vals))
        if f32:
            near = [np.nextafter(np.float32(t), np.float32(0)), np.nextafter(np.float32(t), np.float32(7))]
        else:
            b = int(to_bf16_bits(np.array([t]))[0])
            near = list(x_f32(np.array([b - 1, b + 1], np.uint16)))
        vals += [t] + [v for v in near if abs(v) <= 6.0]
    n = len(vals)
    vals += [-v for v in vals]
    vals += [-0.0, -1e-30, -0.1, -0.25, 2.0 ** -130, -(2.0 ** -130)]
    row = np.zeros(K)
    row[:len(vals)] = vals
    return row, pos, [n + p for p in pos], 2 * n


@pytest.mark.parametrize("f32", [False, True])
def test_quantize_fp4_rounding_boundaries(f32):
    """E2M1 rounding at every tie and next to it: nearest, ties to the even mantissa, negative
    values that round to zero give code 0."""
    torch_cuda()
    K = 256
    row, pos, neg, tail = fp4_boundary_row(K, f32)
    rows = np.stack([row, row[::-1].copy()])
    x = rows.astype(np.float32) if f32 else to_bf16_bits(rows)
    nib, _, d, _ = O.quant_fp4(x_f32(x), EPS, pow2=True)
    np.testing.assert_array_equal(d, np.ones(2, np.float32))
    # the oracle against the rule itself at the ties, at their negatives and at the signed zeros
    for (t, code), p, q in zip(FP4_TIES, pos, neg):
        assert nib[0, p] == code, (t, nib[0, p])
        assert nib[0, q] == (code | 8 if code else 0), (-t, nib[0, q])
    np.testing.assert_array_equal(nib[0, tail:tail + 6], np.zeros(6, np.uint8))
    for fmt, pow2 in (("fp4_pow2", True), ("fp4", False)):
        codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), fmt, eps=EPS)
        nib_o, _, d_o, _ = O.quant_fp4(x_f32(x), EPS, pow2=pow2)
        np.testing.assert_array_equal(nibbles(host(codes)), nib_o)
        np.testing.assert_array_equal(host(scale), d_o)


def int4_tie_row(K, seed):
    """A float32 row whose probe elements land x s exactly on the INT4 rounding ties k + 1/2
    (k = -9 .. 7, so -8.5 and 7.5 meet the clip too), with s = sqrt7 / (beta + eps) the row's scale,
    each beside its neighbours one unit in the last place away, and values that round to -0, +0 and
    -0 itself. The probes move beta only in its last bits, so placing them again until beta no
    longer changes settles it. Returns the row and the number of probes that sit exactly on a tie."""
    rng = np.random.default_rng(seed)
    row = rng.standard_normal(K).astype(np.float32)
    ties = [np.float32(k + 0.5) for k in range(-9, 8)]
    f = np.float32

    def scale(r):
        _, _, beta = O.quant_int4(r[None], EPS)
        return f(O.SQRT7_F32 / f(beta[0] + f(EPS)))

    s = scale(row)
    for _ in range(10):
        j = 0
        for t in ties:
            x = f(t / s)
            for _ in range(8):                      # walk to the float whose product is the tie
                y = f(x * s)
                if y == t:
                    break
                x = np.nextafter(x, f(np.inf) if (y < t) == (s > 0) else f(-np.inf))
            row[j:j + 3] = [np.nextafter(x, f(-np.inf)), x, np.nextafter(x, f(np.inf))]
            j += 3
        row[j:j + 5] = [f(-0.2) / s, -1e-30, 0.0, -0.0, f(0.49) / s]
        s_new = scale(row)
        if s_new == s:
            break
        s = s_new
    exact = sum(int(f(row[3 * i + 1] * s) == t) for i, t in enumerate(ties))
    return row, exact


@pytest.mark.parametrize("fmt", ["int4", "int4_e3m2"])
def test_quantize_int4_rounding_ties(fmt):
    """INT4 rounding at every tie k + 1/2 of x s and next to it, the clip at -8 and 7, and values
    that round to -0: half to even, and the nibble and E3M2 codes equal the oracle's."""
    torch_cuda()
    K = 512
    rows = np.stack([int4_tie_row(K, 77 + i)[0] for i in range(3)])
    exact = min(int4_tie_row(K, 77 + i)[1] for i in range(3))
    assert exact >= 12, exact                       # the probes really sit on the ties
    c, d, _ = O.quant_int4(rows, EPS)
    codes, scale, _ = tw.bitlinear_quantize_act(dev_f32(rows), fmt, eps=EPS)
    got = int4_values(host(codes)) if fmt == "int4" else e3m2_values(host(codes), 3)
    np.testing.assert_array_equal(got, c)
    np.testing.assert_array_equal(host(scale), d)


@pytest.mark.parametrize("fmt", ["int4", "int4_e3m2", "fp4", "fp4_pow2", "int8"])
@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("M,K", [(1, 256), (9, 640), (7, 768), (33, 4096), (130, 1024), (5, 8192)])
def test_quantize_per_tensor(M, K, f32, fmt):
    """One scale for the whole tensor: codes bit-exact, the scale repeated in every row."""
    torch = torch_cuda()
    x = make_x(4100 + M + K, M, K, f32)
    ws = torch.full((tw.bitlinear_quantize_per_tensor_workspace_bytes(M),), 0xAB, dtype=torch.uint8, device="cuda")
    codes, scale = tw.bitlinear_quantize_act_per_tensor(to_dev(x), fmt, eps=EPS, workspace=ws)
    xf = x_f32(x)
    if fmt in ("int4", "int4_e3m2"):
        c, d, _ = O.quant_int4(xf, EPS, per_tensor=True)
        got = int4_values(host(codes)) if fmt == "int4" else e3m2_values(host(codes), M)
        np.testing.assert_array_equal(got, c)
    elif fmt == "int8":
        c, _, d, _ = O.quant_int8(xf, EPS, per_tensor=True)
        np.testing.assert_array_equal(int8_values(host(codes)), c)
    else:
        nib, _, d, _ = O.quant_fp4(xf, EPS, pow2=fmt == "fp4_pow2", per_tensor=True)
        np.testing.assert_array_equal(nibbles(host(codes)), nib)
    np.testing.assert_array_equal(host(scale), d)
    # a second call over the same (dirty) workspace gives the same result
    codes2, scale2 = tw.bitlinear_quantize_act_per_tensor(to_dev(x), fmt, eps=EPS, workspace=ws)
    if fmt == "int4_e3m2":      # tile rows past M are padding the quantizer does not write
        np.testing.assert_array_equal(e3m2_values(host(codes2), M), e3m2_values(host(codes), M))
    else:
        np.testing.assert_array_equal(host(codes2), host(codes))
    np.testing.assert_array_equal(host(scale2), host(scale))


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("M,K", QSHAPES)
def test_quantize_fp4(M, K, f32):
    torch = torch_cuda()
    x = make_x(2000 + M + K, M, K, f32)
    codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), "fp4", eps=EPS)
    nib, _, d, g = O.quant_fp4(x_f32(x), EPS)
    np.testing.assert_array_equal(nibbles(host(codes)), nib)
    np.testing.assert_array_equal(host(scale), d)
    # the row-max hint path gives the same result
    codes2, scale2, _ = tw.bitlinear_quantize_act(to_dev(x), "fp4", eps=EPS, row_absmax_hint=dev_f32(g))
    np.testing.assert_array_equal(host(codes2), host(codes))
    torch.cuda.synchronize()


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("M,K", QSHAPES)
@pytest.mark.parametrize("keep_frac", [None, 0.0, 0.5, 1.0, "one", "k-1"])
def test_quantize_int8_topk(M, K, f32, keep_frac):
    torch_cuda()
    if keep_frac is None:
        keep = -1
    elif keep_frac == "one":
        keep = 1
    elif keep_frac == "k-1":
        keep = K - 1
    else:
        keep = int(keep_frac * K)
    x = make_x(3000 + M + K, M, K, f32)
    codes, scale, mask = tw.bitlinear_quantize_act(to_dev(x), "int8", topk_keep=keep, eps=EPS, want_mask=True)
    c, m, d, g = O.quant_int8(x_f32(x), EPS, None if keep < 0 else keep)
    np.testing.assert_array_equal(mask_bits(host(mask), K), m)
    np.testing.assert_array_equal(int8_values(host(codes)), c)
    np.testing.assert_array_equal(host(scale), d)


@pytest.mark.parametrize("M,K", [(5, 768), (33, 4096), (6, 8192)])
def test_quantize_int8_topk_with_hint(M, K):
    """Top-K of bf16 rows with the row maximum given: the same codes, mask and scales as the oracle
    (the threshold search runs without the block's own max reduction)."""
    torch_cuda()
    x = make_x(3500 + M + K, M, K, False)
    keep = K // 2
    c, m, d, g = O.quant_int8(x_f32(x), EPS, keep)
    codes, scale, mask = tw.bitlinear_quantize_act(to_dev(x), "int8", topk_keep=keep, eps=EPS, want_mask=True,
                                                   row_absmax_hint=dev_f32(g))
    np.testing.assert_array_equal(mask_bits(host(mask), K), m)
    np.testing.assert_array_equal(int8_values(host(codes)), c)
    np.testing.assert_array_equal(host(scale), d)


@pytest.mark.parametrize("M,K", [(4000, 768), (2500, 4096), (1700, 8192)])
@pytest.mark.parametrize("keep_frac", [0.5, 1.0, 0.0, "one", "hint"])
def test_quantize_int8_topk_many_rows(M, K, keep_frac):
    """More bf16 rows than the device holds blocks of the Top-K kernel at once, so that every block
    works through several rows (the next row's copy in flight while one is quantized): with and
    without the threshold search (keep = K and keep = 0 skip it), and with a given row maximum."""
    torch_cuda()
    keep = 1 if keep_frac == "one" else K // 2 if keep_frac == "hint" else int(keep_frac * K)
    x = make_x(3700 + M + K, M, K, False)
    c, m, d, g = O.quant_int8(x_f32(x), EPS, keep)
    hint = dev_f32(g) if keep_frac == "hint" else None
    codes, scale, mask = tw.bitlinear_quantize_act(to_dev(x), "int8", topk_keep=keep, eps=EPS, want_mask=True,
                                                   row_absmax_hint=hint)
    np.testing.assert_array_equal(mask_bits(host(mask), K), m)
    np.testing.assert_array_equal(int8_values(host(codes)), c)
    np.testing.assert_array_equal(host(scale), d)


@pytest.mark.parametrize("K", [768, 4096, 8192])
def test_quantize_int8_topk_threshold_depth(K):
    """Rows whose Top-K threshold lies 0 to 12 binary exponents below the row maximum: a few
    elements near 3.0 set the maximum, the rest are N(0, 1) scaled by 2^-d. The threshold search
    resolves thresholds near the maximum's exponent with small histograms and falls back to the
    full search below that; both sides of that boundary must give the oracle's mask and codes."""
    torch_cuda()
    rng = np.random.default_rng(4242 + K)
    rows = []
    for d in range(0, 13):
        r = rng.standard_normal(K) * 2.0 ** -d
        r[rng.choice(K, 8, replace=False)] = 3.0 + rng.random(8)
        rows.append(r)
    x = to_bf16_bits(np.array(rows))
    for keep in (K // 2, K // 8, K - 3):
        c, m, d_, g = O.quant_int8(x_f32(x), EPS, keep)
        codes, scale, mask = tw.bitlinear_quantize_act(to_dev(x), "int8", topk_keep=keep, eps=EPS, want_mask=True)
        np.testing.assert_array_equal(mask_bits(host(mask), K), m)
        np.testing.assert_array_equal(int8_values(host(codes)), c)
        np.testing.assert_array_equal(host(scale), d_)


def test_quantize_int8_hint_matches_max_pass():
    torch_cuda()
    x = make_x(77, 12, 11008, True)
    _, _, _, g = O.quant_int8(x, EPS)
    a = tw.bitlinear_quantize_act(dev_f32(x), "int8", eps=EPS)
    b = tw.bitlinear_quantize_act(dev_f32(x), "int8", eps=EPS, row_absmax_hint=dev_f32(g))
    np.testing.assert_array_equal(host(a[0]), host(b[0]))
    np.testing.assert_array_equal(host(a[1]), host(b[1]))


def test_quantize_strided_rows():
    torch_cuda()
    x = make_x(5, 10, 1024 + 256)
    xs = to_dev(x)[:, :1024]                      # row stride 1280 elements
    codes, scale, _ = tw.bitlinear_quantize_act(xs, "int4", eps=EPS)
    c, d, _ = O.quant_int4(x_f32(x)[:, :1024], EPS)
    np.testing.assert_array_equal(int4_values(host(codes)), c)
    np.testing.assert_array_equal(host(scale), d)


def test_quantize_is_deterministic():
    torch_cuda()
    x = to_dev(make_x(6, 64, 4096))
    a = tw.bitlinear_quantize_act(x, "int8", topk_keep=2048, want_mask=True)
    b = tw.bitlinear_quantize_act(x, "int8", topk_keep=2048, want_mask=True)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(host(u), host(v))


# ----------------------------------------------------------------------------- GEMMs
GSHAPES = [(1, 16, 256), (37, 80, 384), (200, 272, 512), (129, 144, 768), (64, 2048, 2048)]


def _quant(x, fmt, keep=-1):
    codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), fmt, topk_keep=keep, eps=EPS)
    if fmt in ("int4", "int4_e3m2"):
        c, d, _ = O.quant_int4(x_f32(x), EPS)
        return codes, scale, c, d, 1.0
    if fmt == "fp4":
        _, c, d, _ = O.quant_fp4(x_f32(x), EPS)
        return codes, scale, c, d, 0.5
    c, _, d, _ = O.quant_int8(x_f32(x), EPS, None if keep < 0 else keep)
    return codes, scale, c, d, 1.0


A4_FMTS = ["int4", "int4_e3m2", "fp4"]


@pytest.mark.parametrize("fmt", A4_FMTS)
@pytest.mark.parametrize("M,N,K", GSHAPES + [(300, 528, 1280)])
def test_gemm_a4(fmt, M, N, K):
    torch_cuda()
    x = make_x(4000 + M, M, K)
    _, t, alpha, packed, a = packed_weights(4100 + N, N, K)
    codes, scale, c, d, unit = _quant(x, fmt)
    y = tw.bitlinear_gemm_w158a4(fmt, codes, scale, K, packed, a, N)
    assert_y_close(host(y), O.gemm_int(c, t), d, alpha, unit)


@pytest.mark.parametrize("fmt", A4_FMTS)
@pytest.mark.parametrize("M,N,K", [(200, 272, 512), (3, 48, 1024)])
def test_gemm_a4_residual_inplace(fmt, M, N, K):
    torch_cuda()
    x = make_x(4200 + M, M, K)
    _, t, alpha, packed, a = packed_weights(4300 + N, N, K)
    codes, scale, c, d, unit = _quant(x, fmt)
    r = normal(4400, M * N).reshape(M, N).astype(np.float32)
    y = dev_f32(r)
    tw.bitlinear_gemm_w158a4(fmt, codes, scale, K, packed, a, N, y=y, residual=y)   # y aliases residual
    assert_y_close(host(y), O.gemm_int(c, t), d, alpha, unit, residual=r)


@pytest.mark.parametrize("fmt", A4_FMTS)
@pytest.mark.parametrize("M,N,K", [(200, 272, 512), (64, 2048, 2048), (257, 400, 768)])
def test_gemm_a4_relu2_glu(fmt, M, N, K):
    torch = torch_cuda()
    x = make_x(4500 + M, M, K, special=False)     # (rows scaled by 2^70 would overflow g^2: out of contract)
    x[1] = 0                                       # a zero row stays in
    _, tg, ag, pg, dag = packed_weights(4600 + N, N, K)
    _, tu, au, pu, dau = packed_weights(4700 + N, N, K)
    codes, scale, c, d, unit = _quant(x, fmt)
    rowmax = torch.full((M,), 123.0, dtype=torch.float32, device="cuda")          # must be cleared by the call
    h = tw.bitlinear_gemm_w158a4(fmt, codes, scale, K, pg, dag, N, up_packed=pu, up_alpha=dau, row_absmax=rowmax)
    g = O.dequant_f32(O.gemm_int(c, tg), d, ag, unit)
    u = O.dequant_f32(O.gemm_int(c, tu), d, au, unit)
    h_ref = O.relu2_glu(g, u)
    np.testing.assert_array_equal(host(h).view(np.uint32), h_ref.view(np.uint32))
    np.testing.assert_array_equal(host(rowmax), np.abs(h_ref).max(axis=1))


@pytest.mark.parametrize("M,N,K", GSHAPES + [(40, 64, 11008), (300, 528, 1280)])
@pytest.mark.parametrize("keep_frac", [None, 0.5])
def test_gemm_a8_sparse(M, N, K, keep_frac):
    torch_cuda()
    x = make_x(5000 + M, M, K, f32=True)
    x[M // 2:, : K // 2] = 0.0                      # whole zero K slices exercise the skip path
    _, t, alpha, packed, a = packed_weights(5100 + N, N, K, a8=True)
    keep = -1 if keep_frac is None else int(keep_frac * K)
    codes, scale, c, d, _ = _quant(x, "int8", keep)
    y = tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, a, N)
    assert_y_close(host(y), O.gemm_int(c, t), d, alpha)


@pytest.mark.parametrize("M,N,K,epi", [(130, 80, 1280, "none"), (300, 528, 768, "residual"), (64, 272, 2048, "relu2")])
def test_gemm_a8_structured_zero_slices(M, N, K, epi):
    """A seeded half of the 16-row x 128-column code slices set to zero (the structured-sparsity input
    of the benchmark, at small sizes): in some K steps the first subtile of a 64-row wave strip is
    zero while later ones are live, in others every subtile of a strip is zero; all epilogues."""
    torch = torch_cuda()
    rng = np.random.default_rng(5600 + M + K)
    x = x_f32(make_x(5600 + M, M, K, f32=True, special=False))
    dead = rng.random(((M + 15) // 16, K // 128)) < 0.5
    dead[0, 0], dead[1, 0], dead[2, 0], dead[3, 0] = True, False, True, False   # strip 0, step 0
    x[np.repeat(np.repeat(dead, 16, 0), 128, 1)[:M]] = 0.0
    _, t, alpha, packed, a = packed_weights(5700 + N, N, K, a8=True)
    codes, scale, c, d, _ = _quant(x, "int8", -1)
    acc = O.gemm_int(c, t)
    if epi == "none":
        y = tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, a, N)
        assert_y_close(host(y), acc, d, alpha)
    elif epi == "residual":
        r = normal(5800, M * N).reshape(M, N).astype(np.float32)
        y = tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, a, N, residual=dev_f32(r))
        assert_y_close(host(y), acc, d, alpha, residual=r)
    else:
        _, tu, au, pu, dau = packed_weights(5900 + N, N, K, a8=True)
        h = tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, a, N, up_packed=pu, up_alpha=dau)
        h_ref = O.relu2_glu(O.dequant_f32(acc, d, alpha), O.dequant_f32(O.gemm_int(c, tu), d, au))
        np.testing.assert_array_equal(host(h).view(np.uint32), h_ref.view(np.uint32))
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K", [(200, 272, 512), (33, 64, 11008)])
def test_gemm_a8_residual_and_relu2(M, N, K):
    torch = torch_cuda()
    x = make_x(5200 + M, M, K, f32=True, special=False)
    x[1] = 0.0
    _, t, alpha, packed, a = packed_weights(5300 + N, N, K, a8=True)
    codes, scale, c, d, _ = _quant(x, "int8", K // 2)
    acc = O.gemm_int(c, t)
    r = normal(5400, M * N).reshape(M, N).astype(np.float32)
    y = tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, a, N, residual=dev_f32(r))
    assert_y_close(host(y), acc, d, alpha, residual=r)
    _, tu, au, pu, dau = packed_weights(5500 + N, N, K, a8=True)
    rowmax = torch.zeros(M, dtype=torch.float32, device="cuda")
    h = tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, a, N, up_packed=pu, up_alpha=dau, row_absmax=rowmax)
    h_ref = O.relu2_glu(O.dequant_f32(acc, d, alpha), O.dequant_f32(O.gemm_int(c, tu), d, au))
    np.testing.assert_array_equal(host(h).view(np.uint32), h_ref.view(np.uint32))
    np.testing.assert_array_equal(host(rowmax), np.abs(h_ref).max(axis=1))


# ----------------------------------------------------------------------------- decode
@pytest.mark.parametrize("fmt", ["int4", "int8"])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 7, 8])
@pytest.mark.parametrize("N,K", [(80, 384), (48, 512), (1024, 4096), (64, 11008), (32, 8192), (48, 12800),
                                 (32, 16512)])
def test_decode(fmt, M, N, K):
    torch_cuda()
    x = make_x(6000 + M + K, M, K, special=False)
    if fmt == "int8":
        x = x_f32(x)
        x[:, 256:1024] = 0.0                      # zero slices: their weight loads are skipped
    _, t, alpha, packed, a = packed_weights(6100 + N, N, K, a8=fmt == "int8")
    codes, scale, c, d, _ = _quant(x, fmt, -1)
    y = tw.bitlinear_gemv_decode(fmt, codes, scale, K, packed, a, N)
    assert_y_close(host(y), O.gemm_int(c, t), d, alpha)


@pytest.mark.parametrize("fmt", ["int4", "int8"])
def test_decode_epilogues(fmt):
    torch = torch_cuda()
    M, N, K = 6, 96, 1024
    x = x_f32(make_x(6200, M, K, special=False))
    _, t, alpha, packed, a = packed_weights(6300, N, K, a8=fmt == "int8")
    codes, scale, c, d, _ = _quant(x, fmt, -1)
    acc = O.gemm_int(c, t)
    r = normal(6400, M * N).reshape(M, N).astype(np.float32)
    y = tw.bitlinear_gemv_decode(fmt, codes, scale, K, packed, a, N, residual=dev_f32(r))
    assert_y_close(host(y), acc, d, alpha, residual=r)
    _, tu, au, pu, dau = packed_weights(6500, N, K, a8=fmt == "int8")
    rowmax = torch.zeros(M, dtype=torch.float32, device="cuda")
    h = tw.bitlinear_gemv_decode(fmt, codes, scale, K, packed, a, N, up_packed=pu, up_alpha=dau, row_absmax=rowmax)
    h_ref = O.relu2_glu(O.dequant_f32(acc, d, alpha), O.dequant_f32(O.gemm_int(c, tu), d, au))
    np.testing.assert_array_equal(host(h).view(np.uint32), h_ref.view(np.uint32))
    np.testing.assert_array_equal(host(rowmax), np.abs(h_ref).max(axis=1))


def test_gemm_fp4_pow2_codes():
    """FP4 codes of the power-of-two scale variant run through the FP4 GEMM unchanged."""
    torch_cuda()
    M, N, K = 70, 160, 768
    x = make_x(6950, M, K, special=False)
    _, t, alpha, packed, a = packed_weights(6960, N, K)
    codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), "fp4_pow2", eps=EPS)
    y = tw.bitlinear_gemm_w158a4("fp4", codes, scale, K, packed, a, N)
    r = O.bitlinear_a4(x_f32(x), t, alpha, EPS, fmt="fp4_pow2")
    assert_y_close(host(y), r["acc"], r["dscale"], alpha, 0.5)


def test_gemm_formats_agree():
    """INT4 on int8 cores and the same codes in E3M2 on FP6 cores give identical outputs."""
    torch_cuda()
    M, N, K = 520, 784, 2304
    x = make_x(6800, M, K, special=False)
    _, t, alpha, packed, a = packed_weights(6900, N, K)
    c4, s4, _, _, _ = _quant(x, "int4")
    c6, s6, _, _, _ = _quant(x, "int4_e3m2")
    np.testing.assert_array_equal(host(s4), host(s6))
    y4 = tw.bitlinear_gemm_w158a4("int4", c4, s4, K, packed, a, N)
    y6 = tw.bitlinear_gemm_w158a4("int4_e3m2", c6, s6, K, packed, a, N)
    np.testing.assert_array_equal(host(y4), host(y6))


def test_decode_matches_gemm():
    torch_cuda()
    M, N, K = 8, 512, 4096
    x = make_x(6600, M, K, special=False)
    _, t, alpha, packed, a = packed_weights(6700, N, K)
    codes, scale, _, _, _ = _quant(x, "int4")
    y1 = tw.bitlinear_gemv_decode("int4", codes, scale, K, packed, a, N)
    y2 = tw.bitlinear_gemm_w158a4("int4", codes, scale, K, packed, a, N)
    np.testing.assert_array_equal(host(y1), host(y2))


# ----------------------------------------------------------------------------- conditional up projection
@pytest.mark.parametrize("M", [1, 3, 8])
@pytest.mark.parametrize("N,K", [(16, 256), (48, 384), (48, 768), (80, 4352), (1024, 4096), (32, 8192), (32, 8320)])
def test_glu_conditional(M, N, K):
    """Gate first, up only where the gate is positive: gate, h (bit patterns, +0 where g <= 0) and
    the row maxima equal the oracle's; h equals the fused GLU decode as numbers. K = 8320 with
    M = 8 has more code bytes (33280) than the kernel stages in LDS and takes the global-load path,
    K = 8192 with M = 8 exactly fills the 32 KiB stage; M = 3 runs without the row maxima."""
    torch = torch_cuda()
    x = make_x(7000 + M + K, M, K, special=False)
    wg = latent_weights(7100 + N, N, K)
    wu = latent_weights(7200 + N, N, K)
    tg, ag = O.ternarize(wg, EPS)
    tu, au = O.ternarize(wu, EPS)
    pg, dag = tw.bitlinear_pack_ternary(dev_f32(wg), EPS)
    pu_rows, dau = tw.bitlinear_pack_ternary_rows(dev_f32(wu), EPS)
    pu, _ = tw.bitlinear_pack_ternary(dev_f32(wu), EPS)
    codes, scale, _, _, _ = _quant(x, "int4")
    rowmax = torch.empty(M, dtype=torch.float32, device="cuda") if M != 3 else None
    gate, h = tw.bitlinear_gemv_decode_glu_conditional(codes, scale, K, pg, dag, pu_rows, dau, N, row_absmax=rowmax)
    r = O.ffn_gate_up_conditional_ref(x_f32(x), tg, ag, tu, au, EPS)
    np.testing.assert_array_equal(host(gate).view(np.uint32), r["g"].view(np.uint32))
    np.testing.assert_array_equal(host(h).view(np.uint32), r["h"].view(np.uint32))
    if rowmax is not None:
        np.testing.assert_array_equal(host(rowmax), r["h_absmax"])
    full = tw.bitlinear_gemv_decode("int4", codes, scale, K, pg, dag, N, up_packed=pu, up_alpha=dau)
    np.testing.assert_array_equal(host(full), host(h))


# ----------------------------------------------------------------------------- longest accepted K
MAXK = 262016      # 2^18 - 128: the longest reduction the matmul entry points accept


@pytest.mark.parametrize("kind,fmt", [("gemm", "int4"), ("gemm", "int4_e3m2"), ("gemm", "fp4"), ("a8", "int8"),
                                      ("gemv", "int4"), ("gemv", "int8")])
def test_matmul_extreme_codes_at_longest_k(kind, fmt):
    """Every activation code at its largest magnitude against all -1 weights at the longest accepted
    K: the int32 sums of the int8-core paths (1024 * 8 * K for INT4 nibbles, 64 * 127 * K for INT8)
    and the fp32 sums of the FP6 / FP4 paths stay exact, and the outputs equal the oracle's."""
    torch = torch_cuda()
    K, N = MAXK, 16
    M = 8 if kind == "gemv" else 20
    w = -np.ones((N, K), dtype=np.float32)
    t, a = O.ternarize(w, EPS)
    pack = tw.bitlinear_pack_ternary_a8 if fmt == "int8" else tw.bitlinear_pack_ternary
    packed, alpha = pack(torch.from_numpy(w).cuda(), EPS)
    assert alpha.item() == a
    rows, nbytes = tw.codes_shape(fmt, M, K)
    if fmt == "int4_e3m2":
        # E3M2 of -8 is 0b111000; four 6-bit codes fill three bytes (0x38, 0x8E, 0xE3, little endian)
        pat = np.frombuffer(bytes([0x38, 0x8E, 0xE3]) * (rows * nbytes // 3), dtype=np.uint8)
        codes = torch.from_numpy(pat.reshape(rows, nbytes).copy()).cuda()
    else:
        fill = {"int4": 0x88, "fp4": 0xFF, "int8": 0x81}[fmt]      # nibbles -8, E2M1 -6, int8 -127
        codes = torch.full((rows, nbytes), fill, dtype=torch.uint8, device="cuda")
    cval, unit = {"int4": (-8, 1.0), "int4_e3m2": (-8, 1.0), "fp4": (-12, 0.5), "int8": (-127, 1.0)}[fmt]
    scale = torch.ones(M, dtype=torch.float32, device="cuda")
    if kind == "gemm":
        y = tw.bitlinear_gemm_w158a4(fmt, codes, scale, K, packed, alpha, N)
    elif kind == "a8":
        y = tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, alpha, N)
    else:
        y = tw.bitlinear_gemv_decode(fmt, codes, scale, K, packed, alpha, N)
    c = np.full((M, K), cval, dtype=np.int64)
    ref = O.dequant_f32(O.gemm_int(c, t), np.ones(M, dtype=np.float32), a, unit)
    assert float(ref[0, 0]) == -cval * K * unit                    # the sum at the bound, held exactly
    np.testing.assert_array_equal(host(y).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("kind", ["a8", "gemv"])
def test_a8_sums_beyond_float32_integers(kind):
    """INT8 codes near 127 against +1 weights at the longest accepted K: the exact sums (about 3.2e7)
    are mostly not float32 integers, so the epilogue's RN32(acc) really rounds; outputs equal the
    oracle's fixed-order float32 epilogue bit for bit."""
    torch = torch_cuda()
    K, N = MAXK, 16
    M = 8 if kind == "gemv" else 20
    rng = np.random.default_rng(77)
    c = rng.integers(100, 128, (M, K)).astype(np.int8)
    w = np.where(rng.random((N, K)) < 0.1, -1.0, 1.0).astype(np.float32)     # mostly +1: sums near 2.6e7
    t, a = O.ternarize(w, EPS)
    packed, alpha = tw.bitlinear_pack_ternary_a8(torch.from_numpy(w).cuda(), EPS)
    assert alpha.item() == a
    codes = torch.from_numpy(c.view(np.uint8)).cuda()
    d = (rng.random(M) * 0.01 + 1e-3).astype(np.float32)
    scale = dev_f32(d)
    if kind == "a8":
        y = tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, alpha, N)
    else:
        y = tw.bitlinear_gemv_decode("int8", codes, scale, K, packed, alpha, N)
    acc = O.gemm_int(c.astype(np.int64), t)
    assert np.abs(acc).min() > 2 ** 24 and np.mean(acc != acc.astype(np.float32).astype(np.int64)) > 0.25
    assert_y_close(host(y), acc, d, a)
