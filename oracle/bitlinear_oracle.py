"""Plain, slow CPU oracle of the BitNet a4.8 BitLinear hot path (numpy).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library. It shares no code,
table or constant generator with the HIP kernels.

Source: "BitNet a4.8: 4-bit Activations for 1-bit LLMs", architecture
write-up (paper-graph-ui page), section 3.4 "Detailed, Sentence-Based
Technical Breakdown", subsections
  [TW]  "Ternary Weight Quantization (BitLinear)"          -- Q_w, alpha (paper Eq. 2), RoundClip
  [A4]  "4-Bit Activation Quantization for Gaussian-Like Inputs"  -- Y = Q_INT4(X) Q_w(W)^T,
        Q_INT4 and beta (paper Eq. 6-7); FP4 MinMax quantizer, E2M1 (paper Eq. 8-9)
  [SP]  "Sparsification Pipeline for Outlier-Heavy Intermediate States"
        -- Y = (Q_INT8(X) . M) Q_w(W)^T, M = Top_k(|X|) (paper Eq. 1), Q_INT8 and gamma
  [GLU] "Squared ReLU Gating and Conditional Computation in the FFN" -- ReLU^2 GLU (paper Eq. 5)
  [KV]  "Low-Bit KV Cache Quantization" -- post-RoPE absmax quantization of Q, K, V heads to
        unsigned integers, 4-bit and 3-bit, BOS-token heads kept at 4 bits (paper Table 3)
and section 3.2 "Big-Picture Architecture" for which projection gets which
quantizer and where the residual add sits.

Precision. Where a floating-point value decides an integer (a quantized code,
a Top-K survivor) the decision is taken in IEEE binary32 with round-to-nearest-
even, one operation at a time (numpy float32 ufuncs never fuse), which is the
precision of the GPU kernels. Sums that define a scale (alpha, beta) are exact
(math.fsum is correctly rounded) before the single rounding steps stated in
each function. Final outputs that decide nothing are formed in float64 from
exact integer accumulators.

Readings of points the pages leave open (each one is also listed with its
reason in the design notes):
  R1 epsilon is a caller-supplied positive float32 (default 1e-5) for every quantizer.
  R2 round() is round-half-to-even (numpy.rint).
  R3 beta, gamma and the Top-K set are per token (per row of X [M, K]).
  R4 alpha is per tensor; weights use the literal division W / (alpha + eps).
  R5 beta = RN32(RN64(S) / K) with S the exact sum of |x| of the row; the same
     form gives alpha with S over the whole tensor and N*K in place of K.
  R6 FP4: the row max maps to the largest E2M1 magnitude 6 (s = 6 / (gamma+eps));
     each scaled value rounds to the nearest E2M1 value, ties to even mantissa,
     magnitudes above 6 saturate to 6; a zero result is encoded +0.
  R7 Top-K keeps exactly ``keep`` entries, ordered by |x| descending then index
     ascending.
  R8 The mask is taken on |x|; codes of masked-out entries are 0; gamma is the max
     over the whole row (which survives whenever keep >= 1).
  R9 FFN: ReLU^2 acts on the gate projection, h = RN32(RN32(g+ * g+) * u) with
     g, u the fp32 dequantized projections; the down input is INT8 without Top-K.
  R14 Conditional up projection: a channel's up output is computed only when its gate is
     positive in some row; entries with g <= 0 are +0 (the full form gives +0 * u, which is
     -0 when u < 0: equal as numbers).
  R15 FP4 power-of-two scale variant: the dequant scale is 2^p with p the smallest integer such that
     6 * 2^p >= max|x| (p >= -126); codes are the E2M1 rounding of x * 2^-p (exact scaling).
  R16 Per-tensor variant (per_tensor=True): beta or gamma is taken over all M*K entries of X at
     once, in the same form as R5 (K replaced by M*K), and every row is quantized with it; the
     per-row dscale then holds that one value in every row.
  R17 KV cache: absmax per (token, head) over the head's D values, symmetric, Qp = 2^(b-1) - 1
     (7 for 4 bits, 3 for 3 bits): c = RoundClip(RN32(x * RN32(Qp / RN32(gamma + eps))), -Qp-1, Qp),
     stored unsigned as u = c + 2^(b-1); dequant scale RN32(gamma / Qp). RoPE is the rotate-half
     form on (x_i, x_{i+D/2}) with caller cos/sin tables, each product and sum rounded to fp32.
     BOS tokens (marked by the caller) get a 4-bit record beside the 3-bit one.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

F32 = np.float32

# RN32(sqrt(7)); checked against exact rational bounds by the oracle's tests.
SQRT7_F32 = F32(math.sqrt(7.0))

# E2M1 magnitudes in code order 0..7 (1 sign, 2 exponent bits with bias 1, 1 mantissa bit).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


# --------------------------------------------------------------------------- helpers
def roundclip(x, a, b):
    """RoundClip(x, a, b) = min(max(round(x), a), b) with round half to even. [TW]"""
    return np.minimum(np.maximum(np.rint(x), a), b)


def exact_abs_sum(values) -> float:
    """RN64 of the exact sum of |values| (math.fsum is correctly rounded).

    Streams in chunks so that tensors of tens of millions of entries fit in memory.
    """
    flat = np.abs(np.asarray(values, dtype=np.float64)).ravel()
    chunks = (flat[i:i + (1 << 20)].tolist() for i in range(0, flat.size, 1 << 20))
    return math.fsum(itertools.chain.from_iterable(chunks))


def _rows_f32(x):
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("activations must be [M, K]")
    return x


# --------------------------------------------------------------------------- weights
def ternarize(w, eps: float = 1e-5):
    """Q_w(W) = alpha * RoundClip(W / (alpha + eps), -1, 1), alpha = mean(|W|). [TW], Eq. 2

    Returns (codes int8 [N, K] in {-1, 0, 1}, alpha float32). The dequantized
    weight is alpha * code (alpha, not alpha + eps).
    """
    w = np.asarray(w, dtype=np.float32)
    S = exact_abs_sum(w)
    alpha = F32(S / w.size)                      # R5
    den = F32(alpha + F32(eps))                  # R4: literal division by alpha + eps
    q = w / den                                  # float32 IEEE division per element
    codes = roundclip(q, -1, 1).astype(np.int8)
    return codes, alpha


# --------------------------------------------------------------------------- activations
def quant_int4(x, eps: float = 1e-5, per_tensor: bool = False):
    """Per-token Q_INT4: codes = RoundClip(sqrt7/(beta+eps) * x, -8, 7), beta = mean|x|. [A4], Eq. 6-7

    per_tensor: beta is the mean over the whole tensor (R16).
    Returns (codes int8 [M, K] in [-8, 7], dscale float32 [M] = beta / sqrt7, beta float32 [M]).
    """
    x = _rows_f32(x)
    M, K = x.shape
    if per_tensor:
        beta = np.full(M, F32(exact_abs_sum(x.ravel()) / (M * K)), dtype=np.float32)
    else:
        beta = np.array([F32(exact_abs_sum(x[m]) / K) for m in range(M)], dtype=np.float32)
    den = (beta + F32(eps)).astype(np.float32)
    s = (SQRT7_F32 / den).astype(np.float32)
    v = (x * s[:, None]).astype(np.float32)
    codes = roundclip(v, -8, 7).astype(np.int8)
    dscale = (beta / SQRT7_F32).astype(np.float32)
    return codes, dscale, beta


def e2m1_round(mag):
    """Nearest E2M1 magnitude index (0..7) of non-negative values, ties to even mantissa,
    saturating at 6. [A4] FP4 quantizer, E2M1 format (R6)."""
    mag = np.asarray(mag, dtype=np.float64)
    mids = (E2M1_GRID[:-1] + E2M1_GRID[1:]) / 2.0          # 0.25 0.75 1.25 1.75 2.5 3.5 5
    idx = np.searchsorted(mids, mag, side="left")           # number of midpoints < mag
    tie = (idx < 7) & (mag == mids[np.minimum(idx, 6)])
    idx = np.where(tie & (idx % 2 == 1), idx + 1, idx)      # tie: pick the even (mantissa 0) neighbour
    return idx.astype(np.int64)


def fp4_pow2_exponent(gamma):
    """Reading R15 of the FP4 scale: the smallest integer p with 6 * 2^p >= gamma, at least -126
    (gamma > 0). [A4], Eq. 8-9 read with a power-of-two dynamic scale."""
    g = np.asarray(gamma, dtype=np.float64)
    frac, e2 = np.frexp(g)                       # g = frac * 2^e2, frac in [0.5, 1)
    e = e2 - 1                                   # g = (2 frac) * 2^e, 2 frac in [1, 2)
    p = np.where(2.0 * frac <= 1.5, e - 2, e - 1)
    return np.maximum(p, -126).astype(np.int64)


def quant_fp4(x, eps: float = 1e-5, pow2: bool = False, per_tensor: bool = False):
    """Per-token FP4 (E2M1) MinMax quantizer. [A4], Eq. 8-9, reading R6 (pow2: reading R15;
    per_tensor: gamma over the whole tensor, R16).

    Returns (nibbles uint8 [M, K] = sign<<3 | magnitude index,
             doubled codes int8 [M, K] = 2 * E2M1 value in {0, +-1, +-2, +-3, +-4, +-6, +-8, +-12},
             dscale float32 [M] = gamma / 6 (pow2: 2^p, 0 for a zero row), gamma float32 [M]).
    """
    x = _rows_f32(x)
    gamma = np.max(np.abs(x), axis=1).astype(np.float32)
    if per_tensor:
        gamma = np.full(x.shape[0], np.max(np.abs(x)) if x.size else 0.0, dtype=np.float32)
    if pow2:
        p = fp4_pow2_exponent(gamma)
        zero = gamma == 0
        s = np.where(zero, 0.0, np.ldexp(1.0, -p)).astype(np.float32)
        dscale_p = np.where(zero, 0.0, np.ldexp(1.0, p)).astype(np.float32)
    else:
        den = (gamma + F32(eps)).astype(np.float32)
        s = (F32(6.0) / den).astype(np.float32)
    v = (x * s[:, None]).astype(np.float32)
    idx = e2m1_round(np.abs(v))
    neg = (v < 0) & (idx > 0)
    nibbles = (idx | (neg.astype(np.int64) << 3)).astype(np.uint8)
    doubled = (2.0 * E2M1_GRID[idx]).astype(np.int64)
    doubled = np.where(neg, -doubled, doubled).astype(np.int8)
    dscale = dscale_p if pow2 else (gamma / F32(6.0)).astype(np.float32)
    return nibbles, doubled, dscale, gamma


def topk_mask(x, keep: int):
    """M = Top_k(|X|) per token: keep exactly ``keep`` entries, |x| descending, index ascending. [SP], Eq. 1 (R7)"""
    x = _rows_f32(x)
    M, K = x.shape
    if not 0 <= keep <= K:
        raise ValueError("keep out of range")
    mask = np.zeros((M, K), dtype=bool)
    a = np.abs(x)
    for m in range(M):
        order = np.argsort(-a[m], kind="stable")     # stable: equal |x| stay in index order
        mask[m, order[:keep]] = True
    return mask


def quant_int8(x, eps: float = 1e-5, keep: int | None = None, per_tensor: bool = False):
    """Q_INT8(X) (.) M per token: codes = RoundClip(127/(gamma+eps) * x, -128, 127), gamma = max|x|. [SP]

    ``keep`` None (or K) means no Top-K mask; per_tensor: gamma over the whole tensor (R16, no
    Top-K). Returns (codes int8 [M, K], mask bool [M, K], dscale float32 [M] = gamma / 127,
    gamma float32 [M]).
    """
    x = _rows_f32(x)
    M, K = x.shape
    if per_tensor and keep is not None and keep != K:
        raise ValueError("the per-tensor variant has no Top-K mask")
    mask = np.ones((M, K), dtype=bool) if keep is None or keep == K else topk_mask(x, keep)
    gamma = np.max(np.abs(x), axis=1).astype(np.float32) if K else np.zeros(M, np.float32)
    if per_tensor:
        gamma = np.full(M, np.max(np.abs(x)) if x.size else 0.0, dtype=np.float32)
    den = (gamma + F32(eps)).astype(np.float32)
    s = (F32(127.0) / den).astype(np.float32)
    v = (x * s[:, None]).astype(np.float32)
    codes = roundclip(v, -128, 127).astype(np.int8)
    codes = np.where(mask, codes, 0).astype(np.int8)
    dscale = (gamma / F32(127.0)).astype(np.float32)
    return codes, mask, dscale, gamma


# --------------------------------------------------------------------------- matmul + epilogues
def gemm_int(a_codes, w_codes):
    """acc[m, n] = sum_k a[m, k] * t[n, k] exactly (int64). Y = Q(X) Q_w(W)^T without scales. [A4], [SP]

    Integer-valued float64 operands make every product and partial sum exact
    (all magnitudes stay far below 2^53), so a BLAS matmul serves as the sum.
    """
    a = np.asarray(a_codes, dtype=np.float64)
    t = np.asarray(w_codes, dtype=np.float64)
    if a.shape[1] != t.shape[1]:
        raise ValueError("K mismatch")
    acc = a @ t.T
    bound = np.abs(a).max(initial=0) * a.shape[1]
    assert bound < 2 ** 31, "int32 accumulator bound exceeded"
    return np.rint(acc).astype(np.int64)


def dequant(acc, dscale, alpha, acc_unit: float = 1.0):
    """Y = acc * acc_unit * dscale[m] * alpha in float64 (acc_unit = 0.5 for doubled FP4 codes)."""
    acc = np.asarray(acc, dtype=np.float64)
    sc = np.asarray(dscale, dtype=np.float64)[:, None] * np.float64(alpha)
    return acc * acc_unit * sc


def dequant_f32(acc, dscale, alpha, acc_unit: float = 1.0):
    """float32 dequantization in a fixed order: RN32(RN32(acc * acc_unit) * RN32(dscale * alpha)).

    Reading R10 of Y = Q(X) Q_w(W)^T ([A4], [SP]): the integer sum is scaled by the product of the
    two scales, each step one IEEE binary32 rounding. Used where the result decides later codes
    (the ReLU^2 GLU intermediate) and as the bit pattern the GPU outputs are graded against.
    RN32(acc) is exact for |acc| <= 2^24 (INT4 and FP4 sums always are); INT8 sums at long K
    (127 K up to 3.3e7) can exceed it and are then rounded to nearest even, like the kernels'
    int32 -> float32 conversion. acc_unit is 1 or 0.5, so the scaling by it is exact.
    """
    sc = (np.asarray(dscale, dtype=np.float32) * F32(alpha)).astype(np.float32)
    a = (np.asarray(acc).astype(np.float32) * F32(acc_unit)).astype(np.float32)
    return (a * sc[:, None]).astype(np.float32)


def relu2_glu(g, u):
    """ReLU^2 GLU: h = ReLU(g)^2 * u, as RN32(RN32(g+ * g+) * u). [GLU], Eq. 5 (R9)"""
    g = np.asarray(g, dtype=np.float32)
    u = np.asarray(u, dtype=np.float32)
    gp = np.where(g > 0, g, F32(0.0)).astype(np.float32)
    return ((gp * gp).astype(np.float32) * u).astype(np.float32)


def relu2_glu_conditional(g, u_fn):
    """Conditional up projection of [GLU] (R14): the up projection is evaluated only for channels
    whose gate is positive in some row; h = RN32(RN32(g * g) * u) where g > 0 and +0 elsewhere.

    u_fn(cols) returns the dequantized up projection for the given column indices only (so the
    reference, like the method, never forms u for a channel whose gate is non-positive in every
    row). Returns (h, live_columns).
    """
    g = np.asarray(g, dtype=np.float32)
    live = np.flatnonzero(np.any(g > 0, axis=0))
    h = np.zeros(g.shape, dtype=np.float32)
    if live.size:
        gl = g[:, live]
        ul = np.asarray(u_fn(live), dtype=np.float32)
        hl = ((gl * gl).astype(np.float32) * ul).astype(np.float32)
        h[:, live] = np.where(gl > 0, hl, F32(0.0))
    return h, live


def ffn_gate_up_conditional_ref(x, wg_codes, alpha_g, wu_codes, alpha_u, eps: float = 1e-5):
    """Decode FFN front half with conditional computation: INT4 input -> gate projection g, then
    the up projection only on the channels where some row of g is positive. [A4], [GLU]"""
    codes, dscale, _ = quant_int4(x, eps)
    acc_g = gemm_int(codes, wg_codes)
    g = dequant_f32(acc_g, dscale, alpha_g)
    wu = np.asarray(wu_codes)

    def u_fn(cols):
        return dequant_f32(gemm_int(codes, wu[cols]), dscale, alpha_u)

    h, live = relu2_glu_conditional(g, u_fn)
    return dict(codes=codes, dscale=dscale, g=g, h=h, live=live,
                h_absmax=np.max(np.abs(h), axis=1).astype(np.float32))


# --------------------------------------------------------------------------- end-to-end
def bitlinear_a4(x, w_codes, alpha, eps: float = 1e-5, fmt: str = "int4"):
    """Y = Q_4bit(X) Q_w(W)^T with a per-token 4-bit quantizer (INT4 absmean or FP4 MinMax). [A4]

    Returns a dict with codes, dscale, acc (int64) and y (float64).
    """
    if fmt == "int4":
        codes, dscale, _ = quant_int4(x, eps)
        acc = gemm_int(codes, w_codes)
        y = dequant(acc, dscale, alpha)
        return dict(codes=codes, dscale=dscale, acc=acc, y=y)
    if fmt in ("fp4", "fp4_pow2"):
        nib, doubled, dscale, _ = quant_fp4(x, eps, pow2=fmt == "fp4_pow2")
        acc = gemm_int(doubled, w_codes)          # doubled codes: acc counts half units
        y = dequant(acc, dscale, alpha, acc_unit=0.5)
        return dict(nibbles=nib, codes=doubled, dscale=dscale, acc=acc, y=y)
    raise ValueError(fmt)


def bitlinear_a8(x, w_codes, alpha, eps: float = 1e-5, keep: int | None = None, residual=None):
    """Y = (Q_INT8(X) (.) M) Q_w(W)^T (+ residual). [SP], Eq. 1; residual add per section 3.2."""
    codes, mask, dscale, _ = quant_int8(x, eps, keep)
    acc = gemm_int(codes, w_codes)
    y = dequant(acc, dscale, alpha)
    if residual is not None:
        y = y + np.asarray(residual, dtype=np.float64)
    return dict(codes=codes, mask=mask, dscale=dscale, acc=acc, y=y)


def ffn_ref(x, wg_codes, alpha_g, wu_codes, alpha_u, wd_codes, alpha_d, eps: float = 1e-5):
    """FFN of section 3.2: INT4 input -> gate, up -> ReLU^2 GLU -> INT8 (no Top-K) -> down. [A4], [GLU], [SP]"""
    codes, dscale, _ = quant_int4(x, eps)
    acc_g = gemm_int(codes, wg_codes)
    acc_u = gemm_int(codes, wu_codes)
    g = dequant_f32(acc_g, dscale, alpha_g)
    u = dequant_f32(acc_u, dscale, alpha_u)
    h = relu2_glu(g, u)
    h_absmax = np.max(np.abs(h), axis=1).astype(np.float32)
    hc, _, hd, _ = quant_int8(h, eps)
    acc_d = gemm_int(hc, wd_codes)
    y = dequant(acc_d, hd, alpha_d)
    return dict(codes=codes, dscale=dscale, acc_g=acc_g, acc_u=acc_u, h=h, h_absmax=h_absmax,
                h_codes=hc, h_dscale=hd, acc_d=acc_d, y=y)


def oproj_ref(x, w_codes, alpha, residual, keep: int, eps: float = 1e-5):
    """Attention output projection: Top-K + INT8, o_proj, residual add. [SP], section 3.2"""
    return bitlinear_a8(x, w_codes, alpha, eps, keep=keep, residual=residual)


# --------------------------------------------------------------------------- KV cache
def rope_rotate_half(x, pos, cos, sin):
    """Rotary position embedding on [T, H, D] heads, rotate-half pairing (i, i + D/2), i < D/2:
    out_i = RN32(RN32(x_i c) - RN32(x_j s)), out_j = RN32(RN32(x_j c) + RN32(x_i s)), j = i + D/2,
    c = cos[pos[t], i], s = sin[pos[t], i] from caller tables [P, D/2]. [KV] (applied before the
    quantizer, "post-RoPE"; R17)"""
    x = np.asarray(x, dtype=np.float32)
    T, H, D = x.shape
    h = D // 2
    c = np.asarray(cos, dtype=np.float32)[np.asarray(pos)][:, None, :]     # [T, 1, D/2]
    s = np.asarray(sin, dtype=np.float32)[np.asarray(pos)][:, None, :]
    a, b = x[..., :h], x[..., h:]
    out = np.empty_like(x)
    out[..., :h] = ((a * c).astype(np.float32) - (b * s).astype(np.float32)).astype(np.float32)
    out[..., h:] = ((b * c).astype(np.float32) + (a * s).astype(np.float32)).astype(np.float32)
    return out


def kv_quant(x, bits: int, eps: float = 1e-5):
    """Absmax quantization of each (token, head) of x [T, H, D] to ``bits``-bit unsigned codes. [KV], R17

    Returns (u uint8 [T, H, D] in [0, 2^bits - 1], dscale float32 [T, H] = gamma / Qp,
    gamma float32 [T, H]); the value of a code is (u - 2^(bits-1)) * dscale.
    """
    if bits not in (3, 4):
        raise ValueError("bits must be 3 or 4")
    x = np.asarray(x, dtype=np.float32)
    qp = F32(2 ** (bits - 1) - 1)
    gamma = np.max(np.abs(x), axis=2).astype(np.float32)
    den = (gamma + F32(eps)).astype(np.float32)
    s = (qp / den).astype(np.float32)
    v = (x * s[..., None]).astype(np.float32)
    c = roundclip(v, -int(qp) - 1, int(qp)).astype(np.int16)
    u = (c + 2 ** (bits - 1)).astype(np.uint8)
    dscale = (gamma / qp).astype(np.float32)
    return u, dscale, gamma


def kv_cache_quant(x, bits: int, eps: float = 1e-5, pos=None, cos=None, sin=None, bos=None):
    """KV-cache write of T tokens: optional RoPE, then ``bits``-bit absmax codes per (token, head);
    with bits == 3, tokens flagged in ``bos`` (bool [T]) also get 4-bit codes. [KV], R17

    Returns dict(u, dscale, bos_u, bos_dscale) with bos_* = None unless bits == 3 and bos is given
    (rows of non-BOS tokens there are undefined: filled with 0).
    """
    x = np.asarray(x, dtype=np.float32)
    if cos is not None:
        x = rope_rotate_half(x, pos, cos, sin)
    u, d, _ = kv_quant(x, bits, eps)
    out = dict(u=u, dscale=d, bos_u=None, bos_dscale=None)
    if bits == 3 and bos is not None:
        bos = np.asarray(bos, dtype=bool)
        u4, d4, _ = kv_quant(x, 4, eps)
        out["bos_u"] = np.where(bos[:, None, None], u4, 0).astype(np.uint8)
        out["bos_dscale"] = np.where(bos[:, None], d4, 0).astype(np.float32)
    return out
