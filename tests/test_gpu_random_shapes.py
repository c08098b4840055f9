"""GPU parity over seeded random shapes: every entry point through the C ABI against the CPU oracle
on configurations drawn from one fixed generator (rows, columns and reductions of every size the
entry points accept up to a few thousand, ragged in every dimension, all formats and epilogues,
random Top-K keeps, KV heads with and without RoPE and BOS records). The case list is the same on
every run; each test id names its shape. Bars as elsewhere: codes, masks and scales bit-exact,
float32 outputs bit-exact against the oracle's fixed-order float32 epilogue and within 1e-5
relative of the float64 value.
"""
import numpy as np
import pytest

import oracle as O
import ternary_weight_quantized_amd as tw
from synth import latent_weights, normal, rope_tables
from tests.gpu_util import (assert_y_close, dev_f32, e3m2_values, host, int4_values, int8_values, mask_bits, nibbles,
                            torch_cuda, x_f32)
from tests.packed_layout import unpack_kv
from tests.test_gpu_parity import EPS, make_x, packed_weights, to_dev

pytestmark = pytest.mark.gpu

_R = np.random.default_rng(20260601)


def _draw(n, fn):
    return [fn(i) for i in range(n)]


def _keep(K):
    return int(_R.choice([-1, 0, 1, K // 2, int(_R.integers(0, K + 1)), K]))


QCASES = _draw(30, lambda i: (int(_R.integers(1, 260)), 128 * int(_R.integers(1, 140)),
                              str(_R.choice(["int4", "int4_e3m2", "fp4", "fp4_pow2", "int8"])), bool(_R.integers(2))))
QCASES = [(M, K, fmt, f32, _keep(K) if fmt == "int8" else -1) for M, K, fmt, f32 in QCASES]
GCASES = _draw(24, lambda i: (int(_R.integers(1, 600)), 16 * int(_R.integers(1, 64)), 128 * int(_R.integers(1, 32)),
                              str(_R.choice(["int4", "int4_e3m2", "fp4"])), str(_R.choice(["none", "residual", "glu"]))))
A8CASES = _draw(16, lambda i: (int(_R.integers(1, 600)), 16 * int(_R.integers(1, 64)), 128 * int(_R.integers(1, 48)),
                               str(_R.choice(["none", "residual", "glu"]))))
A8CASES = [(M, N, K, epi, _keep(K)) for M, N, K, epi in A8CASES]
DCASES = _draw(20, lambda i: (int(_R.integers(1, 9)), 16 * int(_R.integers(1, 128)), 128 * int(_R.integers(1, 100)),
                              str(_R.choice(["int4", "int8"])), str(_R.choice(["none", "residual", "glu"]))))
CCASES = _draw(8, lambda i: (int(_R.integers(1, 9)), 16 * int(_R.integers(1, 64)), 128 * int(_R.integers(1, 64))))
KCASES = _draw(16, lambda i: (int(_R.integers(1, 200)), int(_R.integers(1, 9)), int(_R.choice([64, 128, 256])),
                              int(_R.choice([3, 4])), bool(_R.integers(2)), bool(_R.integers(2))))


def _id(c):
    return "-".join(str(v) for v in c)


@pytest.mark.parametrize("M,K,fmt,f32,keep", QCASES, ids=[_id(c) for c in QCASES])
def test_random_quantizer(M, K, fmt, f32, keep):
    torch_cuda()
    x = make_x(30000 + M + K, M, K, f32)
    xf = x_f32(x)
    if fmt == "int8":
        codes, scale, mask = tw.bitlinear_quantize_act(to_dev(x), "int8", topk_keep=keep, eps=EPS, want_mask=True)
        c, m, d, _ = O.quant_int8(xf, EPS, None if keep < 0 else keep)
        np.testing.assert_array_equal(mask_bits(host(mask), K), m)
        np.testing.assert_array_equal(int8_values(host(codes)), c)
    else:
        codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), fmt, eps=EPS)
        if fmt in ("int4", "int4_e3m2"):
            c, d, _ = O.quant_int4(xf, EPS)
            got = int4_values(host(codes)) if fmt == "int4" else e3m2_values(host(codes), M)
            np.testing.assert_array_equal(got, c)
        else:
            nib, _, d, _ = O.quant_fp4(xf, EPS, pow2=fmt == "fp4_pow2")
            np.testing.assert_array_equal(nibbles(host(codes)), nib)
    np.testing.assert_array_equal(host(scale), d)


def _quantized(x, fmt, keep=-1):
    codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), fmt, topk_keep=keep, eps=EPS)
    xf = x_f32(x)
    if fmt in ("int4", "int4_e3m2"):
        c, d, _ = O.quant_int4(xf, EPS)
        return codes, scale, c, d, 1.0
    if fmt == "fp4":
        _, c, d, _ = O.quant_fp4(xf, EPS)
        return codes, scale, c, d, 0.5
    c, _, d, _ = O.quant_int8(xf, EPS, None if keep < 0 else keep)
    return codes, scale, c, d, 1.0


def _check_epilogue(call, epi, M, N, K, c, d, unit, t, alpha, seed, a8=False):
    """Run call(**kw) for the epilogue and compare with the oracle."""
    torch = torch_cuda()
    acc = O.gemm_int(c, t)
    if epi == "none":
        assert_y_close(host(call()), acc, d, alpha, unit)
    elif epi == "residual":
        r = normal(seed, M * N).reshape(M, N).astype(np.float32)
        assert_y_close(host(call(residual=dev_f32(r))), acc, d, alpha, unit, residual=r)
    else:
        _, tu, au, pu, dau = packed_weights(seed + 1, N, K, a8=a8)
        rowmax = torch.full((M,), 7.0, dtype=torch.float32, device="cuda")
        h = call(up_packed=pu, up_alpha=dau, row_absmax=rowmax)
        h_ref = O.relu2_glu(O.dequant_f32(acc, d, alpha, unit), O.dequant_f32(O.gemm_int(c, tu), d, au, unit))
        np.testing.assert_array_equal(host(h).view(np.uint32), h_ref.view(np.uint32))
        np.testing.assert_array_equal(host(rowmax), np.abs(h_ref).max(axis=1))


@pytest.mark.parametrize("M,N,K,fmt,epi", GCASES, ids=[_id(c) for c in GCASES])
def test_random_gemm_a4(M, N, K, fmt, epi):
    torch_cuda()
    x = make_x(31000 + M + K, M, K, special=epi != "glu")      # 2^70-scaled rows would overflow g^2
    _, t, alpha, packed, a = packed_weights(31500 + N + K, N, K)
    codes, scale, c, d, unit = _quantized(x, fmt)
    _check_epilogue(lambda **kw: tw.bitlinear_gemm_w158a4(fmt, codes, scale, K, packed, a, N, **kw),
                    epi, M, N, K, c, d, unit, t, alpha, 32000 + M)


@pytest.mark.parametrize("M,N,K,epi,keep", A8CASES, ids=[_id(c) for c in A8CASES])
def test_random_gemm_a8(M, N, K, epi, keep):
    torch_cuda()
    x = make_x(33000 + M + K, M, K, f32=True, special=epi != "glu")
    _, t, alpha, packed, a = packed_weights(33500 + N + K, N, K, a8=True)
    codes, scale, c, d, unit = _quantized(x, "int8", keep)
    _check_epilogue(lambda **kw: tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, a, N, **kw),
                    epi, M, N, K, c, d, unit, t, alpha, 34000 + M, a8=True)


@pytest.mark.parametrize("M,N,K,fmt,epi", DCASES, ids=[_id(c) for c in DCASES])
def test_random_decode(M, N, K, fmt, epi):
    torch_cuda()
    x = make_x(35000 + M + K, M, K, special=False)
    if fmt == "int8":
        x = x_f32(x)
    _, t, alpha, packed, a = packed_weights(35500 + N + K, N, K, a8=fmt == "int8")
    codes, scale, c, d, unit = _quantized(x, fmt)
    _check_epilogue(lambda **kw: tw.bitlinear_gemv_decode(fmt, codes, scale, K, packed, a, N, **kw),
                    epi, M, N, K, c, d, unit, t, alpha, 36000 + M, a8=fmt == "int8")


@pytest.mark.parametrize("M,N,K", CCASES, ids=[_id(c) for c in CCASES])
def test_random_glu_conditional(M, N, K):
    torch = torch_cuda()
    x = make_x(37000 + M + K, M, K, special=False)
    wg = latent_weights(37500 + N, N, K)
    wu = latent_weights(37600 + N, N, K)
    tg, ag = O.ternarize(wg, EPS)
    tu, au = O.ternarize(wu, EPS)
    pg, dag = tw.bitlinear_pack_ternary(dev_f32(wg), EPS)
    pu_rows, dau = tw.bitlinear_pack_ternary_rows(dev_f32(wu), EPS)
    codes, scale, _ = tw.bitlinear_quantize_act(to_dev(x), "int4", eps=EPS)
    rowmax = torch.empty(M, dtype=torch.float32, device="cuda")
    gate, h = tw.bitlinear_gemv_decode_glu_conditional(codes, scale, K, pg, dag, pu_rows, dau, N, row_absmax=rowmax)
    r = O.ffn_gate_up_conditional_ref(x_f32(x), tg, ag, tu, au, EPS)
    np.testing.assert_array_equal(host(gate).view(np.uint32), r["g"].view(np.uint32))
    np.testing.assert_array_equal(host(h).view(np.uint32), r["h"].view(np.uint32))
    np.testing.assert_array_equal(host(rowmax), r["h_absmax"])


@pytest.mark.parametrize("T,H,D,bits,rope,f32", KCASES, ids=[_id(c) for c in KCASES])
def test_random_kv_quantize(T, H, D, bits, rope, f32):
    torch = torch_cuda()
    x = make_x(38000 + T + H + D, T, H * D, f32, special=False)
    xf = x_f32(x)
    rng = np.random.default_rng(38500 + T)
    pos = rng.integers(0, 48, T).astype(np.int32)
    bos = rng.random(T) < 0.2
    slots = np.where(bos, np.cumsum(bos) - 1, -1).astype(np.int32)
    cos, sin = rope_tables(48, D)
    kw = {}
    if rope:
        kw.update(pos=torch.from_numpy(pos).cuda(), cos=dev_f32(cos), sin=dev_f32(sin))
    if bits == 3 and bos.any():                  # BOS records need at least one slot
        kw.update(bos_slot=torch.from_numpy(slots).cuda(), n_bos_slots=int(bos.sum()))
    codes, scale, bcodes, bscale = tw.bitlinear_kv_quantize(to_dev(x), H, D, bits, eps=EPS, **kw)
    torch.cuda.synchronize()
    ref = O.kv_cache_quant(xf.reshape(T, H, D), bits, EPS, pos=pos if rope else None, cos=cos if rope else None,
                           sin=sin if rope else None, bos=bos if bits == 3 else None)
    np.testing.assert_array_equal(unpack_kv(host(codes), H, D, bits), ref["u"])
    np.testing.assert_array_equal(host(scale), ref["dscale"])
    if bits == 3 and bos.any():
        np.testing.assert_array_equal(unpack_kv(host(bcodes), H, D, 4), ref["bos_u"][bos])
        np.testing.assert_array_equal(host(bscale), ref["bos_dscale"][bos])


QKVCASES = _draw(12, lambda i: (int(_R.integers(1, 400)), int(_R.integers(1, 5)), 128 * int(_R.integers(1, 24)),
                                str(_R.choice(["int4_e3m2", "fp4"])),
                                tuple(int(b) for b in _R.choice([3, 4], size=3)), bool(_R.integers(2)),
                                float(_R.choice([0.0, 0.05, 0.3])), bool(_R.integers(2))))


@pytest.mark.parametrize("M,H,K,fmt,bits,rope,p_bos,want_y", QKVCASES, ids=[_id(c) for c in QKVCASES])
def test_random_qkv_kv_fused(M, H, K, fmt, bits, rope, p_bos, want_y):
    """The QKV GEMM with the KV-cache quantizer in its epilogue: records, scales and BOS records equal
    the oracle's (fixed-order fp32 epilogue, then RoPE and absmax codes) and the stand-alone
    quantizer's on the GEMM's output; Y, when written, equals the plain GEMM's."""
    from tests.test_gpu_kvcache import _qkv_case, dev_i32
    torch = torch_cuda()
    rng = np.random.default_rng(39000 + M + K)
    bos_tokens = sorted(set([0] + np.flatnonzero(rng.random(M) < p_bos).tolist())) if p_bos > 0 else []
    c = _qkv_case(39500 + M + H + K, M, H, K, fmt, rope, bos_tokens)
    N = c["N"]
    kw = dict(pos=dev_i32(c["pos"]), cos=dev_f32(c["cos"]), sin=dev_f32(c["sin"])) if rope else {}
    with_bos = bool(bos_tokens) and 3 in bits
    bkw = dict(bos_slot=dev_i32(c["slots"]), n_bos_slots=c["nslots"]) if with_bos else {}
    r = tw.bitlinear_gemm_w158a4_kv(fmt, c["codes"], c["scale"], K, c["packed"], c["a"], N, H, bits=bits, eps=EPS,
                                    want_y=want_y, **kw, **bkw)
    y = tw.bitlinear_gemm_w158a4(fmt, c["codes"], c["scale"], K, c["packed"], c["a"], N)
    torch.cuda.synchronize()
    xf = x_f32(c["xb"])
    if fmt == "fp4":
        ref = O.bitlinear_a4(xf, c["t"], c["alpha"], EPS, fmt="fp4")
        y32 = O.dequant_f32(ref["acc"], ref["dscale"], c["alpha"], 0.5)
    else:
        ref = O.bitlinear_a4(xf, c["t"], c["alpha"], EPS)
        y32 = O.dequant_f32(ref["acc"], ref["dscale"], c["alpha"])
    np.testing.assert_array_equal(host(y).view(np.uint32), y32.view(np.uint32))
    if want_y:
        np.testing.assert_array_equal(host(r["y"]).view(np.uint32), y32.view(np.uint32))
    for p in range(3):
        b = bits[p]
        cols = slice(p * H * 128, (p + 1) * H * 128)
        use_rope = rope and p < 2
        o = O.kv_cache_quant(y32[:, cols].reshape(M, H, 128), b, EPS, pos=c["pos"] if use_rope else None,
                             cos=c["cos"] if use_rope else None, sin=c["sin"] if use_rope else None,
                             bos=c["bos"] if (with_bos and b == 3) else None)
        np.testing.assert_array_equal(unpack_kv(host(r["codes"][p]), H, 128, b), o["u"])
        np.testing.assert_array_equal(host(r["scale"][p]), o["dscale"])
        kc, ks, kbc, kbs = tw.bitlinear_kv_quantize(y[:, cols], H, 128, b, eps=EPS, **(kw if use_rope else {}),
                                                    **(bkw if b == 3 else {}))
        np.testing.assert_array_equal(host(r["codes"][p]), host(kc))
        np.testing.assert_array_equal(host(r["scale"][p]), host(ks))
        if with_bos and b == 3:
            sl = c["slots"][c["bos"]]
            np.testing.assert_array_equal(unpack_kv(host(r["bos_codes"][p]), H, 128, 4)[sl], o["bos_u"][c["bos"]])
            np.testing.assert_array_equal(host(r["bos_scale"][p])[sl], o["bos_dscale"][c["bos"]])
            np.testing.assert_array_equal(host(r["bos_codes"][p]), host(kbc))
            np.testing.assert_array_equal(host(r["bos_scale"][p]), host(kbs))
