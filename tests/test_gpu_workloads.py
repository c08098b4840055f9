"""GPU parity at the full sizes of the five synthetic workloads, in the launch configuration the
benchmark times. The GPU computes every row; the oracle recomputes a seeded sample of rows (every
step of the path is row-local, and the weights' alpha and codes are recomputed in full).
"""
import numpy as np
import pytest

import oracle as O
import ternary_weight_quantized_amd as tw
from synth import WORKLOADS, bf16_bits_to_f32, workload_inputs
from tests.gpu_util import (assert_y_close, dev_bf16, dev_f32, e3m2_values, host, int4_values, int8_values,
                            mask_bits, nibbles, torch_cuda)
from tests.packed_layout import unpack_ternary

pytestmark = pytest.mark.gpu

EPS = 1e-5


def sample_rows(M, n=256, seed=0, tile=128):
    """A seeded sample of at least min(n, M) rows: one random row in every 128-row tile of the GEMMs'
    blocks (the ragged last tile included), n random rows, and the first and last row."""
    rng = np.random.default_rng(seed)
    per_tile = [t * tile + int(rng.integers(0, min(tile, M - t * tile))) for t in range((M + tile - 1) // tile)]
    rows = set(per_tile) | set(rng.choice(M, size=min(n, M), replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(rows))


def weights(w, a8=False):
    """The oracle's codes and alpha, and the library's packed weights (a8: the layout of the matmuls
    with INT8 activations)."""
    codes, alpha = O.ternarize(w, EPS)
    packed, a = (tw.bitlinear_pack_ternary_a8 if a8 else tw.bitlinear_pack_ternary)(dev_f32(w), EPS)
    assert host(a)[0] == alpha
    return codes, alpha, packed, a


def test_tiny_a4_full():
    torch_cuda()
    wl = WORKLOADS["tiny_a4"]
    inp = workload_inputs("tiny_a4")
    K, N = wl["K"], wl["N"]
    t, alpha, packed, a = weights(inp["w"])
    np.testing.assert_array_equal(unpack_ternary(host(packed), N, K), t)
    codes, scale, _ = tw.bitlinear_quantize_act(dev_bf16(inp["x"]), "int4", eps=EPS)
    y = tw.bitlinear_gemm_w158a4("int4", codes, scale, K, packed, a, N)
    ref = O.bitlinear_a4(bf16_bits_to_f32(inp["x"]), t, alpha, EPS)
    np.testing.assert_array_equal(int4_values(host(codes)), ref["codes"])
    assert_y_close(host(y), ref["acc"], ref["dscale"], alpha)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_decode_a4_full(M):
    torch_cuda()
    wl = WORKLOADS["decode_a4"]
    inp = workload_inputs("decode_a4")
    K, N = wl["K"], wl["N"]
    t, alpha, packed, a = weights(inp["w"])
    xb = inp["x"][:M]
    codes, scale, _ = tw.bitlinear_quantize_act(dev_bf16(xb), "int4", eps=EPS)
    y = tw.bitlinear_gemv_decode("int4", codes, scale, K, packed, a, N)
    ref = O.bitlinear_a4(bf16_bits_to_f32(xb), t, alpha, EPS)
    assert_y_close(host(y), ref["acc"], ref["dscale"], alpha)


@pytest.mark.parametrize("fmt", ["int4", "int4_e3m2", "fp4"])
def test_prefill_qkv_sampled(fmt):
    torch_cuda()
    wl = WORKLOADS["prefill_qkv"]
    inp = workload_inputs("prefill_qkv")
    M, K, N = wl["M"], wl["K"], wl["N"]
    t, alpha, packed, a = weights(inp["w"])
    codes, scale, _ = tw.bitlinear_quantize_act(dev_bf16(inp["x"]), fmt, eps=EPS)
    y = tw.bitlinear_gemm_w158a4(fmt, codes, scale, K, packed, a, N)
    rows = sample_rows(M, seed=3)
    xs = bf16_bits_to_f32(inp["x"][rows])
    ref = O.bitlinear_a4(xs, t, alpha, EPS, fmt="fp4" if fmt == "fp4" else "int4")
    if fmt == "int4":
        np.testing.assert_array_equal(int4_values(host(codes)[rows]), ref["codes"])
    elif fmt == "int4_e3m2":
        np.testing.assert_array_equal(e3m2_values(host(codes), M)[rows], ref["codes"])
    else:
        np.testing.assert_array_equal(nibbles(host(codes)[rows]), ref["nibbles"])
    np.testing.assert_array_equal(host(scale)[rows], ref["dscale"])
    assert_y_close(host(y)[rows], ref["acc"], ref["dscale"], alpha, 0.5 if fmt == "fp4" else 1.0)


@pytest.mark.parametrize("fmt", ["int4", "fp4_pow2"])
def test_prefill_scale_variants_sampled(fmt):
    """The prefill activations with one scale for the whole 4096 x 4096 tensor (INT4) and with the
    power-of-two FP4 scale, in the launch configuration the benchmark times; the per-tensor beta
    comes from the exact sum over all 16.8M entries, the codes are compared on sampled rows."""
    torch = torch_cuda()
    wl = WORKLOADS["prefill_qkv"]
    inp = workload_inputs("prefill_qkv")
    M, K = wl["M"], wl["K"]
    x = dev_bf16(inp["x"])
    rows = sample_rows(M, seed=5)
    xf = bf16_bits_to_f32(inp["x"])
    if fmt == "int4":
        ws = torch.empty(tw.bitlinear_quantize_per_tensor_workspace_bytes(M), dtype=torch.uint8, device="cuda")
        codes, scale = tw.bitlinear_quantize_act_per_tensor(x, "int4", eps=EPS, workspace=ws)
        c, d, _ = O.quant_int4(xf, EPS, per_tensor=True)
        np.testing.assert_array_equal(int4_values(host(codes)[rows]), c[rows])
        np.testing.assert_array_equal(host(scale), d)
    else:
        codes, scale, _ = tw.bitlinear_quantize_act(x, "fp4_pow2", eps=EPS)
        nib, _, d, _ = O.quant_fp4(xf[rows], EPS, pow2=True)
        np.testing.assert_array_equal(nibbles(host(codes)[rows]), nib)
        np.testing.assert_array_equal(host(scale)[rows], d)


def test_ffn_7b_sampled():
    torch = torch_cuda()
    wl = WORKLOADS["ffn_7b"]
    inp = workload_inputs("ffn_7b")
    M, K, N = wl["M"], wl["K"], wl["N"]
    tg, ag, pg, dag = weights(inp["w_gate"])
    tu, au, pu, dau = weights(inp["w_up"])
    td, ad, pd, dad = weights(inp["w_down"], a8=True)
    codes, scale, _ = tw.bitlinear_quantize_act(dev_bf16(inp["x"]), "int4_e3m2", eps=EPS)
    rowmax = torch.empty(M, dtype=torch.float32, device="cuda")
    h = tw.bitlinear_gemm_w158a4("int4_e3m2", codes, scale, K, pg, dag, N, up_packed=pu, up_alpha=dau,
                                 row_absmax=rowmax)
    hc, hs, _ = tw.bitlinear_quantize_act(h, "int8", eps=EPS, row_absmax_hint=rowmax)
    y = tw.bitlinear_gemm_w158a8_sparse(hc, hs, N, pd, dad, K)
    rows = sample_rows(M, seed=4)
    ref = O.ffn_ref(bf16_bits_to_f32(inp["x"][rows]), tg, ag, tu, au, td, ad, EPS)
    np.testing.assert_array_equal(host(h)[rows].view(np.uint32), ref["h"].view(np.uint32))
    np.testing.assert_array_equal(host(rowmax)[rows], ref["h_absmax"])
    np.testing.assert_array_equal(int8_values(host(hc)[rows]), ref["h_codes"])
    np.testing.assert_array_equal(host(hs)[rows], ref["h_dscale"])
    assert_y_close(host(y)[rows], ref["acc_d"], ref["h_dscale"], ad)
    hz = float((host(h) == 0).mean())
    cz = float((int8_values(host(hc)) == 0).mean())
    print(f"ffn_7b: h exact zeros {hz:.3f}, INT8 zero codes {cz:.3f}")
    assert 0.45 < hz < 0.55                       # ReLU^2 zeroes the non-positive gate half


@pytest.mark.parametrize("M", [1, 8])
def test_decode_a8_ffn_full(M):
    """Decode FFN of the first M tokens of the 7B FFN workload as the benchmark runs it: the fused
    ReLU^2 GLU decode product of their INT4 codes (with row maxima), INT8 codes of h, and the INT8
    down-projection decode product; every output against the oracle."""
    torch = torch_cuda()
    wl = WORKLOADS["ffn_7b"]
    inp = workload_inputs("ffn_7b")
    K, N = wl["K"], wl["N"]
    tg, ag, pg, dag = weights(inp["w_gate"])
    tu, au, pu, dau = weights(inp["w_up"])
    td, ad, pd, dad = weights(inp["w_down"], a8=True)
    xb = inp["x"][:M]
    codes, scale, _ = tw.bitlinear_quantize_act(dev_bf16(xb), "int4", eps=EPS)
    rowmax = torch.zeros(M, dtype=torch.float32, device="cuda")
    h = tw.bitlinear_gemv_decode("int4", codes, scale, K, pg, dag, N, up_packed=pu, up_alpha=dau, row_absmax=rowmax)
    hc, hs, _ = tw.bitlinear_quantize_act(h, "int8", eps=EPS, row_absmax_hint=rowmax)
    y = tw.bitlinear_gemv_decode("int8", hc, hs, N, pd, dad, K)
    ref = O.ffn_ref(bf16_bits_to_f32(xb), tg, ag, tu, au, td, ad, EPS)
    np.testing.assert_array_equal(host(h).view(np.uint32), ref["h"].view(np.uint32))
    np.testing.assert_array_equal(host(rowmax), ref["h_absmax"])
    np.testing.assert_array_equal(int8_values(host(hc)), ref["h_codes"])
    np.testing.assert_array_equal(host(hs), ref["h_dscale"])
    assert_y_close(host(y), ref["acc_d"], ref["h_dscale"], ad)


def test_attn_out_sampled():
    torch_cuda()
    wl = WORKLOADS["attn_out"]
    inp = workload_inputs("attn_out")
    M, K, N, keep = wl["M"], wl["K"], wl["N"], wl["keep"]
    t, alpha, packed, a = weights(inp["w"], a8=True)
    codes, scale, mask = tw.bitlinear_quantize_act(dev_bf16(inp["x"]), "int8", topk_keep=keep, eps=EPS,
                                                   want_mask=True)
    r = dev_f32(inp["residual"])
    y = tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, a, N, residual=r)
    rows = sample_rows(M, seed=5)
    ref = O.oproj_ref(bf16_bits_to_f32(inp["x"][rows]), t, alpha, inp["residual"][rows], keep, EPS)
    np.testing.assert_array_equal(mask_bits(host(mask)[rows], K), ref["mask"])
    np.testing.assert_array_equal(int8_values(host(codes)[rows]), ref["codes"])
    np.testing.assert_array_equal(host(scale)[rows], ref["dscale"])
    assert_y_close(host(y)[rows], ref["acc"], ref["dscale"], alpha, residual=inp["residual"][rows])
    assert np.all(mask_bits(host(mask), K).sum(axis=1) == keep)


@pytest.mark.parametrize("M", [1, 8])
def test_decode_glu_conditional_full(M):
    """Decode FFN front half at the 7B shape (K=4096, N=11008) with the conditional up projection."""
    torch = torch_cuda()
    F = WORKLOADS["ffn_7b"]
    inp = workload_inputs("ffn_7b")
    K, N = F["K"], F["N"]
    xb = workload_inputs("decode_a4")["x"][:M]
    tg, ag, pg, dag = weights(inp["w_gate"])
    tu, au = O.ternarize(inp["w_up"], EPS)
    pu_rows, dau = tw.bitlinear_pack_ternary_rows(dev_f32(inp["w_up"]), EPS)
    codes, scale, _ = tw.bitlinear_quantize_act(dev_bf16(xb), "int4", eps=EPS)
    rowmax = torch.empty(M, dtype=torch.float32, device="cuda")
    gate, h = tw.bitlinear_gemv_decode_glu_conditional(codes, scale, K, pg, dag, pu_rows, dau, N, row_absmax=rowmax)
    r = O.ffn_gate_up_conditional_ref(bf16_bits_to_f32(xb), tg, ag, tu, au, EPS)
    np.testing.assert_array_equal(host(gate).view(np.uint32), r["g"].view(np.uint32))
    np.testing.assert_array_equal(host(h).view(np.uint32), r["h"].view(np.uint32))
    np.testing.assert_array_equal(host(rowmax), r["h_absmax"])
    print(f"decode glu conditional M={M}: live up rows {r['live'].size / N:.3f}")


@pytest.mark.parametrize("fmt", ["int4_e3m2", "int4", "fp4"])
def test_largest_index_space_sampled(fmt):
    """The largest M the 2^31-element limits allow at K = 256 (M*K and M*N just below 2^31): 64-bit
    row offsets in the quantizer, the E3M2 tiles and the GEMM epilogue; sampled rows, including the
    last one, against the oracle."""
    torch = torch_cuda()
    from synth import latent_weights
    K, N = 256, 240
    M = ((1 << 31) - 1) // K                     # 8388607 rows: M*K = 2^31 - 256, M*N = 2013265680
    gen = torch.Generator(device="cuda").manual_seed(1234)
    x = torch.randn((M, K), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    t, alpha, packed, a = weights(latent_weights(77, N, K))
    codes, scale, _ = tw.bitlinear_quantize_act(x, fmt, eps=EPS)
    y = tw.bitlinear_gemm_w158a4(fmt, codes, scale, K, packed, a, N)
    torch.cuda.synchronize()
    rows = sample_rows(M, n=64, seed=11, tile=1 << 16)
    rows_t = torch.from_numpy(rows).cuda()
    xs = x[rows_t].float().cpu().numpy()
    ref = O.bitlinear_a4(xs, t, alpha, EPS, fmt="fp4" if fmt == "fp4" else "int4")
    np.testing.assert_array_equal(scale[rows_t].cpu().numpy(), ref["dscale"])
    assert_y_close(y[rows_t].cpu().numpy(), ref["acc"], ref["dscale"], alpha, 0.5 if fmt == "fp4" else 1.0)
    del x, codes, scale, y
    torch.cuda.empty_cache()


def test_largest_index_space_topk_a8_sampled():
    """Top-K INT8 quantization and the A8 GEMM with residual at M*K and M*N just below 2^31 (bf16
    rows of 4096, keep 2048): sampled rows, including the last one, against the oracle."""
    torch = torch_cuda()
    from synth import latent_weights
    K, N, keep = 4096, 4096, 2048
    M = ((1 << 31) - 1) // K                     # 524287 rows
    gen = torch.Generator(device="cuda").manual_seed(4321)
    x = torch.randn((M, K), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
    r = torch.randn((M, N), generator=gen, device="cuda", dtype=torch.float32)
    t, alpha, packed, a = weights(latent_weights(78, N, K), a8=True)
    codes, scale, mask = tw.bitlinear_quantize_act(x, "int8", topk_keep=keep, eps=EPS, want_mask=True)
    y = tw.bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, a, N, residual=r)
    torch.cuda.synchronize()
    rows = sample_rows(M, n=64, seed=12, tile=1 << 16)
    rows_t = torch.from_numpy(rows).cuda()
    res = r[rows_t].cpu().numpy()
    ref = O.oproj_ref(x[rows_t].float().cpu().numpy(), t, alpha, res, keep, EPS)
    np.testing.assert_array_equal(mask_bits(mask[rows_t].cpu().numpy(), K), ref["mask"])
    np.testing.assert_array_equal(int8_values(codes[rows_t].cpu().numpy()), ref["codes"])
    np.testing.assert_array_equal(scale[rows_t].cpu().numpy(), ref["dscale"])
    assert_y_close(y[rows_t].cpu().numpy(), ref["acc"], ref["dscale"], alpha, residual=res)
    del x, r, codes, scale, mask, y
    torch.cuda.empty_cache()
