"""The allocation-free per-tensor quantizer (fixed device scratch) against the entry point that takes a
caller workspace: identical codes and scales, on two calls in a row (the second with a smaller input,
so it runs on scratch the first call left behind), through the C ABI.
"""
import numpy as np
import pytest

import ternary_weight_quantized_amd as tw
from synth import activations_bf16, normal
from tests.gpu_util import dev_bf16, dev_f32, host, torch_cuda

pytestmark = pytest.mark.gpu

EPS = 1e-5


@pytest.mark.parametrize("fmt", ["int4", "int4_e3m2", "fp4", "fp4_pow2", "int8"])
def test_noalloc_per_tensor_matches_workspace_entry_point(fmt):
    torch = torch_cuda()
    for seed, (M, K, f32) in enumerate([(4096, 4096, False), (129, 1152, True)]):   # second call smaller
        if f32:
            xh = normal(9100 + seed, M * K).reshape(M, K).astype(np.float32)
            xh[5] *= 1e30                                    # a wide exponent span: the exact-bins path
            x = dev_f32(xh)
        else:
            x = dev_bf16(activations_bf16(9100 + seed, M, K))
        c0, s0 = tw.bitlinear_quantize_act_per_tensor(x, fmt, eps=EPS)
        c1 = torch.full_like(c0, 0x5A)
        s1 = torch.full_like(s0, -1.0)
        c1, s1 = tw.bitlinear_quantize_act_per_tensor_noalloc(x, fmt, eps=EPS, codes=c1, scale=s1)
        torch.cuda.synchronize()
        rows = M if fmt != "int4_e3m2" else M            # E3M2 padding rows are never written: compare rows < M
        a, b = host(c0), host(c1)
        if fmt == "int4_e3m2":
            from tests.gpu_util import e3m2_values
            np.testing.assert_array_equal(e3m2_values(b, M), e3m2_values(a, M))
        else:
            np.testing.assert_array_equal(b[:rows], a[:rows])
        np.testing.assert_array_equal(host(s1), host(s0))


def test_noalloc_rejects_rows_beyond_the_scratch():
    torch = torch_cuda()
    M, K = tw.NOALLOC_MAX_M + 1, 128
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(tw.BitlinearError) as e:
        tw.bitlinear_quantize_act_per_tensor_noalloc(x, "int4", eps=EPS)
    assert e.value.status == 4
    # the largest accepted M runs, and equals the workspace entry point
    M = tw.NOALLOC_MAX_M
    x = dev_bf16(activations_bf16(9300, M, K))
    c0, s0 = tw.bitlinear_quantize_act_per_tensor(x, "int8", eps=EPS)
    c1, s1 = tw.bitlinear_quantize_act_per_tensor_noalloc(x, "int8", eps=EPS)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(c1), host(c0))
    np.testing.assert_array_equal(host(s1), host(s0))
