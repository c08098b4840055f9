"""Helpers shared by the GPU parity tests: host <-> device marshalling and code-buffer decoding."""
import numpy as np
import pytest

import oracle as O
from synth import bf16_bits_to_f32


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    return torch


def dev_bf16(bits):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_f32(a):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def nibbles(codes_u8):
    """uint8 [M, K/2] -> nibble values uint8 [M, K] (element 2j low nibble, 2j+1 high)."""
    c = np.asarray(codes_u8, dtype=np.uint8)
    out = np.empty((c.shape[0], c.shape[1] * 2), np.uint8)
    out[:, 0::2] = c & 0xF
    out[:, 1::2] = c >> 4
    return out


def int4_values(codes_u8):
    n = nibbles(codes_u8).astype(np.int16)
    return np.where(n >= 8, n - 16, n).astype(np.int8)


def e3m2_values(codes_u8, M=None):
    """Tiled FP6 E3M2 code buffer (16 rows x 128 codes per 1536-byte tile, 96 bytes per row, code k
    at bits [6k, 6k+6) of the row's bytes) -> int8 [M, K].

    Decoded from the format definition (sign, 3 exponent bits with bias 3, 2 mantissa bits); every
    field must hold an integer in [-8, 7].
    """
    b = np.asarray(codes_u8, dtype=np.uint8)
    Mp, rb = b.shape
    K = rb * 4 // 3
    t = b.reshape(Mp // 16, K // 128, 16, 96).transpose(0, 2, 1, 3).reshape(Mp, K // 128 * 96)   # row-major
    g = t.astype(np.uint32).reshape(Mp, -1, 3)
    w = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)                       # 4 codes per 24 bits
    f = np.stack([(w >> (6 * j)) & 63 for j in range(4)], axis=-1).reshape(Mp, -1)
    f = f[: (Mp if M is None else M)]
    sign = np.where(f & 32, -1.0, 1.0)
    e = (f >> 2) & 7
    m = (f & 3).astype(np.float64)
    mag = np.where(e == 0, m / 16.0, np.exp2(e.astype(np.float64) - 3) * (1 + m / 4))
    v = sign * mag
    assert np.all(v == np.rint(v)) and v.min(initial=0) >= -8 and v.max(initial=0) <= 7, "non-INT4 E3M2 field"
    return v.astype(np.int8)


def int8_values(codes_u8):
    return np.asarray(codes_u8, dtype=np.uint8).view(np.int8)


def mask_bits(mask_i32, K):
    w = np.asarray(mask_i32).view(np.uint32)
    bits = (w[:, :, None] >> np.arange(32, dtype=np.uint32)) & 1
    return bits.reshape(w.shape[0], K).astype(bool)


def x_f32(bits_or_f32):
    a = np.asarray(bits_or_f32)
    return bf16_bits_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)


def assert_y_close(y_gpu, acc, dscale, alpha, acc_unit=1.0, residual=None):
    """Output checks: bit-exact against the fixed-order float32 dequantization of the oracle's exact
    accumulator, and within 1e-5 relative of the float64 value (cancellation-aware with a residual)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float32)
    y32 = O.dequant_f32(acc, dscale, alpha, acc_unit)
    y64 = O.dequant(acc, dscale, alpha, acc_unit)
    if residual is not None:
        r = np.asarray(residual, dtype=np.float32)
        y32 = (y32 + r).astype(np.float32)
        bound = 1e-5 * (np.abs(y64) + np.abs(r.astype(np.float64)))
        y64 = y64 + r.astype(np.float64)
    else:
        bound = 1e-5 * np.abs(y64)
    err = np.abs(y_gpu.astype(np.float64) - y64)
    assert np.all(err <= bound), f"max rel err {np.max(err / np.maximum(bound / 1e-5, 1e-300)):.3g}"
    bad = np.flatnonzero(y_gpu.view(np.uint32) != y32.view(np.uint32))
    assert bad.size == 0, f"{bad.size} outputs differ from the float32 epilogue bit pattern, first {bad[:5]}"
