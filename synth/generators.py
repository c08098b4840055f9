"""Counter-based seeded generators (numpy, vectorised).

* SplitMix64 (Steele, Lea, Flood 2014): state_i = seed + (i+1)*0x9E3779B97F4A7C15,
  output = mix(state_i) with the published mixing constants.
* uniform in (0, 1]: ((z >> 11) + 1) * 2^-53.
* Box-Muller (cosine branch only) for N(0, 1) in float64.
* Student-t with 3 degrees of freedom: Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3).
* bfloat16: round-to-nearest-even of the float32 value (bit pattern as uint16).

Seeds are ``1000 * workload + tensor_id``; every stream of a tensor uses its
own seed so tensors never share draws.
"""
from __future__ import annotations

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """n consecutive SplitMix64 outputs of stream ``seed`` starting at counter ``offset``."""
    with np.errstate(over="ignore"):
        idx = np.arange(offset + 1, offset + n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + idx * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def uniform01(seed: int, n: int, offset: int = 0) -> np.ndarray:
    """Uniform doubles in (0, 1]."""
    z = splitmix64(seed, n, offset)
    return ((z >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def normal(seed: int, n: int) -> np.ndarray:
    """n standard normal float64 draws (Box-Muller, cosine branch)."""
    u = uniform01(seed, 2 * n)
    u1, u2 = u[0::2], u[1::2]
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def student_t3(seed: int, n: int) -> np.ndarray:
    """n Student-t(3) float64 draws built from four independent normal streams."""
    z = normal(seed, 4 * n).reshape(n, 4)
    return z[:, 0] / np.sqrt((z[:, 1] ** 2 + z[:, 2] ** 2 + z[:, 3] ** 2) / 3.0)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float -> bfloat16 bit patterns (uint16), round to nearest even via float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> exactly equal float32 values."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def outlier_channels(seed: int, K: int, fraction: float = 0.001) -> np.ndarray:
    """Indices of round(fraction*K) (at least 1) channels, chosen by a seeded permutation."""
    n = max(1, int(round(fraction * K)))
    keys = splitmix64(seed, K)
    return np.sort(np.argsort(keys, kind="stable")[:n])


def activations_bf16(seed: int, M: int, K: int, outlier_scale: float = 0.0,
                     outlier_kind: str = "scale", outlier_fraction: float = 0.001) -> np.ndarray:
    """bf16 bit patterns [M, K] of N(0,1) activations, optionally with outlier channels.

    outlier_kind="scale": the chosen channels are multiplied by ``outlier_scale``.
    outlier_kind="t3":    the chosen channels are replaced by ``outlier_scale`` * t3 draws.
    """
    x = normal(seed, M * K).reshape(M, K)
    if outlier_scale:
        ch = outlier_channels(seed + 500_000, K, outlier_fraction)
        if outlier_kind == "scale":
            x[:, ch] *= outlier_scale
        elif outlier_kind == "t3":
            x[:, ch] = outlier_scale * student_t3(seed + 600_000, M * len(ch)).reshape(M, len(ch))
        else:
            raise ValueError(outlier_kind)
    return to_bf16_bits(x)


def latent_weights(seed: int, N: int, K: int, sigma: float = 0.02) -> np.ndarray:
    """float32 [N, K] latent weights drawn from N(0, sigma^2)."""
    return (sigma * normal(seed, N * K)).astype(np.float32).reshape(N, K)


# Workload shapes, one entry per synthetic workload of the hot path.
WORKLOADS = {
    "tiny_a4":       dict(M=64, K=2048, N=2048),
    "decode_a4":     dict(Ms=(1, 4, 8), K=4096, N=11008),
    "prefill_qkv":   dict(M=4096, K=4096, N=3 * 4096, outlier_scale=20.0),
    "ffn_7b":        dict(M=2048, K=4096, N=11008),
    "attn_out":      dict(M=8192, K=4096, N=4096, keep=2048, outlier_scale=20.0),
    # Q, K and V heads of the prefill projection output (fp32 [T, 3 H D]), 4 sequences of 1024 tokens
    "kv_cache":      dict(T=4096, H=32, D=128, seq_len=1024),
}
_WL_INDEX = {name: i + 1 for i, name in enumerate(WORKLOADS)}


def rope_tables(P: int, D: int, base: float = 10000.0):
    """cos and sin float32 [P, D/2] of the angles p * base^(-2i/D) (computed in float64)."""
    p = np.arange(P, dtype=np.float64)[:, None]
    inv = base ** (-2.0 * np.arange(D // 2, dtype=np.float64) / D)
    ang = p * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def workload_inputs(name: str, M: int | None = None):
    """Host-side inputs of a workload as a dict of numpy arrays.

    ``M`` overrides the token count (for sampled or reduced parity runs the
    first rows of the full-size draw are NOT reproduced; use the full M and
    slice instead when row identity matters).
    """
    wl = WORKLOADS[name]
    base = 1000 * _WL_INDEX[name]
    if name == "kv_cache":
        T = M if M is not None else wl["T"]
        W = 3 * wl["H"] * wl["D"]
        pos = (np.arange(T) % wl["seq_len"]).astype(np.int32)
        cos, sin = rope_tables(wl["seq_len"], wl["D"])
        return dict(qkv=normal(base + 1, T * W).astype(np.float32).reshape(T, W), pos=pos, cos=cos, sin=sin)
    K, N = wl["K"], wl["N"]
    if name == "decode_a4":
        Mx = M if M is not None else max(wl["Ms"])
        return dict(x=activations_bf16(base + 1, Mx, K), w=latent_weights(base + 2, N, K))
    Mx = M if M is not None else wl["M"]
    if name == "tiny_a4":
        return dict(x=activations_bf16(base + 1, Mx, K), w=latent_weights(base + 2, N, K))
    if name == "prefill_qkv":
        return dict(x=activations_bf16(base + 1, Mx, K, outlier_scale=wl["outlier_scale"]),
                    w=latent_weights(base + 2, N, K))
    if name == "ffn_7b":
        return dict(x=activations_bf16(base + 1, Mx, K),
                    w_gate=latent_weights(base + 2, N, K),
                    w_up=latent_weights(base + 3, N, K),
                    w_down=latent_weights(base + 4, K, N))
    if name == "attn_out":
        return dict(x=activations_bf16(base + 1, Mx, K, outlier_scale=wl["outlier_scale"],
                                       outlier_kind="t3"),
                    residual=normal(base + 5, Mx * N).astype(np.float32).reshape(Mx, N),
                    w=latent_weights(base + 2, N, K))
    raise KeyError(name)
