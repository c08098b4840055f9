"""Decoder of the packed ternary weight layout, written from its description in include/bitlinear.h.

Test-side only: it lets the tests compare the library's packed output with the oracle's codes.
"""
import numpy as np

_POS = np.array([4 * q for q in range(8)] + [4 * q + 2 for q in range(8)], dtype=np.uint32)
# A8 tile layout (bitlinear_pack_ternary_a8): weight q of a word at bits 8 (q % 4) + 2 (q / 4)
_POS_A8 = np.array([8 * (q % 4) + 2 * (q // 4) for q in range(16)], dtype=np.uint32)


def unpack_ternary(packed: np.ndarray, N: int, K: int, a8: bool = False) -> np.ndarray:
    """packed uint8 [N*K/4] -> int8 codes [N, K]; raises on the never-written field value 10b.
    a8: the A8 tile layout (same tiles, lanes and words, another bit position per weight)."""
    w = np.ascontiguousarray(packed, dtype=np.uint8).view("<u4").reshape(K // 128, N // 16, 4, 16, 2)
    # axes: k-tile kt, n-group G, lane group g, row r, word i
    f = (w[..., None] >> (_POS_A8 if a8 else _POS)) & np.uint32(3)   # [..., 16 weights of the word]
    if np.any(f == 2):
        raise ValueError("invalid 2-bit field 10b in packed weights")
    codes = np.where(f == 3, -1, f.astype(np.int64)).astype(np.int8)
    # (kt, G, g, r, i, q) -> (G, r, kt, g, i, q) -> [N, K]
    return codes.transpose(1, 3, 0, 2, 4, 5).reshape(N, K)


def pack_reference(codes: np.ndarray, a8: bool = False) -> np.ndarray:
    """Inverse of unpack_ternary (used to test the decoder itself)."""
    N, K = codes.shape
    c = codes.reshape(N // 16, 16, K // 128, 4, 2, 16).transpose(2, 0, 3, 1, 4, 5)   # kt, G, g, r, i, q
    f = np.where(c < 0, 3, c).astype(np.uint32)
    words = np.bitwise_or.reduce(f << (_POS_A8 if a8 else _POS), axis=-1).astype("<u4")
    return words.reshape(-1).view(np.uint8)


def unpack_ternary_rows(packed: np.ndarray, N: int, K: int) -> np.ndarray:
    """Row-major layout (bitlinear_pack_ternary_rows): row n is K/4 bytes, word i holds k = 16 i .. 16 i + 15."""
    w = np.ascontiguousarray(packed, dtype=np.uint8).view("<u4").reshape(N, K // 16)
    f = (w[..., None] >> _POS) & np.uint32(3)
    if np.any(f == 2):
        raise ValueError("invalid 2-bit field 10b in packed weights")
    return np.where(f == 3, -1, f.astype(np.int64)).astype(np.int8).reshape(N, K)


def pack_rows_reference(codes: np.ndarray) -> np.ndarray:
    """Inverse of unpack_ternary_rows (used to test the decoder itself)."""
    N, K = codes.shape
    f = np.where(codes < 0, 3, codes).astype(np.uint32).reshape(N, K // 16, 16)
    words = np.bitwise_or.reduce(f << _POS, axis=-1).astype("<u4")
    return words.reshape(-1).view(np.uint8)


def unpack_kv(codes_u8, H, D, bits):
    """KV-cache code buffer [T, H * D * bits / 8] -> unsigned codes uint8 [T, H, D], decoded from
    the documented layout: 4 bits, code 2j in the low nibble of byte j of a head record; 3 bits,
    codes 8g .. 8g+7 in the little-endian 24 bits of bytes 3g .. 3g+2, code 8g + q at bits 3q."""
    b = np.asarray(codes_u8, dtype=np.uint8)
    T = b.shape[0]
    b = b.reshape(T, H, D * bits // 8)
    if bits == 4:
        return np.stack([b & 15, b >> 4], axis=-1).reshape(T, H, D)
    g = b.reshape(T, H, D // 8, 3).astype(np.uint32)
    w = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
    return np.stack([(w >> (3 * q)) & 7 for q in range(8)], axis=-1).reshape(T, H, D).astype(np.uint8)
