"""Python binding of libbitlinear (ctypes): argument marshalling only.

Every function here has the name of the C entry point it calls (include/bitlinear.h). PyTorch
provides device memory and the current HIP stream; every step of the computation runs in the
library's HIP kernels. There is no fallback: if the library is missing or fails to load, the
functions raise.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbitlinear.so")

BL_OK = 0
BL_ACT_INT4, BL_ACT_FP4_E2M1, BL_ACT_INT8, BL_ACT_INT4_E3M2, BL_ACT_FP4_E2M1_POW2 = 0, 1, 2, 3, 4
BL_IN_BF16, BL_IN_F32 = 0, 1
BL_EPI_NONE, BL_EPI_RESIDUAL, BL_EPI_RELU2_GLU = 0, 1, 2
OPS = {"quantize_act": 0, "quantize_act_per_tensor": 1, "pack_ternary": 2, "pack_ternary_rows": 3,
       "gemm_w158a4": 4, "gemm_w158a8_sparse": 5, "gemv_decode": 6, "gemv_decode_glu_conditional": 7,
       "kv_quantize": 8, "pack_ternary_a8": 9}

FORMATS = {"int4": BL_ACT_INT4, "fp4": BL_ACT_FP4_E2M1, "int8": BL_ACT_INT8, "int4_e3m2": BL_ACT_INT4_E3M2,
           "fp4_pow2": BL_ACT_FP4_E2M1_POW2}

EXPORTED = (
    "bitlinear_quantize_act", "bitlinear_pack_ternary", "bitlinear_pack_ternary_rows", "bitlinear_pack_ternary_a8",
    "bitlinear_packed_bytes",
    "bitlinear_pack_workspace_bytes", "bitlinear_gemm_w158a4", "bitlinear_gemm_w158a8_sparse",
    "bitlinear_gemv_decode", "bitlinear_gemv_decode_glu_conditional", "bitlinear_status_string",
    "bitlinear_abi_version", "bitlinear_quantize_act_per_tensor", "bitlinear_quantize_per_tensor_workspace_bytes",
    "bitlinear_kv_quantize", "bitlinear_calibrate_mfma", "bitlinear_calibrate_read", "bitlinear_workspace_size",
    "bitlinear_quantize_act_per_tensor_noalloc", "bitlinear_noalloc_scratch_bytes", "bitlinear_gemm_w158a4_kv",
)
NOALLOC_MAX_M = 65536


class BitlinearError(RuntimeError):
    """A non-zero bl_status returned by the library."""

    def __init__(self, status: int, where: str):
        self.status = status
        msg = _lib().bitlinear_status_string(status).decode() if _LIB is not None else str(status)
        super().__init__(f"{where}: status {status} ({msg})")


class bl_epilogue(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("d_residual", ctypes.c_void_p),
        ("ldr", ctypes.c_int64),
        ("d_up_packed", ctypes.c_void_p),
        ("d_up_alpha", ctypes.c_void_p),
        ("d_row_absmax", ctypes.c_void_p),
    ]


class bl_kv_epilogue(ctypes.Structure):
    _fields_ = [
        ("H", ctypes.c_int64),
        ("eps", ctypes.c_float),
        ("bits", ctypes.c_int32 * 3),
        ("d_codes", ctypes.c_void_p * 3),
        ("d_scale", ctypes.c_void_p * 3),
        ("d_pos", ctypes.c_void_p),
        ("d_cos", ctypes.c_void_p),
        ("d_sin", ctypes.c_void_p),
        ("P", ctypes.c_int64),
        ("d_bos_slot", ctypes.c_void_p),
        ("n_bos_slots", ctypes.c_int64),
        ("d_bos_codes", ctypes.c_void_p * 3),
        ("d_bos_scale", ctypes.c_void_p * 3),
    ]


_LIB = None


def _lib():
    """Load libbitlinear.so once; raise if it is absent (no CPU fallback exists)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not built: run `python -m ternary_weight_quantized_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        ep = ctypes.POINTER(bl_epilogue)
        lib.bitlinear_quantize_act.argtypes = [vp, i32, i64, i64, i64, i32, i32, f32, vp, vp, vp, vp, vp]
        lib.bitlinear_quantize_act.restype = i32
        lib.bitlinear_packed_bytes.argtypes = [i64, i64]
        lib.bitlinear_packed_bytes.restype = sz
        lib.bitlinear_pack_workspace_bytes.argtypes = []
        lib.bitlinear_pack_workspace_bytes.restype = sz
        lib.bitlinear_workspace_size.argtypes = [i32, i64, i64, i64]
        lib.bitlinear_workspace_size.restype = sz
        lib.bitlinear_pack_ternary.argtypes = [vp, i64, i64, f32, vp, vp, vp, sz, vp]
        lib.bitlinear_pack_ternary.restype = i32
        lib.bitlinear_kv_quantize.argtypes = [vp, i32, i64, i64, i64, i64, vp, vp, vp, i64, i32, f32, vp, vp, vp, i64,
                                              vp, vp, vp]
        lib.bitlinear_kv_quantize.restype = i32
        lib.bitlinear_calibrate_mfma.argtypes = [i32, i32, vp, vp]
        lib.bitlinear_calibrate_read.argtypes = [vp, i64, vp, vp]
        lib.bitlinear_calibrate_read.restype = i32
        lib.bitlinear_calibrate_mfma.restype = i32
        lib.bitlinear_quantize_act_per_tensor.argtypes = [vp, i32, i64, i64, i64, i32, f32, vp, sz, vp, vp, vp]
        lib.bitlinear_quantize_act_per_tensor.restype = i32
        lib.bitlinear_quantize_per_tensor_workspace_bytes.argtypes = [i64]
        lib.bitlinear_quantize_act_per_tensor_noalloc.argtypes = [vp, i32, i64, i64, i64, i32, f32, vp, vp, vp]
        lib.bitlinear_quantize_act_per_tensor_noalloc.restype = i32
        lib.bitlinear_noalloc_scratch_bytes.argtypes = []
        lib.bitlinear_noalloc_scratch_bytes.restype = sz
        lib.bitlinear_quantize_per_tensor_workspace_bytes.restype = sz
        for name in ("bitlinear_pack_ternary_rows", "bitlinear_pack_ternary_a8"):
            getattr(lib, name).argtypes = [vp, i64, i64, f32, vp, vp, vp, sz, vp]
            getattr(lib, name).restype = i32
        lib.bitlinear_gemv_decode_glu_conditional.argtypes = [vp, vp, i64, i64, vp, vp, vp, vp, i64, vp, i64, vp,
                                                              i64, vp, vp]
        lib.bitlinear_gemv_decode_glu_conditional.restype = i32
        for name in ("bitlinear_gemm_w158a4", "bitlinear_gemv_decode"):
            getattr(lib, name).argtypes = [i32, vp, vp, i64, i64, vp, vp, i64, vp, i64, ep, vp]
            getattr(lib, name).restype = i32
        lib.bitlinear_gemm_w158a4_kv.argtypes = [i32, vp, vp, i64, i64, vp, vp, i64, vp, i64,
                                                 ctypes.POINTER(bl_kv_epilogue), vp]
        lib.bitlinear_gemm_w158a4_kv.restype = i32
        lib.bitlinear_gemm_w158a8_sparse.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, i64, ep, vp]
        lib.bitlinear_gemm_w158a8_sparse.restype = i32
        lib.bitlinear_status_string.argtypes = [i32]
        lib.bitlinear_status_string.restype = ctypes.c_char_p
        lib.bitlinear_abi_version.argtypes = []
        lib.bitlinear_abi_version.restype = i32
        _LIB = lib
    return _LIB


def library():
    """The loaded ctypes library (raises if it is missing)."""
    return _lib()


def _check(status: int, where: str):
    if status != BL_OK:
        raise BitlinearError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _fmt(fmt):
    return FORMATS[fmt] if isinstance(fmt, str) else int(fmt)


def codes_shape(fmt, M, K):
    """(rows, bytes per row) of the code buffer of a format (E3M2: tiled, rows padded to 16)."""
    f = _fmt(fmt)
    if f == BL_ACT_INT4_E3M2:
        return ((M + 15) // 16 * 16, 3 * K // 4)
    return (M, K if f == BL_ACT_INT8 else K // 2)


# ------------------------------------------------------------------------------- entry points
def bitlinear_quantize_act(x, fmt, topk_keep=-1, eps=1e-5, row_absmax_hint=None, want_mask=False,
                           codes=None, scale=None, mask=None, stream=None):
    """Per-token quantization of x [M, K] (bf16 or float32, CUDA). Returns (codes uint8, scale f32 [M], mask|None)."""
    import torch
    f = _fmt(fmt)
    M, K = x.shape
    in_dtype = {torch.bfloat16: BL_IN_BF16, torch.float32: BL_IN_F32}[x.dtype]
    if codes is None:
        codes = torch.empty(codes_shape(f, M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(M, dtype=torch.float32, device=x.device)
    if want_mask and mask is None:
        mask = torch.empty((M, K // 32), dtype=torch.int32, device=x.device)
    st = _lib().bitlinear_quantize_act(_ptr(x), in_dtype, M, K, x.stride(0), f, int(topk_keep), float(eps),
                                       _ptr(row_absmax_hint), _ptr(codes), _ptr(scale), _ptr(mask), _stream(stream))
    _check(st, "bitlinear_quantize_act")
    return codes, scale, mask


def bitlinear_quantize_per_tensor_workspace_bytes(M):
    return int(_lib().bitlinear_quantize_per_tensor_workspace_bytes(M))


def bitlinear_quantize_act_per_tensor(x, fmt, eps=1e-5, codes=None, scale=None, workspace=None, stream=None):
    """Quantization of x [M, K] with one scale for the whole tensor. Returns (codes, scale f32 [M])."""
    import torch
    f = _fmt(fmt)
    M, K = x.shape
    in_dtype = {torch.bfloat16: BL_IN_BF16, torch.float32: BL_IN_F32}[x.dtype]
    if codes is None:
        codes = torch.empty(codes_shape(f, M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(M, dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = torch.empty(bitlinear_quantize_per_tensor_workspace_bytes(M), dtype=torch.uint8, device=x.device)
    st = _lib().bitlinear_quantize_act_per_tensor(_ptr(x), in_dtype, M, K, x.stride(0), f, float(eps), _ptr(workspace),
                                                  workspace.numel(), _ptr(codes), _ptr(scale), _stream(stream))
    _check(st, "bitlinear_quantize_act_per_tensor")
    return codes, scale


def bitlinear_noalloc_scratch_bytes():
    return int(_lib().bitlinear_noalloc_scratch_bytes())


def bitlinear_quantize_act_per_tensor_noalloc(x, fmt, eps=1e-5, codes=None, scale=None, stream=None):
    """The per-tensor quantizer without a workspace (the library's fixed scratch; M <= NOALLOC_MAX_M).
    Returns (codes, scale f32 [M]); pass codes and scale to allocate nothing at all."""
    import torch
    f = _fmt(fmt)
    M, K = x.shape
    in_dtype = {torch.bfloat16: BL_IN_BF16, torch.float32: BL_IN_F32}[x.dtype]
    if codes is None:
        codes = torch.empty(codes_shape(f, M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(M, dtype=torch.float32, device=x.device)
    st = _lib().bitlinear_quantize_act_per_tensor_noalloc(_ptr(x), in_dtype, M, K, x.stride(0), f, float(eps),
                                                          _ptr(codes), _ptr(scale), _stream(stream))
    _check(st, "bitlinear_quantize_act_per_tensor_noalloc")
    return codes, scale


def kv_record_bytes(D, bits):
    return D * bits // 8


def bitlinear_kv_quantize(x, H, D, bits, eps=1e-5, pos=None, cos=None, sin=None, bos_slot=None, n_bos_slots=0,
                          codes=None, scale=None, bos_codes=None, bos_scale=None, stream=None):
    """Post-RoPE absmax KV-cache quantization of x [T, >= H*D] (bf16 or float32 rows).

    Returns (codes uint8 [T, H * D * bits / 8], scale f32 [T, H], bos_codes, bos_scale); the BOS
    buffers ([n_bos_slots, H * D / 2] and [n_bos_slots, H]) only when bos_slot is given."""
    import torch
    T = x.shape[0]
    in_dtype = {torch.bfloat16: BL_IN_BF16, torch.float32: BL_IN_F32}[x.dtype]
    if codes is None:
        codes = torch.empty((T, H * kv_record_bytes(D, bits)), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((T, H), dtype=torch.float32, device=x.device)
    if bos_slot is not None:
        if bos_codes is None:
            bos_codes = torch.zeros((n_bos_slots, H * D // 2), dtype=torch.uint8, device=x.device)
        if bos_scale is None:
            bos_scale = torch.zeros((n_bos_slots, H), dtype=torch.float32, device=x.device)
    P = cos.shape[0] if cos is not None else 0
    st = _lib().bitlinear_kv_quantize(_ptr(x), in_dtype, T, H, D, x.stride(0), _ptr(pos), _ptr(cos), _ptr(sin), P,
                                      bits, float(eps), _ptr(codes), _ptr(scale), _ptr(bos_slot), n_bos_slots,
                                      _ptr(bos_codes), _ptr(bos_scale), _stream(stream))
    _check(st, "bitlinear_kv_quantize")
    return codes, scale, bos_codes, bos_scale


def bitlinear_calibrate_read(src, sink, nbytes=None, stream=None):
    """Measurement aid: one plain streaming read of src (a device tensor, nbytes of it); sink: >= 4 bytes."""
    b = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check(_lib().bitlinear_calibrate_read(_ptr(src), b, _ptr(sink), _stream(stream)), "bitlinear_calibrate_read")


def bitlinear_calibrate_mfma(blocks, iters, out=None, stream=None):
    """Measurement aid (not part of the BitLinear path): FP6 x FP4 matrix-core-only loop of
    blocks * iters * 8388608 ops in the GEMM's wave shape, on operands with the GEMM's statistics.
    Returns the buffer: element 256 b holds block b's shader-clock ticks per 100 MHz real-time tick
    (x 0.1 = GHz); the other elements carry no meaning."""
    import torch
    if out is None:
        out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = _lib().bitlinear_calibrate_mfma(blocks, iters, _ptr(out), _stream(stream))
    _check(st, "bitlinear_calibrate_mfma")
    return out


def bitlinear_packed_bytes(N, K):
    return int(_lib().bitlinear_packed_bytes(N, K))


def bitlinear_pack_workspace_bytes():
    return int(_lib().bitlinear_pack_workspace_bytes())


def bitlinear_workspace_size(op, M, N, K):
    """Workspace bytes of an operation (name from OPS or the bl_op value); SIZE_MAX for an unknown op."""
    return int(_lib().bitlinear_workspace_size(OPS[op] if isinstance(op, str) else int(op), M, N, K))


def _pack(fn_name, w, eps, packed, alpha, workspace, stream):
    import torch
    N, K = w.shape
    if packed is None:
        packed = torch.empty(bitlinear_packed_bytes(N, K), dtype=torch.uint8, device=w.device)
    if alpha is None:
        alpha = torch.empty(1, dtype=torch.float32, device=w.device)
    if workspace is None:
        workspace = torch.empty(bitlinear_pack_workspace_bytes(), dtype=torch.uint8, device=w.device)
    st = getattr(_lib(), fn_name)(_ptr(w), N, K, float(eps), _ptr(packed), _ptr(alpha), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, fn_name)
    return packed, alpha


def bitlinear_pack_ternary(w, eps=1e-5, packed=None, alpha=None, workspace=None, stream=None):
    """Ternarize and pack w [N, K] float32 (CUDA), tiled layout. Returns (packed uint8 [N*K/4], alpha f32 [1])."""
    return _pack("bitlinear_pack_ternary", w, eps, packed, alpha, workspace, stream)


def bitlinear_pack_ternary_a8(w, eps=1e-5, packed=None, alpha=None, workspace=None, stream=None):
    """Ternarize and pack w [N, K] float32 (CUDA), A8 tile layout (the weights of the INT8 matmuls)."""
    return _pack("bitlinear_pack_ternary_a8", w, eps, packed, alpha, workspace, stream)


def bitlinear_pack_ternary_rows(w, eps=1e-5, packed=None, alpha=None, workspace=None, stream=None):
    """Ternarize and pack w [N, K] float32 (CUDA), row-major layout (gathered up projection)."""
    return _pack("bitlinear_pack_ternary_rows", w, eps, packed, alpha, workspace, stream)


def _epilogue(residual=None, up_packed=None, up_alpha=None, row_absmax=None):
    if residual is not None:
        return bl_epilogue(BL_EPI_RESIDUAL, residual.data_ptr(), residual.stride(0), None, None, None)
    if up_packed is not None:
        return bl_epilogue(BL_EPI_RELU2_GLU, None, 0, up_packed.data_ptr(), up_alpha.data_ptr(),
                           None if row_absmax is None else row_absmax.data_ptr())
    return None


def _mm(fn_name, fmt, codes, scale, M, K, packed, alpha, N, y, residual, up_packed, up_alpha, row_absmax, stream):
    import torch
    if y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    epi = _epilogue(residual, up_packed, up_alpha, row_absmax)
    epi_ref = ctypes.byref(epi) if epi is not None else None
    fn = getattr(_lib(), fn_name)
    args = [_ptr(codes), _ptr(scale), M, K, _ptr(packed), _ptr(alpha), N, _ptr(y), y.stride(0), epi_ref, _stream(stream)]
    if fn_name != "bitlinear_gemm_w158a8_sparse":
        args.insert(0, _fmt(fmt))
    _check(fn(*args), fn_name)
    return y


def bitlinear_gemm_w158a4(fmt, codes, scale, K, packed, alpha, N, y=None, residual=None, up_packed=None,
                          up_alpha=None, row_absmax=None, stream=None):
    """Y [M, N] = Q_4bit(X) Q_w(W)^T with an optional epilogue (residual or ReLU^2 GLU with W_up)."""
    return _mm("bitlinear_gemm_w158a4", fmt, codes, scale, scale.shape[0], K, packed, alpha, N, y, residual,
               up_packed, up_alpha, row_absmax, stream)


def bitlinear_gemm_w158a4_kv(fmt, codes, scale, K, packed, alpha, N, H, bits=(4, 3, 3), eps=1e-5, pos=None, cos=None,
                             sin=None, bos_slot=None, n_bos_slots=0, y=None, want_y=False, out=None, stream=None):
    """QKV projection with the KV-cache quantizer in its epilogue (head size 128, N = 3 H 128).

    Returns dict(y (or None), codes=[q, k, v], scale=[q, k, v], bos_codes=[...], bos_scale=[...]);
    `out` may give preallocated buffers under the same keys."""
    import torch
    f = _fmt(fmt)
    M = scale.shape[0]
    dev = codes.device
    if want_y and y is None:
        y = torch.empty((M, N), dtype=torch.float32, device=dev)
    out = dict(out or {})
    if "codes" not in out:
        out["codes"] = [torch.empty((M, H * 16 * b), dtype=torch.uint8, device=dev) for b in bits]
        out["scale"] = [torch.empty((M, H), dtype=torch.float32, device=dev) for _ in bits]
    if bos_slot is not None and "bos_codes" not in out:
        out["bos_codes"] = [torch.empty((n_bos_slots, H * 64), dtype=torch.uint8, device=dev) if b == 3 else None
                            for b in bits]
        out["bos_scale"] = [torch.empty((n_bos_slots, H), dtype=torch.float32, device=dev) if b == 3 else None
                            for b in bits]
    e = bl_kv_epilogue()
    e.H, e.eps = H, float(eps)
    for p in range(3):
        e.bits[p] = bits[p]
        e.d_codes[p] = out["codes"][p].data_ptr()
        e.d_scale[p] = out["scale"][p].data_ptr()
        if bos_slot is not None and out["bos_codes"][p] is not None:
            e.d_bos_codes[p] = out["bos_codes"][p].data_ptr()
            e.d_bos_scale[p] = out["bos_scale"][p].data_ptr()
    if cos is not None:
        e.d_pos, e.d_cos, e.d_sin, e.P = pos.data_ptr(), cos.data_ptr(), sin.data_ptr(), cos.shape[0]
    if bos_slot is not None:
        e.d_bos_slot, e.n_bos_slots = bos_slot.data_ptr(), n_bos_slots
    st = _lib().bitlinear_gemm_w158a4_kv(f, _ptr(codes), _ptr(scale), M, K, _ptr(packed), _ptr(alpha), N, _ptr(y),
                                         N if y is None else y.stride(0), ctypes.byref(e), _stream(stream))
    _check(st, "bitlinear_gemm_w158a4_kv")
    out["y"] = y
    return out


def bitlinear_gemm_w158a8_sparse(codes, scale, K, packed, alpha, N, y=None, residual=None, up_packed=None,
                                 up_alpha=None, row_absmax=None, stream=None):
    """Y [M, N] = (Q_INT8(X) . M) Q_w(W)^T with an optional epilogue."""
    return _mm("bitlinear_gemm_w158a8_sparse", BL_ACT_INT8, codes, scale, scale.shape[0], K, packed, alpha, N, y,
               residual, up_packed, up_alpha, row_absmax, stream)


def bitlinear_gemv_decode(fmt, codes, scale, K, packed, alpha, N, y=None, residual=None, up_packed=None,
                          up_alpha=None, row_absmax=None, stream=None):
    """Decode product for 1 <= M <= 8 tokens (INT4 or INT8 codes)."""
    return _mm("bitlinear_gemv_decode", fmt, codes, scale, scale.shape[0], K, packed, alpha, N, y, residual,
               up_packed, up_alpha, row_absmax, stream)


def bitlinear_gemv_decode_glu_conditional(codes, scale, K, gate_packed, gate_alpha, up_rows, up_alpha, N,
                                           gate=None, h=None, row_absmax=None, stream=None):
    """Decode gate projection, then the up projection only where the gate is positive.
    Returns (gate [M, N] f32, h [M, N] f32)."""
    import torch
    M = scale.shape[0]
    if gate is None:
        gate = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    if h is None:
        h = torch.empty((M, N), dtype=torch.float32, device=codes.device)
    st = _lib().bitlinear_gemv_decode_glu_conditional(_ptr(codes), _ptr(scale), M, K, _ptr(gate_packed),
                                                      _ptr(gate_alpha), _ptr(up_rows), _ptr(up_alpha), N,
                                                      _ptr(gate), gate.stride(0), _ptr(h), h.stride(0),
                                                      _ptr(row_absmax), _stream(stream))
    _check(st, "bitlinear_gemv_decode_glu_conditional")
    return gate, h


def bitlinear_abi_version():
    return int(_lib().bitlinear_abi_version())


def bitlinear_status_string(status):
    return _lib().bitlinear_status_string(int(status)).decode()
