"""Host-side checks of the C ABI (no GPU needed, no kernel is ever launched here).

* the built library loads and exports every function declared in include/bitlinear.h;
* every invalid-argument path returns its status before any HIP call (fake device pointers are
  safe because validation rejects the call first);
* the test-side decoder of the packed weight layout round-trips.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import ternary_weight_quantized_amd as tw
from tests.packed_layout import pack_reference, pack_rows_reference, unpack_ternary, unpack_ternary_rows

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bitlinear.h")

needs_lib = pytest.mark.skipif(not os.path.exists(tw.LIB_PATH), reason="libbitlinear.so not built (run build())")

P = ctypes.c_void_p(4096)   # a fake, 16-byte aligned "device pointer" (never dereferenced)
P_MIS = ctypes.c_void_p(4100)


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:[\w\s\*]+?)\b(bitlinear_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_hot_path_calls():
    fns = header_functions()
    for f in ("bitlinear_quantize_act", "bitlinear_pack_ternary", "bitlinear_gemm_w158a4",
              "bitlinear_gemm_w158a8_sparse", "bitlinear_gemv_decode", "bitlinear_pack_ternary_rows",
              "bitlinear_gemv_decode_glu_conditional", "bitlinear_quantize_act_per_tensor", "bitlinear_kv_quantize"):
        assert f in fns


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(tw.LIB_PATH)
    for f in header_functions():
        assert hasattr(lib, f), f
    assert set(tw.EXPORTED) == set(header_functions())


@needs_lib
def test_version_and_status_strings():
    assert tw.bitlinear_abi_version() == 2
    assert tw.bitlinear_status_string(0) == "ok"
    assert "argument" in tw.bitlinear_status_string(1)
    assert tw.bitlinear_packed_bytes(4096, 11008) == 4096 * 11008 // 4
    assert tw.bitlinear_pack_workspace_bytes() >= 2048


@needs_lib
def test_workspace_size_query():
    """One query for every operation: the per-op helpers' values where a workspace is taken, 0 where
    none is, SIZE_MAX for an unknown op."""
    for M in (1, 8, 4096, 1 << 20):
        assert tw.bitlinear_workspace_size("quantize_act_per_tensor", M, 0, 4096) == \
            tw.bitlinear_quantize_per_tensor_workspace_bytes(M)
    for op in ("pack_ternary", "pack_ternary_rows", "pack_ternary_a8"):
        assert tw.bitlinear_workspace_size(op, 0, 11008, 4096) == tw.bitlinear_pack_workspace_bytes()
    for op in ("quantize_act", "gemm_w158a4", "gemm_w158a8_sparse", "gemv_decode", "gemv_decode_glu_conditional",
               "kv_quantize"):
        assert tw.bitlinear_workspace_size(op, 4096, 12288, 4096) == 0
    assert tw.bitlinear_workspace_size(99, 1, 1, 128) == 2 ** 64 - 1
    assert tw.bitlinear_workspace_size(-1, 1, 1, 128) == 2 ** 64 - 1


def _q(**kw):
    a = dict(x=P, dt=0, M=4, K=256, ldx=256, fmt=0, keep=-1, eps=1e-5, hint=None, codes=P, scale=P, mask=None)
    a.update(kw)
    return tw.library().bitlinear_quantize_act(a["x"], a["dt"], a["M"], a["K"], a["ldx"], a["fmt"], a["keep"],
                                               a["eps"], a["hint"], a["codes"], a["scale"], a["mask"], None)


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(scale=None), 1),
    (dict(dt=7), 1), (dict(fmt=9), 1), (dict(eps=0.0), 1), (dict(eps=-1.0), 1), (dict(eps=float("nan")), 1),
    (dict(M=0), 2), (dict(K=0), 2), (dict(K=100, ldx=100), 2), (dict(K=320, ldx=320), 2),
    (dict(ldx=128), 1), (dict(fmt=0, keep=3), 1), (dict(fmt=1, mask=P), 1), (dict(fmt=2, keep=257), 1),
    (dict(fmt=4, keep=3), 1), (dict(fmt=4, mask=P), 1), (dict(fmt=5), 1),
    (dict(x=P_MIS), 3), (dict(codes=P_MIS), 3), (dict(ldx=260), 3), (dict(fmt=2, keep=5, mask=P_MIS), 3),
    (dict(M=1 << 20, K=4096, ldx=4096), 2),
])
def test_quantize_validation(kw, status):
    assert _q(**kw) == status


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(w=None), 1), (dict(packed=None), 1), (dict(alpha=None), 1), (dict(ws=None), 1),
    (dict(eps=0.0), 1), (dict(N=10), 2), (dict(K=300), 2), (dict(N=0), 2),
    (dict(wsb=100), 4), (dict(w=P_MIS), 3), (dict(packed=P_MIS), 3),
])
@pytest.mark.parametrize("entry", ["bitlinear_pack_ternary", "bitlinear_pack_ternary_a8", "bitlinear_pack_ternary_rows"])
def test_pack_validation(kw, status, entry):
    a = dict(w=P, N=32, K=256, eps=1e-5, packed=P, alpha=P, ws=P, wsb=4096)
    a.update(kw)
    st = getattr(tw.library(), entry)(a["w"], a["N"], a["K"], a["eps"], a["packed"], a["alpha"], a["ws"],
                                      a["wsb"], None)
    assert st == status


def _mm(name, **kw):
    a = dict(fmt=0, codes=P, scale=P, M=4, K=256, packed=P, alpha=P, N=32, y=P, ldy=32, epi=None)
    a.update(kw)
    lib = tw.library()
    epi = ctypes.byref(a["epi"]) if a["epi"] is not None else None
    args = [a["codes"], a["scale"], a["M"], a["K"], a["packed"], a["alpha"], a["N"], a["y"], a["ldy"], epi, None]
    if name != "bitlinear_gemm_w158a8_sparse":
        args.insert(0, a["fmt"])
    return getattr(lib, name)(*args)


MM_CASES = [
    (dict(codes=None), 1), (dict(scale=None), 1), (dict(packed=None), 1), (dict(alpha=None), 1), (dict(y=None), 1),
    (dict(K=192), 2), (dict(K=64), 2), (dict(N=24), 2), (dict(M=0), 2), (dict(ldy=16), 1), (dict(ldy=33), 3),
    (dict(K=262144), 2), (dict(K=262016 + 128), 2), (dict(M=1, N=16, K=1 << 20), 2),   # beyond the exact-accumulation K
    (dict(codes=P_MIS), 3), (dict(packed=P_MIS), 3), (dict(y=P_MIS), 3),
    (dict(epi=tw.bl_epilogue(1, None, 32, None, None, None)), 1),
    (dict(epi=tw.bl_epilogue(1, 4096, 8, None, None, None)), 1),
    (dict(epi=tw.bl_epilogue(1, 4100, 32, None, None, None)), 3),
    (dict(epi=tw.bl_epilogue(1, 4096, 33, None, None, None)), 3),
    (dict(epi=tw.bl_epilogue(2, None, 0, None, 4096, None)), 1),
    (dict(epi=tw.bl_epilogue(2, None, 0, 4100, 4096, None)), 3),
    (dict(epi=tw.bl_epilogue(7, None, 0, None, None, None)), 1),
]


@needs_lib
@pytest.mark.parametrize("name", ["bitlinear_gemm_w158a4", "bitlinear_gemm_w158a8_sparse", "bitlinear_gemv_decode"])
@pytest.mark.parametrize("kw,status", MM_CASES)
def test_matmul_validation(name, kw, status):
    assert _mm(name, **kw) == status


@needs_lib
def test_format_restrictions():
    assert _mm("bitlinear_gemm_w158a4", fmt=2) == 1          # INT8 goes through the sparse A8 entry point
    assert _mm("bitlinear_gemv_decode", fmt=1) == 1          # decode takes INT4 or INT8
    assert _mm("bitlinear_gemv_decode", fmt=3) == 1
    assert _mm("bitlinear_gemv_decode", M=9) == 2            # decode is for at most 8 tokens
    assert _mm("bitlinear_gemm_w158a4", fmt=5) == 1
    assert _mm("bitlinear_gemm_w158a4", fmt=4) == 1          # FP4 power-of-two codes run as fmt 1


@pytest.mark.parametrize("a8", [False, True])
def test_packed_layout_decoder_roundtrip(a8):
    rng = np.random.default_rng(0)
    codes = rng.integers(-1, 2, (48, 768)).astype(np.int8)
    packed = pack_reference(codes, a8)
    assert packed.size == 48 * 768 // 4
    np.testing.assert_array_equal(unpack_ternary(packed, 48, 768, a8), codes)


def test_a8_word_expands_in_code_order():
    """The A8 word layout is the one whose int8 expansion (the word shifted left by 6, 4, 2, 0 and
    masked with 0xC0C0C0C0) yields the 16 weights as bytes in k order, 64 t each, the order of
    16 INT8 codes in memory; the standard layout yields k 0 2 4 6, 8 10 12 14, 1 3 5 7, 9 11 13 15."""
    rng = np.random.default_rng(1)
    for a8, order in ((True, list(range(16))), (False, [0, 2, 4, 6, 8, 10, 12, 14, 1, 3, 5, 7, 9, 11, 13, 15])):
        for _ in range(20):
            t = rng.integers(-1, 2, (16, 128)).astype(np.int8)
            w = pack_reference(t, a8).view("<u4")[0]                 # row 0, k 0..15
            out = []
            for sh in (6, 4, 2, 0):
                d = (int(w) << sh) & 0xC0C0C0C0
                out += [np.int8(np.uint8((d >> (8 * b)) & 0xFF)) for b in range(4)]
            np.testing.assert_array_equal(np.array(out, dtype=np.int64), 64 * t[0, order].astype(np.int64))


def test_packed_layout_decoder_positions():
    """A single +1 at (n, k) lands in the tile, lane, word and bit the header describes."""
    N, K = 32, 512
    for n, k in [(0, 0), (5, 7), (17, 8), (31, 511), (3, 300), (20, 64 + 16 + 9), (9, 127), (9, 128)]:
        codes = np.zeros((N, K), np.int8)
        codes[n, k] = 1
        packed = pack_reference(codes)
        kk = k % 128
        tile = (k // 128) * (N // 16) + n // 16
        lane = 16 * (kk // 32) + n % 16
        word = (kk % 32) // 16
        q = kk % 16
        bit = 4 * q if q < 8 else 4 * (q - 8) + 2
        words = packed.view("<u4")
        idx = tile * 128 + lane * 2 + word
        assert words[idx] == (1 << bit)
        assert np.count_nonzero(words) == 1


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(w=None), 1), (dict(packed=None), 1), (dict(eps=0.0), 1), (dict(N=10), 2), (dict(K=300), 2),
    (dict(wsb=100), 4), (dict(packed=P_MIS), 3),
])
def test_pack_rows_validation(kw, status):
    a = dict(w=P, N=32, K=256, eps=1e-5, packed=P, alpha=P, ws=P, wsb=4096)
    a.update(kw)
    st = tw.library().bitlinear_pack_ternary_rows(a["w"], a["N"], a["K"], a["eps"], a["packed"], a["alpha"], a["ws"],
                                                  a["wsb"], None)
    assert st == status


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(codes=None), 1), (dict(up=None), 1), (dict(upa=None), 1), (dict(h=None), 1), (dict(gate=None), 1),
    (dict(M=9), 2), (dict(K=192), 2), (dict(N=24), 2),
    (dict(ldh=16), 1), (dict(ldg=16), 1), (dict(up=P_MIS), 3), (dict(h=P_MIS), 3), (dict(ldh=33), 3),
])
def test_glu_conditional_validation(kw, status):
    a = dict(codes=P, scale=P, M=4, K=256, gp=P, ga=P, up=P, upa=P, N=32, gate=P, ldg=32, h=P, ldh=32, rm=None)
    a.update(kw)
    st = tw.library().bitlinear_gemv_decode_glu_conditional(a["codes"], a["scale"], a["M"], a["K"], a["gp"], a["ga"],
                                                            a["up"], a["upa"], a["N"], a["gate"], a["ldg"], a["h"],
                                                            a["ldh"], a["rm"], None)
    assert st == status


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(scale=None), 1), (dict(ws=None), 1),
    (dict(dt=7), 1), (dict(fmt=9), 1), (dict(eps=0.0), 1), (dict(M=0), 2), (dict(K=100, ldx=100), 2),
    (dict(ldx=128), 1), (dict(wsb=100), 4), (dict(x=P_MIS), 3), (dict(ws=P_MIS), 3), (dict(ldx=260), 3),
    (dict(M=1 << 20, K=4096, ldx=4096, wsb=1 << 24), 2), (dict(M=300000, wsb=1 << 20), 4), (dict(wsb=51200), 4),
])
def test_quantize_per_tensor_validation(kw, status):
    a = dict(x=P, dt=0, M=4, K=256, ldx=256, fmt=0, eps=1e-5, ws=P, wsb=1 << 21, codes=P, scale=P)
    a.update(kw)
    st = tw.library().bitlinear_quantize_act_per_tensor(a["x"], a["dt"], a["M"], a["K"], a["ldx"], a["fmt"], a["eps"],
                                                        a["ws"], a["wsb"], a["codes"], a["scale"], None)
    assert st == status
    assert tw.bitlinear_quantize_per_tensor_workspace_bytes(4) >= 512 * 12 * 8 + 512 * 4 + 16


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(scale=None), 1), (dict(dt=5), 1), (dict(bits=2), 1),
    (dict(bits=8), 1), (dict(eps=0.0), 1), (dict(cos=P), 1), (dict(cos=P, sin=P), 1),
    (dict(cos=P, sin=P, pos=P, Pn=0), 1), (dict(slot=P), 1), (dict(slot=P, bcodes=P, bscale=P, bits=4, ns=2), 1),
    (dict(slot=P, bcodes=P, bscale=P, ns=0), 1), (dict(H=0), 2), (dict(D=96), 2), (dict(D=32, ldx=128), 2),
    (dict(D=512, ldx=2048), 2), (dict(T=-1), 2), (dict(ldx=100), 1), (dict(x=P_MIS), 3), (dict(codes=P_MIS), 3),
    (dict(ldx=258), 3), (dict(cos=P_MIS, sin=P, pos=P, Pn=4), 3), (dict(slot=P, bcodes=P_MIS, bscale=P, ns=2), 3),
    (dict(T=1 << 20, H=32, D=128, ldx=4096), 2), (dict(T=0), 0),
])
def test_kv_quantize_validation(kw, status):
    a = dict(x=P, dt=0, T=4, H=2, D=64, ldx=128, pos=None, cos=None, sin=None, Pn=0, bits=3, eps=1e-5, codes=P,
             scale=P, slot=None, ns=0, bcodes=None, bscale=None)
    a.update(kw)
    st = tw.library().bitlinear_kv_quantize(a["x"], a["dt"], a["T"], a["H"], a["D"], a["ldx"], a["pos"], a["cos"],
                                            a["sin"], a["Pn"], a["bits"], a["eps"], a["codes"], a["scale"],
                                            a["slot"], a["ns"], a["bcodes"], a["bscale"], None)
    assert st == status


@pytest.mark.parametrize("bits", [3, 4])
def test_kv_decoder_positions(bits):
    """A single set bit lands where the documented KV layout says."""
    from tests.packed_layout import unpack_kv
    H, D = 2, 64
    rb = D * bits // 8
    for byte in (0, 1, 5, rb - 1, rb, 2 * rb - 1):
        for bit in (0, 3, 7):
            buf = np.zeros((1, H * rb), np.uint8)
            buf[0, byte] = 1 << bit
            dec = unpack_kv(buf, H, D, bits)
            h, r = divmod(byte, rb)
            pos = (8 * r + bit) // bits
            assert dec[0, h, pos] == 1 << ((8 * r + bit) % bits)
            assert np.count_nonzero(dec) == 1


def test_packed_rows_decoder_roundtrip_and_positions():
    rng = np.random.default_rng(1)
    codes = rng.integers(-1, 2, (24, 512)).astype(np.int8)
    np.testing.assert_array_equal(unpack_ternary_rows(pack_rows_reference(codes), 24, 512), codes)
    for n, k in [(0, 0), (3, 9), (7, 16), (23, 511)]:
        c = np.zeros((24, 512), np.int8)
        c[n, k] = -1
        words = pack_rows_reference(c).view("<u4")
        q = k % 16
        bit = 4 * q if q < 8 else 4 * (q - 8) + 2
        assert words[n * 512 // 16 + k // 16] == (3 << bit)
        assert np.count_nonzero(words) == 1


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(out=None), 1), (dict(blocks=0), 2), (dict(blocks=65537), 2), (dict(iters=-1), 2),
    (dict(iters=(1 << 20) + 1), 2),
])
def test_calibrate_mfma_validation(kw, status):
    a = dict(blocks=512, iters=10, out=P)
    a.update(kw)
    assert tw.library().bitlinear_calibrate_mfma(a["blocks"], a["iters"], a["out"], None) == status


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(codes=None), 1), (dict(scale=None), 1), (dict(dt=7), 1), (dict(fmt=9), 1),
    (dict(eps=0.0), 1), (dict(M=0), 2), (dict(K=100, ldx=100), 2), (dict(ldx=128), 1), (dict(x=P_MIS), 3),
    (dict(ldx=260), 3), (dict(M=(1 << 16) + 1), 4), (dict(M=1 << 20, K=4096, ldx=4096), 2),
])
def test_quantize_per_tensor_noalloc_validation(kw, status):
    """Every rejection happens on the host, before the scratch array is looked up (no GPU here)."""
    a = dict(x=P, dt=0, M=4, K=256, ldx=256, fmt=0, eps=1e-5, codes=P, scale=P)
    a.update(kw)
    st = tw.library().bitlinear_quantize_act_per_tensor_noalloc(a["x"], a["dt"], a["M"], a["K"], a["ldx"], a["fmt"],
                                                                a["eps"], a["codes"], a["scale"], None)
    assert st == status


@needs_lib
def test_noalloc_scratch_size():
    assert tw.bitlinear_noalloc_scratch_bytes() == tw.bitlinear_quantize_per_tensor_workspace_bytes(tw.NOALLOC_MAX_M)
    assert tw.bitlinear_noalloc_scratch_bytes() < 1 << 20


@needs_lib
def test_calibrate_read_validation():
    lib = tw.library()
    assert lib.bitlinear_calibrate_read(None, 1024, P, None) == 1
    assert lib.bitlinear_calibrate_read(P, 1024, None, None) == 1
    for b in (0, 8, 1000, 1 << 31):
        assert lib.bitlinear_calibrate_read(P, b, P, None) == 2
    assert lib.bitlinear_calibrate_read(P_MIS, 1024, P, None) == 3



def _kvmm(**kw):
    a = dict(fmt=3, codes=P, scale=P, M=4, K=256, packed=P, alpha=P, N=384, y=None, ldy=384, H=1, eps=1e-5,
             bits=(4, 3, 3), c=(P, P, P), s=(P, P, P), pos=None, cos=None, sin=None, Pn=0, bos=None, ns=0,
             bc=(None, None, None), bs=(None, None, None))
    a.update(kw)
    e = tw.bl_kv_epilogue()
    e.H, e.eps, e.P, e.n_bos_slots = a["H"], a["eps"], a["Pn"], a["ns"]
    for i in range(3):
        e.bits[i] = a["bits"][i]
        e.d_codes[i] = a["c"][i].value if a["c"][i] is not None else None
        e.d_scale[i] = a["s"][i].value if a["s"][i] is not None else None
        e.d_bos_codes[i] = a["bc"][i].value if a["bc"][i] is not None else None
        e.d_bos_scale[i] = a["bs"][i].value if a["bs"][i] is not None else None
    for f in ("pos", "cos", "sin", "bos"):
        setattr(e, {"pos": "d_pos", "cos": "d_cos", "sin": "d_sin", "bos": "d_bos_slot"}[f],
                a[f].value if a[f] is not None else None)
    return tw.library().bitlinear_gemm_w158a4_kv(a["fmt"], a["codes"], a["scale"], a["M"], a["K"], a["packed"],
                                                 a["alpha"], a["N"], a["y"], a["ldy"], ctypes.byref(e), None)


@needs_lib
@pytest.mark.parametrize("kw,status", [
    (dict(fmt=0), 1), (dict(fmt=2), 1), (dict(codes=None), 1), (dict(N=256), 2), (dict(H=2), 2), (dict(H=0), 2),
    (dict(bits=(4, 5, 3)), 1), (dict(c=(P, None, P)), 1), (dict(s=(None, P, P)), 1), (dict(c=(P, P_MIS, P)), 3),
    (dict(eps=0.0), 1), (dict(cos=P), 1), (dict(cos=P, sin=P), 1), (dict(cos=P, sin=P, pos=P), 1),
    (dict(cos=P_MIS, sin=P, pos=P, Pn=8), 3), (dict(bos=P), 1), (dict(bos=P, ns=1), 1),
    (dict(bos=P, ns=1, bits=(4, 4, 4), bc=(P, P, P), bs=(P, P, P)), 1),
    (dict(bos=P, ns=1, bc=(None, P_MIS, P), bs=(None, P, P)), 3),
    (dict(y=P, ldy=100), 1), (dict(y=P_MIS), 3), (dict(K=192), 2), (dict(M=0), 2),
])
def test_gemm_kv_validation(kw, status):
    """Every rejection of the fused QKV + KV entry point happens on the host (no GPU here)."""
    assert _kvmm(**kw) == status
