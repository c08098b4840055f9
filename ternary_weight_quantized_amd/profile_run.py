"""Minimal driver for hardware-counter runs of the BitLinear kernels (few launches, no benchmark loop).

    python -m ternary_weight_quantized_amd.profile_run --gemm fp6 --reps 3 --copy-calibration
    python -m ternary_weight_quantized_amd.profile_run --decode --copy-calibration
    python -m ternary_weight_quantized_amd.profile_run --a8 --reps 3
    python -m ternary_weight_quantized_amd.profile_run --quant --reps 3 --copy-calibration

--gemm quantizes the prefill workload (M=4096, K=4096, N=12288, seeded synthetic bf16 activations and
latent weights) and launches the selected W1.58A4 GEMM `reps` times. --decode launches, each over 24
rotating copies of its weights (as the benchmark's graphs do): the INT4 decode GEMV of 1 token
(11008x4096), the fused gate+up ReLU^2 GLU decode GEMV of 1 token (12 copies of both 11008x4096
matrices), the gate-first conditional up projection of the same token (12 copies of the gate and of the
row-major up matrix) and the INT8 decode GEMV of one row of the FFN's h codes against the 4096x11008 down
projection. --a8 launches the two W1.58A8 GEMMs of the FFN (down) and attention-output workloads; --kv the
prefill QKV GEMM with the KV-cache quantizer fused into its epilogue (Q4 RoPE, K3 RoPE + BOS, V3 + BOS);
--quant every activation quantizer of the workloads (prefill INT4 nibbles, E3M2, FP4, FP4 power-of-two and
per-tensor INT4 of the 4096x4096 bf16 input; INT8 of an fp32 2048x11008 h with its row maxima; Top-K INT8
of the 8192x4096 bf16 attention output) and the three KV quantizers of a 4096 x 3 x 32 x 128 fp32 QKV output.
With --copy-calibration a 256 MiB device-to-device copy runs first; its FETCH_SIZE and WRITE_SIZE
readings give the factor that turns those counters into bytes.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

EPS = 1e-5
FORMATS = {"fp6": "int4_e3m2", "int4": "int4", "fp4": "fp4"}


def dev_bf16(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--gemm", choices=sorted(FORMATS), default=None)
    p.add_argument("--decode", action="store_true")
    p.add_argument("--a8", action="store_true")
    p.add_argument("--kv", action="store_true", help="the prefill QKV GEMM with the fused KV-cache epilogue")
    p.add_argument("--quant", action="store_true", help="every activation and KV-cache quantizer of the workloads")
    p.add_argument("--reps", type=int, default=3)
    p.add_argument("--copy-calibration", action="store_true")
    args = p.parse_args()
    if not (args.gemm or args.decode or args.a8 or args.kv or args.quant):
        args.gemm = "fp6"

    import torch

    import ternary_weight_quantized_amd as tw
    from synth import WORKLOADS, workload_inputs

    tw.library()

    def pack(w, a8=False):
        f = tw.bitlinear_pack_ternary_a8 if a8 else tw.bitlinear_pack_ternary
        return f(torch.from_numpy(w).cuda(), EPS)

    work = []
    if args.gemm:
        P = WORKLOADS["prefill_qkv"]
        inp = workload_inputs("prefill_qkv")
        x = dev_bf16(torch, inp["x"])
        packed, alpha = pack(inp["w"])
        fmt = FORMATS[args.gemm]
        codes, scale, _ = tw.bitlinear_quantize_act(x, fmt, eps=EPS)
        y = torch.empty((P["M"], P["N"]), dtype=torch.float32, device="cuda")
        work.append((f"{args.reps} x {fmt} GEMM M={P['M']} K={P['K']} N={P['N']}",
                     lambda: [tw.bitlinear_gemm_w158a4(fmt, codes, scale, P["K"], packed, alpha, P["N"], y=y)
                              for _ in range(args.reps)]))
    if args.kv:
        P = WORKLOADS["prefill_qkv"]
        KV = WORKLOADS["kv_cache"]
        import numpy as np
        from synth import rope_tables
        inp = workload_inputs("prefill_qkv")
        kx = dev_bf16(torch, inp["x"])
        kW, kA = pack(inp["w"])
        kc, ks, _ = tw.bitlinear_quantize_act(kx, "int4_e3m2", eps=EPS)
        H = P["N"] // 384
        pos_np = (np.arange(P["M"]) % KV["seq_len"]).astype(np.int32)
        bos = pos_np == 0
        kpos = torch.from_numpy(pos_np).cuda()
        kslot = torch.from_numpy(np.where(bos, np.cumsum(bos) - 1, -1).astype(np.int32)).cuda()
        c_np, s_np = rope_tables(KV["seq_len"], 128)
        kcos, ksin = torch.from_numpy(c_np).cuda(), torch.from_numpy(s_np).cuda()
        kv_out = tw.bitlinear_gemm_w158a4_kv("int4_e3m2", kc, ks, P["K"], kW, kA, P["N"], H, bits=(4, 3, 3), eps=EPS,
                                             pos=kpos, cos=kcos, sin=ksin, bos_slot=kslot,
                                             n_bos_slots=int(bos.sum()))
        work.append((f"{args.reps} x fused QKV + KV GEMM M={P['M']} K={P['K']} N={P['N']}",
                     lambda: [tw.bitlinear_gemm_w158a4_kv("int4_e3m2", kc, ks, P["K"], kW, kA, P["N"], H,
                                                          bits=(4, 3, 3), eps=EPS, pos=kpos, cos=kcos, sin=ksin,
                                                          bos_slot=kslot, n_bos_slots=int(bos.sum()), out=kv_out)
                              for _ in range(args.reps)]))
    if args.decode or args.a8:
        F = WORKLOADS["ffn_7b"]
        fin = workload_inputs("ffn_7b")
        gW, gA = pack(fin["w_gate"])
        uW, uA = pack(fin["w_up"])
        dW, dA = pack(fin["w_down"], a8=True)       # the INT8 matmuls take the A8 weight layout
        fx = dev_bf16(torch, fin["x"])
        uWr = None
        if args.decode:
            uWr, _ = tw.bitlinear_pack_ternary_rows(torch.from_numpy(fin["w_up"]).cuda(), EPS)
        del fin
        fc, fs, _ = tw.bitlinear_quantize_act(fx, "int4_e3m2", eps=EPS)
        frm = torch.empty(F["M"], dtype=torch.float32, device="cuda")
        fh = tw.bitlinear_gemm_w158a4("int4_e3m2", fc, fs, F["K"], gW, gA, F["N"], up_packed=uW, up_alpha=uA,
                                      row_absmax=frm)
        fhc, fhs, _ = tw.bitlinear_quantize_act(fh, "int8", eps=EPS, row_absmax_hint=frm)
    if args.decode:
        D = WORKLOADS["decode_a4"]
        din = workload_inputs("decode_a4")
        w0, a0 = pack(din["w"])
        dc, ds, _ = tw.bitlinear_quantize_act(dev_bf16(torch, din["x"][:1]), "int4", eps=EPS)
        dWs = [w0] + [w0.clone() for _ in range(23)]
        gWs = [gW] + [gW.clone() for _ in range(11)]
        uWs = [uW] + [uW.clone() for _ in range(11)]
        uWrs = [uWr] + [uWr.clone() for _ in range(11)]
        d8Ws = [dW] + [dW.clone() for _ in range(23)]
        y1 = torch.empty((1, D["N"]), dtype=torch.float32, device="cuda")
        h1 = torch.empty((1, F["N"]), dtype=torch.float32, device="cuda")
        g1 = torch.empty((1, F["N"]), dtype=torch.float32, device="cuda")
        y8 = torch.empty((1, F["K"]), dtype=torch.float32, device="cuda")

        def decode():
            for r in range(24):
                tw.bitlinear_gemv_decode("int4", dc, ds, D["K"], dWs[r], a0, D["N"], y=y1)
            for r in range(12):
                tw.bitlinear_gemv_decode("int4", dc, ds, D["K"], gWs[r], gA, F["N"], y=h1, up_packed=uWs[r],
                                         up_alpha=uA)
            for r in range(12):
                tw.bitlinear_gemv_decode_glu_conditional(dc, ds, D["K"], gWs[r], gA, uWrs[r], uA, F["N"], gate=g1, h=h1)
            for r in range(24):
                tw.bitlinear_gemv_decode("int8", fhc[:1], fhs[:1], F["N"], d8Ws[r], dA, F["K"], y=y8)
        work.append(("decode: 24 INT4 GEMV M=1, 12 fused GLU GEMV M=1, 12 conditional GLU M=1, 24 INT8 GEMV M=1",
                     decode))
    if args.a8:
        A = WORKLOADS["attn_out"]
        ain = workload_inputs("attn_out")
        ax = dev_bf16(torch, ain["x"])
        ar = torch.from_numpy(ain["residual"]).cuda()
        oW, oA = pack(ain["w"], a8=True)
        del ain
        ac, as_, _ = tw.bitlinear_quantize_act(ax, "int8", topk_keep=A["keep"], eps=EPS)
        fy = torch.empty((F["M"], F["K"]), dtype=torch.float32, device="cuda")
        ay = torch.empty((A["M"], A["N"]), dtype=torch.float32, device="cuda")

        def a8():
            for _ in range(args.reps):
                tw.bitlinear_gemm_w158a8_sparse(fhc, fhs, F["N"], dW, dA, F["K"], y=fy)
                tw.bitlinear_gemm_w158a8_sparse(ac, as_, A["K"], oW, oA, A["N"], y=ay, residual=ar)
        work.append((f"{args.reps} x (A8 down 2048x11008x4096, A8 o_proj+residual 8192x4096x4096)", a8))
    if args.quant:
        import numpy as np
        from synth import rope_tables
        P = WORKLOADS["prefill_qkv"]
        px = dev_bf16(torch, workload_inputs("prefill_qkv")["x"])
        Fq = WORKLOADS["ffn_7b"]
        # the FFN's h [2048, 11008] as float32, with its row maxima: any fp32 rows of that shape load the same bytes
        qh = torch.from_numpy(np.random.default_rng(5).standard_normal((Fq["M"], Fq["N"]), dtype=np.float32)).cuda()
        qrm = qh.abs().amax(dim=1).contiguous()
        A = WORKLOADS["attn_out"]
        qax = dev_bf16(torch, workload_inputs("attn_out")["x"])
        KV = WORKLOADS["kv_cache"]
        kT, kH, kD = KV["T"], KV["H"], KV["D"]
        # the QKV projection output [4096, 3 * 32 * 128] in float32 (any values: the kernels read all of it)
        qkv = torch.from_numpy(np.random.default_rng(6).standard_normal((kT, 3 * kH * kD), dtype=np.float32)).cuda()
        kpos_np = (np.arange(kT) % KV["seq_len"]).astype(np.int32)
        kpos = torch.from_numpy(kpos_np).cuda()
        kbos = kpos_np == 0
        kslot = torch.from_numpy(np.where(kbos, np.cumsum(kbos) - 1, -1).astype(np.int32)).cuda()
        c_np, s_np = rope_tables(KV["seq_len"], kD)
        kcos, ksin = torch.from_numpy(c_np).cuda(), torch.from_numpy(s_np).cuda()
        pws = torch.empty(tw.bitlinear_quantize_per_tensor_workspace_bytes(P["M"]), dtype=torch.uint8, device="cuda")

        # every prefill quantizer reads its own copy of the rows, and each repetition streams about 530 MB,
        # more than the 256 MB last-level cache holds, so no launch finds its input there (the per-tensor
        # call's second pass re-reads the rows its first pass just read, as it does in use)
        pxs = [px] + [px.clone() for _ in range(4)]

        def quant():
            for _ in range(args.reps):
                for i, fmt in enumerate(("int4", "int4_e3m2", "fp4", "fp4_pow2")):
                    tw.bitlinear_quantize_act(pxs[i], fmt, eps=EPS)
                tw.bitlinear_quantize_act_per_tensor(pxs[4], "int4", eps=EPS, workspace=pws)
                tw.bitlinear_quantize_act(qh, "int8", eps=EPS, row_absmax_hint=qrm)
                tw.bitlinear_quantize_act(qax, "int8", topk_keep=A["keep"], eps=EPS)
                tw.bitlinear_kv_quantize(qkv[:, :kH * kD], kH, kD, 4, eps=EPS, pos=kpos, cos=kcos, sin=ksin)
                tw.bitlinear_kv_quantize(qkv[:, kH * kD:2 * kH * kD], kH, kD, 3, eps=EPS, pos=kpos, cos=kcos, sin=ksin,
                                         bos_slot=kslot, n_bos_slots=int(kbos.sum()))
                tw.bitlinear_kv_quantize(qkv[:, 2 * kH * kD:], kH, kD, 3, eps=EPS, bos_slot=kslot,
                                         n_bos_slots=int(kbos.sum()))
        work.append((f"{args.reps} x every quantizer (prefill INT4/E3M2/FP4/FP4 pow2/per-tensor, INT8 h, Top-K INT8, "
                     "KV Q4/K3/V3)", quant))
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for name, fn in work:
        fn()
        torch.cuda.synchronize()
        print(f"profile_run: {name}", flush=True)


if __name__ == "__main__":
    main()
