"""Benchmark of the BitNet a4.8 BitLinear hot path on one MI355X.

One step = one pass of every hot-path operation over the synthetic workloads, inputs resident in HBM:
  prefill_qkv  (M=4096, K=4096, N=12288, bf16 N(0,1) with 0.1% x20 outlier channels):
               INT4 quantize + W1.58A4 int8-MFMA GEMM; FP4 quantize + W1.58A4 FP4-MFMA GEMM
  ffn_7b       (M=2048, K=4096, N=11008): INT4 quantize, gate+up GEMM with the ReLU^2 GLU epilogue,
               INT8 quantize of h (row max from the epilogue), W1.58A8 down GEMM
  attn_out     (M=8192, K=N=4096, Student-t outlier channels): Top-K 50% + INT8 quantize,
               W1.58A8 o_proj GEMM with the residual add
  decode_a4    (M=1,4,8, K=4096, N=11008): INT4 quantize + decode GEMV, replayed from a HIP graph over
               24 rotating weight copies (270 MB, larger than the 256 MB last-level cache); decode FFN
               gate+up at the same shape, fused ReLU^2 GLU GEMV vs gate first + conditional up projection
               (12 rotating copies of both matrices)
The headline value is the W1.58A4 INT4 prefill GEMM throughput in TOPS (2*M*N*K / average kernel time,
HIP events on the launch stream); the decode GEMV bandwidth and every kernel's time and roofline
fraction are reported beside it. The memory-bound quantizers are also timed back to back from a HIP
graph over input copies larger than the last-level cache (us_graph), which leaves out the dispatch gap
that the eager sequence's events include. The weights are ternarized and packed once, outside the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
INT8_PEAK_TOPS = 5000.0      # dense int8 MFMA
FP4_PEAK_TOPS = 10100.0      # dense FP4/FP6 MFMA
EPS = 1e-5
ROTATE = 24
ROTATE_GLU = 12                # 12 copies of gate + up (tiled and row-major) weights: 405 MB


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=4096, help="rows of the prefill workload the oracle runs")
    p.add_argument("--copy-calibration", action="store_true",
                   help="copy 256 MiB device to device once before the steps (scale for HBM byte counters)")
    return p.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_mx_fp6_prefill_traffic.md")
GEMM_SOURCE = os.path.join(ROOT, "ternary_weight_quantized_amd", "csrc", "gemm.hip")


def measured_traffic():
    """HBM bytes per launch of the FP6 prefill GEMM from the committed counter summary, or None when
    the summary is missing or was taken on another version of the GEMM source."""
    import hashlib
    try:
        text = open(TRAFFIC_FILE).read()
        src = hashlib.sha256(open(GEMM_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = dict(line.split(":", 1) for line in text.splitlines() if line.startswith(("source_sha256:",
                                                                                      "traffic_bytes_per_launch:")))
    if fields.get("source_sha256", "").strip() != src:
        return None
    try:
        return int(float(fields["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def bf16_dev(torch, bits):
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the path would shard by "
              "tokens or output columns without communication, and only one GPU's share is measured here.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import ternary_weight_quantized_amd as tw
    from synth import WORKLOADS, workload_inputs

    tw.library()
    torch.cuda.set_device(0)
    dev = "cuda"
    t_setup = time.time()

    # ------------------------------------------------------------------ inputs and packed weights
    def pack(w, a8=False):
        f = tw.bitlinear_pack_ternary_a8 if a8 else tw.bitlinear_pack_ternary
        return f(torch.from_numpy(w).to(dev), EPS)

    P = WORKLOADS["prefill_qkv"]
    pin = workload_inputs("prefill_qkv")
    px = bf16_dev(torch, pin["x"])
    pW, pA = pack(pin["w"])
    del pin
    pc4 = torch.empty((P["M"], P["K"] // 2), dtype=torch.uint8, device=dev)
    ps4 = torch.empty(P["M"], dtype=torch.float32, device=dev)
    pc6 = torch.empty((P["M"], 3 * P["K"] // 4), dtype=torch.uint8, device=dev)
    ps6 = torch.empty(P["M"], dtype=torch.float32, device=dev)
    pcf = torch.empty_like(pc4)
    psf = torch.empty_like(ps4)
    pcp = torch.empty_like(pc4)          # FP4 with power-of-two scales
    psp = torch.empty_like(ps4)
    pct = torch.empty_like(pc4)          # INT4 with one scale for the whole tensor
    pst = torch.empty_like(ps4)
    pws = torch.empty(tw.bitlinear_quantize_per_tensor_workspace_bytes(P["M"]), dtype=torch.uint8, device=dev)
    py4 = torch.empty((P["M"], P["N"]), dtype=torch.float32, device=dev)
    pyf = torch.empty_like(py4)

    F = WORKLOADS["ffn_7b"]
    fin = workload_inputs("ffn_7b")
    fx = bf16_dev(torch, fin["x"])
    gW, gA = pack(fin["w_gate"])
    uW, uA = pack(fin["w_up"])
    uWr, _ = tw.bitlinear_pack_ternary_rows(torch.from_numpy(fin["w_up"]).to(dev), EPS)
    dW, dA = pack(fin["w_down"], a8=True)        # the INT8 matmuls take the A8 weight layout
    wg_latent = fin["w_gate"]            # kept for the gate-sparse decode input below
    del fin
    fc = torch.empty((F["M"], 3 * F["K"] // 4), dtype=torch.uint8, device=dev)
    fs = torch.empty(F["M"], dtype=torch.float32, device=dev)
    fh = torch.empty((F["M"], F["N"]), dtype=torch.float32, device=dev)
    frm = torch.empty(F["M"], dtype=torch.float32, device=dev)
    fhc = torch.empty((F["M"], F["N"]), dtype=torch.uint8, device=dev)
    fhs = torch.empty(F["M"], dtype=torch.float32, device=dev)
    fy = torch.empty((F["M"], F["K"]), dtype=torch.float32, device=dev)

    A = WORKLOADS["attn_out"]
    ain = workload_inputs("attn_out")
    ax = bf16_dev(torch, ain["x"])
    ar = torch.from_numpy(ain["residual"]).to(dev)
    oW, oA = pack(ain["w"], a8=True)
    del ain
    ac = torch.empty((A["M"], A["K"]), dtype=torch.uint8, device=dev)
    as_ = torch.empty(A["M"], dtype=torch.float32, device=dev)
    am = torch.empty((A["M"], A["K"] // 32), dtype=torch.int32, device=dev)
    ay = torch.empty((A["M"], A["N"]), dtype=torch.float32, device=dev)

    # KV cache (post-RoPE, Q at 4 bits, K and V at 3 bits with BOS records at 4) read from the
    # prefill QKV projection output [4096, 3 * 32 * 128]
    KV = WORKLOADS["kv_cache"]
    from synth import rope_tables
    kT, kH, kD = KV["T"], KV["H"], KV["D"]
    assert kT == P["M"] and 3 * kH * kD == P["N"]
    kpos_np = (np.arange(kT) % KV["seq_len"]).astype(np.int32)
    kpos = torch.from_numpy(kpos_np).to(dev)
    kbos = kpos_np == 0
    kslot = torch.from_numpy(np.where(kbos, np.cumsum(kbos) - 1, -1).astype(np.int32)).to(dev)
    knslots = int(kbos.sum())
    kcos_np, ksin_np = rope_tables(KV["seq_len"], kD)
    kcos, ksin = torch.from_numpy(kcos_np).to(dev), torch.from_numpy(ksin_np).to(dev)
    kq_c = torch.empty((kT, kH * kD // 2), dtype=torch.uint8, device=dev)
    kq_s = torch.empty((kT, kH), dtype=torch.float32, device=dev)
    kk_c = torch.empty((kT, kH * kD * 3 // 8), dtype=torch.uint8, device=dev)
    kk_s = torch.empty_like(kq_s)
    kv_c = torch.empty_like(kk_c)
    kv_s = torch.empty_like(kq_s)
    kkb_c = torch.empty((knslots, kH * kD // 2), dtype=torch.uint8, device=dev)
    kkb_s = torch.empty((knslots, kH), dtype=torch.float32, device=dev)
    kvb_c = torch.empty_like(kkb_c)
    kvb_s = torch.empty_like(kkb_s)
    # the same records from the QKV GEMM with the KV quantizer fused into its epilogue (no fp32 output)
    kv_fused = {"codes": [torch.empty_like(kq_c), torch.empty_like(kk_c), torch.empty_like(kv_c)],
                "scale": [torch.empty_like(kq_s), torch.empty_like(kk_s), torch.empty_like(kv_s)],
                "bos_codes": [None, torch.empty_like(kkb_c), torch.empty_like(kvb_c)],
                "bos_scale": [None, torch.empty_like(kkb_s), torch.empty_like(kvb_s)]}

    D = WORKLOADS["decode_a4"]
    din = workload_inputs("decode_a4")
    dx = bf16_dev(torch, din["x"])
    w0, a0 = pack(din["w"])
    del din
    dWs = [w0] + [w0.clone() for _ in range(ROTATE - 1)]       # distinct HBM copies of the same weights
    dcs = {m: torch.empty((m, D["K"] // 2), dtype=torch.uint8, device=dev) for m in D["Ms"]}
    dss = {m: torch.empty(m, dtype=torch.float32, device=dev) for m in D["Ms"]}
    dys = {m: torch.empty((m, D["N"]), dtype=torch.float32, device=dev) for m in D["Ms"]}
    # decode FFN gate+up (7B shape): fused ReLU^2 GLU GEMV vs gate-first conditional up projection
    gWs = [gW] + [gW.clone() for _ in range(ROTATE_GLU - 1)]
    uWs = [uW] + [uW.clone() for _ in range(ROTATE_GLU - 1)]
    uWrs = [uWr] + [uWr.clone() for _ in range(ROTATE_GLU - 1)]
    dgs = {m: torch.empty((m, F["N"]), dtype=torch.float32, device=dev) for m in D["Ms"]}
    dhs = {m: torch.empty((m, F["N"]), dtype=torch.float32, device=dev) for m in D["Ms"]}
    # Gate-sparse decode input (M = 1), labelled as such: the pages report 67.5% zero gate outputs for the
    # trained 7B model (32.5% live channels, a nearly threefold smaller up projection), while the i.i.d.
    # weights leave half of them live. Negating a latent gate row negates its ternary codes and its gate
    # value exactly (alpha is unchanged), so a seeded choice of the token's live channels is negated
    # until 32.5% of the channels remain live; the gate is computed once here with the INT4 GEMV.
    tw.bitlinear_quantize_act(dx[:1], "int4", eps=EPS, codes=dcs[1], scale=dss[1])
    g1 = tw.bitlinear_gemv_decode("int4", dcs[1], dss[1], D["K"], gW, gA, F["N"])
    pos = torch.nonzero(g1[0] > 0).flatten().cpu().numpy()
    flip = np.random.default_rng(20241).choice(pos, size=max(len(pos) - round(0.325 * F["N"]), 0), replace=False)
    wg_sparse = wg_latent.copy()
    wg_sparse[flip] *= -1.0
    gWsp, gAsp = pack(wg_sparse)
    del wg_sparse, wg_latent, g1
    gWsps = [gWsp] + [gWsp.clone() for _ in range(ROTATE_GLU - 1)]
    dgsp = torch.empty((1, F["N"]), dtype=torch.float32, device=dev)
    dhsp = torch.empty((1, F["N"]), dtype=torch.float32, device=dev)
    # decode A8: INT8 codes of the first M rows of the FFN's h against the down projection
    d8Ws = [dW] + [dW.clone() for _ in range(ROTATE - 1)]
    d8ys = {m: torch.empty((m, F["K"]), dtype=torch.float32, device=dev) for m in D["Ms"]}
    # Structured-sparsity variants of the two A8 inputs, labelled as such: the i.i.d. codes with a seeded half
    # of their 16-row x 128-column slices (the granularity whose matrix-core work the A8 GEMM skips) set to
    # zero, e.g. channels dead for a group of tokens. For h that gives about 84% zero codes, the pages'
    # figure for the 7B down-projection input; the Top-K codes go from 50% to about 75%. The h codes are
    # computed once here.
    tw.bitlinear_quantize_act(fx, "int4_e3m2", eps=EPS, codes=fc, scale=fs)
    tw.bitlinear_gemm_w158a4("int4_e3m2", fc, fs, F["K"], gW, gA, F["N"], y=fh, up_packed=uW, up_alpha=uA,
                             row_absmax=frm)
    tw.bitlinear_quantize_act(fh, "int8", eps=EPS, row_absmax_hint=frm, codes=fhc, scale=fhs)
    tw.bitlinear_quantize_act(ax, "int8", topk_keep=A["keep"], eps=EPS, codes=ac, scale=as_, mask=am)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(4242)

    def slice_mask(M_, K_, p_zero):
        keep = (torch.rand((M_ // 16, K_ // 128), generator=gen) >= p_zero).to(torch.uint8)
        return keep.repeat_interleave(16, 0).repeat_interleave(128, 1).to(dev)
    fhc_s = fhc * slice_mask(F["M"], F["N"], 0.5)
    ac_s = ac * slice_mask(A["M"], A["K"], 0.5)
    fy_s = torch.empty_like(fy)
    ay_s = torch.empty_like(ay)
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    # ------------------------------------------------------------------ decode graphs (launch-bound)
    side = torch.cuda.Stream()
    graphs = {}
    for m in D["Ms"]:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            tw.bitlinear_quantize_act(dx[:m], "int4", eps=EPS, codes=dcs[m], scale=dss[m])
            for r in range(ROTATE):
                tw.bitlinear_gemv_decode("int4", dcs[m], dss[m], D["K"], dWs[r], a0, D["N"], y=dys[m])
        graphs[m] = g
    glu_graphs, cond_graphs = {}, {}
    for m in D["Ms"]:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for r in range(ROTATE_GLU):
                tw.bitlinear_gemv_decode("int4", dcs[m], dss[m], D["K"], gWs[r], gA, F["N"], y=dhs[m],
                                         up_packed=uWs[r], up_alpha=uA)
        glu_graphs[m] = g
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for r in range(ROTATE_GLU):
                tw.bitlinear_gemv_decode_glu_conditional(dcs[m], dss[m], D["K"], gWs[r], gA, uWrs[r], uA, F["N"],
                                                         gate=dgs[m], h=dhs[m])
        cond_graphs[m] = g
    cond_sparse_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cond_sparse_graph, stream=side):
        for r in range(ROTATE_GLU):
            tw.bitlinear_gemv_decode_glu_conditional(dcs[1], dss[1], D["K"], gWsps[r], gAsp, uWrs[r], uA, F["N"],
                                                     gate=dgsp, h=dhsp)
    # ceilings of a launch that streams one packed matrix: a plain read of the 11.27 MB weights (24 copies,
    # the same rotation) and a launch that reads 16 bytes
    read_sink = torch.zeros(4, dtype=torch.int32, device=dev)
    read_graph, launch_graph = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(read_graph, stream=side):
        for r in range(ROTATE):
            tw.bitlinear_calibrate_read(dWs[r], read_sink)
    with torch.cuda.graph(launch_graph, stream=side):
        for r in range(ROTATE):
            tw.bitlinear_calibrate_read(dWs[r], read_sink, nbytes=16)
    a8_graphs = {}
    for m in D["Ms"]:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for r in range(ROTATE):
                tw.bitlinear_gemv_decode("int8", fhc[:m], fhs[:m], F["N"], d8Ws[r], dA, F["K"], y=d8ys[m])
        a8_graphs[m] = g
    torch.cuda.synchronize()

    names = ["quant_int4_e3m2_prefill", "gemm_a4_int4_fp6_prefill", "quant_int4_prefill", "gemm_a4_int4_i8_prefill",
             "quant_fp4_prefill", "gemm_a4_fp4_prefill", "quant_fp4_pow2_prefill",
             "quant_int4_per_tensor_prefill",
             "quant_int4_e3m2_ffn", "gemm_a4_glu_ffn", "quant_int8_h", "gemm_a8_down", "quant_topk_int8_attn",
             "gemm_a8_oproj_residual", "gemm_a8_down_structured", "gemm_a8_oproj_residual_structured",
             "kv_quant_q4_rope", "kv_quant_k3_rope_bos", "kv_quant_v3_bos", "gemm_a4_qkv_kv_fused",
             "decode_read_floor_graph"] + \
        [f"decode_m{m}_graph" for m in D["Ms"]] + \
        [f"decode_glu_m{m}_graph" for m in D["Ms"]] + [f"decode_glu_cond_m{m}_graph" for m in D["Ms"]] + \
        ["decode_glu_cond_gate_sparse_m1_graph"] + \
        [f"decode_a8_m{m}_graph" for m in D["Ms"]]

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def step(record):
        evs = [ev() for _ in range(len(names) + 1)] if record else None
        i = 0

        def mark():
            nonlocal i
            if record:
                evs[i].record()
            i += 1

        mark()
        tw.bitlinear_quantize_act(px, "int4_e3m2", eps=EPS, codes=pc6, scale=ps6); mark()
        tw.bitlinear_gemm_w158a4("int4_e3m2", pc6, ps6, P["K"], pW, pA, P["N"], y=py4); mark()
        tw.bitlinear_quantize_act(px, "int4", eps=EPS, codes=pc4, scale=ps4); mark()
        tw.bitlinear_gemm_w158a4("int4", pc4, ps4, P["K"], pW, pA, P["N"], y=py4); mark()
        tw.bitlinear_quantize_act(px, "fp4", eps=EPS, codes=pcf, scale=psf); mark()
        tw.bitlinear_gemm_w158a4("fp4", pcf, psf, P["K"], pW, pA, P["N"], y=pyf); mark()
        tw.bitlinear_quantize_act(px, "fp4_pow2", eps=EPS, codes=pcp, scale=psp); mark()
        tw.bitlinear_quantize_act_per_tensor(px, "int4", eps=EPS, codes=pct, scale=pst, workspace=pws); mark()
        tw.bitlinear_quantize_act(fx, "int4_e3m2", eps=EPS, codes=fc, scale=fs); mark()
        tw.bitlinear_gemm_w158a4("int4_e3m2", fc, fs, F["K"], gW, gA, F["N"], y=fh, up_packed=uW, up_alpha=uA,
                                 row_absmax=frm); mark()
        tw.bitlinear_quantize_act(fh, "int8", eps=EPS, row_absmax_hint=frm, codes=fhc, scale=fhs); mark()
        tw.bitlinear_gemm_w158a8_sparse(fhc, fhs, F["N"], dW, dA, F["K"], y=fy); mark()
        tw.bitlinear_quantize_act(ax, "int8", topk_keep=A["keep"], eps=EPS, codes=ac, scale=as_, mask=am); mark()
        tw.bitlinear_gemm_w158a8_sparse(ac, as_, A["K"], oW, oA, A["N"], y=ay, residual=ar); mark()
        tw.bitlinear_gemm_w158a8_sparse(fhc_s, fhs, F["N"], dW, dA, F["K"], y=fy_s); mark()
        tw.bitlinear_gemm_w158a8_sparse(ac_s, as_, A["K"], oW, oA, A["N"], y=ay_s, residual=ar); mark()
        tw.bitlinear_kv_quantize(py4[:, :kH * kD], kH, kD, 4, eps=EPS, pos=kpos, cos=kcos, sin=ksin,
                                 codes=kq_c, scale=kq_s); mark()
        tw.bitlinear_kv_quantize(py4[:, kH * kD:2 * kH * kD], kH, kD, 3, eps=EPS, pos=kpos, cos=kcos, sin=ksin,
                                 bos_slot=kslot, n_bos_slots=knslots, codes=kk_c, scale=kk_s, bos_codes=kkb_c,
                                 bos_scale=kkb_s); mark()
        tw.bitlinear_kv_quantize(py4[:, 2 * kH * kD:], kH, kD, 3, eps=EPS, bos_slot=kslot, n_bos_slots=knslots,
                                 codes=kv_c, scale=kv_s, bos_codes=kvb_c, bos_scale=kvb_s); mark()
        tw.bitlinear_gemm_w158a4_kv("int4_e3m2", pc6, ps6, P["K"], pW, pA, P["N"], kH, bits=(4, 3, 3), eps=EPS,
                                    pos=kpos, cos=kcos, sin=ksin, bos_slot=kslot, n_bos_slots=knslots,
                                    out=kv_fused); mark()
        read_graph.replay(); mark()                # the read floor where the decode graphs run
        for m in D["Ms"]:
            graphs[m].replay(); mark()
        for m in D["Ms"]:
            glu_graphs[m].replay(); mark()
        for m in D["Ms"]:
            cond_graphs[m].replay(); mark()
        cond_sparse_graph.replay(); mark()
        for m in D["Ms"]:
            a8_graphs[m].replay(); mark()
        return evs

    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    # ------------------------------------------------------------------ timed region
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    recs = [step(True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    times = {n: 0.0 for n in names}
    for evs in recs:
        for j, n in enumerate(names):
            times[n] += evs[j].elapsed_time(evs[j + 1]) * 1e3 / args.steps     # microseconds
    gemv_us = {m: times[f"decode_m{m}_graph"] / ROTATE for m in D["Ms"]}     # includes the tiny quantize
    glu_us = {m: times[f"decode_glu_m{m}_graph"] / ROTATE_GLU for m in D["Ms"]}
    cond_us = {m: times[f"decode_glu_cond_m{m}_graph"] / ROTATE_GLU for m in D["Ms"]}
    cond_sparse_us = times["decode_glu_cond_gate_sparse_m1_graph"] / ROTATE_GLU
    a8_us = {m: times[f"decode_a8_m{m}_graph"] / ROTATE for m in D["Ms"]}
    # 32-wide K slices of the down weights that the A8 GEMV reads (some of the M rows nonzero there)
    a8_live = {m: int((fhc[:m].view(torch.int8).view(m, F["N"] // 32, 32) != 0).any(dim=2).any(dim=0).sum().item())
               for m in D["Ms"]}
    peaks = measured_peaks(torch, dev)

    def graph_us(g, reps=20, launches=ROTATE):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps / launches
    read_us, launch_us = graph_us(read_graph), graph_us(launch_graph)
    # Inside the step the decode graphs follow the prefill GEMMs and take longer than alone; the read floor
    # is replayed there too (read_step_us), and every decode graph is timed again here, in the same quiet
    # phase as the floors, so that each floor fraction compares launches timed under the same conditions.
    read_step_us = times["decode_read_floor_graph"] / ROTATE
    q_gemv = {m: graph_us(graphs[m]) for m in D["Ms"]}
    q_glu = {m: graph_us(glu_graphs[m], launches=ROTATE_GLU) for m in D["Ms"]}
    q_cond = {m: graph_us(cond_graphs[m], launches=ROTATE_GLU) for m in D["Ms"]}
    q_cond_sparse = graph_us(cond_sparse_graph, launches=ROTATE_GLU)
    q_a8 = {m: graph_us(a8_graphs[m]) for m in D["Ms"]}
    peaks["decode_read_floor_us"] = round(read_us, 3)
    peaks["decode_read_floor_in_step_us"] = round(read_step_us, 3)
    peaks["decode_read_floor_gbs"] = round(D["N"] * D["K"] / 4 / (read_us * 1e-6) / 1e9, 1)
    peaks["launch_floor_us"] = round(launch_us, 3)
    peaks["how_floors"] = ("graph of 24 plain streaming reads of one packed 11008x4096 matrix (11.27 MB, the "
                           "decode rotation), and of 24 launches reading 16 bytes; microseconds per launch, "
                           "after the timed region; the read graph also runs inside the step, right before "
                           "the decode graphs (decode_read_floor_in_step_us)")
    # The eager sequence times each call between events on the launch stream, so a short quantizer's
    # figure there also holds the dispatch gap before it (every call is issued from Python). Here each
    # memory-bound quantizer runs back to back from a HIP graph, every launch on its own HBM copy of its
    # input, the copies together larger than the 256 MB last-level cache, so that no launch finds its
    # input in a cache: microseconds per launch.
    def spread(t, n=None):
        n = n or max(2, -(-(320 << 20) // (t.numel() * t.element_size())))    # at least 320 MiB in all
        return [t] + [t.clone() for _ in range(n - 1)]

    def per_launch_us(calls, reps=10):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for c in calls:
                c()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps / len(calls)
        del g
        return us

    pxs, fxs, fhs_in, axs = spread(px), spread(fx), spread(fh), spread(ax)
    kvxs = spread(py4, 6)          # six copies of the QKV output: five other 67 MB parts between two reads of one
    kq, kk = slice(0, kH * kD), slice(kH * kD, 2 * kH * kD)
    kvv = slice(2 * kH * kD, 3 * kH * kD)
    qgraph = {
        "quant_int4_e3m2_prefill": [lambda x=x: tw.bitlinear_quantize_act(x, "int4_e3m2", eps=EPS, codes=pc6, scale=ps6)
                                    for x in pxs],
        "quant_int4_prefill": [lambda x=x: tw.bitlinear_quantize_act(x, "int4", eps=EPS, codes=pc4, scale=ps4)
                               for x in pxs],
        "quant_fp4_prefill": [lambda x=x: tw.bitlinear_quantize_act(x, "fp4", eps=EPS, codes=pcf, scale=psf)
                              for x in pxs],
        "quant_fp4_pow2_prefill": [lambda x=x: tw.bitlinear_quantize_act(x, "fp4_pow2", eps=EPS, codes=pcp, scale=psp)
                                   for x in pxs],
        "quant_int4_per_tensor_prefill": [lambda x=x: tw.bitlinear_quantize_act_per_tensor(x, "int4", eps=EPS, codes=pct,
                                                                                          scale=pst, workspace=pws)
                                          for x in pxs],
        "quant_int4_e3m2_ffn": [lambda x=x: tw.bitlinear_quantize_act(x, "int4_e3m2", eps=EPS, codes=fc, scale=fs)
                                for x in fxs],
        "quant_int8_h": [lambda x=x: tw.bitlinear_quantize_act(x, "int8", eps=EPS, row_absmax_hint=frm, codes=fhc,
                                                               scale=fhs) for x in fhs_in],
        "quant_topk_int8_attn": [lambda x=x: tw.bitlinear_quantize_act(x, "int8", topk_keep=A["keep"], eps=EPS, codes=ac,
                                                                       scale=as_, mask=am) for x in axs],
        "kv_quant_q4_rope": [lambda x=x: tw.bitlinear_kv_quantize(x[:, kq], kH, kD, 4, eps=EPS, pos=kpos, cos=kcos,
                                                                  sin=ksin, codes=kq_c, scale=kq_s) for x in kvxs],
        "kv_quant_k3_rope_bos": [lambda x=x: tw.bitlinear_kv_quantize(x[:, kk], kH, kD, 3, eps=EPS, pos=kpos, cos=kcos,
                                                                      sin=ksin, bos_slot=kslot, n_bos_slots=knslots,
                                                                      codes=kk_c, scale=kk_s, bos_codes=kkb_c,
                                                                      bos_scale=kkb_s) for x in kvxs],
        "kv_quant_v3_bos": [lambda x=x: tw.bitlinear_kv_quantize(x[:, kvv], kH, kD, 3, eps=EPS, bos_slot=kslot,
                                                                 n_bos_slots=knslots, codes=kv_c, scale=kv_s,
                                                                 bos_codes=kvb_c, bos_scale=kvb_s) for x in kvxs],
    }
    q_graph_us = {n: per_launch_us(c) for n, c in qgraph.items()}
    del pxs, fxs, fhs_in, axs, kvxs, qgraph
    # live up rows of the conditional projection (channels whose gate is positive in some row)
    live = {m: int((dgs[m] > 0).any(dim=0).sum().item()) for m in D["Ms"]}
    live_sparse = int((dgsp > 0).any(dim=0).sum().item())

    # ------------------------------------------------------------------ algorithmic work per kernel
    Mp, Kp, Np = P["M"], P["K"], P["N"]
    ops_prefill = 2.0 * Mp * Np * Kp
    ops_glu = 2.0 * 2 * F["M"] * F["N"] * F["K"]
    h_codes = fhc.view(torch.int8)
    nnz_h = int((h_codes != 0).sum().item())
    nnz_attn = int((ac.view(torch.int8) != 0).sum().item())
    nnz_h_s = int((fhc_s.view(torch.int8) != 0).sum().item())
    nnz_attn_s = int((ac_s.view(torch.int8) != 0).sum().item())
    ops_down_alg = 2.0 * F["K"] * nnz_h
    ops_down_dense = 2.0 * F["M"] * F["N"] * F["K"]
    ops_oproj_alg = 2.0 * A["N"] * nnz_attn
    ops_oproj_dense = 2.0 * A["M"] * A["N"] * A["K"]
    wbytes = D["N"] * D["K"] / 4

    def dec_bytes(m):
        return wbytes + m * D["K"] / 2 + 4 * m + 4 + 4 * m * D["N"]      # weights + codes + scales + alpha + y

    def tops(ops, us):
        return ops / (us * 1e-6) / 1e12

    def gbs(b, us):
        return b / (us * 1e-6) / 1e9

    kern = {
        "quant_int4_e3m2_prefill": dict(us=times["quant_int4_e3m2_prefill"], bound="hbm",
                                        gbs=gbs(Mp * Kp * 2 + Mp * Kp * 0.75 + 4 * Mp,
                                                times["quant_int4_e3m2_prefill"])),
        "gemm_a4_int4_fp6_prefill": dict(us=times["gemm_a4_int4_fp6_prefill"], bound="mfma",
                                         tops=tops(ops_prefill, times["gemm_a4_int4_fp6_prefill"]),
                                         peak=FP4_PEAK_TOPS),
        "quant_int4_prefill": dict(us=times["quant_int4_prefill"], bound="hbm",
                                   gbs=gbs(Mp * Kp * 2 + Mp * Kp / 2 + 4 * Mp, times["quant_int4_prefill"])),
        "gemm_a4_int4_i8_prefill": dict(us=times["gemm_a4_int4_i8_prefill"], bound="mfma",
                                        tops=tops(ops_prefill, times["gemm_a4_int4_i8_prefill"]), peak=INT8_PEAK_TOPS),
        "quant_fp4_prefill": dict(us=times["quant_fp4_prefill"], bound="hbm",
                                  gbs=gbs(Mp * Kp * 2 + Mp * Kp / 2 + 4 * Mp, times["quant_fp4_prefill"])),
        "gemm_a4_fp4_prefill": dict(us=times["gemm_a4_fp4_prefill"], bound="mfma",
                                    tops=tops(ops_prefill, times["gemm_a4_fp4_prefill"]), peak=FP4_PEAK_TOPS),
        "quant_fp4_pow2_prefill": dict(us=times["quant_fp4_pow2_prefill"], bound="hbm",
                                       gbs=gbs(Mp * Kp * 2 + Mp * Kp / 2 + 4 * Mp, times["quant_fp4_pow2_prefill"])),
        # two passes over x: the tensor-wide exact sum, then the row quantizer with the given beta
        "quant_int4_per_tensor_prefill": dict(us=times["quant_int4_per_tensor_prefill"], bound="hbm",
                                              gbs=gbs(2 * Mp * Kp * 2 + Mp * Kp / 2 + 8 * Mp,
                                                      times["quant_int4_per_tensor_prefill"])),
        "quant_int4_e3m2_ffn": dict(us=times["quant_int4_e3m2_ffn"], bound="hbm",
                                    gbs=gbs(F["M"] * F["K"] * 2.75 + 4 * F["M"], times["quant_int4_e3m2_ffn"])),
        "gemm_a4_glu_ffn": dict(us=times["gemm_a4_glu_ffn"], bound="mfma",
                                tops=tops(ops_glu, times["gemm_a4_glu_ffn"]), peak=FP4_PEAK_TOPS),
        "quant_int8_h": dict(us=times["quant_int8_h"], bound="hbm",
                             gbs=gbs(F["M"] * F["N"] * 5 + 8 * F["M"], times["quant_int8_h"])),
        "gemm_a8_down": dict(us=times["gemm_a8_down"], bound="mfma",
                             tops=tops(ops_down_alg, times["gemm_a8_down"]),
                             dense_tops=tops(ops_down_dense, times["gemm_a8_down"]), peak=INT8_PEAK_TOPS),
        "quant_topk_int8_attn": dict(us=times["quant_topk_int8_attn"], bound="hbm",
                                     gbs=gbs(A["M"] * A["K"] * 3 + A["M"] * A["K"] / 8 + 4 * A["M"],
                                             times["quant_topk_int8_attn"])),
        "gemm_a8_oproj_residual": dict(us=times["gemm_a8_oproj_residual"], bound="mfma",
                                       tops=tops(ops_oproj_alg, times["gemm_a8_oproj_residual"]),
                                       dense_tops=tops(ops_oproj_dense, times["gemm_a8_oproj_residual"]),
                                       peak=INT8_PEAK_TOPS),
        "gemm_a8_down_structured": dict(us=times["gemm_a8_down_structured"], bound="mfma",
                                        tops=tops(2.0 * F["K"] * nnz_h_s, times["gemm_a8_down_structured"]),
                                        dense_tops=tops(ops_down_dense, times["gemm_a8_down_structured"]),
                                        peak=INT8_PEAK_TOPS, input="structured sparsity (labelled variant)"),
        "gemm_a8_oproj_residual_structured": dict(us=times["gemm_a8_oproj_residual_structured"], bound="mfma",
                                                  tops=tops(2.0 * A["N"] * nnz_attn_s,
                                                            times["gemm_a8_oproj_residual_structured"]),
                                                  dense_tops=tops(ops_oproj_dense,
                                                                  times["gemm_a8_oproj_residual_structured"]),
                                                  peak=INT8_PEAK_TOPS, input="structured sparsity (labelled variant)"),
    }
    for name, codes_t in (("gemm_a8_down", fhc), ("gemm_a8_oproj_residual", ac), ("gemm_a8_down_structured", fhc_s),
                          ("gemm_a8_oproj_residual_structured", ac_s)):
        z, zs = zero_slices(torch, codes_t)
        kern[name]["zero_16x128_slices"] = round(z, 4)
        kern[name]["skipped_16x128_slices"] = round(zs, 4)
    kv_rec = kT * kH

    def kv_bytes(bits, rope, bos):
        b = kv_rec * kD * 4 + kv_rec * (kD * bits / 8 + 4)                 # fp32 heads in, codes + scales out
        if rope:
            b += kT * (4 + kD * 4)                                         # position + cos/sin rows
        if bos:
            b += kT * 4 + knslots * kH * (kD / 2 + 4)                      # slots + 4-bit BOS records
        return b

    for n, bits, rope, bos in (("kv_quant_q4_rope", 4, True, False), ("kv_quant_k3_rope_bos", 3, True, True),
                               ("kv_quant_v3_bos", 3, False, True)):
        kern[n] = dict(us=times[n], bound="hbm", gbs=gbs(kv_bytes(bits, rope, bos), times[n]))
    unfused = times["gemm_a4_int4_fp6_prefill"] + sum(times[n] for n in ("kv_quant_q4_rope", "kv_quant_k3_rope_bos",
                                                                          "kv_quant_v3_bos"))
    kern["gemm_a4_qkv_kv_fused"] = dict(us=times["gemm_a4_qkv_kv_fused"], bound="mfma",
                                        tops=tops(ops_prefill, times["gemm_a4_qkv_kv_fused"]), peak=FP4_PEAK_TOPS,
                                        unfused_us=round(unfused, 3),
                                        speedup_vs_unfused=round(unfused / times["gemm_a4_qkv_kv_fused"], 3),
                                        what="INT4-on-FP6 QKV GEMM with RoPE and the Q4/K3/V3 (+BOS) KV quantizer "
                                             "in its epilogue, no fp32 output; unfused = GEMM + three KV kernels")
    for m in D["Ms"]:
        kern[f"decode_m{m}"] = dict(us=gemv_us[m], bound="hbm", gbs=gbs(dec_bytes(m), gemv_us[m]),
                                    us_quiet=q_gemv[m], gbs_quiet=gbs(dec_bytes(m), q_gemv[m]))
    for n, us in q_graph_us.items():
        k = kern[n]
        k["us_graph"] = us
        k["gbs_graph"] = k["gbs"] * k["us"] / us                 # the same algorithmic bytes
        k["frac_graph"] = round(k["gbs_graph"] / HBM_PEAK_GBS, 4)
    for k in kern.values():
        if "tops" in k:
            k["frac"] = round(k["tops"] / k["peak"], 4)
        else:
            k["frac"] = round(k["gbs"] / HBM_PEAK_GBS, 4)
        for f in ("us", "tops", "dense_tops", "gbs", "us_graph", "gbs_graph", "us_quiet", "gbs_quiet"):
            if f in k:
                k[f] = round(k[f], 3)

    head_us = times["gemm_a4_int4_fp6_prefill"]
    value = tops(ops_prefill, head_us)
    roofline = {"bound": "mfma", "achieved": round(value, 2), "peak": FP4_PEAK_TOPS, "unit": "TFLOP/s",
                "frac": round(value / FP4_PEAK_TOPS, 4), "traffic": measured_traffic(),
                "frac_of_int8_peak": round(value / INT8_PEAK_TOPS, 4),
                "frac_of_measured_peak": round(value / peaks["mfma_fp6_fp4_tops"], 4),
                "kernel": "k_gemm_mx<INT4_E3M2,NONE>: INT4 codes on FP6 x FP4 matrix cores "
                          "(prefill_qkv M=4096 K=4096 N=12288)",
                "avg_kernel_us": round(head_us, 3),
                "algorithmic": f"2*M*N*K = {ops_prefill:.4g} ops per launch"}
    # us / gbs / frac_hbm: inside the step; *_quiet: the same graph alone, beside the floors
    def quiet(d, b, us_q):
        d.update({"us_quiet": round(us_q, 3), "gbs_quiet": round(gbs(b, us_q), 1),
                  "frac_hbm_quiet": round(gbs(b, us_q) / HBM_PEAK_GBS, 4)})
        return d

    decode = {f"m{m}": quiet({"us": round(gemv_us[m], 3), "gbs": round(gbs(dec_bytes(m), gemv_us[m]), 1),
                              "frac_hbm": round(gbs(dec_bytes(m), gemv_us[m]) / HBM_PEAK_GBS, 4),
                              "frac_read_floor": round(read_us / q_gemv[m], 4),
                              "frac_read_floor_in_step": round(read_step_us / gemv_us[m], 4)},
                             dec_bytes(m), q_gemv[m]) for m in D["Ms"]}
    glu_w = F["N"] * F["K"] / 4

    def glu_bytes(m, rows_up):
        return glu_w + rows_up * F["K"] / 4 + m * F["K"] / 2 + 8 * m + 8 + 4 * m * F["N"] * (2 if rows_up < F["N"] else 1)

    for m in D["Ms"]:
        b_full, b_cond = glu_bytes(m, F["N"]), glu_bytes(m, live[m])
        decode[f"glu_full_m{m}"] = quiet({"us": round(glu_us[m], 3), "gbs": round(gbs(b_full, glu_us[m]), 1),
                                          "frac_hbm": round(gbs(b_full, glu_us[m]) / HBM_PEAK_GBS, 4)},
                                         b_full, q_glu[m])
        decode[f"glu_conditional_m{m}"] = quiet({
            "us": round(cond_us[m], 3), "gbs": round(gbs(b_cond, cond_us[m]), 1),
            "frac_hbm": round(gbs(b_cond, cond_us[m]) / HBM_PEAK_GBS, 4),
            "live_up_rows": round(live[m] / F["N"], 4), "speedup_vs_fused": round(glu_us[m] / cond_us[m], 3),
            "speedup_vs_fused_quiet": round(q_glu[m] / q_cond[m], 3)}, b_cond, q_cond[m])
    b_sp = glu_bytes(1, live_sparse)
    decode["glu_conditional_gate_sparse_m1"] = quiet({
        "us": round(cond_sparse_us, 3), "gbs": round(gbs(b_sp, cond_sparse_us), 1),
        "frac_hbm": round(gbs(b_sp, cond_sparse_us) / HBM_PEAK_GBS, 4),
        "live_up_rows": round(live_sparse / F["N"], 4), "speedup_vs_fused": round(glu_us[1] / cond_sparse_us, 3),
        "speedup_vs_fused_quiet": round(q_glu[1] / q_cond_sparse, 3),
        "input": "gate weights with a seeded share of the token's live channels negated, 32.5% left live "
                 "(the 67.5% gate sparsity the pages report for 7B); the fused GLU reads every row either way"},
        b_sp, q_cond_sparse)

    for m in D["Ms"]:
        b8 = a8_live[m] * 32 * F["K"] / 4 + m * F["N"] + 4 * m + 4 + 4 * m * F["K"]
        decode[f"a8_m{m}"] = quiet({"us": round(a8_us[m], 3), "gbs": round(gbs(b8, a8_us[m]), 1),
                                    "frac_hbm": round(gbs(b8, a8_us[m]) / HBM_PEAK_GBS, 4),
                                    "live_k_slices": round(a8_live[m] / (F["N"] // 32), 4)}, b8, q_a8[m])

    # whole BitLinear layers, quantizer and matmul together: consecutive launches on one stream, so the
    # sum of their event intervals is the layer's time on the stream (dispatch gaps included)
    def layer(parts, ops, what):
        us = sum(times[n] for n in parts)
        return {"us": round(us, 3), "tops": round(tops(ops, us), 2), "kernels": parts, "what": what}

    layers = {
        "prefill_qkv_int4_fp6": layer(["quant_int4_e3m2_prefill", "gemm_a4_int4_fp6_prefill"], ops_prefill,
                                      "per-token INT4 (E3M2 layout) + W1.58A4 GEMM on FP6 x FP4 cores"),
        "prefill_qkv_int4_int8core": layer(["quant_int4_prefill", "gemm_a4_int4_i8_prefill"], ops_prefill,
                                           "per-token INT4 (nibbles) + W1.58A4 GEMM on int8 cores"),
        "prefill_qkv_fp4": layer(["quant_fp4_prefill", "gemm_a4_fp4_prefill"], ops_prefill,
                                 "per-token FP4 E2M1 + W1.58A4 GEMM on FP4 cores"),
        "ffn_7b": layer(["quant_int4_e3m2_ffn", "gemm_a4_glu_ffn", "quant_int8_h", "gemm_a8_down"],
                        ops_glu + ops_down_dense,
                        "INT4 + gate/up GEMM with ReLU^2 GLU + INT8 of h + W1.58A8 down (dense-equivalent ops)"),
        "attn_out": layer(["quant_topk_int8_attn", "gemm_a8_oproj_residual"], ops_oproj_dense,
                          "Top-K 50% + INT8 + W1.58A8 o_proj with the residual (dense-equivalent ops)"),
    }
    sparsity = {"ffn_h_zero_codes": round(1 - nnz_h / (F["M"] * F["N"]), 4),
                "attn_zero_codes": round(1 - nnz_attn / (A["M"] * A["K"]), 4),
                "ffn_h_zero_codes_structured": round(1 - nnz_h_s / (F["M"] * F["N"]), 4),
                "attn_zero_codes_structured": round(1 - nnz_attn_s / (A["M"] * A["K"]), 4)}

    # ------------------------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.cpu_rows)

    out = {
        "metric": "W1.58A4 GEMM TOPS (% int8 MFMA peak) + decode GEMV GB/s (% HBM peak)",
        "value": round(value, 2),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6(e3m2) x fp4(e2m1) MFMA holding INT4 x ternary codes exactly, fp32 accumulate, fp32 epilogue",
        "data": "synthetic (seeded N(0,1) bf16 activations, N(0,0.02) latent weights, outlier channels)",
        "config": {"workload": "prefill_qkv: W1.58A4 BitLinear M=4096 K=4096 N=12288 (fused QKV, 7B-shaped)",
                   "step": "all hot-path operations: prefill INT4+FP4, ffn_7b, attn_out, KV-cache quantize "
                           "(Q4/K3/V3 of the prefill QKV output), decode M=1/4/8",
                   "global_batch": P["M"], "seq_len": None, "parallelism": "none (1 GPU)"},
        "roofline": roofline,
        "measured_peaks": peaks,
        "decode_gemv": decode,
        "kernels": kern,
        "layers": layers,
        "sparsity": sparsity,
        "cpu_baseline": cpu,
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(out), flush=True)


def zero_slices(torch, codes):
    """Fractions of the 16-row x 128-column slices of INT8 codes that are all zero, and of those the A8 GEMM
    skips (every 16-row subtile except the first of each 64-row wave strip, which also expands the weights)."""
    c = codes.view(torch.int8)
    M_, K_ = c.shape
    z = (c[: M_ // 16 * 16].view(M_ // 16, 16, K_ // 128, 128) != 0).any(dim=3).any(dim=1).logical_not()
    skippable = (torch.arange(M_ // 16, device=c.device) % 4 != 0)[:, None]
    return float(z.float().mean().item()), float((z & skippable).float().mean().item())


def measured_peaks(torch, dev):
    """What this GPU sustains, beside the datasheet peaks: a 256 MiB device-to-device copy (bytes read
    plus written per second) and the library's FP6 x FP4 matrix-core-only loop in the GEMM's wave
    shape (two 256-thread blocks per CU), each the best of three timed runs after a warm-up."""
    import ternary_weight_quantized_amd as tw

    def best_us(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            best = min(best, e0.elapsed_time(e1) * 1e3)
        return best
    src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    copy_us = best_us(lambda: dst.copy_(src))
    del src, dst
    blocks = 2 * torch.cuda.get_device_properties(dev).multi_processor_count
    iters = 4000
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    mfma_us = best_us(lambda: tw.bitlinear_calibrate_mfma(blocks, iters, out=out))
    # thread 0 of every block: shader-clock ticks per 100 MHz real-time tick over its loop
    clk = out.view(blocks, 256)[:, 0].double()
    return {"hbm_copy_gbs": round(2 * (256 << 20) / (copy_us * 1e-6) / 1e9, 1),
            "mfma_fp6_fp4_tops": round(blocks * iters * 8388608 / (mfma_us * 1e-6) / 1e12, 1),
            "mfma_clock_ghz": round(float(clk.mean().item()) * 0.1, 3),
            "how": "256 MiB device copy (read + write bytes); FP6 x FP4 MFMA-only loop on operands with the "
                   "GEMM's statistics (ternary E2M1 weights, bell-shaped INT4 codes in E3M2, eight weight and four "
                   f"activation sets alternating), {blocks} blocks x 4 waves x {iters} x 32 MFMAs 16x16x128, best of "
                   "3 after a warm-up; the clock is the mean shader-clock rate over the blocks' loops"}


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(rows, rows_single=256, min_seconds=10.0, min_seconds_single=6.0, max_reps=30):
    """The oracle as it stands (its integer GEMM is a float64 BLAS matmul of the codes), on the first
    `rows` tokens of the prefill workload with all the threads BLAS uses, and on `rows_single` tokens
    with one thread (quantize + exact integer GEMM + dequantization), each repeated until about
    `min_seconds` of CPU work has been timed; the weights are ternarized beforehand (offline in the
    method)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O
    from synth import WORKLOADS, bf16_bits_to_f32, workload_inputs
    P = WORKLOADS["prefill_qkv"]
    inp = workload_inputs("prefill_qkv")
    t, alpha = O.ternarize(inp["w"], EPS)

    def run(nrows, min_s):
        x = bf16_bits_to_f32(inp["x"][:nrows])
        reps, dt = 0, 0.0
        while reps < max_reps and (reps == 0 or dt < min_s):
            t0 = time.perf_counter()
            O.bitlinear_a4(x, t, alpha, EPS)
            dt += time.perf_counter() - t0
            reps += 1
        return 2.0 * nrows * P["N"] * P["K"] * reps / dt / 1e12, reps, dt

    v_all, reps, dt = run(rows, min_seconds)
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    with threadpool_limits(limits=1):
        v_one, reps1, dt1 = run(rows_single, min_seconds_single)
    return {"value": round(v_all, 5), "unit": "TOPS", "cores": int(threads), "kind": "oracle",
            "sample": f"oracle.bitlinear_a4 (INT4; its integer GEMM is a BLAS float64 matmul of the codes) on "
                      f"{rows} of the 4096 prefill tokens, N=12288, K=4096, {reps} passes: {dt:.2f} s",
            "single_thread": {"value": round(v_one, 5), "unit": "TOPS", "cores": 1,
                              "sample": f"the same on {rows_single} tokens, one BLAS thread, {reps1} passes: "
                                        f"{dt1:.2f} s"},
            "host_cpu": host_cpu_model(), "host_cpus": os.cpu_count()}


if __name__ == "__main__":
    main()
