"""Minimal driver for hardware-counter runs of one BitLinear GEMM (no graphs, few launches).

    python -m ternary_weight_quantized_amd.profile_run --gemm fp6 --reps 3 --copy-calibration

quantizes the prefill workload (M=4096, K=4096, N=12288, seeded synthetic bf16 activations and
latent weights) and launches the selected GEMM `reps` times. With --copy-calibration a 256 MiB
device-to-device copy runs first; its FETCH_SIZE and WRITE_SIZE readings give the factor that
turns those counters into bytes.
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


def main():
    p = argparse.ArgumentParser()
    p.add_argument("--gemm", choices=sorted(FORMATS), default="fp6")
    p.add_argument("--reps", type=int, default=3)
    p.add_argument("--copy-calibration", action="store_true")
    args = p.parse_args()

    import numpy as np
    import torch

    import ternary_weight_quantized_amd as tw
    from synth import WORKLOADS, workload_inputs

    tw.library()
    P = WORKLOADS["prefill_qkv"]
    inp = workload_inputs("prefill_qkv")
    x = torch.from_numpy(np.ascontiguousarray(inp["x"]).view(np.int16)).view(torch.bfloat16).cuda()
    packed, alpha = tw.bitlinear_pack_ternary(torch.from_numpy(inp["w"]).cuda(), EPS)
    fmt = FORMATS[args.gemm]
    codes, scale, _ = tw.bitlinear_quantize_act(x, fmt, eps=EPS)
    y = torch.empty((P["M"], P["N"]), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.reps):
        tw.bitlinear_gemm_w158a4(fmt, codes, scale, P["K"], packed, alpha, P["N"], y=y)
    torch.cuda.synchronize()
    print(f"profile_run: {args.reps} x {fmt} GEMM M={P['M']} K={P['K']} N={P['N']}", flush=True)


if __name__ == "__main__":
    main()
