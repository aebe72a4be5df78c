#!/usr/bin/env python3
"""Benchmark of the fused NF4 QLoRA linear layer on one MI355X.

One step = one forward + backward of the layer on the "down" workload (a Llama down_proj training
step: X bf16 [16384, 14336], W NF4 [4096, 14336] with double-quantised absmax, LoRA r = 32, s = 1,
dY ~ N(0, 1e-2)): T = X A^T, Y = X deq(W)^T + s T B^T, then U = dY B, dX, dA, dB. Inputs are
seeded synthetic tensors of that shape, resident in HBM before timing starts; W is quantised once
(untimed), as a frozen base weight is.

Output: one JSON line with the whole-step throughput (algorithmic matmul flops / step time), the
roofline of the dominant kernel (the fused dequant-GEMM-LoRA forward, timed with HIP events on
the stream it runs on) and the CPU oracle timed on a bounded row sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload down] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused QLoRA fwd+bwd TFLOP/s and weight-stream GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="down")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the CPU oracle sample")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Layer:
    """Preallocated device buffers and direct C-ABI calls for one workload."""

    def __init__(self, w, dev):
        import torch
        import nf4_dequant_gemm_amd as lib
        import workloads as wl
        self.w, self.lib, self.c = w, lib, lib.library()
        t0 = time.time()
        host = {t: wl.tensor(w, t) for t in ("X", "W", "A", "B")}
        if w.backward:
            host["dY"] = wl.tensor(w, "dY")
        log(f"inputs generated in {time.time() - t0:.1f}s")
        self.X = host["X"].to(dev)
        self.A = host["A"].to(dev)
        self.B = host["B"].to(dev)
        self.dY = host["dY"].to(dev) if w.backward else None
        self.q = lib.nf4_quantize(host["W"].to(dev), w.dq_block)
        del host
        M, N, K, r = w.M, w.N, w.K, w.r
        bf = torch.bfloat16
        self.Y = torch.empty(M, N, dtype=bf, device=dev)
        self.T = torch.empty(M, r, dtype=bf, device=dev)
        self.fws = self.c.qlora_fwd_workspace_bytes(M, N, K, r)
        self.ws_f = torch.empty(max(self.fws, 1), dtype=torch.uint8, device=dev)
        if w.backward:
            self.dX = torch.empty(M, K, dtype=bf, device=dev)
            self.dA = torch.empty(r, K, dtype=bf, device=dev)
            self.dB = torch.empty(N, r, dtype=bf, device=dev)
            self.bws = self.c.qlora_bwd_workspace_bytes(M, N, K, r)
            self.ws_b = torch.empty(max(self.bws, 1), dtype=torch.uint8, device=dev)
        self.qs = self.q.c_struct()
        self.stream = torch.cuda.current_stream(dev)
        self.sp = ctypes.c_void_p(self.stream.cuda_stream)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        self.p = {k: p(v) for k, v in self.__dict__.items() if isinstance(v, torch.Tensor)}

    def check(self, st):
        if st != 0:
            raise RuntimeError(self.c.nf4_last_error().decode())

    def lora_down(self):
        w, p = self.w, self.p
        self.check(self.c.qlora_lora_down(p["X"], w.M, w.K, p["A"], w.r, p["T"], p["ws_f"], self.fws, self.sp))

    def fwd_fused(self):
        w, p = self.w, self.p
        self.check(self.c.qlora_fwd_fused(p["X"], w.M, ctypes.byref(self.qs), p["T"], p["B"], w.r,
                                          w.s, p["Y"], self.sp))

    def bwd(self):
        w, p = self.w, self.p
        self.check(self.c.qlora_bwd(p["dY"], p["X"], w.M, ctypes.byref(self.qs), p["A"], p["B"], w.r,
                                    w.s, p["T"], p["dX"], p["dA"], p["dB"], p["ws_b"], self.bws, self.sp))


def run_gpu(args, w):
    import torch
    dev = torch.device("cuda:0")
    L = Layer(w, dev)
    for _ in range(args.warmup):
        L.lora_down()
        L.fwd_fused()
        if w.backward:
            L.bwd()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        e = ev[s]
        e[0].record(L.stream)
        L.lora_down()
        e[1].record(L.stream)
        L.fwd_fused()
        e[2].record(L.stream)
        if w.backward:
            L.bwd()
        e[3].record(L.stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = lambda a, b: sum(ev[s][a].elapsed_time(ev[s][b]) for s in range(args.steps)) / args.steps
    return {
        "ms_per_step": (t1 - t0) * 1e3 / args.steps,
        "lora_down_ms": ms(0, 1), "fused_fwd_ms": ms(1, 2), "bwd_ms": ms(2, 3), "event_step_ms": ms(0, 3),
    }


def run_cpu_baseline(w, target_s):
    """The oracle (float64 numpy/BLAS) on a row sample of the same step."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import workloads as wl
    from oracle import nf4, qlora
    W = wl.tensor(w, "W").float().numpy()
    Wd = nf4.dequantize_f32(nf4.quantize(W, w.dq_block))
    A, B = wl.tensor(w, "A").float().numpy(), wl.tensor(w, "B").float().numpy()

    Xall = wl.tensor(w, "X").float().numpy()
    dYall = wl.tensor(w, "dY").float().numpy() if w.backward else None

    def step(rows):
        X = Xall[:rows]
        dY = dYall[:rows] if w.backward else None
        t = time.perf_counter()
        qlora.forward(X, Wd, A, B, w.s)
        if w.backward:
            qlora.backward(dY, X, Wd, A, B, w.s)
        return time.perf_counter() - t

    rows = min(64, w.M)
    dt = step(rows)
    while dt < 0.4 * target_s and rows < w.M:       # grow the sample until it takes ~target_s
        rows = int(min(w.M, max(2 * rows, rows * target_s / max(dt, 1e-3))))
        rows = max(64, rows // 64 * 64) if w.M >= 64 else w.M
        dt = step(rows)
    flops = (w.fwd_flops() + (w.bwd_flops() if w.backward else 0)) * rows / w.M
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{rows} of {w.M} rows of the {w.name} workload, forward+backward in float64 "
                      f"(numpy/BLAS), {dt:.1f}s wall; W dequantised once outside the timing"}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    import workloads as wl
    w = wl.WORKLOADS[args.workload]
    g = run_gpu(args, w)
    flops = w.fwd_flops() + (w.bwd_flops() if w.backward else 0)
    value = flops / (g["ms_per_step"] * 1e-3) / 1e12
    fused_flops = 2 * w.M * w.N * w.K + 2 * w.M * w.N * w.r
    achieved = fused_flops / (g["fused_fwd_ms"] * 1e-3) / 1e12
    log(json.dumps(g))
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(g["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: X [{w.M},{w.K}] bf16, W NF4 [{w.N},{w.K}] block 64"
                               f"{' double-quant int8/256' if w.dq_block else ' fp32 absmax'}, "
                               f"LoRA r={w.r} s={w.s}, {'fwd+bwd' if w.backward else 'fwd'}",
                   "M": w.M, "K": w.K, "N": w.N, "r": w.r,
                   "phase_ms": {k: round(v, 4) for k, v in g.items() if k != "ms_per_step"}},
        "roofline": {"kernel": "qlora_fwd_fused (fused NF4-dequant GEMM + LoRA, one launch)",
                     "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = run_cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
