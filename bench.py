#!/usr/bin/env python3
"""Benchmark of the fused NF4 QLoRA linear layer on one MI355X.

One step = one forward + backward of the layer on the "down" workload (a Llama down_proj training
step: X bf16 [16384, 14336], W NF4 [4096, 14336] with double-quantised absmax, LoRA r = 32, s = 1,
dY ~ N(0, 1e-2)):

    qlora_lora_down   T = X A^T
    qlora_fwd_fused   Y = X deq(W)^T + s T B^T             (one launch)
    qlora_bwd (dX=0)  U = dY B, dA = s U^T X, dB = s dY^T T
    qlora_bwd_dx      dX = dY deq(W) + s U A                (one launch)

Inputs are seeded synthetic tensors of that shape, resident in HBM before timing starts. W is
quantised once (untimed), as a frozen base weight is, and then copied so that the steps rotate
over enough distinct copies (>= 512 MB together) that no step finds its weight in the 256 MB
last-level cache or the L2 left there by the step before (the weight is the only input read by
every step; X and dY of the large workloads are far larger than the caches).

Output: one JSON line with the whole-step throughput (algorithmic matmul flops / step time on the
host clock), the roofline of the dominant kernel (the larger of the two fused dequant-GEMM
launches, timed with HIP events on the stream it runs on), the weight-stream rate of the
decode-shaped forward (M = 16, K = 8192, N = 28672: weight-stream bytes / whole qlora_fwd time)
the CPU oracle timed on a bounded row sample of the same workload, and (context) measured-achievable
references on this machine: the vendor bf16 GEMM and the unfused forward on the same data for the
matrix-core-bound shapes, a device copy for the HBM-bound one.

    python bench.py [--steps K] [--warmup W] [--workload down] [--no-cpu-baseline]
                    [--no-weight-stream] [--copy-calibration]

--workload mlp_swiglu measures the gate/up SwiGLU pair instead (a step: qlora_swiglu_fwd +
qlora_swiglu_bwd on the mlp_up shape, two projections); --workload moe_mlp_up the grouped
mixture-of-experts layer (a step: qlora_moe_fwd + qlora_moe_bwd, 8 experts of the mlp_up shape,
16384 routed rows); --workload mlp_up_e2m1 the single layer of the mlp_up shape with an E2M1 base
weight (4-bit floats, E4M3 scale per 16, float32 tensor scale) instead of NF4.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import sys
import time
import types

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused QLoRA fwd+bwd TFLOP/s and weight-stream GB/s, % of MI355X roofline"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
COLD_BYTES = 512 << 20        # rotate weight copies until they add up to this
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {"qlora_fwd_fused": "fwd.hip", "qlora_bwd_dx": "dx.hip",
                  "qlora_fwd_fused (decode)": "decode16.hip"}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="down")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the vendor-GEMM / device-copy reference measurements")
    ap.add_argument("--no-weight-stream", action="store_true",
                    help="skip the decode-shaped weight-stream measurement")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target wall time of the CPU oracle sample")
    ap.add_argument("--wcopies", type=int, default=0,
                    help="distinct weight copies to rotate over (0: enough for 512 MB)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pct(vals, q):
    v = sorted(vals)
    i = min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))
    return v[i]


class Layer:
    """Preallocated device buffers and direct C-ABI calls for one workload."""

    def __init__(self, w, dev, wcopies=0):
        import torch
        import nf4_dequant_gemm_amd as lib
        import workloads as wl
        self.w, self.lib, self.c = w, lib, lib.library()
        t0 = time.time()
        host = {t: wl.tensor(w, t) for t in ("X", "W", "A", "B")}
        if w.backward:
            host["dY"] = wl.tensor(w, "dY")
        log(f"{w.name}: inputs generated in {time.time() - t0:.1f}s")
        self.X = host["X"].to(dev)
        self.A = host["A"].to(dev)
        self.B = host["B"].to(dev)
        self.dY = host["dY"].to(dev) if w.backward else None
        q = (lib.fp4_quantize(host["W"].to(dev)) if w.fmt == "e2m1"
             else lib.nf4_quantize(host["W"].to(dev), w.dq_block))
        del host
        n = wcopies or max(1, min(64, math.ceil(COLD_BYTES / w.weight_stream_bytes())))
        self.copies = [q] + [q.clone() for _ in range(n - 1)]
        self.qs = [c.c_struct() for c in self.copies]
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
        self.stream = torch.cuda.current_stream(dev)
        self.sp = ctypes.c_void_p(self.stream.cuda_stream)
        p = lambda t: ctypes.c_void_p(t.data_ptr())
        self.p = {k: p(v) for k, v in self.__dict__.items() if isinstance(v, torch.Tensor)}

    def check(self, st):
        if st != 0:
            raise RuntimeError(self.c.nf4_last_error().decode())

    def lora_down(self, i):
        w, p = self.w, self.p
        self.check(self.c.qlora_lora_down(p["X"], w.M, w.K, p["A"], w.r, p["T"], p["ws_f"], self.fws, self.sp))

    def fwd_fused(self, i):
        w, p = self.w, self.p
        self.check(self.c.qlora_fwd_fused(p["X"], w.M, ctypes.byref(self.qs[i % len(self.qs)]), p["T"],
                                          p["B"], w.r, w.s, p["Y"], self.sp))

    def fwd_whole(self, i):
        """The whole forward call (T pre-pass and fused kernel), as a caller makes it."""
        w, p = self.w, self.p
        self.check(self.c.qlora_fwd(p["X"], w.M, ctypes.byref(self.qs[i % len(self.qs)]), p["A"], p["B"],
                                    w.r, w.s, p["Y"], p["T"], p["ws_f"], self.fws, self.sp))

    def bwd_lora(self, i):
        """U (left at the start of the workspace), dA and dB: qlora_bwd without dX."""
        w, p = self.w, self.p
        self.check(self.c.qlora_bwd(p["dY"], p["X"], w.M, ctypes.byref(self.qs[i % len(self.qs)]), p["A"],
                                    p["B"], w.r, w.s, p["T"], None, p["dA"], p["dB"], p["ws_b"], self.bws,
                                    self.sp))

    def bwd_dx(self, i):
        w, p = self.w, self.p
        self.check(self.c.qlora_bwd_dx(p["dY"], w.M, ctypes.byref(self.qs[i % len(self.qs)]), p["ws_b"],
                                       p["A"], w.r, w.s, p["dX"], self.sp))


PHASES = ("lora_down", "fwd_fused", "bwd_lora", "bwd_dx")


def time_layer(L, steps, warmup):
    """Run warmup + steps steps; per-phase HIP-event times (ms) and the host-clock step time."""
    import torch
    w = L.w
    calls = [L.lora_down, L.fwd_fused] + ([L.bwd_lora, L.bwd_dx] if w.backward else [])
    for i in range(warmup):
        for c in calls:
            c(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        e = ev[s]
        e[0].record(L.stream)
        for j, c in enumerate(calls):
            c(warmup + s)
            e[j + 1].record(L.stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    per = {}
    for j in range(len(calls)):
        v = [ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(steps)]
        per[PHASES[j]] = {"mean": sum(v) / len(v), "median": pct(v, 0.5), "p10": pct(v, 0.1),
                          "p90": pct(v, 0.9)}
    return (t1 - t0) * 1e3 / steps, per


def time_call(L, fn, steps, warmup):
    """HIP-event times (ms) of one call over rotating weight copies: median, p10, p90."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for s, (a, b) in enumerate(ev):
        a.record(L.stream)
        fn(warmup + s)
        b.record(L.stream)
    torch.cuda.synchronize()
    v = [a.elapsed_time(b) for a, b in ev]
    return {"median": pct(v, 0.5), "p10": pct(v, 0.1), "p90": pct(v, 0.9)}


def source_sha(name):
    path = os.path.join(ROOT, "nf4_dequant_gemm_amd", "csrc", KERNEL_SOURCES[name])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def traffic_for(name, workload):
    """HBM bytes per launch from the committed counter summary, if it still matches the source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f).get(f"{name}@{workload}")
    except (OSError, ValueError):
        return None
    if not t or t.get("sha256") != source_sha(name):
        return None
    return t.get("bytes_per_launch")


def run_weight_stream(dev, steps, warmup):
    """Decode-shaped forward (M = 16): weight-stream bytes / whole qlora_fwd time, cold weights."""
    import workloads as wl
    w = wl.WORKLOADS["decode"]
    L = Layer(w, dev)
    _, per = time_layer(L, steps, warmup)
    fwd_ms = time_call(L, L.fwd_whole, steps, warmup)["median"]
    wb = w.weight_stream_bytes()
    gbs = wb / (fwd_ms * 1e-3) / 1e9
    kern = wb / (per["fwd_fused"]["median"] * 1e-3) / 1e9
    out = {"workload": f"decode: X [16,8192] bf16, W NF4 [28672,8192] double-quant int8/256, LoRA r=16, fwd",
           "weight_stream_bytes": wb, "qlora_fwd_us": round(fwd_ms * 1e3, 2),
           "value": round(gbs, 1), "unit": "GB/s", "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
           "fused_kernel_us": round(per["fwd_fused"]["median"] * 1e3, 2),
           "fused_kernel_GBps": round(kern, 1),
           "cold": f"{len(L.copies)} rotating weight copies"}
    del L
    return out


def run_merge(L, steps, warmup):
    """LoRA merge of the workload's weight (qlora_merge, W' = bf16(deq(W) + s B A)), cold weights:
    bytes moved (weight stream + A, B read; W' written) / HIP-event time, against HBM."""
    import torch
    w, c = L.w, L.c
    out = torch.empty(w.N, w.K, dtype=torch.bfloat16, device=L.X.device)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def fn(i):
        L.check(c.qlora_merge(ctypes.byref(L.qs[i % len(L.qs)]), P(L.A), P(L.B), w.r, w.s, P(out), L.sp))
    t = time_call(L, fn, steps, warmup)
    nbytes = w.weight_stream_bytes() + 2 * w.r * w.K + 2 * w.N * w.r + 2 * w.N * w.K
    gbs = nbytes / (t["median"] * 1e-3) / 1e9
    del out
    return {"what": f"qlora_merge of the {w.name} weight [{w.N},{w.K}], r={w.r}: W' = bf16(deq(W) + s B A)",
            "us": round(t["median"] * 1e3, 2), "bytes": nbytes, "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def run_cpu_baseline(w, target_s):
    """The oracle (float64 numpy/BLAS) on a row sample of the same step."""
    from threadpoolctl import threadpool_info

    import workloads as wl
    from oracle import nf4, qlora
    W = wl.tensor(w, "W").float().numpy()
    if w.fmt == "e2m1":
        from oracle import fp4
        Wd = fp4.dequantize_f32(fp4.quantize(W))
    else:
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
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "cpu": model, "wall_s": round(dt, 2),
            "sample": f"{rows} of {w.M} rows of the {w.name} workload, forward+backward in float64 "
                      f"(numpy/BLAS), {dt:.1f}s wall; W dequantised once outside the timing"}


def run_pair(args, pw, dev):
    """The gate/up SwiGLU pair (qlora_swiglu_fwd + qlora_swiglu_bwd per step) on pair workload pw."""
    import torch
    import nf4_dequant_gemm_amd as lib
    import workloads as wl
    c = lib.library()
    M, K, N, r, s = pw.M, pw.K, pw.N, pw.r, pw.s
    host = {t: wl.pair_tensor(pw, t) for t in ("X", "Wgu", "Agu", "Bg", "Bu", "dH")}
    d = {t: v.to(dev) for t, v in host.items() if t != "Wgu"}
    q = lib.nf4_quantize(host["Wgu"].to(dev), pw.dq_block)
    del host
    ncopies = args.wcopies or max(1, min(64, math.ceil(COLD_BYTES / pw.weight_stream_bytes())))
    copies = [q] + [q.clone() for _ in range(ncopies - 1)]
    qs = [x.c_struct() for x in copies]
    bf = torch.bfloat16
    H = torch.empty(M, N, dtype=bf, device=dev)
    Ygu = torch.empty(M, 2 * N, dtype=bf, device=dev)
    Tgu = torch.empty(M, 2 * r, dtype=bf, device=dev)
    dX = torch.empty(M, K, dtype=bf, device=dev)
    dAgu = torch.empty(2 * r, K, dtype=bf, device=dev)
    dBg = torch.empty(N, r, dtype=bf, device=dev)
    dBu = torch.empty(N, r, dtype=bf, device=dev)
    wsb = c.qlora_swiglu_workspace_bytes(M, N, K, r)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def check(st):
        if st != 0:
            raise RuntimeError(c.nf4_last_error().decode())

    def fwd(i):
        check(c.qlora_swiglu_fwd(P(d["X"]), M, ctypes.byref(qs[i % ncopies]), P(d["Agu"]), P(d["Bg"]),
                                 P(d["Bu"]), r, s, P(H), P(Ygu), P(Tgu), P(ws), wsb, sp))

    def bwd(i):
        check(c.qlora_swiglu_bwd(P(d["dH"]), P(d["X"]), M, ctypes.byref(qs[i % ncopies]), P(d["Agu"]),
                                 P(d["Bg"]), P(d["Bu"]), r, s, P(Ygu), P(Tgu), P(dX), P(dAgu), P(dBg),
                                 P(dBu), P(ws), wsb, sp))

    calls = (fwd, bwd)
    for i in range(args.warmup):
        for f in calls:
            f(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for st in range(args.steps):
        ev[st][0].record(stream)
        for j, f in enumerate(calls):
            f(args.warmup + st)
            ev[st][j + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    per = {}
    for j, name in enumerate(("swiglu_fwd", "swiglu_bwd")):
        v = [ev[st][j].elapsed_time(ev[st][j + 1]) for st in range(args.steps)]
        per[name] = {"mean": sum(v) / len(v), "median": pct(v, 0.5), "p10": pct(v, 0.1), "p90": pct(v, 0.9)}
    # The dominant launch: the fused forward of the stacked layer ([Wg; Wu] with the block-diagonal
    # up projection), timed on its own with T from the forward. qlora_swiglu_fwd runs the same
    # GEMM in the kernel's pair form, which adds the activation to the epilogue; the plain
    # stacked launch is the one the C ABI exposes alone.
    B2 = torch.zeros(2 * N, 2 * r, dtype=bf, device=dev)
    B2[:N, :r] = d["Bg"]
    B2[N:, r:] = d["Bu"]

    def fused(i):
        check(c.qlora_fwd_fused(P(d["X"]), M, ctypes.byref(qs[i % ncopies]), P(Tgu), P(B2), 2 * r, s,
                                P(Ygu), sp))
    t = time_call(types.SimpleNamespace(stream=stream), fused, args.steps, args.warmup)
    work = 2 * M * (2 * N) * K + 2 * M * (2 * N) * (2 * r)
    achieved = work / (t["median"] * 1e-3) / 1e12
    roof = {"kernel": "qlora_fwd_fused (stacked gate/up; the pair's own launch adds the activation epilogue)", "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "kernel_us": {k: round(v * 1e3, 2) for k, v in t.items()}, "traffic": None}
    context = None
    if not args.no_context:
        Wd = lib.nf4_dequantize(q, torch.bfloat16)
        context = {"mfma_loop": run_mfma_loop(Wd, d["X"])}
        roof["frac_of_mfma_loop"] = round(achieved / context["mfma_loop"]["TFLOP/s"], 4)
        del Wd
    del copies, qs, d, H, Ygu, Tgu, dX, dAgu, dBg, dBu, ws, B2
    torch.cuda.empty_cache()
    flops = pw.fwd_flops() + pw.bwd_flops()
    out = {
        "metric": METRIC, "value": round(flops / (step_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{pw.name}: gate/up pair, X [{M},{K}] bf16, W NF4 [{N},{K}] x 2 (stacked) "
                               f"double-quant int8/256, LoRA r={r} x 2 s={s}, H = silu(Yg) * Yu, fwd+bwd",
                   "M": M, "K": K, "N": N, "r": r, "weight_copies": ncopies,
                   "phase_ms": {k: {x: round(y, 4) for x, y in v.items()} for k, v in per.items()}},
        "roofline": roof,
    }
    if context:
        out["context"] = context
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = run_pair_cpu_baseline(pw, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def run_moe(args, mw, dev):
    """The grouped MoE layer (qlora_moe_fwd + qlora_moe_bwd per step) on MoE workload mw."""
    import torch
    import nf4_dequant_gemm_amd as lib
    import workloads as wl
    c = lib.library()
    E, M, K, N, r, s = mw.E, mw.M, mw.K, mw.N, mw.r, mw.s
    counts = mw.counts()
    cnt = (ctypes.c_int64 * E)(*counts)
    host = {t: wl.moe_tensor(mw, t) for t in ("X", "W", "A", "B", "dY")}
    d = {t: v.to(dev) for t, v in host.items() if t != "W"}
    q = lib.nf4_quantize(host["W"].to(dev), mw.dq_block)
    del host
    ncopies = args.wcopies or max(1, min(64, math.ceil(COLD_BYTES / mw.weight_stream_bytes())))
    copies = [q] + [q.clone() for _ in range(ncopies - 1)]
    qs = [x.c_struct() for x in copies]
    bf = torch.bfloat16
    Y = torch.empty(M, N, dtype=bf, device=dev)
    T = torch.empty(M, r, dtype=bf, device=dev)
    dX = torch.empty(M, K, dtype=bf, device=dev)
    dA = torch.empty(E * r, K, dtype=bf, device=dev)
    dB = torch.empty(E * N, r, dtype=bf, device=dev)
    wsb = c.qlora_moe_workspace_bytes(cnt, E, N, K, r)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def check(st):
        if st != 0:
            raise RuntimeError(c.nf4_last_error().decode())

    def fwd(i):
        check(c.qlora_moe_fwd(P(d["X"]), cnt, E, ctypes.byref(qs[i % ncopies]), P(d["A"]), P(d["B"]), r, s,
                              P(Y), P(T), P(ws), wsb, sp))

    def bwd(i):
        check(c.qlora_moe_bwd(P(d["dY"]), P(d["X"]), cnt, E, ctypes.byref(qs[i % ncopies]), P(d["A"]),
                              P(d["B"]), r, s, P(T), P(dX), P(dA), P(dB), P(ws), wsb, sp))

    calls = (fwd, bwd)
    for i in range(args.warmup):
        for f in calls:
            f(i)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for st in range(args.steps):
        ev[st][0].record(stream)
        for j, f in enumerate(calls):
            f(args.warmup + st)
            ev[st][j + 1].record(stream)
    torch.cuda.synchronize()
    step_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    per = {}
    for j, name in enumerate(("moe_fwd", "moe_bwd")):
        v = [ev[st][j].elapsed_time(ev[st][j + 1]) for st in range(args.steps)]
        per[name] = {"mean": sum(v) / len(v), "median": pct(v, 0.5), "p10": pct(v, 0.1), "p90": pct(v, 0.9)}

    # The dominant forward launch: the grouped fused kernel (every expert's tiles), given T.
    def fused(i):
        check(c.qlora_moe_fwd_fused(P(d["X"]), cnt, E, ctypes.byref(qs[i % ncopies]), P(T), P(d["B"]), r, s,
                                    P(Y), sp))
    t = time_call(types.SimpleNamespace(stream=stream), fused, args.steps, args.warmup)
    work = 2 * M * N * K + 2 * M * N * r
    achieved = work / (t["median"] * 1e-3) / 1e12
    roof = {"kernel": "qlora_moe_fwd_fused (grouped)", "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "kernel_us": {k: round(v * 1e3, 2) for k, v in t.items()}, "traffic": None}
    context = None
    if not args.no_context:
        Wd = lib.nf4_dequantize(q, torch.bfloat16)[:N]
        context = {"mfma_loop": run_mfma_loop(Wd, d["X"])}
        roof["frac_of_mfma_loop"] = round(achieved / context["mfma_loop"]["TFLOP/s"], 4)
        del Wd
    del copies, qs, d, Y, T, dX, dA, dB, ws
    torch.cuda.empty_cache()
    flops = mw.fwd_flops() + mw.bwd_flops()
    out = {
        "metric": METRIC, "value": round(flops / (step_ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{mw.name}: {E} experts, {mw.tokens} tokens x top-{mw.top_k} = {M} rows "
                               f"grouped by expert, X [{M},{K}] bf16, W NF4 [{E}x{N},{K}] double-quant "
                               f"int8/256, LoRA r={r} per expert s={s}, fwd+bwd",
                   "E": E, "M": M, "K": K, "N": N, "r": r, "counts": counts, "weight_copies": ncopies,
                   "phase_ms": {k: {x: round(y, 4) for x, y in v.items()} for k, v in per.items()}},
        "roofline": roof,
    }
    if context:
        out["context"] = context
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = run_moe_cpu_baseline(mw, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def run_moe_cpu_baseline(mw, target_s):
    """The oracle's grouped layer (float64) on a sample: the first rows of every expert's group,
    in proportion to its count."""
    from threadpoolctl import threadpool_info

    import numpy as np
    import workloads as wl
    from oracle import moe, nf4
    counts = mw.counts()
    off = moe.offsets(counts)
    Wd = nf4.dequantize_f32(nf4.quantize(wl.moe_tensor(mw, "W").float().numpy(), mw.dq_block))
    A, B = wl.moe_tensor(mw, "A").float().numpy(), wl.moe_tensor(mw, "B").float().numpy()
    Xall, dYall = wl.moe_tensor(mw, "X").float().numpy(), wl.moe_tensor(mw, "dY").float().numpy()

    def step(frac):
        cs = [int(c * frac) for c in counts]
        rows = np.concatenate([np.arange(off[e], off[e] + cs[e]) for e in range(mw.E)])
        X, dY = Xall[rows], dYall[rows]
        t = time.perf_counter()
        moe.forward(X, cs, Wd, A, B, mw.s)
        moe.backward(dY, X, cs, Wd, A, B, mw.s)
        return time.perf_counter() - t, sum(cs)

    frac = 64 / mw.M * mw.E
    dt, rows = step(frac)
    while dt < 0.4 * target_s and frac < 1:
        frac = min(1.0, max(2 * frac, frac * target_s / max(dt, 1e-3)))
        dt, rows = step(frac)
    flops = (mw.fwd_flops() + mw.bwd_flops()) * rows / mw.M
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "wall_s": round(dt, 2),
            "sample": f"{rows} of {mw.M} rows of the {mw.name} layer (the first rows of each expert's group, "
                      f"in proportion), forward+backward in float64 (numpy/BLAS), {dt:.1f}s wall; the weights "
                      f"dequantised once outside the timing"}


def run_pair_cpu_baseline(pw, target_s):
    """The oracle's gate/up pair (float64) on a row sample of the same step."""
    from threadpoolctl import threadpool_info

    import workloads as wl
    from oracle import nf4, swiglu
    Wd = nf4.dequantize_f32(nf4.quantize(wl.pair_tensor(pw, "Wgu").float().numpy(), pw.dq_block))
    N, r = pw.N, pw.r
    Agu = wl.pair_tensor(pw, "Agu").float().numpy()
    Bg, Bu = wl.pair_tensor(pw, "Bg").float().numpy(), wl.pair_tensor(pw, "Bu").float().numpy()
    Xall = wl.pair_tensor(pw, "X").float().numpy()
    dHall = wl.pair_tensor(pw, "dH").float().numpy()

    def step(rows):
        t = time.perf_counter()
        swiglu.forward(Xall[:rows], Wd[:N], Wd[N:], Agu[:r], Agu[r:], Bg, Bu, pw.s)
        swiglu.backward(dHall[:rows], Xall[:rows], Wd[:N], Wd[N:], Agu[:r], Agu[r:], Bg, Bu, pw.s)
        return time.perf_counter() - t

    rows = 64
    dt = step(rows)
    while dt < 0.4 * target_s and rows < pw.M:
        rows = int(min(pw.M, max(2 * rows, rows * target_s / max(dt, 1e-3))))
        rows = max(64, rows // 64 * 64)
        dt = step(rows)
    flops = (pw.fwd_flops() + pw.bwd_flops()) * rows / pw.M
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "wall_s": round(dt, 2),
            "sample": f"{rows} of {pw.M} rows of the {pw.name} pair, forward+backward in float64 "
                      f"(numpy/BLAS), {dt:.1f}s wall; the weights dequantised once outside the timing"}


def _median_ms(fn, reps, warmup=2):
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in ev)
    return t[len(t) // 2]


def run_context(L):
    """Measured-achievable references on this machine, beside the fused path (context, not the target).

    MFMA-bound shapes: the vendor bf16 GEMM (torch.matmul -> hipBLASLt) of X by the dequantised
    weight, same shape and data, and the unfused forward (nf4_dequantize, then that GEMM and the two
    LoRA GEMMs). Both run on the same data as the fused kernels: with realistic data the chip's
    clock falls under sustained matrix-core load, so the vendor GEMM measures what is reachable
    here. HBM-bound shapes: a plain 1 GiB device copy (bytes read + written / time)."""
    import torch
    w = L.w
    M, N, K, r = w.M, w.N, w.K, w.r
    out = {}
    if M > 64:
        q = L.copies[0]
        Wd = L.lib.nf4_dequantize(q, torch.bfloat16)                  # [N, K]
        Wt = Wd.t().contiguous()                                      # [K, N]
        At = L.A.t().contiguous()                                     # [K, r]
        Bt = (w.s * L.B.float()).to(torch.bfloat16).t().contiguous()  # [r, N]
        ms = _median_ms(lambda: torch.matmul(L.X, Wt), 10)
        out["vendor_bf16_gemm"] = {"what": "torch.matmul X [M,K] @ deq(W)^T [K,N], bf16 (hipBLASLt)",
                                   "ms": round(ms, 4), "TFLOP/s": round(2 * M * N * K / (ms * 1e-3) / 1e12, 2)}

        def unfused():
            Wu = L.lib.nf4_dequantize(q, torch.bfloat16).t().contiguous()
            T = torch.matmul(L.X, At)
            return torch.matmul(L.X, Wu) + torch.matmul(T, Bt)
        ms_u = _median_ms(unfused, 5)
        out["unfused_fwd"] = {"what": "nf4_dequantize + vendor GEMM + LoRA GEMMs (forward)",
                              "ms": round(ms_u, 4),
                              "TFLOP/s": round(w.fwd_flops() / (ms_u * 1e-3) / 1e12, 2)}
        out["mfma_loop"] = run_mfma_loop(Wd, L.X)
        del Wd, Wt, At, Bt
    else:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        ms = _median_ms(lambda: dst.copy_(src), 5)
        out["device_copy"] = {"what": "1 GiB device-to-device copy", "ms": round(ms, 4),
                              "GB/s": round(2 * n / (ms * 1e-3) / 1e9, 1)}
        del src, dst
    torch.cuda.empty_cache()
    return out


def run_mfma_loop(a, b, workgroups=2048, iters=2048):
    """The dense bf16 MFMA rate this chip sustains: libnf4probe's loop of back-to-back MFMA
    16x16x32 on register operands (values taken from the dequantised weight and from X, since the
    rate under the power limit depends on the data), 8 workgroups of 4 waves per CU."""
    import ctypes
    import torch
    from nf4_dequant_gemm_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        raise ImportError(f"{PROBE_LIB} is not built; run python -m nf4_dequant_gemm_amd.build")
    lib = ctypes.CDLL(PROBE_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.nf4probe_mfma_loop.argtypes = [vp, vp, i64, i64, i32, vp, vp]
    lib.nf4probe_mfma_loop.restype = ctypes.c_int
    lib.nf4probe_mfma_loop_flops.argtypes = [i64, i32]
    lib.nf4probe_mfma_loop_flops.restype = ctypes.c_double
    nbytes = min(a.numel() * a.element_size(), b.numel() * b.element_size())
    out = torch.empty(workgroups * 256, dtype=torch.float32, device=a.device)
    st = torch.cuda.current_stream().cuda_stream

    def launch():
        rc = lib.nf4probe_mfma_loop(a.data_ptr(), b.data_ptr(), nbytes, workgroups, iters,
                                    out.data_ptr(), st)
        if rc != 0:
            raise RuntimeError(f"nf4probe_mfma_loop returned {rc}")
    ms = _median_ms(launch, 5)
    flops = lib.nf4probe_mfma_loop_flops(workgroups, iters)
    return {"what": "bf16 MFMA 16x16x32 loop on register operands (values of deq(W) and X), "
                    f"{workgroups} workgroups x 4 waves x {iters} x 8 MFMAs",
            "ms": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2)}


def copy_calibration():
    """A plain 1 GiB device-to-device copy, five times: the reference for HBM byte counters."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "repeats": 5}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1).", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    import workloads as wl
    dev = torch.device("cuda:0")
    if args.workload in wl.PAIRS:
        run_pair(args, wl.PAIRS[args.workload], dev)
        return
    if args.workload in wl.MOES:
        run_moe(args, wl.MOES[args.workload], dev)
        return
    w = wl.WORKLOADS[args.workload]
    L = Layer(w, dev, args.wcopies)
    step_ms, per = time_layer(L, args.steps, args.warmup)
    whole_fwd = time_call(L, L.fwd_whole, args.steps, args.warmup) if not w.backward else None
    ncopies = len(L.copies)
    merge = run_merge(L, args.steps, args.warmup) if w.M > 64 and w.fmt == "nf4" else None
    context = None if args.no_context else run_context(L)
    del L
    torch.cuda.empty_cache()
    flops = w.fwd_flops() + (w.bwd_flops() if w.backward else 0)
    value = flops / (step_ms * 1e-3) / 1e12
    M, N, K, r = w.M, w.N, w.K, w.r
    kern = {"qlora_fwd_fused": (per["fwd_fused"], 2 * M * N * K + 2 * M * N * r)}
    if w.backward:
        kern["qlora_bwd_dx"] = (per["bwd_dx"], 2 * M * N * K + 2 * M * r * K)
    name = max(kern, key=lambda k: kern[k][0]["mean"])
    t, work = kern[name]
    if M <= 64:     # the decode-shaped forward: bound by the weight stream
        name = "qlora_fwd_fused (decode)"
        achieved = w.weight_stream_bytes() / (t["mean"] * 1e-3) / 1e9
        roof = {"kernel": name, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4)}
    else:
        achieved = work / (t["mean"] * 1e-3) / 1e12
        roof = {"kernel": name, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
    roof["kernel_us"] = {k: round(v * 1e3, 2) for k, v in t.items()}
    roof["traffic"] = traffic_for(name, w.name)
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: X [{M},{K}] bf16, "
                               + (f"W E2M1 [{N},{K}] E4M3 scale per 16 + fp32 tensor scale, " if w.fmt == "e2m1"
                                  else f"W NF4 [{N},{K}] block 64"
                                  f"{' double-quant int8/256' if w.dq_block else ' fp32 absmax'}, ") +
                               f"LoRA r={r} s={w.s}, {'fwd+bwd' if w.backward else 'fwd'}",
                   "M": M, "K": K, "N": N, "r": r, "weight_copies": ncopies,
                   "phase_ms": {k: {q: round(x, 4) for q, x in v.items()} for k, v in per.items()}},
        "roofline": roof,
    }
    if merge:
        out["merge"] = merge
    if whole_fwd:
        out["config"]["qlora_fwd_ms"] = {q: round(x, 4) for q, x in whole_fwd.items()}
        if M <= 64:
            gbs = w.weight_stream_bytes() / (whole_fwd["median"] * 1e-3) / 1e9
            out["config"]["weight_stream_GBps"] = round(gbs, 1)
    if context:
        ref = context.get("vendor_bf16_gemm", {}).get("TFLOP/s") or context.get("device_copy", {}).get("GB/s")
        if ref:
            roof["frac_of_measured_achievable"] = round(roof["achieved"] / ref, 4)
        loop = context.get("mfma_loop", {}).get("TFLOP/s")
        if loop:
            roof["frac_of_mfma_loop"] = round(roof["achieved"] / loop, 4)
        out["context"] = context
    if not args.no_weight_stream and w.name != "decode":
        out["weight_stream"] = run_weight_stream(dev, 20, 5)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = run_cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
