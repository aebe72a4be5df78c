#!/usr/bin/env python3
"""Benchmark of the fused NF4 QLoRA linear layer on one MI355X.

The default run measures the five layer workloads one after the other and prints ONE JSON line.
Its top level is the "down" workload (a Llama down_proj training step: X bf16 [16384, 14336],
W NF4 [4096, 14336] with double-quantised absmax, LoRA r = 32, s = 1, dY ~ N(0, 1e-2)), the
largest forward + backward shape, where one step is

    qlora_lora_down   T = X A^T
    qlora_fwd_fused   Y = X deq(W)^T + s T B^T             (one launch)
    qlora_bwd (dX=0)  U = dY B, dA = s U^T X, dB = s dY^T T
    qlora_bwd_dx      dX = dY deq(W) + s U A                (one launch)

and its "configs" object holds one entry per workload, each with its own step time, roofline
and CPU baseline:

    small   M=64    K=256   N=256    r=8   fp32 absmax      fwd+bwd  (launch latency only)
    q_proj  M=4096  K=4096  N=4096   r=16  int8/256 absmax  fwd      (matrix-core bound)
    mlp_up  M=8192  K=4096  N=11008  r=64  int8/256 absmax  fwd+bwd  (matrix-core bound)
    decode  M=16    K=8192  N=28672  r=16  int8/256 absmax  fwd      (weight-stream bound: GB/s)
    down    M=16384 K=14336 N=4096   r=32  int8/256 absmax  fwd+bwd  (matrix-core bound)

Inputs are seeded synthetic tensors of those shapes, resident in HBM before timing starts. W is
quantised once per workload (untimed), as a frozen base weight is, then copied so that the steps
rotate over enough distinct copies (>= 512 MB together) that no step finds its weight in the
256 MB last-level cache or the L2 left there by the step before.

Timing, per workload: W warm-up steps, then K steps between two synchronisations (host clock:
ms_per_step and value), with a HIP event pair on the launch stream around every call of the
step (phase_ms). The roofline of each workload is that of its dominant fused launch (forward
and, with a backward, dX; decode: the forward's stream kernel, which on this shape is the whole
qlora_fwd call, T = X A^T included), from its mean duration over the timed steps: algorithmic
flops (or weight-stream bytes) per launch / mean duration. For the decode workload the value is
the weight-stream rate of the whole qlora_fwd call (weight-stream bytes / call time). cpu_baseline times the CPU oracle
(float64) on a bounded sample of the same workload on this host.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-context] [--copy-calibration] [--summarize-trace DIR]

--workload runs one workload alone (its entry becomes the top level). mlp_swiglu measures the
gate/up SwiGLU pair instead (a step: qlora_swiglu_fwd + qlora_swiglu_bwd on the mlp_up shape, two
projections); moe_mlp_up the grouped mixture-of-experts layer (a step: qlora_moe_fwd +
qlora_moe_bwd, 8 experts of the mlp_up shape, 16384 routed rows); mlp_up_e2m1 / decode_e2m1 the
single layer with an E2M1 base weight (4-bit floats, E4M3 scale per 16, float32 tensor scale).
--summarize-trace DIR reads a rocprofv3 kernel trace of this command and prints the per-workload
kernel durations (split by grid size) that the profiles record.
"""
from __future__ import annotations

import argparse
import ctypes
import csv
import glob
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
                  "qlora_fwd (decode)": "decode16.hip", "qlora_fwd_fused (decode)": "decode16.hip"}
DEFAULT_CONFIGS = ("small", "q_proj", "mlp_up", "decode", "down")
HEADLINE = "down"


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None,
                    help="run one workload alone (default: the five layer workloads)")
    ap.add_argument("--order", default=None,
                    help="comma-separated layer workloads to run, in this order (default: the five, "
                         "headline first)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the vendor-GEMM / MFMA-loop / device-copy reference measurements")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target wall time of each CPU oracle sample")
    ap.add_argument("--wcopies", type=int, default=0,
                    help="distinct weight copies to rotate over (0: enough for 512 MB)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--summarize-trace", default=None, metavar="DIR",
                    help="summarise a rocprofv3 kernel trace of this command (no GPU needed)")
    ap.add_argument("--summarize-counters", default=None, nargs="+", metavar="DIR",
                    help="summarise rocprofv3 --pmc runs of this command (no GPU needed)")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def pct(vals, q):
    v = sorted(vals)
    i = min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))
    return v[i]


def stats(v):
    return {"mean": sum(v) / len(v), "median": pct(v, 0.5), "p10": pct(v, 0.1), "p90": pct(v, 0.9)}


def host_cores():
    """Cores this process may run on (the CPU baseline's thread pool is sized to them)."""
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def blas_threads():
    from threadpoolctl import threadpool_info
    return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        return ""


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

    def q(self, i):
        return ctypes.byref(self.qs[i % len(self.qs)])

    def lora_down(self, i):
        w, p = self.w, self.p
        self.check(self.c.qlora_lora_down(p["X"], w.M, w.K, p["A"], w.r, p["T"], p["ws_f"], self.fws, self.sp))

    def fwd_fused(self, i):
        w, p = self.w, self.p
        self.check(self.c.qlora_fwd_fused(p["X"], w.M, self.q(i), p["T"], p["B"], w.r, w.s, p["Y"], self.sp))

    def fwd_whole(self, i):
        """The whole forward call (T pre-pass and fused kernel), as a caller makes it."""
        w, p = self.w, self.p
        self.check(self.c.qlora_fwd(p["X"], w.M, self.q(i), p["A"], p["B"], w.r, w.s, p["Y"], p["T"],
                                    p["ws_f"], self.fws, self.sp))

    def bwd_whole(self, i):
        """The whole backward call (U, dX, dA, dB)."""
        w, p = self.w, self.p
        self.check(self.c.qlora_bwd(p["dY"], p["X"], w.M, self.q(i), p["A"], p["B"], w.r, w.s, p["T"],
                                    p["dX"], p["dA"], p["dB"], p["ws_b"], self.bws, self.sp))

    def bwd_lora(self, i):
        """U (left at the start of the workspace), dA and dB: qlora_bwd without dX."""
        w, p = self.w, self.p
        self.check(self.c.qlora_bwd(p["dY"], p["X"], w.M, self.q(i), p["A"], p["B"], w.r, w.s, p["T"],
                                    None, p["dA"], p["dB"], p["ws_b"], self.bws, self.sp))

    def bwd_dx(self, i):
        w, p = self.w, self.p
        self.check(self.c.qlora_bwd_dx(p["dY"], w.M, self.q(i), p["ws_b"], p["A"], w.r, w.s, p["dX"],
                                       self.sp))


def step_calls(L):
    """The calls of one step, by phase name. Forward-only workloads call qlora_fwd whole (the
    decode shapes take the T pre-pass into the stream kernel's prologue only there); forward +
    backward workloads call the launches separately so that the two fused launches can be timed
    on their own (the same kernels as qlora_fwd + qlora_bwd). The small workload calls qlora_fwd
    and qlora_bwd whole: it is timed for latency."""
    w = L.w
    if w.name == "small" or (w.backward and w.M <= 64):
        return [("qlora_fwd", L.fwd_whole), ("qlora_bwd", L.bwd_whole)]
    if not w.backward:
        return [("qlora_fwd", L.fwd_whole)]
    return [("lora_down", L.lora_down), ("fwd_fused", L.fwd_fused), ("bwd_lora", L.bwd_lora),
            ("bwd_dx", L.bwd_dx)]


HOLD_CYCLES = 10_000_000   # ~4 ms of GPU spin ahead of each timed region


def hold_stream():
    """Keep the launch stream busy (a spin kernel) while the host enqueues the timed launches and
    their events, so that no timed interval contains host issue time: the short launches of the
    decode and small workloads are issued more slowly than they run."""
    import torch
    torch.cuda._sleep(HOLD_CYCLES)


def time_steps(L, calls, steps, warmup):
    """warmup + steps steps, three times. First the plain steps between two synchronisations: the
    host-clock time per step. Then the GPU time per step (one HIP event pair around the whole
    timed region on the launch stream, the launches queued behind a spin kernel). Then the same
    steps with a HIP event pair around every call: the per-call times (ms). Returns (host
    ms/step, GPU ms/step, per-call stats)."""
    import torch
    for i in range(warmup):
        for _, c in calls:
            c(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record(L.stream)
    for s in range(steps):
        for _, c in calls:
            c(warmup + s)
    b.record(L.stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    host_ms = (t1 - t0) * 1e3 / steps
    # the GPU time per step: the same steps again, enqueued behind a spin kernel so that the GPU
    # runs them back to back whatever the host's issue rate
    hold_stream()
    a.record(L.stream)
    for s in range(steps):
        for _, c in calls:
            c(warmup + s)
    b.record(L.stream)
    torch.cuda.synchronize()
    gpu_ms = a.elapsed_time(b) / steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(steps)]
    hold_stream()
    for s in range(steps):
        e = ev[s]
        e[0].record(L.stream)
        for j, (_, c) in enumerate(calls):
            c(warmup + steps + s)
            e[j + 1].record(L.stream)
    torch.cuda.synchronize()
    per = {}
    for j, (name, _) in enumerate(calls):
        per[name] = stats([ev[s][j].elapsed_time(ev[s][j + 1]) for s in range(steps)])
    return host_ms, gpu_ms, per


def time_call(L, fn, steps, warmup):
    """HIP-event times (ms) of one call over rotating weight copies. The mean is the average
    launch duration: one event pair around `steps` back-to-back launches, queued behind a spin
    kernel (no host gaps, no per-launch event overhead, which is about 1.5 us and would inflate a
    30 us launch by 5%). The spread (median, p10, p90) comes from an event pair around each
    launch of a second pass; its own mean is kept as mean_per_launch_events."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_stream()
    a.record(L.stream)
    for s in range(steps):
        fn(warmup + s)
    b.record(L.stream)
    torch.cuda.synchronize()
    mean = a.elapsed_time(b) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    hold_stream()
    for s, (a, b) in enumerate(ev):
        a.record(L.stream)
        fn(warmup + steps + s)
        b.record(L.stream)
    torch.cuda.synchronize()
    st = stats([a.elapsed_time(b) for a, b in ev])
    st["mean_per_launch_events"] = st["mean"]
    st["mean"] = mean
    return st


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


def roofline_mfma(kernel, t_ms, flops, workload):
    achieved = flops / (t_ms["mean"] * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "flops_per_launch": flops,
            "kernel_us": {k: round(v * 1e3, 2) for k, v in t_ms.items()},
            "traffic": traffic_for(kernel, workload)}


def roofline_hbm(kernel, t_ms, nbytes, workload):
    achieved = nbytes / (t_ms["mean"] * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4), "bytes_per_launch": nbytes,
            "kernel_us": {k: round(v * 1e3, 2) for k, v in t_ms.items()},
            "traffic": traffic_for(kernel, workload)}


def single_launch_decode(w):
    """qlora_fwd is one launch of the stream kernel (which forms T itself): M <= 16, K % 256 == 0,
    r % 8 == 0 and 8 <= r <= 64 with a double-quantised NF4 weight, 8 <= r <= 16 with E2M1."""
    if w.M > 16 or w.K % 256 or w.r % 8 or w.r < 8:
        return False
    return w.r <= 16 if w.fmt == "e2m1" else (w.dq_block > 0 and w.r <= 64)


def describe(w):
    return (f"{w.name}: X [{w.M},{w.K}] bf16, "
            + (f"W E2M1 [{w.N},{w.K}] E4M3 scale per 16 + fp32 tensor scale, " if w.fmt == "e2m1"
               else f"W NF4 [{w.N},{w.K}] block 64"
               f"{' double-quant int8/256' if w.dq_block else ' fp32 absmax'}, ")
            + f"LoRA r={w.r} s={w.s}, {'fwd+bwd' if w.backward else 'fwd'}")


def run_config(w, dev, args, cpu=True):
    """One workload: step time, per-call times, the roofline of its dominant fused launch and
    (cpu) the CPU oracle on a sample. Returns the JSON object and the Layer (for the context)."""
    L = Layer(w, dev, args.wcopies)
    calls = step_calls(L)
    host_ms, gpu_ms, per = time_steps(L, calls, args.steps, args.warmup)
    # the GPU time per step (the host may be slower than the GPU at issuing the short steps of
    # the small and decode workloads); the host-clock time is reported beside it
    step_ms = gpu_ms
    M, N, K, r = w.M, w.N, w.K, w.r
    out = {"workload": describe(w), "M": M, "K": K, "N": N, "r": r, "weight_copies": len(L.copies),
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
           "host_ms_per_step": round(host_ms, 4),
           "phase_ms": {k: {q: round(x, 4) for q, x in v.items()} for k, v in per.items()}}
    kernels = {}
    if w.name == "small" or (w.backward and M <= 64):
        out.update(bound="latency", value=round(step_ms * 1e3, 2), unit="us per fwd+bwd step",
                   higher_is_better=False)
    elif not w.backward:
        # forward only: the whole qlora_fwd call is the step. Its fused launch is timed alone too;
        # on the NF4 decode shape (M <= 16, r % 8 == 0, r <= 64) the call is that one launch (the
        # stream kernel forms T itself), so the call is what is timed.
        if M <= 64:
            one = single_launch_decode(w)
            fwd_only = time_call(L, L.fwd_whole if one else L.fwd_fused, args.steps, args.warmup)
            wb = w.weight_stream_bytes()
            gbs = wb / (step_ms * 1e-3) / 1e9
            out.update(bound="hbm", value=round(gbs, 1), unit="GB/s", higher_is_better=True,
                       weight_stream_bytes=wb, frac_of_hbm_peak=round(gbs / PEAK_HBM_GBS, 4))
            label = "qlora_fwd (decode)" if one else "qlora_fwd_fused (decode)"
            kernels[label] = roofline_hbm(label, fwd_only, wb, w.name)
        else:
            fwd_only = time_call(L, L.fwd_fused, args.steps, args.warmup)
            fl = w.fwd_flops()
            out.update(bound="mfma", value=round(fl / (step_ms * 1e-3) / 1e12, 2), unit="TFLOP/s",
                       higher_is_better=True)
            kernels["qlora_fwd_fused"] = roofline_mfma("qlora_fwd_fused", fwd_only,
                                                       2 * M * N * K + 2 * M * N * r, w.name)
        out["qlora_fwd_ms" if M <= 64 and single_launch_decode(w) else "qlora_fwd_fused_ms"] = \
            {q: round(x, 4) for q, x in fwd_only.items()}
    else:
        fl = w.fwd_flops() + w.bwd_flops()
        out.update(bound="mfma", value=round(fl / (step_ms * 1e-3) / 1e12, 2), unit="TFLOP/s",
                   higher_is_better=True)
        kernels["qlora_fwd_fused"] = roofline_mfma("qlora_fwd_fused", per["fwd_fused"],
                                                   2 * M * N * K + 2 * M * N * r, w.name)
        kernels["qlora_bwd_dx"] = roofline_mfma("qlora_bwd_dx", per["bwd_dx"],
                                                2 * M * N * K + 2 * M * r * K, w.name)
    if kernels:
        dom = max(kernels, key=lambda k: kernels[k]["kernel_us"]["mean"])
        out["roofline"] = kernels[dom]
        if len(kernels) > 1:
            out["kernels"] = kernels
    if cpu and not args.no_cpu_baseline:
        out["cpu_baseline"] = run_cpu_baseline(w, args.cpu_seconds)
    return out, L


def run_merge(L, steps, warmup):
    """LoRA merge of the workload's weight (qlora_merge, W' = bf16(deq(W) + s B A)), cold weights:
    bytes moved (weight stream + A, B read; W' written) / HIP-event time, against HBM."""
    import torch
    w, c = L.w, L.c
    out = torch.empty(w.N, w.K, dtype=torch.bfloat16, device=L.X.device)
    P = lambda t: ctypes.c_void_p(t.data_ptr())

    def fn(i):
        L.check(c.qlora_merge(L.q(i), P(L.A), P(L.B), w.r, w.s, P(out), L.sp))
    t = time_call(L, fn, steps, warmup)
    nbytes = w.weight_stream_bytes() + 2 * w.r * w.K + 2 * w.N * w.r + 2 * w.N * w.K
    gbs = nbytes / (t["mean"] * 1e-3) / 1e9
    del out
    return {"what": f"qlora_merge of the {w.name} weight [{w.N},{w.K}], r={w.r}: W' = bf16(deq(W) + s B A)",
            "us": round(t["mean"] * 1e3, 2), "bytes": nbytes, "GB/s": round(gbs, 1),
            "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def run_cpu_baseline(w, target_s):
    """The oracle (float64 numpy/BLAS) on a bounded row sample of the same step, in the workload's
    unit: TFLOP/s of algorithmic flops, or (decode) GB/s of weight-stream bytes."""
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

    def step(rows, reps=1):
        X = Xall[:rows]
        dY = dYall[:rows] if w.backward else None
        t = time.perf_counter()
        for _ in range(reps):
            qlora.forward(X, Wd, A, B, w.s)
            if w.backward:
                qlora.backward(dY, X, Wd, A, B, w.s)
        return time.perf_counter() - t

    rows, reps = min(64, w.M), 1
    dt = step(rows)
    while dt < 0.4 * target_s and rows < w.M:       # grow the sample until it takes ~target_s
        rows = int(min(w.M, max(2 * rows, rows * target_s / max(dt, 1e-3))))
        rows = max(64, rows // 64 * 64) if w.M >= 64 else w.M
        dt = step(rows)
    while dt < 0.4 * target_s:                      # whole workload is quick: repeat it
        reps = int(max(2 * reps, reps * target_s / max(dt, 1e-3)))
        dt = step(rows, reps)
    frac = rows * reps / w.M
    out = {"kind": "oracle", "cores": host_cores(), "threads": blas_threads(), "cpu": cpu_model(),
           "wall_s": round(dt, 2)}
    if not w.backward and w.M <= 64:
        out.update(value=round(w.weight_stream_bytes() * frac / dt / 1e9, 4), unit="GB/s")
    else:
        flops = (w.fwd_flops() + (w.bwd_flops() if w.backward else 0)) * frac
        out.update(value=round(flops / dt / 1e12, 5), unit="TFLOP/s")
    out["sample"] = (f"{rows} of {w.M} rows of the {w.name} workload"
                     + (f", {reps} times" if reps > 1 else "")
                     + f", {'forward+backward' if w.backward else 'forward'} in float64 (numpy/BLAS),"
                     f" {dt:.1f}s wall; W dequantised once outside the timing")
    return out


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
    # The roofline launch: the pair's own fused kernel (the one qlora_swiglu_fwd makes at this
    # shape after T = X Agu^T): the stacked gate/up GEMM with the NF4 decode, the LoRA steps (the
    # block-diagonal up projection applied as B is staged) and H = silu(Yg) * Yu in the epilogue.
    def fused(i):
        check(c.qlora_swiglu_fwd_fused(P(d["X"]), M, ctypes.byref(qs[i % ncopies]), P(Tgu), P(d["Bg"]),
                                       P(d["Bu"]), r, s, P(H), P(Ygu), sp))
    t = time_call(types.SimpleNamespace(stream=stream), fused, args.steps, args.warmup)
    # algorithmic flops: each of the 2N output columns sums K + r products per row (the kernel
    # also runs the r zero ranks of the other half of the block-diagonal B)
    work = 2 * M * (2 * N) * (K + r)
    achieved = work / (t["mean"] * 1e-3) / 1e12
    roof = {"kernel": "qlora_swiglu_fwd_fused (pair kernel: stacked gate/up GEMM, LoRA steps, SwiGLU epilogue)",
            "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "kernel_us": {k: round(v * 1e3, 2) for k, v in t.items()}, "traffic": None}
    context = None
    if not args.no_context:
        Wd = lib.nf4_dequantize(q, torch.bfloat16)
        context = {"mfma_loop": run_mfma_loop(Wd, d["X"])}
        roof["frac_of_mfma_loop"] = round(achieved / context["mfma_loop"]["TFLOP/s"], 4)
        del Wd
    del copies, qs, d, H, Ygu, Tgu, dX, dAgu, dBg, dBu, ws
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
    achieved = work / (t["mean"] * 1e-3) / 1e12
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
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": host_cores(),
            "threads": blas_threads(), "kind": "oracle",
            "wall_s": round(dt, 2),
            "sample": f"{rows} of {mw.M} rows of the {mw.name} layer (the first rows of each expert's group, "
                      f"in proportion), forward+backward in float64 (numpy/BLAS), {dt:.1f}s wall; the weights "
                      f"dequantised once outside the timing"}


def run_pair_cpu_baseline(pw, target_s):
    """The oracle's gate/up pair (float64) on a row sample of the same step."""
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
    return {"value": round(flops / dt / 1e12, 5), "unit": "TFLOP/s", "cores": host_cores(),
            "threads": blas_threads(), "kind": "oracle",
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
        # the same forward without fusion: the weight dequantised to bf16 in HBM, then read back
        # by the vendor GEMM, and the two LoRA products (its HBM bytes beside the fused launch's
        # are in the counter profiles)
        q = L.copies[0]
        At = L.A.t().contiguous()
        Bt = (w.s * L.B.float()).to(torch.bfloat16).t().contiguous()

        def unfused():
            Wd = L.lib.nf4_dequantize(q, torch.bfloat16)
            return torch.matmul(L.X, Wd.t()) + torch.matmul(torch.matmul(L.X, At), Bt)
        ms_u = _median_ms(unfused, 5)
        out["unfused_fwd"] = {"what": "nf4_dequantize (bf16 W written) + vendor GEMM + LoRA GEMMs (forward)",
                              "ms": round(ms_u, 4),
                              "GB/s": round(w.weight_stream_bytes() / (ms_u * 1e-3) / 1e9, 1)}
        del At, Bt
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


def trace_groups(names=DEFAULT_CONFIGS):
    """(kernel name part, workgroups) -> (workload, launch) for the fused launches of a run of the
    named layer workloads (default: the default run): the tile counts of the 256 x 256 forward
    and dX kernels and of the 112-row stream kernel, from the workload shapes."""
    import workloads as wl
    out = {}
    for name in names:
        w = wl.WORKLOADS[name]
        cd = lambda a, b: -(-a // b)
        if w.M <= 16 and (w.dq_block or w.fmt == "e2m1") and w.K % 256 == 0:
            out[("decode16_fwd_kernel", cd(w.N, 112))] = \
                (name, "qlora_fwd (decode)" if single_launch_decode(w) else "qlora_fwd_fused (decode)")
        elif w.M > 48 or w.K % 256:
            out[("fwd_fused_kernel", cd(w.N, 256) * cd(w.M, 256))] = (name, "qlora_fwd_fused")
        if w.backward:
            out[("dx_fused_kernel", cd(w.K, 256) * cd(w.M, 256))] = (name, "qlora_bwd_dx")
    return out


def timed_launches(v, steps, warmup):
    """The launches of a fused kernel that bench.py's roofline times, in launch order. time_steps
    issues warmup + 3 steps launches of each call of the step (host pass, GPU pass, per-call
    pass); a forward-only workload then times its fused launch alone (time_call: warmup +
    2 steps launches), and that block is the roofline's. Warm-up launches are left out."""
    if len(v) >= 2 * warmup + 5 * steps:             # forward only: the time_call block
        return v[warmup + 3 * steps + warmup:]
    return v[warmup:warmup + 3 * steps] or v


def summarize_trace(path, steps, warmup, names=DEFAULT_CONFIGS):
    """Per-(kernel, grid) durations from a rocprofv3 kernel trace (CSV) of this command: the fused
    kernels of different workloads share names, so they are told apart by their workgroup count.
    mean_timed leaves out the warm-up launches (see timed_launches), as the bench's own means do."""
    files = sorted(glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True))
    if not files:
        raise SystemExit(f"no *kernel_trace.csv under {path}")
    groups = {}
    for fn in files:
        with open(fn, newline="") as f:
            for row in csv.DictReader(f):
                name = row["Kernel_Name"]
                wgs = 1
                for ax in "XYZ":
                    grid = int(row.get(f"Grid_Size_{ax}", 1) or 1)
                    wg = int(row.get(f"Workgroup_Size_{ax}", 1) or 1)
                    wgs *= -(-grid // max(wg, 1))
                dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
                groups.setdefault((name, wgs), []).append((int(row["Start_Timestamp"]), dur))
    known = trace_groups(names)
    print(f"# source: {', '.join(os.path.relpath(f, path) for f in files)}")
    print("# durations in microseconds (End_Timestamp - Start_Timestamp of each dispatch); wgs = workgroups")
    print(f"{'calls':>5} {'mean_us':>10} {'mean_timed':>10} {'median_us':>10} {'min_us':>10} {'max_us':>10}"
          f"  {'wgs':>6}  {'workload/launch':<34} kernel")
    rows = []
    for (name, wgs), tv in groups.items():
        v = [d for _, d in sorted(tv)]
        tag = next((f"{wl_}/{launch}" for (part, n), (wl_, launch) in known.items()
                    if n == wgs and part in name), "")
        timed = timed_launches(v, steps, warmup) if tag else v
        rows.append((sum(v), name, wgs, v, timed or v, tag))
    for _, name, wgs, v, timed, tag in sorted(rows, reverse=True):
        s = stats(v)
        print(f"{len(v):5d} {s['mean']:10.2f} {sum(timed) / len(timed):10.2f} {s['median']:10.2f} "
              f"{min(v):10.2f} {max(v):10.2f}  {wgs:6d}  {tag:<34} {name[:100]}")


def summarize_counters(paths):
    """Per-(kernel, grid) means of rocprofv3 --pmc counters (run_counter_collection.csv under each
    path), with derived figures where their inputs were collected: matrix-core busy share and
    clock (SQ counters summed over the 1024 SIMDs, GRBM_GUI_ACTIVE over the 8 XCDs), vector
    instructions per MFMA, LDS busy share, and HBM-side KiB per dispatch."""
    import collections
    rows = collections.defaultdict(lambda: collections.defaultdict(list))
    known = trace_groups()
    for path in paths:
        for fn in sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)):
            per = collections.defaultdict(lambda: collections.defaultdict(float))
            meta = {}
            with open(fn, newline="") as f:
                for r in csv.DictReader(f):
                    wgs = max(1, int(float(r["Grid_Size"])) // max(1, int(float(r["Workgroup_Size"]))))
                    key = (r["Kernel_Name"], wgs)
                    per[(key, r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
                    meta[(key, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
            for (key, d), cs in per.items():
                for c, v in cs.items():
                    rows[key][c].append(v)
                rows[key]["_us"].append(meta[(key, d)])
    print("# means per dispatch; durations are the profiler's (counter collection replays kernels)")
    for (name, wgs), cs in sorted(rows.items(), key=lambda kv: -sum(kv[1]["_us"])):
        tag = next((f"{w}/{launch}" for (part, n), (w, launch) in known.items() if n == wgs and part in name), "")
        m = {c: sum(v) / len(v) for c, v in cs.items()}
        out = [f"dispatches {len(cs['_us'])}", f"us {m['_us']:.1f}"]
        gui = m.get("GRBM_GUI_ACTIVE")
        if gui:
            out.append(f"clk_GHz {gui / 8 / (m['_us'] * 1e3):.3f}")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
                out.append(f"mfma_busy {m['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / (gui / 8):.3f}")
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in m:
                out.append(f"coexec {m['SQ_VALU_MFMA_COEXEC_CYCLES'] / 1024 / (gui / 8):.3f}")
            if "SQ_LDS_IDX_ACTIVE" in m:
                out.append(f"lds_busy {m['SQ_LDS_IDX_ACTIVE'] / 256 / (gui / 8):.3f}")
            if "SQ_ACTIVE_INST_VALU" in m:
                out.append(f"valu_busy {4 * m['SQ_ACTIVE_INST_VALU'] / 1024 / (gui / 8):.3f}")
        if "SQ_INSTS_MFMA" in m and "SQ_INSTS_VALU" in m and m["SQ_INSTS_MFMA"]:
            out.append(f"valu_per_mfma {(m['SQ_INSTS_VALU'] - m['SQ_INSTS_MFMA']) / m['SQ_INSTS_MFMA']:.2f}")
        for c in ("FETCH_SIZE", "WRITE_SIZE"):
            if c in m:
                out.append(f"{c}_KiB {m[c]:.0f}")
        for c in sorted(m):
            if c.startswith("SQ_") or c.startswith("TCC_") or c.startswith("TCP_"):
                out.append(f"{c} {m[c]:.4g}")
        print(f"{tag or '-'}  wgs {wgs}  {name[:90]}")
        print("    " + "  ".join(out))


def main():
    args = parse()
    if args.summarize_trace:
        import workloads as wl
        names = [args.workload] if args.workload in wl.WORKLOADS else DEFAULT_CONFIGS
        summarize_trace(args.summarize_trace, args.steps, args.warmup, names)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters)
        return
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
    if args.workload is not None and args.workload not in wl.WORKLOADS:
        raise SystemExit(f"unknown workload {args.workload}; one of "
                         f"{sorted(wl.WORKLOADS) + sorted(wl.PAIRS) + sorted(wl.MOES)}")
    names = [args.workload] if args.workload else (args.order.split(",") if args.order else list(DEFAULT_CONFIGS))
    if not args.workload and HEADLINE not in names:
        raise SystemExit(f"--order must include the headline workload {HEADLINE}")
    head = args.workload or HEADLINE
    configs, extra = {}, {}
    for name in names:
        w = wl.WORKLOADS[name]
        log(f"== {name}")
        res, L = run_config(w, dev, args)
        if res["bound"] == "mfma" and not args.no_context:
            ctx = run_context(L)
            loop = ctx.get("mfma_loop", {}).get("TFLOP/s")
            vendor = ctx.get("vendor_bf16_gemm", {}).get("TFLOP/s")
            for k in res.get("kernels", {"_": res["roofline"]}).values():
                if loop:
                    k["frac_of_mfma_loop"] = round(k["achieved"] / loop, 4)
                if vendor:
                    k["frac_of_vendor_gemm"] = round(k["achieved"] / vendor, 4)
            res["context"] = ctx
        elif res["bound"] == "hbm" and not args.no_context:
            ctx = run_context(L)
            copy = ctx.get("device_copy", {}).get("GB/s")
            if copy:
                res["roofline"]["frac_of_device_copy"] = round(res["roofline"]["achieved"] / copy, 4)
            res["context"] = ctx
        if name == head and w.M > 64 and w.fmt == "nf4":
            extra["merge"] = run_merge(L, args.steps, args.warmup)
        del L
        torch.cuda.empty_cache()
        configs[name] = res
        log(f"   {name}: {res['value']} {res['unit']}"
            + (f", roofline {res['roofline']['kernel']} frac {res['roofline']['frac']}" if "roofline" in res else ""))
    h = configs[head]
    cfg = {k: h[k] for k in ("workload", "M", "K", "N", "r", "weight_copies", "phase_ms")}
    out = {
        "metric": METRIC, "value": h["value"], "unit": h["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": h["ms_per_step"],
        "higher_is_better": h["higher_is_better"], "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic", "config": cfg,
    }
    if "roofline" in h:
        out["roofline"] = h["roofline"]
    if "cpu_baseline" in h:
        out["cpu_baseline"] = h["cpu_baseline"]
    if len(names) > 1:
        out["configs"] = configs
    else:
        for k in ("kernels", "context", "qlora_fwd_fused_ms", "qlora_fwd_ms"):
            if k in h:
                out[k] = h[k]
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
