"""The grouped (mixture-of-experts) layer with its routing in device memory
(qlora_moe_fwd_dev / qlora_moe_bwd_dev).

The counts live in a device tensor and only the number of routed rows is given on the host, so
the calls need no host synchronisation: they are checked bit for bit against the host-routed
calls (the same kernels, split counts that depend on the row total only) and within 1e-2 of the
float64 oracle, with up to 256 experts, empty experts (exact zero adapter gradients) and one-row
experts. A graph captured once with the device-routed calls then follows a different routing on
every replay: the counts, X and dY buffers are rewritten between replays, and each replay equals
the host-routed calls for its own routing.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import moe, nf4
from tests.gpu_helpers import check_close, f32, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def routing(E, M, seed):
    """Seeded uneven counts summing to M, with every seventh expert empty and expert 1 given one
    row (when M allows)."""
    rng = np.random.default_rng(seed)
    p = np.exp(rng.standard_normal(E) * 0.8)
    p[::7] = 0
    p /= p.sum()
    c = rng.multinomial(M - (1 if E > 1 else 0), p).astype(np.int64)
    if E > 1:
        c[1] += 1
    assert c.sum() == M
    return [int(x) for x in c]


def layer(counts, K, N, r, seed):
    E, M = len(counts), int(sum(counts))
    X = wl.normal_bf16(seed + 1, (M, K), 1.0)
    W = wl.normal_bf16(seed + 2, (E * N, K), 0.02)
    A = wl.normal_bf16(seed + 3, (E * r, K), K ** -0.5)
    B = wl.normal_bf16(seed + 4, (E * N, r), 0.1)
    dY = wl.normal_bf16(seed + 5, (M, N), 1.0)
    return X, W, A, B, dY


def device_calls(lib, Xd, dYd, cd, q, Ad, Bd, s, M, E, N, K, r, out=None):
    bf = torch.bfloat16
    if out is None:
        out = dict(Y=torch.empty(M, N, dtype=bf, device=DEV),
                   T=torch.empty(M, r, dtype=bf, device=DEV) if r else None,
                   dX=torch.empty(M, K, dtype=bf, device=DEV),
                   dA=torch.empty(E * r, K, dtype=bf, device=DEV) if r else None,
                   dB=torch.empty(E * N, r, dtype=bf, device=DEV) if r else None,
                   ws=torch.empty(max(lib.moe_workspace_bytes_dev(M, E, N, K, r), 1), dtype=torch.uint8,
                                  device=DEV))
    lib.qlora_moe_fwd_dev(Xd, cd, q, Ad, Bd, s, out["Y"], out["T"], out["ws"])
    lib.qlora_moe_bwd_dev(dYd, Xd, cd, q, Ad, Bd, s, out["T"], out["dX"], out["dA"], out["dB"], out["ws"])
    return out


CASES = [
    # E, M, K, N, r, dq, s
    (256, 2000, 256, 64, 8, 256, 1.0),
    (256, 300, 512, 72, 16, 0, -0.5),      # most experts empty or one row
    (8, 700, 320, 264, 32, 256, 2.0),
    (64, 64, 256, 128, 0, 256, 1.0),        # no adapters
    (8, 7000, 2304, 512, 16, 256, 0.5),     # dX: a round of 256 tiles and a tail split into pieces
]


@pytest.mark.parametrize("E,M,K,N,r,dq,s", CASES)
def test_device_routing_equals_host_routing(lib, E, M, K, N, r, dq, s):
    counts = routing(E, M, 17 * E + M)
    say(f"moe device routing E={E} M={M} K={K} N={N} r={r} dq={dq} (empty experts: {counts.count(0)})")
    X, W, A, B, dY = layer(counts, K, N, r, 31 * E + M)
    q = lib.nf4_quantize(W.to(DEV), dq)
    Xd, dYd = X.to(DEV), dY.to(DEV)
    Ad, Bd = (A.to(DEV), B.to(DEV)) if r else (None, None)
    Yh, Th = lib.qlora_moe_fwd(Xd, counts, q, Ad, Bd, s)
    dXh, dAh, dBh = lib.qlora_moe_bwd(dYd, Xd, counts, q, Ad, Bd, s, Th)
    cd = torch.tensor(counts, dtype=torch.int64, device=DEV)
    o = device_calls(lib, Xd, dYd, cd, q, Ad, Bd, s, M, E, N, K, r)
    torch.cuda.synchronize()
    for name, got, want in (("Y", o["Y"], Yh), ("T", o["T"], Th), ("dX", o["dX"], dXh),
                            ("dA", o["dA"], dAh), ("dB", o["dB"], dBh)):
        if want is None:
            continue
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{name}: device routing differs"
    Wd = nf4.dequantize_f32(nf4.quantize(W.float().numpy(), dq))
    Yr, Tr = moe.forward(f32(X), counts, Wd, f32(A), f32(B), s)
    dXr, dAr, dBr = moe.backward(f32(dY), f32(X), counts, Wd, f32(A), f32(B), s)
    check_close("Y", f32(o["Y"]), Yr)
    check_close("dX", f32(o["dX"]), dXr)
    if r:
        check_close("T", f32(o["T"]), Tr)
        # with hundreds of experts most hold a handful of rows, whose adapter gradients sum few
        # products (the bf16 rounding of T and U does not average out): warn above 8e-3 there
        check_close("dA", f32(o["dA"]), dAr, warn_above=8e-3)
        check_close("dB", f32(o["dB"]), dBr, warn_above=8e-3)
        dA3 = f32(o["dA"]).reshape(E, r, K)
        dB3 = f32(o["dB"]).reshape(E, N, r)
        for e in range(E):
            if counts[e] == 0:
                assert not dA3[e].any() and not dB3[e].any(), f"expert {e} has no rows: zero gradients"


def test_graph_replays_follow_device_routing(lib):
    """One capture, three replays with three different routings written into the same device
    buffers; every replay equals the host-routed calls for its routing, bit for bit."""
    E, M, K, N, r, s = 32, 1024, 256, 128, 16, 0.5
    base = routing(E, M, 5)
    X, W, A, B, dY = layer(base, K, N, r, 77)
    q = lib.nf4_quantize(W.to(DEV), 256)
    Ad, Bd = A.to(DEV), B.to(DEV)
    Xd, dYd = X.to(DEV), dY.to(DEV)
    cd = torch.tensor(base, dtype=torch.int64, device=DEV)
    out = device_calls(lib, Xd, dYd, cd, q, Ad, Bd, s, M, E, N, K, r)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        device_calls(lib, Xd, dYd, cd, q, Ad, Bd, s, M, E, N, K, r, out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        device_calls(lib, Xd, dYd, cd, q, Ad, Bd, s, M, E, N, K, r, out)
    torch.cuda.synchronize()
    for rep in range(3):
        counts = routing(E, M, 100 + rep)
        say(f"replay {rep}: empty experts {counts.count(0)}, largest {max(counts)}")
        cd.copy_(torch.tensor(counts, dtype=torch.int64))
        Xd.copy_(wl.normal_bf16(200 + rep, (M, K), 1.0))
        dYd.copy_(wl.normal_bf16(300 + rep, (M, N), 1.0))
        for name in ("Y", "T", "dX", "dA", "dB"):
            out[name].fill_(7)
        g.replay()
        torch.cuda.synchronize()
        Yh, Th = lib.qlora_moe_fwd(Xd, counts, q, Ad, Bd, s)
        dXh, dAh, dBh = lib.qlora_moe_bwd(dYd, Xd, counts, q, Ad, Bd, s, Th)
        torch.cuda.synchronize()
        for name, want in (("Y", Yh), ("T", Th), ("dX", dXh), ("dA", dAh), ("dB", dBh)):
            assert torch.equal(out[name].view(torch.int16), want.view(torch.int16)), \
                f"replay {rep}: {name} differs from the host-routed calls"


def test_device_counts_are_clipped(lib):
    """Counts that do not sum to m: negative counts count as 0 and the experts' row ranges are
    clipped at m, so the result equals the host-routed call with the clipped counts; a count
    near the int64 limit does not overflow the running offsets."""
    E, M, K, N, r, s = 6, 300, 256, 64, 8, 1.0
    raw = [5, -3, 1000, 2 ** 62, 7, 0]
    clipped = [5, 0, 295, 0, 0, 0]
    say(f"moe device routing with clipped counts {raw} -> {clipped}")
    X, W, A, B, dY = layer(clipped, K, N, r, 4242)
    q = lib.nf4_quantize(W.to(DEV), 256)
    Xd, dYd, Ad, Bd = X.to(DEV), dY.to(DEV), A.to(DEV), B.to(DEV)
    Yh, Th = lib.qlora_moe_fwd(Xd, clipped, q, Ad, Bd, s)
    dXh, dAh, dBh = lib.qlora_moe_bwd(dYd, Xd, clipped, q, Ad, Bd, s, Th)
    cd = torch.tensor(raw, dtype=torch.int64, device=DEV)
    o = device_calls(lib, Xd, dYd, cd, q, Ad, Bd, s, M, E, N, K, r)
    torch.cuda.synchronize()
    for name, got, want in (("Y", o["Y"], Yh), ("T", o["T"], Th), ("dX", o["dX"], dXh),
                            ("dA", o["dA"], dAh), ("dB", o["dB"], dBh)):
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{name}: clipped routing differs"
