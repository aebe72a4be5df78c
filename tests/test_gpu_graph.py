"""The layer's calls under HIP graph capture.

Every launch path of the forward and backward is kernels only (no memset nodes, no allocation,
no host synchronisation), so a caller can capture them. The test captures one forward + backward
of a QLoRA layer (large-M kernels and the decode-shaped path) into a graph, replays it several
times with the program's own eager work and synchronisations in between, and checks every replay
against the eager calls bit for bit (the kernels are deterministic).
"""
import pytest
import torch

import workloads as wl
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _replay_check(step):
    """Capture step() in a graph (after a warm-up on the capture stream), replay it three times
    with every output overwritten first and an eager step() in between, and require every replay
    and every eager call to equal the first eager call bit for bit."""
    eager = step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(7)
        g.replay()
        torch.cuda.synchronize()
        again = step()
        torch.cuda.synchronize()
        for i, (got, want, e2) in enumerate(zip(outs, eager, again)):
            assert torch.equal(got, want), f"replay {rep}: output {i} differs from the eager call"
            assert torch.equal(e2, want), f"eager call {rep}: output {i} changed"


@pytest.mark.parametrize("M,K,N,r", [(300, 512, 264, 16), (8, 1024, 512, 16)])
def test_forward_backward_replay_equals_eager(lib, M, K, N, r):
    say(f"graph M={M} K={K} N={N} r={r}")
    X = wl.normal_bf16(1, (M, K), 1.0).to(DEV)
    W = wl.normal_bf16(2, (N, K), 0.02).to(DEV)
    A = wl.normal_bf16(3, (r, K), K ** -0.5).to(DEV)
    B = wl.normal_bf16(4, (N, r), 0.1).to(DEV)
    dY = wl.normal_bf16(5, (M, N), 1.0).to(DEV)
    q = lib.nf4_quantize(W, 256)

    def step():
        Y, T = lib.qlora_fwd(X, q, A, B, 0.5)
        return (Y, T) + tuple(lib.qlora_bwd(dY, X, q, A, B, 0.5, T))

    _replay_check(step)


def test_swiglu_pair_replay_equals_eager(lib):
    """The gate/up pair (the fused kernel's pair form, the activation backward) under capture."""
    M, K, N, r, s = 300, 512, 136, 8, 0.5
    X = wl.normal_bf16(11, (M, K), 1.0).to(DEV)
    Wgu = wl.normal_bf16(12, (2 * N, K), 0.02).to(DEV)
    Agu = wl.normal_bf16(13, (2 * r, K), K ** -0.5).to(DEV)
    Bg, Bu = wl.normal_bf16(14, (N, r), 0.1).to(DEV), wl.normal_bf16(15, (N, r), 0.1).to(DEV)
    dH = wl.normal_bf16(16, (M, N), 1.0).to(DEV)
    q = lib.nf4_quantize(Wgu, 256)

    def step():
        H, Ygu, Tgu = lib.qlora_swiglu_fwd(X, q, Agu, Bg, Bu, s)
        return (H, Ygu, Tgu) + tuple(lib.qlora_swiglu_bwd(dH, X, q, Agu, Bg, Bu, s, Ygu, Tgu))

    _replay_check(step)


def test_moe_replay_equals_eager(lib):
    """The grouped MoE layer (grouped row projections, fused kernels and M-reductions) under
    capture; the routing counts are host values fixed at capture time."""
    counts, K, N, r, s = [70, 0, 200, 9], 512, 72, 16, 1.5
    E, M = len(counts), sum(counts)
    X = wl.normal_bf16(21, (M, K), 1.0).to(DEV)
    W = wl.normal_bf16(22, (E * N, K), 0.02).to(DEV)
    A = wl.normal_bf16(23, (E * r, K), K ** -0.5).to(DEV)
    B = wl.normal_bf16(24, (E * N, r), 0.1).to(DEV)
    dY = wl.normal_bf16(25, (M, N), 1.0).to(DEV)
    q = lib.nf4_quantize(W, 256)

    def step():
        Y, T = lib.qlora_moe_fwd(X, counts, q, A, B, s)
        return (Y, T) + tuple(lib.qlora_moe_bwd(dY, X, counts, q, A, B, s, T))

    _replay_check(step)
