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


@pytest.mark.parametrize("M,K,N,r", [(300, 512, 264, 16), (8, 1024, 512, 16)])
def test_forward_backward_replay_equals_eager(lib, M, K, N, r):
    say(f"graph M={M} K={K} N={N} r={r}")
    X = wl.normal_bf16(1, (M, K), 1.0).to(DEV)
    W = wl.normal_bf16(2, (N, K), 0.02).to(DEV)
    A = wl.normal_bf16(3, (r, K), K ** -0.5).to(DEV)
    B = wl.normal_bf16(4, (N, r), 0.1).to(DEV)
    dY = wl.normal_bf16(5, (M, N), 1.0).to(DEV)
    q = lib.nf4_quantize(W, 256)
    s = 0.5

    def step():
        Y, T = lib.qlora_fwd(X, q, A, B, s)
        dX, dA, dB = lib.qlora_bwd(dY, X, q, A, B, s, T)
        return Y, T, dX, dA, dB

    eager = step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # warm the allocator on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:
            t.fill_(7)                        # replays must overwrite every output
        g.replay()
        torch.cuda.synchronize()
        again = step()                        # eager work between the replays
        torch.cuda.synchronize()
        for name, got, want, e2 in zip(("Y", "T", "dX", "dA", "dB"), outs, eager, again):
            assert torch.equal(got, want), f"replay {rep}: {name} differs from the eager call"
            assert torch.equal(e2, want), f"eager call {rep}: {name} changed"
