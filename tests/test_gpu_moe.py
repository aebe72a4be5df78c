"""GPU parity of the grouped (mixture-of-experts) layer (qlora_moe_fwd / qlora_moe_bwd) against
the oracle.

The stacked expert weight [W_0; ...; W_{E-1}] is bit-exact against the oracle's quantisation of
the same stacked weight; Y, T, dX, dA and dB are within max|got - ref| / max|ref| <= 1e-2 of the
float64 oracle (oracle/moe.py), per expert as well as over all rows (an expert with few rows must
not hide under the others' scale). The cases cover empty experts (zero adapter gradients), an
expert with one row, expert row counts that straddle the 256-row tile, ragged n against the
256-column tile, runs of the double quantisation that straddle two experts, r = 0, the largest
rank and 64 experts. With one expert the grouped layer is the plain layer, bit for bit.

An expert with a handful of rows sums few products into dB = s dY^T T, so the bf16 rounding of
T does not average out there and its relative error can sit near two roundings (the warning
level for its per-expert check is 8e-3, the bar stays 1e-2).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import moe, nf4
from tests.gpu_helpers import assert_quant_equal, check_close, f32, say

pytestmark = pytest.mark.gpu

DEV = "cuda"

CASES = [
    # counts, K, N, r, dq, s
    ([0, 37, 300, 5], 512, 128, 8, 256, 1.0),
    ([64, 1, 200], 320, 72, 16, 0, -0.5),
    ([33, 250, 9], 320, 72, 16, 256, 1.5),         # runs of 256 block constants straddle experts
    ([257, 0], 256, 256, 0, 256, 1.0),             # no adapters
    ([40, 90, 3, 0, 260, 17, 1, 128], 1024, 264, 64, 256, 0.5),
    ([130, 0, 0, 70], 1024, 64, 128, 0, 2.0),      # the largest rank
]


def rand_moe(counts, K, N, r, seed):
    E, M = len(counts), int(sum(counts))
    X = wl.normal_bf16(seed + 1, (M, K), 1.0)
    W = wl.normal_bf16(seed + 2, (E * N, K), 0.02)
    A = wl.normal_bf16(seed + 3, (E * r, K), K ** -0.5)
    B = wl.normal_bf16(seed + 4, (E * N, r), 0.1)      # large enough that the LoRA term shows in Y
    dY = wl.normal_bf16(seed + 5, (M, N), 1.0)
    return X, W, A, B, dY


def check_experts(name, got, ref, off, what="rows"):
    """Each expert's part on its own scale, then the whole."""
    for e in range(len(off) - 1):
        lo, hi = off[e], off[e + 1]
        if hi > lo and np.abs(ref[lo:hi]).max() > 0:
            check_close(f"{name}[{what} of expert {e}]", got[lo:hi], ref[lo:hi], warn_above=8e-3)
    check_close(name, got, ref)


@pytest.mark.parametrize("counts,K,N,r,dq,s", CASES)
def test_moe_parity(lib, counts, K, N, r, dq, s):
    E = len(counts)
    say(f"moe E={E} counts={counts} K={K} N={N} r={r} dq={dq} s={s}")
    X, W, A, B, dY = rand_moe(counts, K, N, r, seed=7 * sum(counts) + N)
    qg = lib.nf4_quantize(W.to(DEV), dq)
    d = lambda t: t.to(DEV) if r else None
    Y, T = lib.qlora_moe_fwd(X.to(DEV), counts, qg, d(A), d(B), s)
    dX, dA, dB = lib.qlora_moe_bwd(dY.to(DEV), X.to(DEV), counts, qg, d(A), d(B), s, T)
    torch.cuda.synchronize()
    qo = nf4.quantize(W.float().numpy(), dq)
    assert_quant_equal(qg, qo)
    Wd = nf4.dequantize_f32(qo)
    Yr, Tr = moe.forward(f32(X), counts, Wd, f32(A), f32(B), s)
    dXr, dAr, dBr = moe.backward(f32(dY), f32(X), counts, Wd, f32(A), f32(B), s)
    off = moe.offsets(counts)
    check_experts("Y", f32(Y), Yr, off)
    check_experts("dX", f32(dX), dXr, off)
    if r:
        check_experts("T", f32(T), Tr, off)
        check_experts("dA", f32(dA), dAr, [e * r for e in range(E + 1)], "ranks")
        check_experts("dB", f32(dB), dBr, [e * N for e in range(E + 1)], "ranks")
        for e in range(E):
            if counts[e] == 0:     # no rows routed: the gradients are exactly zero
                assert not torch.any(dA[e * r:(e + 1) * r]) and not torch.any(dB[e * N:(e + 1) * N])
    else:
        assert T is None and dA is None and dB is None


def test_moe_sixty_four_experts(lib):
    """The most experts the grouped launch takes, mostly small groups (the decode-like case)."""
    rng = np.random.default_rng(64)
    counts = [int(c) for c in rng.integers(0, 9, size=64)]
    K, N, r, s = 256, 64, 8, 1.0
    X, W, A, B, dY = rand_moe(counts, K, N, r, seed=640)
    qg = lib.nf4_quantize(W.to(DEV), 0)
    Y, T = lib.qlora_moe_fwd(X.to(DEV), counts, qg, A.to(DEV), B.to(DEV), s)
    dX, dA, dB = lib.qlora_moe_bwd(dY.to(DEV), X.to(DEV), counts, qg, A.to(DEV), B.to(DEV), s, None)
    torch.cuda.synchronize()
    Wd = nf4.dequantize_f32(nf4.quantize(W.float().numpy(), 0))
    Yr, Tr = moe.forward(f32(X), counts, Wd, f32(A), f32(B), s)
    dXr, dAr, dBr = moe.backward(f32(dY), f32(X), counts, Wd, f32(A), f32(B), s)
    check_close("Y", f32(Y), Yr)
    check_close("T", f32(T), Tr)
    check_close("dX", f32(dX), dXr)
    check_close("dA", f32(dA), dAr)
    check_close("dB", f32(dB), dBr)


def test_moe_one_expert_is_the_plain_layer(lib):
    """E = 1: the grouped launches run the fused kernels on the same tiles as qlora_fwd and
    qlora_bwd, and U, T, dA, dB take the same row projections and reductions, so every output
    agrees bit for bit."""
    M, K, N, r, s = 300, 512, 264, 16, 0.75
    X, W, A, B, dY = rand_moe([M], K, N, r, seed=1)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    Xd, Ad, Bd, dYd = X.to(DEV), A.to(DEV), B.to(DEV), dY.to(DEV)
    Y1, T1 = lib.qlora_moe_fwd(Xd, [M], qg, Ad, Bd, s)
    Y0, T0 = lib.qlora_fwd(Xd, qg, Ad, Bd, s)
    Y2 = lib.qlora_moe_fwd_fused(Xd, [M], qg, T1, Bd, s)
    g1 = lib.qlora_moe_bwd(dYd, Xd, [M], qg, Ad, Bd, s, T1)
    g0 = lib.qlora_bwd(dYd, Xd, qg, Ad, Bd, s, T0)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y0) and torch.equal(T1, T0) and torch.equal(Y2, Y0)
    for a, b in zip(g1, g0):
        assert torch.equal(a, b)


def test_moe_recomputes_missing_t(lib):
    """T = None in the backward recomputes each expert's T exactly as the forward computes it."""
    counts, K, N, r, s = [70, 0, 19, 300], 512, 96, 16, -1.25
    X, W, A, B, dY = rand_moe(counts, K, N, r, seed=33)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    Xd, Ad, Bd, dYd = X.to(DEV), A.to(DEV), B.to(DEV), dY.to(DEV)
    Y, T = lib.qlora_moe_fwd(Xd, counts, qg, Ad, Bd, s)
    a = lib.qlora_moe_bwd(dYd, Xd, counts, qg, Ad, Bd, s, T)
    b = lib.qlora_moe_bwd(dYd, Xd, counts, qg, Ad, Bd, s, None)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_moe_full_size(lib):
    """The moe_mlp_up layer at full size, as bench.py launches it (8 experts of K 4096, N 11008,
    16384 routed rows, r 16): the stacked weight bit for bit; Y, T and dX on sampled rows of
    every expert, dA on sampled columns and dB on sampled rows of every expert's block, against
    the float64 oracle on the same seeded inputs."""
    from tests.test_gpu_workloads import sample
    mw = wl.MOES["moe_mlp_up"]
    counts, E, K, N, r, s = mw.counts(), mw.E, mw.K, mw.N, mw.r, mw.s
    say(f"moe {mw.name}: E={E} counts={counts} K={K} N={N} r={r} s={s}")
    W = wl.moe_tensor(mw, "W")
    X, A, B, dY = (wl.moe_tensor(mw, t) for t in ("X", "A", "B", "dY"))
    qg = lib.nf4_quantize(W.to(DEV), mw.dq_block)
    Xd, Ad, Bd = X.to(DEV), A.to(DEV), B.to(DEV)
    Y, T = lib.qlora_moe_fwd(Xd, counts, qg, Ad, Bd, s)
    dX, dA, dB = lib.qlora_moe_bwd(dY.to(DEV), Xd, counts, qg, Ad, Bd, s, T)
    torch.cuda.synchronize()
    say("  fwd + bwd done")
    qo = nf4.quantize(W.float().numpy(), mw.dq_block)
    assert_quant_equal(qg, qo)
    del W
    Wd = nf4.dequantize_f32(qo)
    Xf, Af, Bf, dYf = (f32(t).astype(np.float64) for t in (X, A, B, dY))
    off = moe.offsets(counts)
    Yg, Tg, dXg = f32(Y), f32(T), f32(dX)
    dAg, dBg = f32(dA), f32(dB)
    for e in range(E):
        lo, hi = int(off[e]), int(off[e + 1])
        We = Wd[e * N:(e + 1) * N].astype(np.float64)
        Ae, Be = Af[e * r:(e + 1) * r], Bf[e * N:(e + 1) * N]
        rows = lo + sample(hi - lo, 16, 100 + e)
        Te = Xf[lo:hi] @ Ae.T                                   # [me, r]
        Ue = dYf[lo:hi] @ Be                                    # [me, r]
        check_close(f"Y[expert {e}]", Yg[rows], Xf[rows] @ We.T + s * (Te[rows - lo] @ Be.T))
        check_close(f"T[expert {e}]", Tg[rows], Te[rows - lo])
        check_close(f"dX[expert {e}]", dXg[rows], dYf[rows] @ We + s * (Ue[rows - lo] @ Ae))
        cols = sample(K, 32, 200 + e)
        check_close(f"dA[expert {e}]", dAg[e * r:(e + 1) * r][:, cols], s * (Ue.T @ Xf[lo:hi, cols]))
        nrows = sample(N, 32, 300 + e)
        check_close(f"dB[expert {e}]", dBg[e * N:(e + 1) * N][nrows], s * (dYf[lo:hi, nrows].T @ Te))
