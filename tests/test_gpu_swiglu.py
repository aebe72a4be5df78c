"""GPU parity of the gate/up SwiGLU pair (qlora_swiglu_fwd / qlora_swiglu_bwd) against the oracle.

The stacked NF4 weight [Wg; Wu] is bit-exact against the oracle's quantisation of the same
stacked weight (double-quant runs may straddle the gate/up boundary on both sides alike); H, the
saved Ygu and Tgu, and dX, dAgu, dBg, dBu are within max|got - ref| / max|ref| <= 1e-2 of the
float64 oracle (oracle/swiglu.py). Shapes span several 256-wide tiles with ragged tails, the
M <= 16 kernels, r = 0 and the largest rank (2r = 128).

Where the pair rounds twice and one layer rounds once, its errors sit near twice the
one-rounding floor, so the warning level for a bug hiding under the bar is 8e-3 there (4e-3 for
one layer): the backward (dYg, dYu are rounded to bf16 before the backward GEMMs take them as
their dY) and H on the decode shapes (the activation kernel reads the bf16 Ygu). Above the decode
shapes the fused kernel computes H from the float32 sums of Yg and Yu: one rounding, 4e-3.
"""
import numpy as np
import pytest
import torch

import nf4_dequant_gemm_amd as lib_mod
import workloads as wl
from oracle import nf4, swiglu
from tests.gpu_helpers import assert_quant_equal, check_close as _check_close, f32, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def check_close(name, got, ref, warn_above=8e-3):
    return _check_close(name, got, ref, warn_above=warn_above)


def decode_shaped(M, K):
    """Shapes whose stacked forward takes the decode kernels (H then from the bf16 Ygu)."""
    return M <= 48 and K % 256 == 0

CASES = [
    # M, K, N, r, dq, s
    (64, 256, 128, 8, 256, 2.0),
    (200, 320, 72, 16, 0, -0.5),
    (7, 512, 264, 8, 256, 1.0),        # M <= 16: the stacked forward takes the decode kernel
    (12, 256, 40, 16, 0, 1.5),         # M <= 16 without double quantisation
    (33, 256, 40, 0, 256, 1.0),        # no adapters
    (300, 1024, 520, 64, 256, 0.5),    # 2r = 128, the layer's largest rank
]


def rand_pair(M, K, N, r, seed):
    X = wl.normal_bf16(seed + 1, (M, K), 1.0)
    Wgu = wl.normal_bf16(seed + 2, (2 * N, K), 0.02)
    Agu = wl.normal_bf16(seed + 3, (2 * r, K), K ** -0.5)
    # adapters large enough that the LoRA terms are visible in H
    Bg = wl.normal_bf16(seed + 4, (N, r), 0.1)
    Bu = wl.normal_bf16(seed + 5, (N, r), 0.1)
    dH = wl.normal_bf16(seed + 6, (M, N), 1.0)
    return X, Wgu, Agu, Bg, Bu, dH


def run_pair(lib, M, K, N, r, dq, s, seed):
    X, Wgu, Agu, Bg, Bu, dH = rand_pair(M, K, N, r, seed)
    qo = nf4.quantize(Wgu.float().numpy(), dq)
    Wd = nf4.dequantize_f32(qo)
    f = lambda t: t.float().numpy()
    Ag, Au = (f(Agu[:r]), f(Agu[r:])) if r else (np.zeros((0, K)), np.zeros((0, K)))
    Bgo, Buo = (f(Bg), f(Bu)) if r else (np.zeros((N, 0)), np.zeros((N, 0)))
    ref_fwd = swiglu.forward(f(X), Wd[:N], Wd[N:], Ag, Au, Bgo, Buo, s)
    ref_bwd = swiglu.backward(f(dH), f(X), Wd[:N], Wd[N:], Ag, Au, Bgo, Buo, s)
    qg = lib.nf4_quantize(Wgu.to(DEV), dq)
    d = lambda t: t.to(DEV) if r else None
    H, Ygu, Tgu = lib.qlora_swiglu_fwd(X.to(DEV), qg, d(Agu), d(Bg), d(Bu), s)
    dX, dAgu, dBg, dBu = lib.qlora_swiglu_bwd(dH.to(DEV), X.to(DEV), qg, d(Agu), d(Bg), d(Bu), s, Ygu, Tgu)
    torch.cuda.synchronize()
    assert_quant_equal(qg, qo)
    return (H, Ygu, Tgu, dX, dAgu, dBg, dBu), ref_fwd, ref_bwd


@pytest.mark.parametrize("M,K,N,r,dq,s", CASES)
def test_swiglu_pair_parity(lib, M, K, N, r, dq, s):
    say(f"swiglu pair M={M} K={K} N={N} r={r} dq={dq} s={s}")
    (H, Ygu, Tgu, dX, dAgu, dBg, dBu), (Hr, Yg, Yu, Tg, Tu), (dXr, dAg, dAu, dBgr, dBur) = \
        run_pair(lib, M, K, N, r, dq, s, seed=M * 11 + N)
    check_close("H", f32(H), Hr, warn_above=8e-3 if decode_shaped(M, K) else 4e-3)
    check_close("Ygu", f32(Ygu), np.concatenate([Yg, Yu], axis=1), warn_above=4e-3)
    check_close("dX", f32(dX), dXr)
    if r:
        check_close("Tgu", f32(Tgu), np.concatenate([Tg, Tu], axis=1), warn_above=4e-3)
        check_close("dAgu", f32(dAgu), np.concatenate([dAg, dAu]))
        check_close("dBg", f32(dBg), dBgr)
        check_close("dBu", f32(dBu), dBur)
    else:
        assert Tgu is None and dAgu is None and dBg is None and dBu is None


def test_swiglu_recomputes_missing_tgu(lib):
    """Tgu = None in the backward recomputes it exactly as the forward computes it."""
    M, K, N, r, s = 40, 256, 64, 8, 1.0
    X, Wgu, Agu, Bg, Bu, dH = rand_pair(M, K, N, r, 77)
    qg = lib.nf4_quantize(Wgu.to(DEV), 256)
    X, Agu, Bg, Bu, dH = (t.to(DEV) for t in (X, Agu, Bg, Bu, dH))
    H, Ygu, Tgu = lib.qlora_swiglu_fwd(X, qg, Agu, Bg, Bu, s)
    a = lib.qlora_swiglu_bwd(dH, X, qg, Agu, Bg, Bu, s, Ygu, Tgu)
    b = lib.qlora_swiglu_bwd(dH, X, qg, Agu, Bg, Bu, s, Ygu, None)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_swiglu_autograd_function(lib):
    M, K, N, r, s = 48, 256, 64, 8, 0.5
    X, Wgu, Agu, Bg, Bu, dH = rand_pair(M, K, N, r, 91)
    qg = lib.nf4_quantize(Wgu.to(DEV), 256)
    Xd = X.to(DEV).requires_grad_(True)
    Ad, Bgd, Bud = (t.to(DEV).requires_grad_(True) for t in (Agu, Bg, Bu))
    H = lib_mod.QLoRASwiGLUFunction.apply(Xd, qg, Ad, Bgd, Bud, s)
    H.backward(dH.to(DEV))
    H2, Ygu, Tgu = lib.qlora_swiglu_fwd(X.to(DEV), qg, Agu.to(DEV), Bg.to(DEV), Bu.to(DEV), s)
    ref = lib.qlora_swiglu_bwd(dH.to(DEV), X.to(DEV), qg, Agu.to(DEV), Bg.to(DEV), Bu.to(DEV), s, Ygu, Tgu)
    torch.cuda.synchronize()
    assert torch.equal(H.detach(), H2)
    for got, want in zip((Xd.grad, Ad.grad, Bgd.grad, Bud.grad), ref):
        assert torch.equal(got, want)


def test_swiglu_pair_full_size(lib):
    """The mlp_swiglu pair at full size, as bench.py launches it: the stacked weight bit for bit;
    H, Ygu, Tgu and dX on sampled rows, dAgu on sampled columns, dBg and dBu on sampled rows,
    against the float64 oracle on the same seeded inputs."""
    from tests.test_gpu_workloads import sample, t_full
    p = wl.PAIRS["mlp_swiglu"]
    M, K, N, r, s = p.M, p.K, p.N, p.r, p.s
    say(f"pair {p.name}: M={M} K={K} N={N} r={r} s={s}")
    Wgu = wl.pair_tensor(p, "Wgu")
    X, Agu, Bg, Bu, dH = (wl.pair_tensor(p, t) for t in ("X", "Agu", "Bg", "Bu", "dH"))
    qg = lib.nf4_quantize(Wgu.to(DEV), p.dq_block)
    Xd, Ad, Bgd, Bud = X.to(DEV), Agu.to(DEV), Bg.to(DEV), Bu.to(DEV)
    H, Ygu, Tgu = lib.qlora_swiglu_fwd(Xd, qg, Ad, Bgd, Bud, s)
    dX, dAgu, dBgg, dBug = lib.qlora_swiglu_bwd(dH.to(DEV), Xd, qg, Ad, Bgd, Bud, s, Ygu, Tgu)
    torch.cuda.synchronize()
    say("  fwd + bwd done")
    qo = nf4.quantize(Wgu.float().numpy(), p.dq_block)
    assert_quant_equal(qg, qo)
    del Wgu
    Wd = nf4.dequantize_f32(qo).astype(np.float64)
    Xf, Af, Bgf, Buf, dHf = (f32(t).astype(np.float64) for t in (X, Agu, Bg, Bu, dH))
    Ag, Au = Af[:r], Af[r:]
    Tg, Tu = t_full(f32(X), f32(Agu)[:r]), t_full(f32(X), f32(Agu)[r:])
    # full gate and up outputs in float64 (the gradients of the adapters sum over every row)
    Yg = np.empty((M, N))
    Yu = np.empty((M, N))
    for lo in range(0, M, 1024):
        Yg[lo:lo + 1024] = Xf[lo:lo + 1024] @ Wd[:N].T + s * (Tg[lo:lo + 1024] @ Bgf.T)
        Yu[lo:lo + 1024] = Xf[lo:lo + 1024] @ Wd[N:].T + s * (Tu[lo:lo + 1024] @ Buf.T)
    sg = swiglu.sigmoid(Yg)
    dYg = dHf * Yu * (sg * (1 + Yg * (1 - sg)))
    dYu = dHf * Yg * sg
    rows = sample(M, 48, p.index)
    rt = torch.from_numpy(rows).to(DEV)
    check_close("H", f32(H[rt]), (Yg * sg * Yu)[rows], warn_above=4e-3)
    check_close("Ygu", f32(Ygu[rt]), np.concatenate([Yg[rows], Yu[rows]], axis=1), warn_above=4e-3)
    check_close("Tgu", f32(Tgu[rt]), np.concatenate([Tg[rows], Tu[rows]], axis=1), warn_above=4e-3)
    Ug, Uu = dYg @ Bgf, dYu @ Buf
    dXs = dYg[rows] @ Wd[:N] + dYu[rows] @ Wd[N:] + s * (Ug[rows] @ Ag + Uu[rows] @ Au)
    check_close("dX", f32(dX[rt]), dXs)
    cols = sample(K, 64, p.index + 1)
    dAs = s * np.concatenate([Ug.T @ Xf[:, cols], Uu.T @ Xf[:, cols]])
    check_close("dAgu", f32(dAgu)[:, cols], dAs)
    nrows = sample(N, 64, p.index + 2)
    check_close("dBg", f32(dBgg)[nrows], s * (dYg[:, nrows].T @ Tg))
    check_close("dBu", f32(dBug)[nrows], s * (dYu[:, nrows].T @ Tu))


@pytest.mark.parametrize("M,K,N,r", [(300, 1024, 520, 16), (64, 256, 128, 8), (200, 320, 72, 0),
                                     (264, 320, 136, 5), (300, 512, 264, 32), (72, 256, 200, 64)])
def test_pair_kernel_equals_stacked_layer(lib, M, K, N, r):
    """Above the decode shapes the pair runs as ONE launch of the fused kernel with the activation
    in its epilogue, the block-diagonal up projection applied as B is staged; its Ygu equals the
    plain stacked layer (qlora_fwd with [Wg; Wu] and the block-diagonal B stored) bit for bit,
    ragged last tiles (N % 128 != 0) and a rank that is not a multiple of 8 (element-wise B
    staging) included; with r a multiple of 32 the waves of each half skip the other half's rank
    slices (all-zero B there) and the result is still the same."""
    X, Wgu, Agu, Bg, Bu, _ = rand_pair(M, K, N, r, 300 + M)
    qg = lib.nf4_quantize(Wgu.to(DEV), 256)
    d = lambda t: t.to(DEV) if r else None
    H, Ygu, Tgu = lib.qlora_swiglu_fwd(X.to(DEV), qg, d(Agu), d(Bg), d(Bu), 0.5)
    B2 = None
    if r:
        B2 = torch.zeros(2 * N, 2 * r, dtype=torch.bfloat16)
        B2[:N, :r], B2[N:, r:] = Bg, Bu
        B2 = B2.to(DEV)
    Y2, T2 = lib.qlora_fwd(X.to(DEV), qg, d(Agu), B2, 0.5)
    torch.cuda.synchronize()
    assert torch.equal(Ygu, Y2)
    if r:
        assert torch.equal(Tgu, T2)
    Yg, Yu = f32(Ygu)[:, :N].astype(np.float64), f32(Ygu)[:, N:].astype(np.float64)
    check_close("H from Ygu", f32(H), Yg * swiglu.sigmoid(Yg) * Yu)


@pytest.mark.parametrize("M,K,N,r,s", [(300, 1024, 520, 16, 0.5), (200, 320, 72, 5, -1.5),
                                       (64, 256, 128, 0, 1.0), (9, 512, 264, 8, 2.0)])
def test_swiglu_fwd_fused_entry(lib, M, K, N, r, s):
    """qlora_swiglu_fwd_fused (Tgu given, one launch, no workspace) is the launch qlora_swiglu_fwd
    makes above the decode shapes: the same H and Ygu bit for bit there. On a decode shape (M = 9),
    where qlora_swiglu_fwd runs the decode kernels, it still runs the pair kernel: H and Ygu
    against the oracle."""
    say(f"swiglu fused entry M={M} K={K} N={N} r={r} s={s}")
    X, Wgu, Agu, Bg, Bu, _ = rand_pair(M, K, N, r, 700 + M)
    qg = lib.nf4_quantize(Wgu.to(DEV), 256)
    d = lambda t: t.to(DEV) if r else None
    H, Ygu, Tgu = lib.qlora_swiglu_fwd(X.to(DEV), qg, d(Agu), d(Bg), d(Bu), s)
    H2, Y2 = lib.qlora_swiglu_fwd_fused(X.to(DEV), qg, Tgu, d(Bg), d(Bu), s)
    torch.cuda.synchronize()
    if not decode_shaped(M, K):
        assert torch.equal(Y2, Ygu)
        assert torch.equal(H2, H)
    qo = nf4.quantize(Wgu.float().numpy(), 256)
    Wd = nf4.dequantize_f32(qo)
    f = lambda t: t.float().numpy()
    Ag, Au = (f(Agu[:r]), f(Agu[r:])) if r else (np.zeros((0, K)), np.zeros((0, K)))
    Bgo, Buo = (f(Bg), f(Bu)) if r else (np.zeros((N, 0)), np.zeros((N, 0)))
    Hr, Yg, Yu, _, _ = swiglu.forward(f(X), Wd[:N], Wd[N:], Ag, Au, Bgo, Buo, s)
    check_close("H", f32(H2), Hr, warn_above=4e-3)
    check_close("Ygu", f32(Y2), np.concatenate([Yg, Yu], axis=1), warn_above=4e-3)
