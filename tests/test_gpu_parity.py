"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Quantise and dequantise are bit-exact. Y, dX, dA, dB are within max|got - ref| / max|ref| <= 1e-2
of the float64 oracle. Small shapes span several 256-wide tiles with ragged tails and are
compared element by element; the identity and zero-base probes pin the fused dequantisation and
the LoRA path on their own. The five full-size workloads live in test_gpu_workloads.py.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import nf4, qlora
from tests.gpu_helpers import assert_quant_equal, check_close, f32, say, u16

pytestmark = pytest.mark.gpu

DEV = "cuda"


def rand_layer(M, K, N, r, seed, wstd=0.02, dq=256):
    X = wl.normal_bf16(seed + 1, (M, K), 1.0)
    W = wl.normal_bf16(seed + 2, (N, K), wstd)
    A = wl.normal_bf16(seed + 3, (r, K), K ** -0.5)
    B = wl.normal_bf16(seed + 4, (N, r), 0.01)
    dY = wl.normal_bf16(seed + 5, (M, N), 1.0)
    return X, W, A, B, dY


# ------------------------------------------------------------------------------- quantiser
@pytest.mark.parametrize("n,k,dq,f32in", [(1, 64, 0, False), (3, 192, 256, False), (17, 320, 256, False),
                                          (256, 256, 0, True), (40, 4160, 256, True), (129, 1024, 256, False)])
def test_quantize_bit_exact(lib, n, k, dq, f32in):
    say(f"quantize n={n} k={k} dq={dq} f32={f32in}")
    W = wl.normal_bf16(100 + n, (n, k), 0.02)
    if f32in:
        W = W.float() * (1 + wl.uniform_f32(200 + n, (n, k), 0, 1e-3))   # not bf16-representable
    qg = lib.nf4_quantize(W.to(DEV), dq)
    torch.cuda.synchronize()
    assert_quant_equal(qg, nf4.quantize(W.float().numpy(), dq))


def sweep_weight(a: float) -> np.ndarray:
    """Every finite bf16 value v with |v| <= a, 63 per block after a leading block maximum a."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = nf4.bf16_value(bits)
    v = v[np.isfinite(v) & (np.abs(v) <= a)]
    pad = (-v.size) % 63
    v = np.concatenate([v, np.zeros(pad, np.float32)]).reshape(-1, 63)
    lead = np.full((v.shape[0], 1), a, np.float32)
    lead[1::2] = -a
    return np.concatenate([lead, v], axis=1).reshape(-1)


@pytest.mark.parametrize("a", [1.0, 0.0234375, 3.3895313892515355e38, 1.1754943508222875e-38, 0.7421875])
@pytest.mark.parametrize("dq", [0, 256])
def test_quantize_exhaustive_bf16_sweep(lib, a, dq):
    say(f"bf16 sweep a={a} dq={dq}")
    w = sweep_weight(a)
    w = np.concatenate([w, np.zeros((-w.size) % 256, np.float32)]).reshape(-1, 256)
    Wt = torch.from_numpy(w).to(torch.bfloat16)
    assert np.array_equal(Wt.float().numpy(), w)   # exactly bf16
    qg = lib.nf4_quantize(Wt.to(DEV), dq)
    torch.cuda.synchronize()
    assert_quant_equal(qg, nf4.quantize(w, dq))


def test_quantize_special_blocks(lib):
    w = np.zeros((4, 256), np.float32)
    w[1, 64:128] = -0.0
    w[2, 130] = -5.0
    w[3, 200] = 7.0
    w[3, 201] = -7.0
    for dq in (0, 256):
        qg = lib.nf4_quantize(torch.from_numpy(w).to(torch.bfloat16).to(DEV), dq)
        torch.cuda.synchronize()
        assert_quant_equal(qg, nf4.quantize(w, dq))


@pytest.mark.parametrize("dq", [0, 256])
def test_dequantize_bit_exact(lib, dq):
    say(f"dequantize dq={dq}")
    W = wl.normal_bf16(300 + dq, (72, 640), 0.02)
    qo = nf4.quantize(W.float().numpy(), dq)
    qg = lib.nf4_quantize(W.to(DEV), dq)
    d32 = lib.nf4_dequantize(qg, torch.float32)
    d16 = lib.nf4_dequantize(qg, torch.bfloat16)
    torch.cuda.synchronize()
    assert np.array_equal(d32.cpu().numpy().view(np.uint32), nf4.dequantize_f32(qo).view(np.uint32))
    assert np.array_equal(u16(d16), nf4.dequantize_bf16(qo))


def test_round_trip_on_codebook_points(lib):
    levels = nf4.codebook()
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 16, (8, 512))
    idx[:, ::64] = 0
    e = rng.integers(-10, 3, (8, 8)).astype(np.float64)
    w = (levels[idx].astype(np.float64) * np.repeat(2.0 ** e, 64, axis=1)).astype(np.float32)
    qg = lib.nf4_quantize(torch.from_numpy(w).to(DEV), 0)
    out = lib.nf4_dequantize(qg, torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), w)


# ------------------------------------------------------------------------------- layer
LAYER_CASES = [
    # M, K, N, r, dq, s
    (64, 256, 256, 8, 0, 2.0),
    (1, 64, 8, 1, 0, 1.0),
    (300, 320, 264, 24, 256, 0.5),
    (257, 512, 520, 5, 256, -1.5),
    (33, 128, 16, 128, 0, 0.25),
    (513, 640, 776, 0, 256, 1.0),
    (200, 1024, 96, 64, 256, 2.0),
    # at most 16 rows (the short-reduction row projection) with N not a multiple of 32, so the
    # U = dY B reduction ends inside a 32-column slice
    (12, 256, 200, 16, 256, 1.5),
    (16, 320, 72, 8, 0, -0.5),
    (3, 128, 40, 24, 256, 2.0),
]


def oracle_layer(X, W, A, B, dY, s, dq):
    qo = nf4.quantize(W.float().numpy(), dq)
    Wd = nf4.dequantize_f32(qo)
    Y, T = qlora.forward(f32(X), Wd, f32(A), f32(B), s)
    dX, dA, dB = qlora.backward(f32(dY), f32(X), Wd, f32(A), f32(B), s)
    return qo, Y, T, dX, dA, dB


@pytest.mark.parametrize("M,K,N,r,dq,s", LAYER_CASES)
def test_layer_parity(lib, M, K, N, r, dq, s):
    say(f"layer M={M} K={K} N={N} r={r} dq={dq} s={s}")
    X, W, A, B, dY = rand_layer(M, K, N, r, seed=M * 7 + N)
    qo, Y, T, dX, dA, dB = oracle_layer(X, W, A, B, dY, s, dq)
    qg = lib.nf4_quantize(W.to(DEV), dq)
    Ad, Bd = (A.to(DEV), B.to(DEV)) if r else (None, None)
    Yg, Tg = lib.qlora_fwd(X.to(DEV), qg, Ad, Bd, s)
    dXg, dAg, dBg = lib.qlora_bwd(dY.to(DEV), X.to(DEV), qg, Ad, Bd, s, Tg)
    torch.cuda.synchronize()
    assert_quant_equal(qg, qo)
    check_close("Y", f32(Yg), Y)
    check_close("dX", f32(dXg), dX)
    if r:
        check_close("T", f32(Tg), T)
        check_close("dA", f32(dAg), dA)
        check_close("dB", f32(dBg), dB)


# Forward with at most 64 rows of X and K % 256 == 0 takes the weight-streaming kernel: stage
# counts 1..9 of 512 columns (one to three stages after the two-stage main loop), half-live last
# stages, ragged last 64-row tile, every 16-row m-tile count. K % 256 != 0 falls back to the
# large-M kernel (last two cases).
DECODE_CASES = [
    # M, K, N, r, dq
    (1, 256, 8, 1, 0),
    (16, 768, 200, 16, 256),
    (17, 1280, 72, 8, 0),
    (40, 2048, 136, 4, 256),
    (64, 2560, 64, 32, 256),
    (5, 4352, 264, 0, 0),
    (33, 4352, 136, 16, 256),
    (48, 3328, 520, 64, 0),
    (16, 576, 200, 16, 256),
    (9, 1600, 72, 8, 0),
    # M <= 16 with double quantisation (the 112-row stage-ring kernel): one stage, stage counts
    # around the 8-stage loop and its 4-stage code windows, ragged and multi-workgroup N
    (1, 256, 8, 0, 256),
    (3, 1792, 112, 1, 256),
    (7, 2304, 120, 8, 256),
    (16, 4352, 1000, 64, 256),
    (16, 8192, 336, 16, 256),
]


@pytest.mark.parametrize("M,K,N,r,dq", DECODE_CASES)
def test_decode_forward_parity(lib, M, K, N, r, dq):
    s = 1.5
    say(f"decode-shaped forward M={M} K={K} N={N} r={r} dq={dq}")
    X, W, A, _, _ = rand_layer(M, K, N, r, seed=M * 11 + K + N)
    B = wl.normal_bf16(M * 11 + K + N + 9, (N, r), 0.1)   # LoRA term comparable to the base term
    qo = nf4.quantize(W.float().numpy(), dq)
    Y, T = qlora.forward(f32(X), nf4.dequantize_f32(qo), f32(A), f32(B), s)
    qg = lib.nf4_quantize(W.to(DEV), dq)
    Ad, Bd = (A.to(DEV), B.to(DEV)) if r else (None, None)
    Yg, Tg = lib.qlora_fwd(X.to(DEV), qg, Ad, Bd, s)
    torch.cuda.synchronize()
    check_close("Y", f32(Yg), Y)
    if r:
        check_close("T", f32(Tg), T)


def test_identity_probe_forward(lib):
    """X = I_K, r = 0: Y = bf16(deq(W))^T bit for bit (one exact product per output)."""
    K, N = 256, 264
    W = wl.normal_bf16(901, (N, K), 0.02)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    X = torch.eye(K, dtype=torch.bfloat16, device=DEV)
    Yg, _ = lib.qlora_fwd(X, qg, None, None, 1.0)
    torch.cuda.synchronize()
    want = nf4.dequantize_bf16(nf4.quantize(W.float().numpy(), 256)).T
    assert np.array_equal(u16(Yg), want)


def test_identity_probe_dx(lib):
    """dY = I_N, r = 0: dX = bf16(deq(W)) bit for bit (the transposed weight read of dX)."""
    K, N = 320, 264
    W = wl.normal_bf16(902, (N, K), 0.02)
    qg = lib.nf4_quantize(W.to(DEV), 0)
    dY = torch.eye(N, dtype=torch.bfloat16, device=DEV)
    X = torch.zeros(N, K, dtype=torch.bfloat16, device=DEV)
    dXg, _, _ = lib.qlora_bwd(dY, X, qg, None, None, 1.0, None)
    torch.cuda.synchronize()
    want = nf4.dequantize_bf16(nf4.quantize(W.float().numpy(), 0))
    assert np.array_equal(u16(dXg), want)


def test_rank_zero_equals_b_zero(lib):
    """r = 0 and B = 0 give bitwise-identical Y (the LoRA steps add exact zeros)."""
    M, K, N, r = 300, 384, 272, 16
    X, W, A, B, dY = rand_layer(M, K, N, r, seed=77)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    Y0, _ = lib.qlora_fwd(X.to(DEV), qg, None, None, 2.0)
    Yb, _ = lib.qlora_fwd(X.to(DEV), qg, A.to(DEV), torch.zeros_like(B).to(DEV), 2.0)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Yb.view(torch.int16))
    qo = nf4.quantize(W.float().numpy(), 256)
    plain = f32(X).astype(np.float64) @ nf4.dequantize_f32(qo).T.astype(np.float64)
    check_close("Y(r=0)", f32(Y0), plain)


def test_zero_base_probe(lib):
    """W = 0: Y = s T B^T and dX = s U A, the LoRA path alone."""
    M, K, N, r, s = 130, 256, 136, 32, 0.5
    X, _, A, B, dY = rand_layer(M, K, N, r, seed=88)
    B = wl.normal_bf16(99, (N, r), 1.0)
    W = torch.zeros(N, K, dtype=torch.bfloat16)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    Yg, Tg = lib.qlora_fwd(X.to(DEV), qg, A.to(DEV), B.to(DEV), s)
    dXg, dAg, dBg = lib.qlora_bwd(dY.to(DEV), X.to(DEV), qg, A.to(DEV), B.to(DEV), s, Tg)
    torch.cuda.synchronize()
    Wd = np.zeros((N, K))
    Y, _ = qlora.forward(f32(X), Wd, f32(A), f32(B), s)
    dX, dA, dB = qlora.backward(f32(dY), f32(X), Wd, f32(A), f32(B), s)
    check_close("Y", f32(Yg), Y)
    check_close("dX", f32(dXg), dX)
    check_close("dA", f32(dAg), dA)
    check_close("dB", f32(dBg), dB)


def test_deterministic(lib):
    M, K, N, r = 700, 1024, 520, 16
    X, W, A, B, dY = rand_layer(M, K, N, r, seed=55)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    outs = []
    for _ in range(2):
        Y, T = lib.qlora_fwd(X.to(DEV), qg, A.to(DEV), B.to(DEV), 1.0)
        dX, dA, dB = lib.qlora_bwd(dY.to(DEV), X.to(DEV), qg, A.to(DEV), B.to(DEV), 1.0, T)
        outs.append([t.view(torch.int16).clone() for t in (Y, T, dX, dA, dB)])
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_autograd_function(lib):
    M, K, N, r, s = 96, 256, 200, 8, 2.0
    X, W, A, B, dY = rand_layer(M, K, N, r, seed=66)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    Xd = X.to(DEV).requires_grad_(True)
    Ad = A.to(DEV).requires_grad_(True)
    Bd = B.to(DEV).requires_grad_(True)
    Y = lib.QLoRALinearFunction.apply(Xd, qg, Ad, Bd, s)
    Y.backward(dY.to(DEV))
    torch.cuda.synchronize()
    qo, Yo, _, dXo, dAo, dBo = oracle_layer(X, W, A, B, dY, s, 256)
    check_close("Y", f32(Y), Yo)
    check_close("dX", f32(Xd.grad), dXo)
    check_close("dA", f32(Ad.grad), dAo)
    check_close("dB", f32(Bd.grad), dBo)


def test_bwd_split_matches_bwd(lib):
    """qlora_bwd without dX leaves U at the start of the workspace; qlora_bwd_dx on that U gives
    the dX of a full qlora_bwd bit for bit, and U matches dY B from the oracle."""
    import ctypes
    M, K, N, r, s = 200, 512, 264, 16, 0.5
    X, W, A, B, dY = rand_layer(M, K, N, r, seed=123)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    Xd, Ad, Bd, dYd = X.to(DEV), A.to(DEV), B.to(DEV), dY.to(DEV)
    _, T = lib.qlora_fwd(Xd, qg, Ad, Bd, s)
    dX_full, dA_full, dB_full = lib.qlora_bwd(dYd, Xd, qg, Ad, Bd, s, T)
    c = lib.library()
    wsb = c.qlora_bwd_workspace_bytes(M, N, K, r)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    dA = torch.empty(r, K, dtype=torch.bfloat16, device=DEV)
    dB = torch.empty(N, r, dtype=torch.bfloat16, device=DEV)
    st = qg.c_struct()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert c.qlora_bwd(p(dYd), p(Xd), M, ctypes.byref(st), p(Ad), p(Bd), r, s, p(T), None, p(dA), p(dB),
                       p(ws), wsb, sp) == 0
    U = ws[: M * r * 2].view(torch.bfloat16).view(M, r)
    dX = lib.qlora_bwd_dx(dYd, qg, U, Ad, s)
    torch.cuda.synchronize()
    assert torch.equal(dX.view(torch.int16), dX_full.view(torch.int16))
    assert torch.equal(dA.view(torch.int16), dA_full.view(torch.int16))
    assert torch.equal(dB.view(torch.int16), dB_full.view(torch.int16))
    check_close("U", f32(U), f32(dY).astype(np.float64) @ f32(B).astype(np.float64))


@pytest.mark.parametrize("M,K,N,r", [(16, 2048, 448, 128), (5, 1024, 200, 96)])
def test_decode_qlora_fwd_matches_two_calls(lib, M, K, N, r):
    """On decode shapes with r > 64 qlora_fwd adds the split partials of T inside the fused
    kernel; Y and T equal those of qlora_lora_down followed by qlora_fwd_fused bit for bit (same
    partials, same summation order), and T matches X A^T from the oracle."""
    s = 2.0
    X, W, A, _, _ = rand_layer(M, K, N, r, seed=M * 7 + K + N)
    B = wl.normal_bf16(M + K + N + 5, (N, r), 0.1)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    Xd, Ad, Bd = X.to(DEV), A.to(DEV), B.to(DEV)
    Y1, T1 = lib.qlora_fwd(Xd, qg, Ad, Bd, s)
    T2 = lib.qlora_lora_down(Xd, Ad)
    Y2 = lib.qlora_fwd_fused(Xd, qg, T2, Bd, s)
    torch.cuda.synchronize()
    assert torch.equal(T1.view(torch.int16), T2.view(torch.int16))
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    check_close("T", f32(T1), f32(X).astype(np.float64) @ f32(A).astype(np.float64).T)


@pytest.mark.parametrize("M,K,N,r", [(16, 8192, 336, 16), (7, 2304, 120, 8), (1, 768, 232, 64),
                                     (16, 4096, 1000, 32), (3, 512, 120, 48)])
def test_decode_qlora_fwd_forms_T(lib, M, K, N, r):
    """On decode shapes with r <= 64 the stream kernel forms T = X A^T itself (one launch). T and Y
    match the oracle; where no workgroup's walk over K is rotated (fewer than 8 stages, or a
    count not a multiple of 4), every workgroup sums T in the same order, so Y equals
    qlora_fwd_fused given that T bit for bit."""
    s = 2.0
    X, W, A, _, _ = rand_layer(M, K, N, r, seed=M * 5 + K + N + r)
    B = wl.normal_bf16(M + K + N + 6, (N, r), 0.1)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    Xd, Ad, Bd = X.to(DEV), A.to(DEV), B.to(DEV)
    Y1, T1 = lib.qlora_fwd(Xd, qg, Ad, Bd, s)
    Y2 = lib.qlora_fwd_fused(Xd, qg, T1, Bd, s)
    torch.cuda.synchronize()
    nst = K // 256
    if nst < 8 or nst % 4:
        assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    qo = nf4.quantize(W.float().numpy(), 256)
    Yo, To = qlora.forward(f32(X), nf4.dequantize_f32(qo), f32(A), f32(B), s)
    check_close("T", f32(T1), To)
    check_close("Y", f32(Y1), Yo)


@pytest.mark.parametrize("M,K,N,r", [(200, 512, 264, 16), (16, 2304, 120, 8)])
def test_bwd_recomputes_missing_T(lib, M, K, N, r):
    """qlora_bwd with T = NULL recomputes T = X A^T in its workspace by the row projection of
    qlora_lora_down: dX, dA and dB equal those of a call given that T, bit for bit."""
    s = 0.5
    X, W, A, B, dY = rand_layer(M, K, N, r, seed=M + 3 * K + N)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    Xd, Ad, Bd, dYd = X.to(DEV), A.to(DEV), B.to(DEV), dY.to(DEV)
    T = lib.qlora_lora_down(Xd, Ad)
    g1 = lib.qlora_bwd(dYd, Xd, qg, Ad, Bd, s, T)
    g2 = lib.qlora_bwd(dYd, Xd, qg, Ad, Bd, s, None)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
