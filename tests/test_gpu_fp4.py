"""GPU parity of the 4-bit floating-point (E2M1) weight format against the oracle (oracle/fp4.py).

* quantisation bit-exact: codes, E4M3 group scales and the float32 tensor scale, for bf16 and
  float32 inputs, an all-zero weight, all-zero groups, tiny and large magnitudes;
* dequantisation exact (float32) and its bf16 rounding;
* the fused layer with an E2M1 base (qlora_fwd, qlora_bwd through the fused forward and dX
  kernels): Y, T, dX, dA, dB within max|got - ref| / max|ref| <= 1e-2 of the float64 oracle on
  ragged shapes, r = 0 and r = 128, M <= 16;
* identity probes: X = I gives Y = bf16(deq(W))^T and dY = I gives dX = bf16(deq(W)), bit for
  bit (the decoded operand e2m1 * s is exact in bf16 and the tensor scale is applied once, in
  float32, so both equal one rounding of the exact dequantised value);
* the grouped (MoE) layer and the gate/up SwiGLU pair with E2M1 weights;
* the LoRA merge of an E2M1 base: within one bf16 ulp of the oracle, r = 0 equal to the bf16
  dequantisation, and its re-quantisation to E2M1 (a compressed FP4 export) bit-exact.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import fp4, merge, moe, nf4, qlora, swiglu
from tests.gpu_helpers import assert_fp4_equal, check_close, f32, say, u16

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("n,k,std,f32_in", [
    (64, 256, 0.02, False),
    (200, 320, 1.0, True),
    (8, 64, 3e-4, False),
    (264, 1024, 0.02, True),
])
def test_quantize_bit_exact(lib, n, k, std, f32_in):
    say(f"fp4 quantize n={n} k={k} std={std} f32={f32_in}")
    W = wl.normal_bf16(900 + n, (n, k), std)
    Wf = W.float()
    if f32_in:   # float32 values off the bf16 grid
        Wf = Wf + torch.from_numpy(np.random.default_rng(n).standard_normal((n, k)).astype(np.float32)) * std * 1e-3
    Wf[1, 16:48] = 0.0                                   # two all-zero groups
    Wf[n - 1, k - 1] = 50 * std                          # one large value: many groups get small scales
    src = Wf if f32_in else Wf.to(torch.bfloat16)
    qg = lib.fp4_quantize(src.to(DEV))
    torch.cuda.synchronize()
    qo = fp4.quantize(src.float().numpy())
    assert_fp4_equal(qg, qo)
    ref = fp4.dequantize_f32(qo)
    d32 = lib.nf4_dequantize(qg, torch.float32).cpu().numpy()
    assert np.array_equal(d32.view(np.uint32), ref.view(np.uint32))
    d16 = u16(lib.nf4_dequantize(qg, torch.bfloat16))
    assert np.array_equal(d16, nf4.bf16_bits(ref))


def test_quantize_all_zero(lib):
    qg = lib.fp4_quantize(torch.zeros(16, 128, dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert not qg.codes.any() and not qg.absmax.any() and qg.scale[0].item() == 0.0
    assert not lib.nf4_dequantize(qg, torch.float32).any()


LAYER_CASES = [
    # M, K, N, r, s
    (64, 256, 128, 8, 2.0),
    (300, 320, 72, 16, -0.5),
    (7, 512, 264, 8, 1.0),           # M <= 16, K % 256 == 0: the stream kernel's E2M1 form
    (1, 1024, 264, 8, 1.0),
    (16, 8192, 512, 16, 2.0),
    (5, 768, 232, 12, 0.5),          # r % 8 != 0: T by the separate projection, the LoRA term
                                     # element by element; ragged last workgroup
    (12, 2304, 448, 0, 1.0),         # no adapters, four full workgroups
    (9, 320, 136, 8, 1.0),           # K % 256 != 0: the large-M kernel's E2M1 form
    (40, 512, 136, 8, 0.5),          # 16 < M <= 48: the large-M kernel (E2M1 stream form: M <= 16)
    (257, 1024, 64, 0, 1.0),         # no adapters
    (130, 512, 136, 128, 0.25),      # the largest rank
]


@pytest.mark.parametrize("M,K,N,r,s", LAYER_CASES)
def test_layer_parity(lib, M, K, N, r, s):
    say(f"fp4 layer M={M} K={K} N={N} r={r} s={s}")
    X = wl.normal_bf16(M + 1, (M, K), 1.0)
    W = wl.normal_bf16(N + 2, (N, K), 0.02)
    A = wl.normal_bf16(r + 3, (r, K), K ** -0.5)
    B = wl.normal_bf16(r + 4, (N, r), 0.1)
    dY = wl.normal_bf16(M + 5, (M, N), 1.0)
    qg = lib.fp4_quantize(W.to(DEV))
    d = lambda t: t.to(DEV) if r else None
    Y, T = lib.qlora_fwd(X.to(DEV), qg, d(A), d(B), s)
    dX, dA, dB = lib.qlora_bwd(dY.to(DEV), X.to(DEV), qg, d(A), d(B), s, T)
    torch.cuda.synchronize()
    qo = fp4.quantize(W.float().numpy())
    assert_fp4_equal(qg, qo)
    Wd = fp4.dequantize_f32(qo)
    Yr, Tr = qlora.forward(f32(X), Wd, f32(A), f32(B), s)
    dXr, dAr, dBr = qlora.backward(f32(dY), f32(X), Wd, f32(A), f32(B), s)
    check_close("Y", f32(Y), Yr)
    check_close("dX", f32(dX), dXr)
    if r:
        check_close("T", f32(T), Tr)
        check_close("dA", f32(dA), dAr)
        check_close("dB", f32(dB), dBr)


def test_identity_probes_are_exact(lib):
    K, N = 320, 200
    W = wl.normal_bf16(77, (N, K), 0.02)
    W[3, :] *= 40                                          # spread the group scales
    qg = lib.fp4_quantize(W.to(DEV))
    deq16 = lib.nf4_dequantize(qg, torch.bfloat16)
    # forward: X = I_K gives Y = deq(W)^T
    I_K = torch.eye(K, dtype=torch.bfloat16, device=DEV)
    Y, _ = lib.qlora_fwd(I_K, qg, None, None, 1.0)
    # backward: dY = I_N gives dX = deq(W)
    I_N = torch.eye(N, dtype=torch.bfloat16, device=DEV)
    dX, _, _ = lib.qlora_bwd(I_N, torch.zeros(N, K, dtype=torch.bfloat16, device=DEV), qg, None, None,
                             1.0, None)
    # the decode kernel (M <= 16): the first 16 rows of the identity give the first 16 columns
    Y16, _ = lib.qlora_fwd(I_K[:16].contiguous(), qg, None, None, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(Y, deq16.t().contiguous())
    assert torch.equal(dX, deq16)
    assert torch.equal(Y16, deq16[:, :16].t().contiguous())


@pytest.mark.parametrize("counts,K,N,r,s", [
    ([40, 0, 300, 7], 512, 72, 16, 1.5),
    # the grouped dX launch has a full round of 256 tiles and a tail it splits into pieces, whose
    # adding launch applies the tensor scale
    ([1300, 0, 700, 2000, 900, 1100, 1000, 0], 2304, 264, 16, 0.5),
])
def test_moe_with_fp4_experts(lib, counts, K, N, r, s):
    E, M = len(counts), sum(counts)
    X = wl.normal_bf16(11, (M, K), 1.0)
    W = wl.normal_bf16(12, (E * N, K), 0.02)
    A = wl.normal_bf16(13, (E * r, K), K ** -0.5)
    B = wl.normal_bf16(14, (E * N, r), 0.1)
    dY = wl.normal_bf16(15, (M, N), 1.0)
    qg = lib.fp4_quantize(W.to(DEV))
    Y, T = lib.qlora_moe_fwd(X.to(DEV), counts, qg, A.to(DEV), B.to(DEV), s)
    dX, dA, dB = lib.qlora_moe_bwd(dY.to(DEV), X.to(DEV), counts, qg, A.to(DEV), B.to(DEV), s, T)
    torch.cuda.synchronize()
    Wd = fp4.dequantize_f32(fp4.quantize(W.float().numpy()))
    Yr, Tr = moe.forward(f32(X), counts, Wd, f32(A), f32(B), s)
    dXr, dAr, dBr = moe.backward(f32(dY), f32(X), counts, Wd, f32(A), f32(B), s)
    for name, got, ref in (("Y", Y, Yr), ("T", T, Tr), ("dX", dX, dXr), ("dA", dA, dAr), ("dB", dB, dBr)):
        check_close(name, f32(got), ref)


@pytest.mark.parametrize("M", [96, 8])   # the pair kernel; the decode kernel's E2M1 form
def test_swiglu_pair_with_fp4_weight(lib, M):
    K, N, r, s = 256, 64, 8, 0.5
    X = wl.normal_bf16(21, (M, K), 1.0)
    Wgu = wl.normal_bf16(22, (2 * N, K), 0.02)
    Agu = wl.normal_bf16(23, (2 * r, K), K ** -0.5)
    Bg, Bu = wl.normal_bf16(24, (N, r), 0.1), wl.normal_bf16(25, (N, r), 0.1)
    dH = wl.normal_bf16(26, (M, N), 1.0)
    qg = lib.fp4_quantize(Wgu.to(DEV))
    H, Ygu, Tgu = lib.qlora_swiglu_fwd(X.to(DEV), qg, Agu.to(DEV), Bg.to(DEV), Bu.to(DEV), s)
    dX, dAgu, dBg, dBu = lib.qlora_swiglu_bwd(dH.to(DEV), X.to(DEV), qg, Agu.to(DEV), Bg.to(DEV),
                                              Bu.to(DEV), s, Ygu, Tgu)
    torch.cuda.synchronize()
    Wd = fp4.dequantize_f32(fp4.quantize(Wgu.float().numpy()))
    Hr = swiglu.forward(f32(X), Wd[:N], Wd[N:], f32(Agu)[:r], f32(Agu)[r:], f32(Bg), f32(Bu), s)[0]
    dXr, dAg, dAu, dBgr, dBur = swiglu.backward(f32(dH), f32(X), Wd[:N], Wd[N:], f32(Agu)[:r],
                                                f32(Agu)[r:], f32(Bg), f32(Bu), s)
    # H: one rounding from the pair kernel's float32 sums (M = 96), two through the bf16 Ygu on
    # the decode shape (M = 8); the backward takes dYg, dYu rounded to bf16 (two roundings)
    check_close("H", f32(H), Hr, warn_above=4e-3 if M > 16 else 8e-3)
    check_close("dX", f32(dX), dXr, warn_above=8e-3)
    check_close("dAgu", f32(dAgu), np.concatenate([dAg, dAu]), warn_above=8e-3)
    check_close("dBg", f32(dBg), dBgr, warn_above=8e-3)
    check_close("dBu", f32(dBu), dBur, warn_above=8e-3)


@pytest.mark.parametrize("n,k,r,s", [(64, 256, 16, 2.0), (200, 320, 5, -0.5), (40, 1024, 128, 0.25)])
def test_merge_and_fp4_export(lib, n, k, r, s):
    say(f"fp4 merge n={n} k={k} r={r} s={s}")
    W = wl.normal_bf16(700 + n, (n, k), 0.02)
    A = wl.normal_bf16(701 + n, (r, k), k ** -0.5)
    B = wl.normal_bf16(702 + n, (n, r), 0.05)
    qg = lib.fp4_quantize(W.to(DEV))
    Wm = lib.qlora_merge(qg, A.to(DEV), B.to(DEV), s)
    q2 = lib.fp4_quantize(Wm)
    W0 = lib.qlora_merge(qg, None, None, s)
    D0 = lib.nf4_dequantize(qg, torch.bfloat16)
    torch.cuda.synchronize()
    qo = fp4.quantize(W.float().numpy())
    assert_fp4_equal(qg, qo)
    ref = merge.merge(fp4.dequantize_f32(qo), f32(A), f32(B), s)
    got = f32(Wm).astype(np.float64)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), np.finfo(np.float32).tiny))) - 7)
    err = (np.abs(got - ref) / ulp).max()
    say(f"  max error {err:.3f} bf16 ulp")
    assert err <= 1.0
    assert torch.equal(W0, D0)
    assert_fp4_equal(q2, fp4.quantize(f32(Wm)))
