"""Pins for the oracle's gate/up SwiGLU pair (CPU only).

* silu against scipy's logistic function (an independent implementation), and its derivative
  against central differences of that function;
* the forward against the gated composition silu(Yg) * Yu built from scipy and the (separately
  pinned) single-projection oracle;
* the backward against central finite differences of <dH, H> along random directions of X, Ag,
  Au, Bg and Bu (H is not linear, so this is the check that fixes every gradient);
* the stacked form the library computes: [Wg; Wu], [Ag; Au] and the block-diagonal B give
  [Yg | Yu], and one stacked backward gives dX, [dAg; dAu] and dBg, dBu on the diagonal blocks;
* a zero up projection zeroes the output and the gate adapters' gradients.
"""
import math

import numpy as np
import pytest
from scipy.special import expit

from oracle import nf4, qlora, swiglu


def make(M, K, N, r, seed, dq=0):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    Wg = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Wu = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    Ag = rng.standard_normal((r, K)) / math.sqrt(K)
    Au = rng.standard_normal((r, K)) / math.sqrt(K)
    Bg = rng.standard_normal((N, r)) * 0.01
    Bu = rng.standard_normal((N, r)) * 0.01
    dH = rng.standard_normal((M, N))
    Wdg = nf4.dequantize_f32(nf4.quantize(Wg, dq))
    Wdu = nf4.dequantize_f32(nf4.quantize(Wu, dq))
    return X, Wdg, Wdu, Ag, Au, Bg, Bu, dH


def test_silu_matches_scipy_logistic():
    x = np.concatenate([np.linspace(-40, 40, 20001), [-750.0, -100.0, 0.0, 100.0, 750.0]])
    np.testing.assert_allclose(swiglu.silu(x), x * expit(x), rtol=1e-14, atol=1e-300)
    assert swiglu.silu(np.array([0.0]))[0] == 0.0
    h = 1e-5
    xs = np.linspace(-12, 12, 2401)
    fd = ((xs + h) * expit(xs + h) - (xs - h) * expit(xs - h)) / (2 * h)
    np.testing.assert_allclose(swiglu.silu_grad(xs), fd, rtol=1e-8, atol=1e-10)


@pytest.mark.parametrize("M,K,N,r,dq,s", [(5, 128, 7, 3, 0, 1.5), (4, 64, 9, 2, 256, -0.5)])
def test_forward_is_the_gated_composition(M, K, N, r, dq, s):
    X, Wdg, Wdu, Ag, Au, Bg, Bu, _ = make(M, K, N, r, 3, dq)
    H, Yg, Yu, Tg, Tu = swiglu.forward(X, Wdg, Wdu, Ag, Au, Bg, Bu, s)
    Yg0, Tg0 = qlora.forward(X, Wdg, Ag, Bg, s)
    Yu0, Tu0 = qlora.forward(X, Wdu, Au, Bu, s)
    assert np.array_equal(Yg, Yg0) and np.array_equal(Yu, Yu0)
    assert np.array_equal(Tg, Tg0) and np.array_equal(Tu, Tu0)
    np.testing.assert_allclose(H, Yg0 * expit(Yg0) * Yu0, rtol=1e-13, atol=1e-300)


@pytest.mark.parametrize("seed,s", [(5, 2.0), (6, -0.75)])
def test_backward_matches_finite_differences(seed, s):
    M, K, N, r = 4, 64, 6, 3
    X, Wdg, Wdu, Ag, Au, Bg, Bu, dH = make(M, K, N, r, seed)
    # larger adapters so that the LoRA paths carry weight in the check
    Bg, Bu = Bg * 30, Bu * 30
    dX, dAg, dAu, dBg, dBu = swiglu.backward(dH, X, Wdg, Wdu, Ag, Au, Bg, Bu, s)
    params = {"X": X, "Ag": Ag, "Au": Au, "Bg": Bg, "Bu": Bu}
    grads = {"X": dX, "Ag": dAg, "Au": dAu, "Bg": dBg, "Bu": dBu}

    def loss(p):
        H = swiglu.forward(p["X"], Wdg, Wdu, p["Ag"], p["Au"], p["Bg"], p["Bu"], s)[0]
        return float(np.sum(dH * H))

    rng = np.random.default_rng(seed + 100)
    for name in params:
        V = rng.standard_normal(params[name].shape)
        h = 1e-4 / max(1.0, float(np.abs(params[name]).max()))
        plus = dict(params, **{name: params[name] + h * V})
        minus = dict(params, **{name: params[name] - h * V})
        fd = (loss(plus) - loss(minus)) / (2 * h)
        an = float(np.sum(grads[name] * V))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_stacked_form_equals_the_pair():
    M, K, N, r, s = 5, 128, 6, 4, 0.5
    X, Wdg, Wdu, Ag, Au, Bg, Bu, dH = make(M, K, N, r, 9)
    H, Yg, Yu, Tg, Tu = swiglu.forward(X, Wdg, Wdu, Ag, Au, Bg, Bu, s)
    W2 = np.concatenate([Wdg, Wdu])                       # [2N, K]
    A2 = np.concatenate([Ag, Au])                         # [2r, K]
    B2 = np.zeros((2 * N, 2 * r))                         # block-diagonal [2N, 2r]
    B2[:N, :r], B2[N:, r:] = Bg, Bu
    Y2, T2 = qlora.forward(X, W2, A2, B2, s)
    assert qlora.rel_err(Y2, np.concatenate([Yg, Yu], axis=1)) < 1e-13
    assert qlora.rel_err(T2, np.concatenate([Tg, Tu], axis=1)) < 1e-13
    dYg = dH * Yu * swiglu.silu_grad(Yg)
    dYu = dH * swiglu.silu(Yg)
    dX2, dA2, dB2 = qlora.backward(np.concatenate([dYg, dYu], axis=1), X, W2, A2, B2, s)
    dX, dAg, dAu, dBg, dBu = swiglu.backward(dH, X, Wdg, Wdu, Ag, Au, Bg, Bu, s)
    assert qlora.rel_err(dX2, dX) < 1e-13
    assert qlora.rel_err(dA2, np.concatenate([dAg, dAu])) < 1e-13
    assert qlora.rel_err(dB2[:N, :r], dBg) < 1e-13 and qlora.rel_err(dB2[N:, r:], dBu) < 1e-13


def test_zero_up_projection():
    M, K, N, r, s = 4, 64, 5, 2, 1.0
    X, Wdg, _, Ag, Au, Bg, _, dH = make(M, K, N, r, 12)
    Wdu, Bu = np.zeros_like(Wdg), np.zeros_like(Bg)
    H = swiglu.forward(X, Wdg, Wdu, Ag, Au, Bg, Bu, s)[0]
    assert not np.any(H)
    dX, dAg, dAu, dBg, dBu = swiglu.backward(dH, X, Wdg, Wdu, Ag, Au, Bg, Bu, s)
    assert not np.any(dAg) and not np.any(dBg) and not np.any(dAu)
    assert np.any(dBu)            # the up adapter still gets a gradient through silu(Yg)
