"""Pins for the oracle's QLoRA forward and backward (CPU only).

* Brute force: pure-Python loops on tiny shapes, reading the packed NF4 bytes nibble by nibble
  and looking levels up explicitly, must equal the oracle to 1e-12.
* Adjoints: Y is linear in X, A and B, so <dY, Y(X)> = <dX, X>, <dY, s T B^T> = <dB, B> and
  <dY, s X A^T B^T> = <dA, A> hold exactly; checked to 1e-12 relative in float64.
* Finite differences: by linearity Y(B + E) - Y(B) = s T E^T and Y(A + E) - Y(A) = s X E^T B^T.
* Reductions: r = 0 equals B = 0 equals the plain dequant GEMM; a zero base leaves s T B^T.
"""
import math

import numpy as np
import pytest

from oracle import nf4, qlora

C = nf4.codebook()


def make(M, K, N, r, seed, dq=0, wstd=0.02):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K))
    W = (rng.standard_normal((N, K)) * wstd).astype(np.float32)
    A = rng.standard_normal((r, K)) / math.sqrt(K)
    B = rng.standard_normal((N, r)) * 0.01
    dY = rng.standard_normal((M, N))
    q = nf4.quantize(W, dq)
    return X, q, A, B, dY


def brute_deq(q, n, k):
    """Dequantised element (n, k) read straight from the packed bytes."""
    flat = n * q.k + k
    byte = int(q.codes[flat // 2])
    code = (byte >> 4) if flat % 2 == 0 else (byte & 0x0F)
    blk = flat // 64
    if q.dq_block:
        a = np.float32(np.float32(int(q.absmax[blk])) * q.scale[blk // q.dq_block])
    else:
        a = np.float32(q.absmax[blk])
    return float(np.float32(C[code] * a))


def brute_forward(X, q, A, B, s):
    M, K = X.shape
    N, r = q.n, A.shape[0]
    Wd = [[brute_deq(q, n, k) for k in range(K)] for n in range(N)]
    Y = [[0.0] * N for _ in range(M)]
    for m in range(M):
        T = [sum(float(X[m, k]) * float(A[j, k]) for k in range(K)) for j in range(r)]
        for n in range(N):
            base = sum(float(X[m, k]) * Wd[n][k] for k in range(K))
            lora = sum(T[j] * float(B[n, j]) for j in range(r))
            Y[m][n] = base + s * lora
    return np.array(Y)


def brute_backward(dY, X, q, A, B, s):
    M, K = X.shape
    N, r = q.n, A.shape[0]
    Wd = [[brute_deq(q, n, k) for k in range(K)] for n in range(N)]
    T = [[sum(float(X[m, k]) * float(A[j, k]) for k in range(K)) for j in range(r)] for m in range(M)]
    U = [[sum(float(dY[m, n]) * float(B[n, j]) for n in range(N)) for j in range(r)] for m in range(M)]
    dX = [[sum(float(dY[m, n]) * Wd[n][k] for n in range(N)) + s * sum(U[m][j] * float(A[j, k]) for j in range(r))
           for k in range(K)] for m in range(M)]
    dA = [[s * sum(U[m][j] * float(X[m, k]) for m in range(M)) for k in range(K)] for j in range(r)]
    dB = [[s * sum(float(dY[m, n]) * T[m][j] for m in range(M)) for j in range(r)] for n in range(N)]
    return np.array(dX), np.array(dA).reshape(r, K), np.array(dB).reshape(N, r)


@pytest.mark.parametrize("M,K,N,r,dq,s", [(3, 64, 5, 2, 0, 2.0), (4, 128, 3, 3, 256, 0.5),
                                          (1, 64, 2, 1, 0, -1.25), (2, 128, 4, 4, 256, 1.0)])
def test_forward_backward_brute_force(M, K, N, r, dq, s):
    X, q, A, B, dY = make(M, K, N, r, seed=M * 100 + N, dq=dq)
    Wd = nf4.dequantize_f32(q)
    Y, T = qlora.forward(X, Wd, A, B, s)
    assert qlora.rel_err(Y, brute_forward(X, q, A, B, s)) < 1e-12
    assert qlora.rel_err(T, X @ A.T) < 1e-12
    dX, dA, dB = qlora.backward(dY, X, Wd, A, B, s)
    bX, bA, bB = brute_backward(dY, X, q, A, B, s)
    assert qlora.rel_err(dX, bX) < 1e-12
    assert qlora.rel_err(dA, bA) < 1e-12
    assert qlora.rel_err(dB, bB) < 1e-12


def _ip(a, b):
    return float(np.sum(np.asarray(a, np.float64) * np.asarray(b, np.float64)))


@pytest.mark.parametrize("seed", [1, 2])
def test_adjoint_identities(seed):
    M, K, N, r, s = 9, 192, 11, 5, 0.75
    X, q, A, B, dY = make(M, K, N, r, seed)
    Wd = nf4.dequantize_f32(q)
    Y, T = qlora.forward(X, Wd, A, B, s)
    dX, dA, dB = qlora.backward(dY, X, Wd, A, B, s)
    lhs = _ip(dY, Y)
    assert abs(lhs - _ip(dX, X)) <= 1e-12 * (abs(lhs) + _ip(np.abs(dY), np.abs(Y)))
    lora = s * (X @ A.T) @ B.T
    lb = _ip(dY, lora)
    assert abs(lb - _ip(dB, B)) <= 1e-12 * _ip(np.abs(dY), np.abs(lora))
    assert abs(lb - _ip(dA, A)) <= 1e-12 * _ip(np.abs(dY), np.abs(lora))


def test_finite_differences_are_exact_by_linearity():
    M, K, N, r, s = 6, 128, 7, 3, 1.5
    X, q, A, B, _ = make(M, K, N, r, 21)
    Wd = nf4.dequantize_f32(q)
    rng = np.random.default_rng(22)
    E = rng.standard_normal(B.shape)
    Y0, T = qlora.forward(X, Wd, A, B, s)
    Y1, _ = qlora.forward(X, Wd, A, B + E, s)
    assert qlora.rel_err(Y1 - Y0, s * T @ E.T) < 1e-9
    F = rng.standard_normal(A.shape)
    Y2, _ = qlora.forward(X, Wd, A + F, B, s)
    assert qlora.rel_err(Y2 - Y0, s * (X @ F.T) @ B.T) < 1e-9


def test_rank_zero_equals_b_zero_equals_plain_gemm():
    M, K, N, r, s = 5, 128, 6, 4, 2.0
    X, q, A, B, dY = make(M, K, N, r, 31)
    Wd = nf4.dequantize_f32(q)
    Y0, _ = qlora.forward(X, Wd, A[:0], B[:, :0], s)
    Yb, _ = qlora.forward(X, Wd, A, np.zeros_like(B), s)
    plain = np.array([[sum(X[m, k] * Wd[n, k] for k in range(K)) for n in range(N)] for m in range(M)])
    assert np.array_equal(Y0, Yb)
    assert qlora.rel_err(Y0, plain) < 1e-12
    dX0, dA0, dB0 = qlora.backward(dY, X, Wd, A[:0], B[:, :0], s)
    assert dA0.shape == (0, K) and dB0.shape == (N, 0)
    plain_dx = np.array([[sum(dY[m, n] * Wd[n, k] for n in range(N)) for k in range(K)] for m in range(M)])
    assert qlora.rel_err(dX0, plain_dx) < 1e-12


def test_zero_base_leaves_lora_term():
    M, K, N, r, s = 4, 64, 5, 3, 0.5
    X, q, A, B, dY = make(M, K, N, r, 41)
    Wd = np.zeros((N, K))
    Y, T = qlora.forward(X, Wd, A, B, s)
    want = [[s * sum(sum(X[m, k] * A[j, k] for k in range(K)) * B[n, j] for j in range(r))
             for n in range(N)] for m in range(M)]
    assert qlora.rel_err(Y, np.array(want)) < 1e-12


def test_identity_input_returns_dequantised_weight():
    """X = I_K, r = 0 gives Y = deq(W)^T; dY = I_N gives dX = deq(W)."""
    K, N = 128, 64
    _, q, _, _, _ = make(1, K, N, 1, 51, dq=256)
    Wd = nf4.dequantize_f32(q)
    Y, _ = qlora.forward(np.eye(K), Wd, np.zeros((0, K)), np.zeros((N, 0)), 1.0)
    assert np.array_equal(Y, Wd.T.astype(np.float64))
    dX, _, _ = qlora.backward(np.eye(N), np.zeros((N, K)), Wd, np.zeros((0, K)), np.zeros((N, 0)), 1.0)
    assert np.array_equal(dX, Wd.astype(np.float64))


def test_rel_err_definition():
    ref = np.array([[1.0, -4.0], [2.0, 0.0]])
    got = ref + np.array([[0.0, 0.04], [0.0, -0.02]])
    assert abs(qlora.rel_err(got, ref) - 0.01) < 1e-15
    assert qlora.rel_err(np.zeros(3), np.zeros(3)) == 0.0


@pytest.mark.parametrize("M,K,N,r", [(37, 128, 24, 4), (70, 192, 40, 0), (5, 64, 8, 3)])
def test_sampled_backward_equals_backward(M, K, N, r):
    """backward_sampled (the full-size parity references) selects exactly the rows and columns of
    backward(); forward_rows the rows of forward()."""
    X, q, A, B, dY = make(M, K, N, r, 800 + M)
    Wd = nf4.dequantize_f32(q)
    rng = np.random.default_rng(M)
    rows = np.sort(rng.choice(M, min(M, 9), replace=False))
    cols = np.sort(rng.choice(K, 11, replace=False))
    nrows = np.sort(rng.choice(N, min(N, 7), replace=False))
    dX, dA, dB = qlora.backward(dY, X, Wd, A, B, 1.5)
    sX, sA, sB = qlora.backward_sampled(dY, X, Wd, A, B, 1.5, rows, cols, nrows, chunk=16)
    assert np.allclose(sX, dX[rows], rtol=1e-13, atol=1e-13)
    assert np.allclose(sA, dA[:, cols], rtol=1e-13, atol=1e-13)
    assert np.allclose(sB, dB[nrows], rtol=1e-13, atol=1e-13)
    Y, T = qlora.forward(X, Wd, A, B, 1.5)
    fY, fT = qlora.forward_rows(X, Wd, A, B, 1.5, rows)
    assert np.allclose(fY, Y[rows], rtol=1e-13, atol=1e-13)
    assert np.allclose(fT, T[rows], rtol=1e-13, atol=1e-13)
