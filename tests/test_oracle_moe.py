"""Pins for the oracle's grouped (MoE) QLoRA layer (CPU only).

* one expert is the single layer (the separately pinned oracle), exactly;
* brute force: every output row from the explicit formula with its own expert's tensors, looked up
  by walking the counts (no offsets array), on tiny shapes;
* an expert with no rows gets zero adapter gradients and inserting it changes nothing else;
* reordering the experts (their row blocks and their stacked tensors together) reorders the
  outputs and gradients the same way, exactly.
"""
import math

import numpy as np

from oracle import moe, nf4, qlora


def make(E, N, K, r, counts, seed, dq=0):
    rng = np.random.default_rng(seed)
    M = int(sum(counts))
    X = rng.standard_normal((M, K))
    W = (rng.standard_normal((E * N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((E * r, K)) / math.sqrt(K)
    B = rng.standard_normal((E * N, r)) * 0.05
    dY = rng.standard_normal((M, N))
    return X, nf4.dequantize_f32(nf4.quantize(W, dq)), A, B, dY


def test_one_expert_is_the_single_layer():
    X, Wd, A, B, dY = make(1, 6, 128, 3, [9], 1)
    Y, T = moe.forward(X, [9], Wd, A, B, 1.5)
    Y0, T0 = qlora.forward(X, Wd, A, B, 1.5)
    assert np.array_equal(Y, Y0) and np.array_equal(T, T0)
    for a, b in zip(moe.backward(dY, X, [9], Wd, A, B, 1.5), qlora.backward(dY, X, Wd, A, B, 1.5)):
        assert np.array_equal(a, b)


def test_brute_force_rows():
    counts, E, N, K, r, s = [2, 0, 3], 3, 4, 64, 2, -0.5
    X, Wd, A, B, dY = make(E, N, K, r, counts, 2)
    Y, _ = moe.forward(X, counts, Wd, A, B, s)
    dX, dA, dB = moe.backward(dY, X, counts, Wd, A, B, s)
    row = 0
    for e, c in enumerate(counts):
        for _ in range(c):
            for n in range(N):
                t = [sum(X[row, k] * A[e * r + j, k] for k in range(K)) for j in range(r)]
                ref = sum(X[row, k] * Wd[e * N + n, k] for k in range(K)) + s * sum(t[j] * B[e * N + n, j] for j in range(r))
                assert abs(Y[row, n] - ref) <= 1e-12 * max(1.0, abs(ref))
            for k in range(0, K, 7):
                u = [sum(dY[row, n] * B[e * N + n, j] for n in range(N)) for j in range(r)]
                ref = sum(dY[row, n] * Wd[e * N + n, k] for n in range(N)) + s * sum(u[j] * A[e * r + j, k] for j in range(r))
                assert abs(dX[row, k] - ref) <= 1e-12 * max(1.0, abs(ref))
            row += 1
    # adapter gradients: sums over the expert's own rows
    e, lo = 2, 2
    U = dY[lo:lo + 3] @ B[e * N:(e + 1) * N]
    assert qlora.rel_err(dA[e * r:(e + 1) * r], s * U.T @ X[lo:lo + 3]) < 1e-12
    assert qlora.rel_err(dB[e * N:(e + 1) * N], s * dY[lo:lo + 3].T @ (X[lo:lo + 3] @ A[e * r:(e + 1) * r].T)) < 1e-12


def test_empty_expert():
    counts, E, N, K, r = [5, 0, 4], 3, 6, 128, 3
    X, Wd, A, B, dY = make(E, N, K, r, counts, 3, 256)
    dX, dA, dB = moe.backward(dY, X, counts, Wd, A, B, 2.0)
    assert not np.any(dA[r:2 * r]) and not np.any(dB[N:2 * N])
    # the same without the empty expert
    keep = np.r_[0:N, 2 * N:3 * N]
    Y, _ = moe.forward(X, counts, Wd, A, B, 2.0)
    Y2, _ = moe.forward(X, [5, 4], Wd[keep], A[np.r_[0:r, 2 * r:3 * r]], B[keep], 2.0)
    assert np.array_equal(Y, Y2)


def test_expert_reordering():
    counts, E, N, K, r, s = [3, 4, 2], 3, 5, 64, 2, 0.75
    X, Wd, A, B, dY = make(E, N, K, r, counts, 4)
    perm = [2, 0, 1]
    off = moe.offsets(counts)
    rows = np.concatenate([np.arange(off[e], off[e + 1]) for e in perm])
    wrows = np.concatenate([np.arange(e * N, (e + 1) * N) for e in perm])
    arows = np.concatenate([np.arange(e * r, (e + 1) * r) for e in perm])
    Y, T = moe.forward(X, counts, Wd, A, B, s)
    Yp, Tp = moe.forward(X[rows], [counts[e] for e in perm], Wd[wrows], A[arows], B[wrows], s)
    assert np.array_equal(Yp, Y[rows]) and np.array_equal(Tp, T[rows])
    dX, dA, dB = moe.backward(dY, X, counts, Wd, A, B, s)
    dXp, dAp, dBp = moe.backward(dY[rows], X[rows], [counts[e] for e in perm], Wd[wrows], A[arows], B[wrows], s)
    assert np.array_equal(dXp, dX[rows]) and np.array_equal(dAp, dA[arows]) and np.array_equal(dBp, dB[wrows])
