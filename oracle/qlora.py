"""The QLoRA linear layer in float64 -- test infrastructure (see the package docstring).

The pages state the adapter algebra (Delta W = B A with rank r, only the adapters train, the
4-bit base is frozen) [Unsloth v0.1.463-beta release article, "About the Unsloth Project"]. The
fused kernel folds the low-rank delta into the product with the dequantised base rather than
running it as extra separate products [pyshine Unsloth code tour, "Why You Need This", the
kernels/fast_lora.py paragraph; "Inside Unsloth" listing, "What You'll Learn", "LoRA and QLoRA"],
and the rewrite is numerically equivalent to the plain layer [v0.1.47-beta article, section on
lowering the fine-tuning barrier]. So the layer is the plain definition, written out here:

    T  = X A^T                      [M, r]
    Y  = X deq(W)^T + s T B^T       [M, N]
    U  = dY B                       [M, r]
    dX = dY deq(W) + s U A          [M, K]
    dA = s U^T X                    [r, K]
    dB = s dY^T T                   [N, r]

W gets no gradient (it is frozen). Readings: s is passed as given (alpha / r by the usual LoRA
convention); there is no bias and no adapter dropout (the pages name neither). Every product is
taken in float64 from the exact values of the bf16 inputs and of the float32 dequantised weight,
with no intermediate rounding; numpy's matmul is the only library step.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def forward(X, Wd, A, B, s: float):
    """(Y, T) for X [M,K], dequantised W [N,K], A [r,K], B [N,r]."""
    X, Wd, A, B = _f64(X), _f64(Wd), _f64(A), _f64(B)
    T = X @ A.T
    Y = X @ Wd.T + float(s) * (T @ B.T)
    return Y, T


def backward(dY, X, Wd, A, B, s: float):
    """(dX, dA, dB) for upstream gradient dY [M,N]."""
    dY, X, Wd, A, B = _f64(dY), _f64(X), _f64(Wd), _f64(A), _f64(B)
    s = float(s)
    T = X @ A.T
    U = dY @ B
    dX = dY @ Wd + s * (U @ A)
    dA = s * (U.T @ X)
    dB = s * (dY.T @ T)
    return dX, dA, dB


def forward_rows(X, Wd, A, B, s: float, rows):
    """(Y[rows], T[rows]): the forward on a subset of rows (each row of Y and T depends on its
    own row of X only)."""
    return forward(np.asarray(X)[rows], Wd, A, B, s)


def backward_sampled(dY, X, Wd, A, B, s: float, rows, cols, nrows, chunk: int = 2048):
    """(dX[rows], dA[:, cols], dB[nrows]) of the backward, for full-size workloads where the
    whole of dX is too costly: U = dY B and T = X A^T over every row (the adapter gradients sum
    over all of them), taken in row chunks to bound host memory, then the same products as
    backward() on the selected rows and columns."""
    dY, X = np.asarray(dY), np.asarray(X)
    Wd, A, B = _f64(Wd), _f64(A), _f64(B)
    s = float(s)
    M = dY.shape[0]
    U = np.empty((M, B.shape[1]))
    T = np.empty((M, A.shape[0]))
    for lo in range(0, M, chunk):
        U[lo:lo + chunk] = _f64(dY[lo:lo + chunk]) @ B
        T[lo:lo + chunk] = _f64(X[lo:lo + chunk]) @ A.T
    dX = _f64(dY[rows]) @ Wd + s * (U[rows] @ A)
    dA = s * (U.T @ _f64(X[:, cols]))
    dB = s * (_f64(dY[:, nrows]).T @ T)
    return dX, dA, dB


def rel_err(got, ref) -> float:
    """Normwise error max|got - ref| / max|ref| (0 when both are all zero)."""
    got, ref = _f64(got), _f64(ref)
    den = np.abs(ref).max() if ref.size else 0.0
    num = np.abs(got - ref).max() if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)
