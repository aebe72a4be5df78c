"""Grouped (mixture-of-experts) QLoRA layer in float64 -- test infrastructure (see the package
docstring).

Each token's row goes through the QLoRA layer of the expert it was routed to, every expert with
its own frozen NF4 base and its own (A, B) adapters [NVFP4 update article, "Comprehensive
Improvements in Training Performance and Stability": grouped MoE and LoRA on the experts' MLP
layers, and its MoE background paragraph; pyshine Unsloth code tour, "Why You Need This": the
grouped-GEMM interface for MoE experts]. The routing itself (which rows go where) is an input: the
rows of X arrive grouped by expert, counts[e] of them for expert e, in expert order, and

    Y[rows of e] = X[rows of e] deq(W_e)^T + s (X[rows of e] A_e^T) B_e^T

with the backward of each expert's layer on its own rows (dX row by row; dA_e, dB_e summed over
expert e's rows only, zero for an expert with no rows). Storage: the experts' tensors stacked in
expert order, W [E*N, K], A [E*r, K], B [E*N, r].
"""
from __future__ import annotations

import numpy as np

from . import qlora

_f64 = qlora._f64


def offsets(counts):
    return np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))])


def forward(X, counts, Wd, A, B, s: float):
    """(Y, T) for rows X [sum(counts), K] grouped by expert and the stacked expert tensors."""
    X, Wd, A, B = _f64(X), _f64(Wd), _f64(A), _f64(B)
    E = len(counts)
    N, r = Wd.shape[0] // E, A.shape[0] // E
    off = offsets(counts)
    Y = np.zeros((X.shape[0], N))
    T = np.zeros((X.shape[0], r))
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        Y[rows], T[rows] = qlora.forward(X[rows], Wd[e * N:(e + 1) * N], A[e * r:(e + 1) * r],
                                         B[e * N:(e + 1) * N], s)
    return Y, T


def backward(dY, X, counts, Wd, A, B, s: float):
    """(dX, dA [E*r, K], dB [E*N, r]) for the upstream gradient dY [sum(counts), N]."""
    dY, X, Wd, A, B = _f64(dY), _f64(X), _f64(Wd), _f64(A), _f64(B)
    E = len(counts)
    N, r = Wd.shape[0] // E, A.shape[0] // E
    off = offsets(counts)
    dX = np.zeros_like(X)
    dA = np.zeros_like(A)
    dB = np.zeros_like(B)
    for e in range(E):
        rows = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:
            continue
        dX[rows], dA[e * r:(e + 1) * r], dB[e * N:(e + 1) * N] = qlora.backward(
            dY[rows], X[rows], Wd[e * N:(e + 1) * N], A[e * r:(e + 1) * r], B[e * N:(e + 1) * N], s)
    return dX, dA, dB
