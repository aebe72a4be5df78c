"""The gate/up pair of QLoRA projections with the SwiGLU activation, in float64 -- test
infrastructure (see the package docstring).

The pages name a fused gated-MLP activation kernel next to the fused LoRA matmul, with a
backward pass that reuses its input buffers [pyshine Unsloth code tour, "Why You Need This":
swiglu.py fuses the gated MLP activation; "Inside Unsloth" listing, "What You'll Learn", "Triton
Kernel Internals": the SwiGLU backward reuses input buffers; NVFP4 update article, section on
Triton hotspot fusion: SwiGLU among the fused operations]. They do not write the activation out;
the reading taken here is the gated MLP of the Llama family, whose gate and up projections are
the shape these kernels serve:

    Yg = X deq(Wg)^T + s (X Ag^T) Bg^T          gate projection  [M, N]
    Yu = X deq(Wu)^T + s (X Au^T) Bu^T          up projection    [M, N]
    H  = silu(Yg) * Yu                          silu(x) = x / (1 + exp(-x))

and its backward for an upstream gradient dH [M, N], by the chain rule:

    dYg = dH * Yu * silu'(Yg),   silu'(x) = sigma(x) (1 + x (1 - sigma(x))),  sigma(x) = 1 / (1 + exp(-x))
    dYu = dH * silu(Yg)

then each projection's QLoRA backward (qlora.backward) with its own dY; dX is the sum of the two
projections' input gradients. Everything is float64 from the exact values of the inputs; the
bases are frozen (no weight gradient).
"""
from __future__ import annotations

import numpy as np

from . import qlora

_f64 = qlora._f64


def sigmoid(x):
    x = _f64(x)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x))


def silu(x):
    x = _f64(x)
    return x * sigmoid(x)


def silu_grad(x):
    """d silu / dx."""
    x = _f64(x)
    sg = sigmoid(x)
    return sg * (1.0 + x * (1.0 - sg))


def forward(X, Wd_g, Wd_u, Ag, Au, Bg, Bu, s: float):
    """(H, Yg, Yu, Tg, Tu) for X [M,K], dequantised gate and up weights [N,K], A [r,K], B [N,r]."""
    Yg, Tg = qlora.forward(X, Wd_g, Ag, Bg, s)
    Yu, Tu = qlora.forward(X, Wd_u, Au, Bu, s)
    H = silu(Yg) * Yu
    return H, Yg, Yu, Tg, Tu


def backward(dH, X, Wd_g, Wd_u, Ag, Au, Bg, Bu, s: float):
    """(dX, dAg, dAu, dBg, dBu) for upstream gradient dH [M,N]."""
    dH = _f64(dH)
    Yg, _ = qlora.forward(X, Wd_g, Ag, Bg, s)
    Yu, _ = qlora.forward(X, Wd_u, Au, Bu, s)
    dYg = dH * Yu * silu_grad(Yg)
    dYu = dH * silu(Yg)
    dXg, dAg, dBg = qlora.backward(dYg, X, Wd_g, Ag, Bg, s)
    dXu, dAu, dBu = qlora.backward(dYu, X, Wd_u, Au, Bu, s)
    return dXg + dXu, dAg, dAu, dBg, dBu
