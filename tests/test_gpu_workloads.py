"""GPU parity on the full-size workloads (small, q_proj, mlp_up, decode, down, and mlp_up with an
E2M1 base weight).

The HIP path runs at full size, exactly as bench.py launches it. The quantised weight is compared
bit for bit in full. Y, T and dX are compared on sampled rows (first, last and random rows), dA
on sampled columns and dB on sampled rows, each computed by the float64 oracle's sampled entries
(oracle.qlora.forward_rows / backward_sampled, pinned to the full forward and backward) from the
same seeded inputs; the small workload is compared in full.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import fp4, nf4, qlora
from tests.gpu_helpers import assert_fp4_equal, assert_quant_equal, check_close, f32, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def sample(n: int, count: int, seed: int) -> np.ndarray:
    if n <= count:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    edge = np.concatenate([np.arange(4), np.arange(n - 4, n)])
    mid = rng.choice(np.arange(4, n - 4), count - 8, replace=False)
    return np.sort(np.concatenate([edge, mid]))


def t_full(X: np.ndarray, A: np.ndarray) -> np.ndarray:
    """X A^T in float64, in row chunks to bound host memory."""
    out = np.empty((X.shape[0], A.shape[0]))
    A64 = A.astype(np.float64)
    for lo in range(0, X.shape[0], 2048):
        out[lo:lo + 2048] = X[lo:lo + 2048].astype(np.float64) @ A64.T
    return out


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_workload(lib, name):
    w = wl.WORKLOADS[name]
    say(f"workload {name}: M={w.M} K={w.K} N={w.N} r={w.r} s={w.s} dq={w.dq_block}")
    W = wl.tensor(w, "W")
    X = wl.tensor(w, "X")
    A = wl.tensor(w, "A")
    B = wl.tensor(w, "B")
    e2m1 = w.fmt == "e2m1"
    qg = lib.fp4_quantize(W.to(DEV)) if e2m1 else lib.nf4_quantize(W.to(DEV), w.dq_block)
    Xd, Ad, Bd = X.to(DEV), A.to(DEV), B.to(DEV)
    Yg, Tg = lib.qlora_fwd(Xd, qg, Ad, Bd, w.s)
    torch.cuda.synchronize()
    say("  fwd done")
    if e2m1:
        qo = fp4.quantize(W.float().numpy())
        assert_fp4_equal(qg, qo)
        Wd = fp4.dequantize_f32(qo)
    else:
        qo = nf4.quantize(W.float().numpy(), w.dq_block)
        assert_quant_equal(qg, qo)
        Wd = nf4.dequantize_f32(qo)
    del W
    Xf, Af, Bf = f32(X), f32(A), f32(B)
    rows = sample(w.M, 48, w.index)
    Ys, Ts = qlora.forward_rows(Xf, Wd, Af, Bf, w.s, rows)
    check_close("Y", f32(Yg[torch.from_numpy(rows).to(DEV)]), Ys)
    check_close("T", f32(Tg[torch.from_numpy(rows).to(DEV)]), Ts)
    del Yg
    if not w.backward:
        return
    dY = wl.tensor(w, "dY")
    dXg, dAg, dBg = lib.qlora_bwd(dY.to(DEV), Xd, qg, Ad, Bd, w.s, Tg)
    torch.cuda.synchronize()
    say("  bwd done")
    cols = sample(w.K, 64, w.index + 1)
    nrows = sample(w.N, 64, w.index + 2)
    dXs, dAs, dBs = qlora.backward_sampled(f32(dY), Xf, Wd, Af, Bf, w.s, rows, cols, nrows)
    check_close("dX", f32(dXg[torch.from_numpy(rows).to(DEV)]), dXs)
    check_close("dA", f32(dAg)[:, cols], dAs)
    check_close("dB", f32(dBg)[nrows], dBs)
