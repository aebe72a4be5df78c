"""qlora_fwd_noalloc (the forward with its scratch in a static per-GPU array) against qlora_fwd
with a caller workspace: the same kernels and the same split-K partial sums, so Y and T must be
equal bit for bit. Two calls in a row, the second with a smaller input (the array keeps the first
call's partial sums), both through the C ABI, then a decode shape whose stream kernel forms T
itself (no scratch) and a larger-row call.
"""
import ctypes

import numpy as np
import pytest
import torch

import nf4_dequant_gemm_amd as lib_mod
import workloads as wl
from oracle import nf4, qlora
from tests.gpu_helpers import check_close, f32, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def layer(M, K, N, r, seed, dq=256):
    X = wl.normal_bf16(seed + 1, (M, K), 1.0)
    W = wl.normal_bf16(seed + 2, (N, K), 0.02)
    A = wl.normal_bf16(seed + 3, (r, K), K ** -0.5)
    B = wl.normal_bf16(seed + 4, (N, r), 0.05)
    return X, W, A, B


def run_both(lib, c, M, K, N, r, s, seed):
    say(f"no-alloc forward M={M} K={K} N={N} r={r}")
    X, W, A, B = layer(M, K, N, r, seed)
    q = lib.nf4_quantize(W.to(DEV), 256)
    Xd, Ad, Bd = X.to(DEV), A.to(DEV), B.to(DEV)
    st = q.c_struct()
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    sp = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # the entry point with a workspace
    Y1 = torch.empty(M, N, dtype=torch.bfloat16, device=DEV)
    T1 = torch.empty(M, r, dtype=torch.bfloat16, device=DEV)
    wsb = c.qlora_fwd_workspace_bytes(M, N, K, r)
    assert 0 < wsb <= lib_mod.NOALLOC_SCRATCH_BYTES
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    assert c.qlora_fwd(P(Xd), M, ctypes.byref(st), P(Ad), P(Bd), r, s, P(Y1), P(T1), P(ws), wsb, sp) == 0
    # the no-allocation entry point
    Y2 = torch.full((M, N), 7.0, dtype=torch.bfloat16, device=DEV)
    T2 = torch.full((M, r), 7.0, dtype=torch.bfloat16, device=DEV)
    rc = c.qlora_fwd_noalloc(P(Xd), M, ctypes.byref(st), P(Ad), P(Bd), r, s, P(Y2), P(T2), sp)
    assert rc == 0, c.nf4_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(T1.view(torch.int16), T2.view(torch.int16))
    Wd = nf4.dequantize_f32(nf4.quantize(W.float().numpy(), 256))
    Yo, To = qlora.forward(f32(X), Wd, f32(A), f32(B), s)
    check_close("Y", f32(Y2), Yo)
    check_close("T", f32(T2), To)


def test_noalloc_forward_matches_qlora_fwd(lib):
    c = lib.library()
    # decode shapes: T's partial sums (in the scratch array) added inside the stream kernel
    # (r > 64), then a smaller one
    run_both(lib, c, 16, 2048, 2240, 128, 2.0, 1100)
    run_both(lib, c, 4, 1024, 448, 96, 0.5, 1200)
    # a decode shape whose stream kernel forms T itself (no scratch)
    run_both(lib, c, 16, 8192, 2240, 16, 2.0, 1150)
    # more rows: the separate row projection with its split partials in the scratch array
    run_both(lib, c, 300, 1024, 264, 24, 1.0, 1300)
