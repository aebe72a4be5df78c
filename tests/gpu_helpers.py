"""Shared helpers of the GPU parity tests: marshal seeded inputs to the HIP library (through the
C-ABI binding) and to the CPU oracle, and compare the results."""
from __future__ import annotations

import sys

import warnings

import numpy as np
import torch

from oracle import fp4, nf4, qlora

TOL = 1e-2   # max |got - ref| / max |ref| for Y, dX, dA, dB (bf16 outputs, fp32 accumulation)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f32(t: torch.Tensor) -> np.ndarray:
    """bf16/float tensor (any device) -> float32 numpy (exact for bf16)."""
    return t.detach().float().cpu().numpy()


def u16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> its bit patterns as uint16 numpy."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def assert_quant_equal(qg, qo: nf4.NF4Weight):
    """GPU NF4Tensor == oracle NF4Weight, bit for bit."""
    codes = qg.codes.cpu().numpy()
    assert codes.shape == qo.codes.shape
    bad = np.nonzero(codes != qo.codes)[0]
    assert bad.size == 0, f"{bad.size} code bytes differ, first at {bad[:5]}"
    if qo.dq_block:
        am = qg.absmax.cpu().numpy()
        assert np.array_equal(am, qo.absmax), "int8 absmax differs"
        sc = qg.scale.cpu().numpy()
        assert np.array_equal(sc.view(np.uint32), qo.scale.view(np.uint32)), "scales differ"
    else:
        am = qg.absmax.cpu().numpy()
        assert np.array_equal(am.view(np.uint32), qo.absmax.view(np.uint32)), "absmax differs"


def assert_fp4_equal(qg, qo: fp4.FP4Weight):
    """GPU E2M1 tensor == oracle FP4Weight, bit for bit (codes, group scales, tensor scale)."""
    codes = qg.codes.cpu().numpy()
    bad = np.nonzero(codes != qo.codes)[0]
    assert bad.size == 0, f"{bad.size} code bytes differ, first at {bad[:5]}"
    sc = qg.absmax.cpu().numpy()
    bad = np.nonzero(sc != qo.scales)[0]
    assert bad.size == 0, f"{bad.size} group scales differ, first at {bad[:5]}"
    S = qg.scale.cpu().numpy()[0]
    assert np.float32(S).view(np.uint32) == np.float32(qo.tscale).view(np.uint32), (S, qo.tscale)


def check_close(name: str, got, ref, tol: float = TOL, warn_above: float = 4e-3):
    """err <= tol; warn above warn_above, well over the bf16 floor (about 2^-9) of one rounding,
    where a bug may hide under the bar."""
    err = qlora.rel_err(got, ref)
    floor = qlora.rel_err(nf4.bf16_value(nf4.bf16_bits(np.asarray(ref, np.float32))), ref)
    say(f"  {name}: rel err {err:.3e} (bf16 output floor {floor:.3e})")
    assert err <= tol, f"{name}: rel err {err:.3e} > {tol}"
    if err > warn_above:
        warnings.warn(f"{name}: rel err {err:.3e} is above {warn_above:g} (bf16 output floor {floor:.3e})")
    return err
