"""LoRA merge of the QLoRA layer in float64 -- test infrastructure (see the package docstring).

After training, the adapters are folded into the base weight for a merged save, optionally
re-quantised for export [pyshine Unsloth code tour, the save.py walkthrough: adapter versus merged
saves, LoRA weights merged layer by layer; NVFP4 update article, "A More Flexible Quantization
Export Pipeline": merged saves with compressed export]. The merged weight is the one whose plain
layer equals the QLoRA layer (Delta W = B A scaled by s):

    W' = deq(W) + s B A          [N, K]

so that X W'^T = X deq(W)^T + s (X A^T) B^T. Re-quantising W' is nf4.quantize of its values.
Float64 from the exact values of the float32 dequantised weight and the bf16 adapters.
"""
from __future__ import annotations

import numpy as np

from . import qlora

_f64 = qlora._f64


def merge(Wd, A, B, s: float):
    """W' = deq(W) + s B A for the dequantised W [N,K], A [r,K], B [N,r]."""
    return _f64(Wd) + float(s) * (_f64(B) @ _f64(A))
