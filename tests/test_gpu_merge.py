"""GPU parity of the LoRA merge (qlora_merge) against the oracle.

W' = bf16(deq(W) + s B A) is compared element by element with the float64 oracle (oracle/merge.py).
The kernel forms deq(W) + s B A in float32 (the rank-r sum on the matrix cores) and rounds once to
bf16, so each element lies within one bf16 unit in the last place of the exact value plus the
float32 error of that sum, which standard analysis bounds by (r + 2) 2^-24 (|deq(W)| + |s| |B| |A|)
(r products summed, one more addition). Where the two terms do not nearly cancel that float32 part
is far below a bf16 unit; where they do (the exact value much smaller than its terms), the float32
error can be several bf16 units of the small result, and the bound says by how much.
With r = 0 it equals nf4_dequantize's bf16 output exactly. Re-quantising W' with
nf4_quantize equals the oracle's quantisation of the same values bit for bit. Shapes are ragged
against the 64 x 128 tile, ranks span the rank-term padding (1, 5, 16, 33, 64, 128) and the
kernel's B prefetch widths (one, two and four 16-byte pieces per thread); the larger shapes give
each workgroup a run of several tiles of its column strip (the software-pipelined loop).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import merge, nf4
from tests.gpu_helpers import assert_quant_equal, f32, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """bf16 spacing at |x| (the normal range; the smallest normal's spacing below it)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def check_merge(got, ref, deq, A, B, s, r, what="merge"):
    """Every element within one bf16 ulp of the exact value plus the float32 error bound of
    deq + s B A; reports the largest error in bf16 ulps and how many elements exceed one."""
    ulps = np.abs(got - ref) / bf16_ulp(ref)
    mag = np.abs(deq).astype(np.float64)
    if r:
        mag = mag + abs(s) * (np.abs(B).astype(np.float64) @ np.abs(A).astype(np.float64))
    bound = bf16_ulp(ref) + (r + 2) * 2.0 ** -24 * mag
    i = np.unravel_index(np.argmax(ulps), ulps.shape)
    say(f"  {what}: max error {ulps.max():.3f} bf16 ulp ({int((ulps > 1).sum())} of {ulps.size} above 1; "
        f"worst: exact {ref[i]:.4e}, got {got[i]:.4e}, terms {mag[i]:.3e})")
    assert (np.abs(got - ref) <= bound).all()


@pytest.mark.parametrize("n,k,r,dq,s", [
    (64, 128, 16, 256, 2.0),
    (200, 320, 5, 0, -0.5),
    (129, 576, 1, 256, 1.0),
    (70, 1024, 33, 256, 0.25),
    (256, 256, 64, 0, 1.5),
    (40, 192, 128, 256, -2.0),
    (1000, 192, 32, 256, 1.0),       # 16 tiles in one strip and a ragged last one
    (2056, 4160, 96, 256, 0.5),      # many strips, a 64-column last strip, runs of tiles
    (3000, 320, 24, 0, -1.0),
])
def test_merge_parity(lib, n, k, r, dq, s):
    say(f"merge n={n} k={k} r={r} dq={dq} s={s}")
    W = wl.normal_bf16(500 + n, (n, k), 0.02)
    A = wl.normal_bf16(501 + n, (r, k), k ** -0.5)
    B = wl.normal_bf16(502 + n, (n, r), 0.05)
    qg = lib.nf4_quantize(W.to(DEV), dq)
    Wm = lib.qlora_merge(qg, A.to(DEV), B.to(DEV), s)
    q2 = lib.nf4_quantize(Wm, 256)
    torch.cuda.synchronize()
    qo = nf4.quantize(W.float().numpy(), dq)
    assert_quant_equal(qg, qo)
    deq = nf4.dequantize_f32(qo)
    ref = merge.merge(deq, f32(A), f32(B), s)
    got = f32(Wm).astype(np.float64)
    check_merge(got, ref, deq, f32(A), f32(B), s, r)
    # re-quantised merged weight: bit for bit the oracle's quantisation of the same values
    assert_quant_equal(q2, nf4.quantize(f32(Wm), 256))


def test_merge_rank_zero_equals_dequantize(lib):
    W = wl.normal_bf16(610, (136, 448), 0.02)
    for dq in (0, 256):
        qg = lib.nf4_quantize(W.to(DEV), dq)
        Wm = lib.qlora_merge(qg, None, None, 3.0)
        Wd = lib.nf4_dequantize(qg, torch.bfloat16)
        torch.cuda.synchronize()
        assert np.array_equal(f32(Wm), f32(Wd))


def test_merge_full_size_down_weight(lib):
    """The merge bench.py times: the down workload's weight [4096, 14336], r = 32, s = 1, on
    sampled rows (all columns) against the oracle, within the bound of check_merge."""
    from tests.test_gpu_workloads import sample
    w = wl.WORKLOADS["down"]
    W, A, B = wl.tensor(w, "W"), wl.tensor(w, "A"), wl.tensor(w, "B")
    qg = lib.nf4_quantize(W.to(DEV), w.dq_block)
    Wm = lib.qlora_merge(qg, A.to(DEV), B.to(DEV), w.s)
    torch.cuda.synchronize()
    qo = nf4.quantize(W.float().numpy(), w.dq_block)
    assert_quant_equal(qg, qo)
    rows = sample(w.N, 64, 55)
    Wd = nf4.dequantize_f32(qo)
    ref = merge.merge(Wd[rows], f32(A), f32(B)[rows], w.s)
    got = f32(Wm[torch.from_numpy(rows).to(DEV)]).astype(np.float64)
    check_merge(got, ref, Wd[rows], f32(A), f32(B)[rows], w.s, w.r, "full-size merge")
