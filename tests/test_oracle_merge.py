"""Pins for the oracle's LoRA merge (CPU only).

* Forward equivalence: the plain layer with the merged weight equals the QLoRA layer with the
  adapters, X W'^T == X deq(W)^T + s (X A^T) B^T (the pinned single-layer oracle), to 1e-12;
* brute force: each element from its own sum on tiny shapes;
* B = 0 and s = 0 leave deq(W) exactly; a rank-1 update equals numpy's outer product.
"""
import math

import numpy as np

from oracle import merge, nf4, qlora


def make(N, K, r, seed, dq=0):
    rng = np.random.default_rng(seed)
    W = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    A = rng.standard_normal((r, K)) / math.sqrt(K)
    B = rng.standard_normal((N, r)) * 0.01
    X = rng.standard_normal((5, K))
    return nf4.dequantize_f32(nf4.quantize(W, dq)), A, B, X


def test_merged_layer_equals_the_qlora_layer():
    for dq, s in ((0, 2.0), (256, -0.75)):
        Wd, A, B, X = make(9, 128, 4, 1, dq)
        Wm = merge.merge(Wd, A, B, s)
        Y_merged, _ = qlora.forward(X, Wm, A[:0], B[:, :0], 1.0)
        Y_lora, _ = qlora.forward(X, Wd, A, B, s)
        assert qlora.rel_err(Y_merged, Y_lora) < 1e-12


def test_merge_brute_force():
    Wd, A, B, _ = make(4, 64, 3, 2)
    s = 1.5
    Wm = merge.merge(Wd, A, B, s)
    for n in range(4):
        for k in range(64):
            ref = float(Wd[n, k]) + s * sum(float(B[n, j]) * float(A[j, k]) for j in range(3))
            assert abs(Wm[n, k] - ref) <= 1e-15 * max(1.0, abs(ref))


def test_merge_special_cases():
    Wd, A, B, _ = make(6, 128, 5, 3, 256)
    assert np.array_equal(merge.merge(Wd, A, np.zeros_like(B), 2.0), Wd.astype(np.float64))
    assert np.array_equal(merge.merge(Wd, A, B, 0.0), Wd.astype(np.float64))
    u, v = B[:, :1], A[:1]
    np.testing.assert_allclose(merge.merge(Wd, v, u, 0.5), Wd + 0.5 * np.outer(u[:, 0], v[0]),
                               rtol=1e-15, atol=1e-18)
