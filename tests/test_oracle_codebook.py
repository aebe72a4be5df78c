"""Pins for the oracle's NF4 codebook and bf16 rounding (CPU only).

The levels follow the QLoRA construction of 4-bit NormalFloat (the pages name NF4 but print no
values; see oracle/nf4.py). They are pinned here against scipy's normal quantile (a library
routine for the same special function), against the normal CDF directly (each level must sit at
its evenly spaced probability), and against the structure the construction fixes.
"""
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import ndtri

from oracle import nf4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nf4_codebook.txt")


def test_quantile_matches_library():
    ps = np.concatenate([np.linspace(0.5, 0.999, 97)[1:], [nf4.DELTA, 0.75, 0.9, 0.99]])
    for p in ps:
        mine = nf4.normal_quantile(float(p))
        ref = float(ndtri(p))
        # conditioning: p itself is known to ~2^-53, which moves the quantile by that / phi(x)
        phi = math.exp(-0.5 * ref * ref) / math.sqrt(2 * math.pi)
        tol = 4 * 2.0 ** -53 / phi + 4e-15 * max(1.0, abs(ref))
        assert abs(mine - ref) <= tol, (p, mine, ref)


def test_codebook_same_from_library_quantile():
    mine = nf4.codebook()
    lib = nf4.nf4_levels_f64(quantile=lambda p: float(ndtri(p))).astype(np.float32)
    assert mine.view(np.uint32).tolist() == lib.view(np.uint32).tolist()


def test_codebook_structure():
    c = nf4.codebook()
    assert c.dtype == np.float32 and c.shape == (16,)
    assert np.all(np.diff(c) > 0)
    assert c[0] == -1.0 and c[15] == 1.0
    assert c[7] == 0.0 and not np.signbit(c[7])
    assert int((c < 0).sum()) == 7 and int((c > 0).sum()) == 8


def test_levels_sit_at_evenly_spaced_probabilities():
    """Phi(level * z_delta) lands on the evenly spaced probabilities of the construction."""
    lv = nf4.nf4_levels_f64()
    z = float(ndtri(nf4.DELTA))
    pos = lv[8:]            # 8 positive levels, ascending
    neg = -lv[:7][::-1]     # 7 negative levels, as magnitudes ascending
    for j, v in enumerate(pos):
        want = 0.5 + (j + 1) * (nf4.DELTA - 0.5) / 8
        assert abs(0.5 * math.erfc(-v * z / math.sqrt(2)) - want) < 1e-13
    for j, v in enumerate(neg):
        want = 0.5 + (j + 1) * (nf4.DELTA - 0.5) / 7
        assert abs(0.5 * math.erfc(-v * z / math.sqrt(2)) - want) < 1e-13


def test_codebook_golden_file():
    """tests/golden/nf4_codebook.txt was written by tests/golden/make_golden.py (oracle only)."""
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    stored = np.array([float.fromhex(r[1]) for r in rows], dtype=np.float32)
    assert stored.view(np.uint32).tolist() == nf4.codebook().view(np.uint32).tolist()


def test_codebook_levels_far_from_fp32_rounding_boundaries():
    """Each float64 level lies at least 0.02 ulp inside its float32 rounding interval (the
    closest is about 0.023 ulp), far more than any accurate quantile's error, so the float32
    table does not depend on how the quantile is computed."""
    lv = nf4.nf4_levels_f64()
    for v in lv:
        f = np.float32(v)
        if v == 0 or abs(v) == 1:
            continue
        ulp = abs(float(np.spacing(f)))
        assert abs(float(f) - v) < 0.48 * ulp


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(7)
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0)
    # exact ties: low 16 bits 0x8000, both parities of the kept lsb
    ties = (rng.integers(0x3F000000 >> 16, 0x4100, 5000, dtype=np.uint32) << 16 | 0x8000)
    x = np.concatenate([x, ties.view(np.float32), -ties.view(np.float32),
                        np.array([0.0, -0.0, 1e-40, -1e-40, 3.0e38], np.float32)])
    mine = nf4.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    back = nf4.bf16_value(mine)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
