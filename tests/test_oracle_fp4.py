"""Pins for the oracle's 4-bit floating-point (E2M1) weight format (CPU only).

* the E2M1 codebook against what the page fixes (1 sign, 2 exponent and 1 mantissa bits, largest
  magnitude 6: this fixes the exponent bias at 1) and the golden file;
* the E4M3 values and the rounding of the group scales against torch's float8_e4m3fn conversion
  (an independent implementation: round to nearest, ties to even);
* the E2M1 encoder against exact-rational brute force (nearest value, ties to the even mantissa),
  at and next to every midpoint and on random groups;
* special cases (all-zero weight, an all-zero group, the group that holds the tensor maximum
  gets the largest scale, signs, saturation), the nibble order, the dequantisation definition
  (one rounding of an exact product) and its error bound; every E2M1 value times every E4M3 scale
  is exact in bf16 (the GPU kernels rely on it).
"""
from fractions import Fraction
import os

import numpy as np
import pytest
import torch

from oracle import fp4, nf4

HERE = os.path.dirname(os.path.abspath(__file__))


def test_e2m1_codebook_matches_the_page():
    c = fp4.e2m1_codebook()
    assert c.shape == (16,)
    mags = c[:8]
    assert mags.max() == 6.0                          # the page: range about +-6.0
    assert mags[0] == 0.0 and np.all(np.diff(mags) > 0)
    assert np.array_equal(c[8:], -mags)               # bit 3 is the sign
    # normal values 2^(e - 1) (1 + m/2): exactly one mantissa bit, three binades 1, 2, 4
    for code in range(2, 8):
        e, m = code >> 1, code & 1
        assert mags[code] == 2.0 ** (e - 1) * (1.0 + 0.5 * m)
    # the subnormals (exponent field 0) are m / 2: 0 and 0.5
    assert mags[1] == 0.5
    rows = [ln.split() for ln in open(os.path.join(HERE, "golden", "e2m1_codebook.txt"))
            if not ln.startswith("#")]
    assert [float.fromhex(r[1]) for r in rows] == list(c)


def test_e4m3_grid_matches_torch():
    b = torch.arange(127, dtype=torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(fp4.e4m3_grid(), ref)
    assert fp4.e4m3_grid()[-1] == fp4.E4M3_MAX


def test_e4m3_rounding_matches_torch():
    g = fp4.e4m3_grid()
    rng = np.random.default_rng(1)
    mids = (g[1:] + g[:-1]) / 2
    x = np.concatenate([rng.uniform(0, 460, 20000), rng.uniform(0, 0.03, 20000), mids, g,
                        np.nextafter(mids.astype(np.float32), np.float32(0)),
                        np.nextafter(mids.astype(np.float32), np.float32(1000))]).astype(np.float32)
    got = g[fp4.round_to_grid(x, g)].astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(got, want)


def test_group_scales_match_torch():
    rng = np.random.default_rng(2)
    w = (rng.standard_normal((8, 512)) * rng.uniform(1e-4, 1.0, (8, 1))).astype(np.float32)
    S = fp4.tensor_scale(w)
    assert S == np.float32(np.abs(w).max() / np.float32(2688))
    amax_g = np.abs(w).reshape(-1, 16).max(axis=1)
    t = (amax_g / np.float32(np.float32(6) * S)).astype(np.float32)
    want = torch.from_numpy(t).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(fp4.group_scales(w, S), want)


def nearest_e2m1(v: Fraction) -> int:
    """Code of the E2M1 value nearest to v by exact distance, ties to the even mantissa."""
    best = None
    for code in range(8):
        val = Fraction(fp4.e2m1_value(code))
        d = abs(abs(v) - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1] | (8 if v < 0 else 0)


def brute_codes(w, scales, S):
    out = []
    grid = fp4.e4m3_grid()
    for gi, grp in enumerate(np.asarray(w, np.float32).reshape(-1, 16)):
        d = np.float32(np.float32(grid[scales[gi]]) * S)
        for x in grp:
            if d == 0:
                out.append(0)
                continue
            v = np.float32(x / d)
            out.append(nearest_e2m1(Fraction(float(v))))
    return np.array(out, dtype=np.uint8)


def test_encode_brute_force_random():
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((6, 64)) * 0.02).astype(np.float32)
    w[2, :16] *= 1e-3                                  # a group far below the tensor maximum
    q = fp4.quantize(w)
    assert np.array_equal(fp4.unpack(q.codes), brute_codes(w, q.scales, q.tscale))


def test_encode_brute_force_at_midpoints():
    """Values that land exactly on, and one float32 step either side of, every midpoint between
    E2M1 magnitudes (and beyond 6): the tie rule and the saturation decide them."""
    mags = fp4.e2m1_codebook()[:8]
    mids = np.concatenate([(mags[1:] + mags[:-1]) / 2, [6.0, 7.5, 100.0]]).astype(np.float32)
    vs = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    vs = np.concatenate([vs, -vs])
    # one group per value, each pinned to scale 1 and tensor scale 1 so that v = w exactly
    S = np.float32(1.0)
    one = np.uint8(56)                                 # E4M3 byte of 1.0
    w = np.zeros((len(vs), 16), np.float32)
    w[:, 0] = vs
    sc = np.full(len(vs), one, np.uint8)
    assert fp4.e4m3_grid()[one] == 1.0
    assert np.array_equal(fp4.encode(w, sc, S), brute_codes(w, sc, S))


def test_special_cases():
    z = np.zeros((4, 64), np.float32)
    q = fp4.quantize(z)
    assert q.tscale == 0 and not q.scales.any() and not q.codes.any()
    assert not fp4.dequantize_f32(q).any()
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    w[1, 16:32] = 0                                    # an all-zero group
    w[3, 50] = -0.5                                    # the tensor maximum, negative
    w[0, 3] = -1e-9                                    # a negative that rounds to zero
    q = fp4.quantize(w)
    codes = fp4.unpack(q.codes).reshape(4, 64)
    assert q.scales[(1 * 64 + 16) // 16] == 0 and not codes[1, 16:32].any()
    g = (3 * 64 + 50) // 16
    assert fp4.e4m3_grid()[q.scales[g]] == fp4.E4M3_MAX           # the largest group scale
    assert codes[3, 50] == 15                                      # -6: sign and saturation
    assert codes[0, 3] == 8                                        # -0
    assert fp4.dequantize_f32(q)[0, 3] == 0.0
    assert np.array_equal(codes >= 8, w < 0)                      # the sign bit


def test_pack_known_pattern():
    codes = np.array([1, 2, 15, 0, 8, 7], np.uint8)
    assert list(fp4.pack(codes)) == [0x12, 0xF0, 0x87]
    assert np.array_equal(fp4.unpack(fp4.pack(codes)), codes)


def test_dequantize_definition_and_bound():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((5, 128)) * 0.05).astype(np.float32)
    q = fp4.quantize(w)
    got = fp4.dequantize_f32(q)
    codes = fp4.unpack(q.codes).reshape(-1, 16)
    s = fp4.e4m3_grid()[q.scales]
    S = float(q.tscale)
    for gi in range(codes.shape[0]):
        for j in range(16):
            exact = fp4.e2m1_value(int(codes[gi, j])) * s[gi] * S      # exact in float64
            assert got.reshape(-1, 16)[gi, j] == np.float32(exact)
    # |w - w'| <= half the widest E2M1 gap (2 / 2) times the group's step d, plus one rounding
    d = (s * S).astype(np.float64)
    err = np.abs(w.reshape(-1, 16).astype(np.float64) - got.reshape(-1, 16))
    assert np.all(err <= d[:, None] * (1.0 + 1e-6) + 1e-12)


def test_every_code_times_every_scale_is_exact_in_bf16():
    v = (fp4.e2m1_codebook()[:, None] * fp4.e4m3_grid()[None, :]).astype(np.float32)
    assert np.array_equal(nf4.bf16_value(nf4.bf16_bits(v)), v)
