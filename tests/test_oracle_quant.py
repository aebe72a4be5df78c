"""Pins for the oracle's NF4 quantiser, double quantisation and dequantiser (CPU only).

Encoding is pinned by brute force in exact rational arithmetic (fractions.Fraction), including
every float32 value near each midpoint between levels; packing by a known byte pattern; the
round trip by exact reconstruction on codebook points; double quantisation by its rounding
definition and error bound.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import nf4

C = nf4.codebook()
CF = [Fraction(float(c)) for c in C]


def nearest_exact(v: float) -> int:
    """Index of the level nearest to v, exact rational distances, ties to the lower index."""
    fv = Fraction(float(v))
    best, bi = None, -1
    for i, c in enumerate(CF):
        d = abs(fv - c)
        if best is None or d < best:
            best, bi = d, i
    return bi


def encode_unit(v: np.ndarray) -> np.ndarray:
    """Codes of float32 values v with a block absmax of exactly 1 (so v / a == v)."""
    v = np.asarray(v, dtype=np.float32)
    pad = (-v.size) % 64
    w = np.concatenate([v, np.zeros(pad, np.float32)])
    a = np.ones(w.size // 64, np.float32)
    return nf4.encode(w, a)[: v.size]


def near_midpoints(span: int = 40) -> np.ndarray:
    out = []
    for i in range(15):
        mid = (float(C[i]) + float(C[i + 1])) / 2      # exact in float64
        f = np.float32(mid)
        bits = np.array([f], np.float32).view(np.int32)[0]
        for d in range(-span, span + 1):
            x = np.array([bits + d if f >= 0 else bits - d], np.int32).view(np.float32)[0]
            out.append(x)
        out.append(np.float32(mid))
    return np.array(out, np.float32)


def test_encode_brute_force_near_midpoints():
    v = near_midpoints()
    got = encode_unit(v)
    want = np.array([nearest_exact(x) for x in v])
    assert np.array_equal(got, want)


def test_encode_brute_force_random():
    rng = np.random.default_rng(11)
    v = rng.uniform(-1, 1, 4000).astype(np.float32)
    got = encode_unit(v)
    want = np.array([nearest_exact(x) for x in v])
    assert np.array_equal(got, want)


def test_encode_ties_go_to_lower_code():
    """Midpoints 2, 6, 7 and 14 are exact in float32; a value there takes the lower code, both
    directly and when it arrives through the division by a power-of-two absmax."""
    exact = []
    for i in range(15):
        mid = (float(C[i]) + float(C[i + 1])) / 2
        if float(np.float32(mid)) == mid:
            exact.append(i)
            assert encode_unit(np.array([mid], np.float32))[0] == i
            w = np.zeros(64, np.float32)
            w[0] = -4.0                                   # absmax 4: v = w / 4 exactly
            w[1] = np.float32(4.0 * mid)
            assert nf4.encode(w, nf4.block_absmax(w))[1] == i
    assert exact == [2, 6, 7, 14]


def test_encode_divides_in_float32():
    """v is fl32(w / a), not the exact quotient: pin on a quotient that rounds across a midpoint."""
    rng = np.random.default_rng(5)
    w = rng.standard_normal(64 * 2000).astype(np.float32)
    a = nf4.block_absmax(w)
    got = nf4.encode(w, a)
    v = (w / np.repeat(a, 64)).astype(np.float32)
    want = np.array([nearest_exact(x) for x in v[:20000]])
    assert np.array_equal(got[:20000], want)


def test_special_blocks():
    z = np.zeros(64, np.float32)
    assert nf4.block_absmax(z)[0] == 0
    assert np.all(nf4.encode(z, nf4.block_absmax(z)) == 7)
    neg0 = np.full(64, -0.0, np.float32)
    assert np.all(nf4.encode(neg0, nf4.block_absmax(neg0)) == 7)
    one = np.zeros(64, np.float32)
    one[17] = -3.5
    codes = nf4.encode(one, nf4.block_absmax(one))
    assert codes[17] == 0 and np.all(np.delete(codes, 17) == 7)
    one[17] = 2.0
    codes = nf4.encode(one, nf4.block_absmax(one))
    assert codes[17] == 15 and np.all(np.delete(codes, 17) == 7)


def test_pack_known_pattern():
    codes = np.arange(32, dtype=np.uint8) % 16
    packed = nf4.pack(codes)
    assert packed.tolist() == [0x01, 0x23, 0x45, 0x67, 0x89, 0xAB, 0xCD, 0xEF] * 2
    assert np.array_equal(nf4.unpack(packed), codes)


def test_round_trip_exact_on_codebook_points():
    rng = np.random.default_rng(3)
    n, k = 12, 256
    idx = rng.integers(0, 16, (n, k))
    idx[:, ::64] = 15                       # every block holds +1 * 2^e, so absmax = 2^e
    e = rng.integers(-20, 5, (n, k // 64)).astype(np.float64)
    scale = np.repeat(2.0 ** e, 64, axis=1)
    w = (C[idx].astype(np.float64) * scale).astype(np.float32)
    q = nf4.quantize(w, 0)
    assert np.array_equal(nf4.unpack(q.codes).reshape(n, k), idx)
    assert np.array_equal(nf4.dequantize_f32(q), w)


def test_quantize_is_idempotent_on_dequantised_weights():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((16, 512)) * 0.02).astype(np.float32)
    q1 = nf4.quantize(w, 0)
    q2 = nf4.quantize(nf4.dequantize_f32(q1), 0)
    assert np.array_equal(q1.codes, q2.codes)
    assert np.array_equal(q1.absmax, q2.absmax)


def test_double_quant_definition_and_bound():
    rng = np.random.default_rng(9)
    a = np.abs(rng.standard_normal(256 * 5 + 77)).astype(np.float32) * np.float32(0.05)
    a[300] = 0.0
    q, S = nf4.double_quant(a, 256)
    assert q.dtype == np.int8 and S.dtype == np.float32 and S.size == 6
    assert q.min() >= 0 and q.max() <= 127
    for j in range(S.size):
        seg = a[j * 256:(j + 1) * 256]
        assert S[j] == np.float32(seg.max() / np.float32(127))
        assert q[j * 256 + int(np.argmax(seg))] == 127
        for t, av in enumerate(seg):
            ratio = float(np.float32(av / S[j]))
            assert int(q[j * 256 + t]) == round(ratio)            # Python round: half to even
    dec = nf4.decode_absmax(nf4.NF4Weight(1, a.size * 64, 256, np.zeros(0, np.uint8), q, S))
    Sx = np.repeat(S, 256)[: a.size].astype(np.float64)
    assert np.all(np.abs(dec.astype(np.float64) - a) <= Sx * (0.5 + 2 ** -20) + 2 ** -24 * a)


def test_double_quant_zero_run():
    q, S = nf4.double_quant(np.zeros(300, np.float32), 256)
    assert np.all(q == 0) and np.all(S == 0)


def test_dequantize_definition():
    rng = np.random.default_rng(10)
    w = (rng.standard_normal((8, 128)) * 0.02).astype(np.float32)
    for dq in (0, 256):
        q = nf4.quantize(w, dq)
        codes = nf4.unpack(q.codes)
        a = nf4.decode_absmax(q)
        d = nf4.dequantize_f32(q).reshape(-1)
        for t in range(0, d.size, 7):
            assert d[t] == np.float32(C[codes[t]] * a[t // 64])
        bits = nf4.dequantize_bf16(q).reshape(-1)
        assert np.array_equal(bits, nf4.bf16_bits(d))


def test_dequantised_error_within_half_step():
    """|w - w'| is at most half the widest level gap times absmax (plus rounding)."""
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((32, 256)) * 0.02).astype(np.float32)
    q = nf4.quantize(w, 0)
    a = np.repeat(q.absmax, 64).reshape(w.shape)
    gap = float(np.max(np.diff(C.astype(np.float64))))
    assert np.all(np.abs(nf4.dequantize_f32(q) - w) <= a * (gap / 2 + 1e-6))


def test_k_not_multiple_of_block_rejected():
    with pytest.raises(ValueError):
        nf4.quantize(np.zeros((2, 96), np.float32))


def test_c_encoder_equals_numpy_encoder():
    """The C twin (oracle/nf4_encode.c) and the numpy encoder agree on every case above."""
    rng = np.random.default_rng(13)
    w = np.concatenate([
        rng.standard_normal(64 * 3000).astype(np.float32) * np.float32(0.02),
        near_midpoints(), np.zeros(64, np.float32), np.full(64, -0.0, np.float32)])
    w = np.concatenate([w, np.zeros((-w.size) % 64, np.float32)])
    for a in (nf4.block_absmax(w), np.ones(w.size // 64, np.float32)):
        assert np.array_equal(nf4.encode_c(w, a), nf4.encode_numpy(w, a))
    v = near_midpoints()
    v = np.concatenate([v, np.zeros((-v.size) % 64, np.float32)])
    got = nf4.encode_c(v, np.ones(v.size // 64, np.float32))
    assert np.array_equal(got[: near_midpoints().size], [nearest_exact(x) for x in near_midpoints()])
