"""The 4-bit floating-point (E2M1) variant of the base-weight format, in plain numpy -- test
infrastructure (see the package docstring).

What the pages fix [NVFP4 update article, "NVFP4: A Quantization Format for the Next Generation
of Hardware"]: each weight is a 4-bit float with 1 sign bit, 2 exponent bits and 1 mantissa bit
(E2M1), whose largest magnitude is 6; weights are quantised in groups of 16 or 32 that share one
FP8 scaling factor. Everything else below is a reading, stated where it is taken:

* E2M1 values: exponent bias 1, no infinities or NaN; exponent field 0 is subnormal, so the
  magnitudes are m/2 (e = 0) and 2^(e-1) (1 + m/2) (e = 1..3): 0, 0.5, 1, 1.5, 2, 3, 4, 6.
  Code = sign << 3 | e << 1 | m.
* Groups of 16 consecutive elements of the row-major weight (the smaller of the two sizes the
  page gives); the group scale is FP8 E4M3 (4 exponent bits, bias 7, 3 mantissa bits, largest
  finite value 448, the FP8 form used for scales), stored as its byte.
* A float32 scale per tensor, S = fl32(amax(W) / 2688) with 2688 = 6 * 448, so that a group scale
  spans the whole E4M3 range: the page's FP8 scale alone could not hold the scales of weights
  whose groups sit far below 1 (E4M3's smallest normal is 2^-6). S == 0 (an all-zero weight) gives
  every group scale 0 and every code 0.
* Group scale: s = E4M3(fl32(amax_g / fl32(6 * S))), rounded to the nearest E4M3 value, ties to
  the even mantissa, saturating at 448.
* Encode: v = fl32(w / fl32(s * S)) (s == 0: code 0); the code is the nearest E2M1 value to v,
  ties to the even mantissa, magnitudes above 6 saturating to 6; the sign bit is set when v < 0.
* Pack: byte i holds element 2i in bits 7..4 and element 2i+1 in bits 3..0 (as the NF4 codes of
  this library).
* Dequantise: w' = fl32(fl32(e2m1[code] * s) * S); the inner product is exact (it needs at most
  6 significant bits), so w' is one rounding of the exact product.
"""
from __future__ import annotations

import dataclasses

import numpy as np

GROUP = 16
E4M3_MAX = 448.0
TSCALE_DIV = 6.0 * E4M3_MAX          # 2688


# ----------------------------------------------------------------------------------- codebooks
def e2m1_value(code: int) -> float:
    """The value of 4-bit code sign|e1 e0|m, from its bit fields (bias 1, e = 0 subnormal)."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m / 2.0 if e == 0 else 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


def e2m1_codebook() -> np.ndarray:
    """The 16 values, indexed by code (float64; all exact)."""
    return np.array([e2m1_value(c) for c in range(16)])


def e4m3_value(byte: int) -> float:
    """Value of a non-negative E4M3 byte 0..126 (bias 7; e = 0 subnormal, m * 2^-9)."""
    e, m = (byte >> 3) & 15, byte & 7
    if e == 0:
        return m * 2.0 ** -9
    return 2.0 ** (e - 7) * (1.0 + m / 8.0)


def e4m3_grid() -> np.ndarray:
    """The 127 non-negative finite E4M3 values, ascending, indexed by byte (float64, exact)."""
    return np.array([e4m3_value(b) for b in range(127)])


def round_to_grid(x: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the nearest grid value to each x >= 0 (ascending grid, index parity = mantissa
    parity), ties to the even index, x beyond the last value saturating to it. Exact: the grid
    values, their midpoints and x (float32) are all exact in float64."""
    x = np.asarray(x, dtype=np.float64)
    mids = (grid[1:] + grid[:-1]) / 2.0
    i = np.searchsorted(mids, x, side="left")        # number of midpoints strictly below x
    tie = (i < len(mids)) & (x == mids[np.minimum(i, len(mids) - 1)])
    # at a tie x sits between grid[i] and grid[i + 1]: take whichever index is even
    i = np.where(tie & (i % 2 == 1), i + 1, i)
    return i


# ----------------------------------------------------------------------------------- weight
@dataclasses.dataclass
class FP4Weight:
    n: int
    k: int
    codes: np.ndarray      # uint8 [n*k/2] packed, element 2i in the high nibble
    scales: np.ndarray     # uint8 [n*k/16] E4M3 bytes of the group scales
    tscale: np.float32     # the tensor scale S


def tensor_scale(w: np.ndarray) -> np.float32:
    amax = np.float32(np.abs(w.astype(np.float32)).max()) if w.size else np.float32(0)
    return np.float32(amax / np.float32(TSCALE_DIV))


def group_scales(w: np.ndarray, S: np.float32) -> np.ndarray:
    """E4M3 bytes of the group scales (uint8 [n*k/16])."""
    g = np.abs(w.astype(np.float32)).reshape(-1, GROUP).max(axis=1)
    if S == 0:
        return np.zeros(g.shape, dtype=np.uint8)
    t = (g / np.float32(np.float32(6.0) * S)).astype(np.float32)
    return round_to_grid(t, e4m3_grid()).astype(np.uint8)


def encode(w: np.ndarray, scales: np.ndarray, S: np.float32) -> np.ndarray:
    """Unpacked codes (uint8, one per element) of w against its group scales."""
    w = w.astype(np.float32).reshape(-1, GROUP)
    s = e4m3_grid()[scales].astype(np.float32)                     # exact in float32
    d = (s * S).astype(np.float32)[:, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(d > 0, w / np.where(d > 0, d, np.float32(1)), np.float32(0)).astype(np.float32)
    mags = e2m1_codebook()[:8]
    idx = round_to_grid(np.abs(v), mags)
    codes = idx.astype(np.uint8) | np.where(v < 0, np.uint8(8), np.uint8(0))
    return codes.reshape(-1)


def pack(codes: np.ndarray) -> np.ndarray:
    c = codes.reshape(-1, 2)
    return ((c[:, 0] << 4) | c[:, 1]).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed >> 4
    out[1::2] = packed & 15
    return out


def quantize(w: np.ndarray) -> FP4Weight:
    """w: float32 (or bf16 values as float32) [n, k], k % 16 == 0."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % GROUP:
        raise ValueError("k must be a multiple of 16")
    S = tensor_scale(w)
    sc = group_scales(w, S)
    return FP4Weight(n, k, pack(encode(w, sc, S)), sc, S)


def dequantize_f32(q: FP4Weight) -> np.ndarray:
    codes = unpack(q.codes).reshape(-1, GROUP)
    vals = e2m1_codebook()[codes].astype(np.float32)
    s = e4m3_grid()[q.scales].astype(np.float32)[:, None]
    inner = (vals * s).astype(np.float32)                         # exact
    return (inner * q.tscale).astype(np.float32).reshape(q.n, q.k)
