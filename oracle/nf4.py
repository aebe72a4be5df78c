"""NF4 quantisation in plain numpy (plus one plain C loop) -- test infrastructure.

See the package docstring for who may use it.

What the pages fix: the frozen base weight is stored as 4-bit NormalFloat (NF4), a code whose
levels suit normally distributed weights, and the quantisation constants are themselves
quantised ("double quantization") [Unsloth v0.1.463-beta release article, "About the Unsloth
Project"; v0.1.47-beta article, section on lowering the fine-tuning barrier]. Everything else
below is a reading, stated where it is taken:

* Levels. The QLoRA construction of NF4: with delta = 1 - (1/30 + 1/32)/2, take the standard
  normal quantiles of 9 probabilities evenly spaced from delta down to 1/2 (dropping 1/2) for the
  positive side and of 8 such probabilities (dropping 1/2) negated for the negative side, add an
  exact zero, sort, divide by the largest; 16 levels, 7 negative, exact 0, 8 positive, ends -1
  and +1. Computed in float64, then rounded to float32 (nearest-even).
* Blocks of 64 consecutive elements of the row-major weight; the per-block constant is the
  absolute maximum in float32 (exact).
* Encode: v = fl32(w / absmax) (IEEE float32 division), code = index of the nearest level to v
  (distance taken exactly, in float64), ties to the lower index. An all-zero block has absmax 0
  and every code 7 (the exact zero level).
* Pack: byte i holds element 2i in bits 7..4 and element 2i+1 in bits 3..0.
* Double quantisation: runs of 256 consecutive absmax values (flattened order, a last partial run
  uses what is left) share S = fl32(max / 127); q = rint(fl32(a / S)) (half to even) clamped to
  [0, 127] and stored as int8; S == 0 gives q = 0. Decode a' = fl32(q * S). Codes are always
  taken against the exact float32 absmax, before double quantisation.
* Dequantise: w' = fl32(level[code] * a'); the bf16 form is w' rounded to nearest-even.

The encoder exists twice: encode_numpy (vectorised numpy) and encode_c (the same definition as a
C loop in nf4_encode.c, for full-size weights); tests pin both to exact-rational brute force and
to each other.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
import subprocess
from typing import Optional

import numpy as np

BLOCK = 64
DELTA = 1.0 - 0.5 * (1.0 / 30.0 + 1.0 / 32.0)


# ----------------------------------------------------------------------------------- codebook
def normal_cdf(x: float) -> float:
    """Phi(x) = erfc(-x / sqrt 2) / 2, in float64."""
    return 0.5 * math.erfc(-x / math.sqrt(2.0))


def normal_quantile(p: float) -> float:
    """Phi^-1(p) for 0 < p < 1 by bisection on normal_cdf, run until the bracket stops shrinking."""
    if not 0.0 < p < 1.0:
        raise ValueError("p must lie in (0, 1)")
    lo, hi = -40.0, 40.0
    while True:
        mid = 0.5 * (lo + hi)
        if mid <= lo or mid >= hi:
            break
        if normal_cdf(mid) < p:
            lo = mid
        else:
            hi = mid
    return lo if abs(normal_cdf(lo) - p) <= abs(normal_cdf(hi) - p) else hi


def nf4_levels_f64(quantile=normal_quantile) -> np.ndarray:
    """The 16 NF4 levels in float64, ascending (QLoRA construction, see module docstring)."""
    pos = [quantile(float(p)) for p in np.linspace(DELTA, 0.5, 9)[:-1]]
    neg = [-quantile(float(p)) for p in np.linspace(DELTA, 0.5, 8)[:-1]]
    vals = sorted(pos + [0.0] + neg)
    top = max(abs(v) for v in vals)
    return np.array([v / top for v in vals], dtype=np.float64)


def codebook() -> np.ndarray:
    """The 16 levels rounded to float32 (nearest-even)."""
    return nf4_levels_f64().astype(np.float32)


_CODEBOOK = codebook()


# ------------------------------------------------------------------------------- bf16 helpers
def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even. Finite inputs."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    return ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ------------------------------------------------------------------------------- quantisation
@dataclasses.dataclass
class NF4Weight:
    n: int
    k: int
    dq_block: int                       # 0 or the double-quant run length (256)
    codes: np.ndarray                   # uint8 [n*k/2], packed
    absmax: np.ndarray                  # float32 [n*k/64] (dq_block == 0) or int8 [n*k/64]
    scale: Optional[np.ndarray] = None  # float32 [ceil(n*k/64 / dq_block)] when dq_block > 0


def block_absmax(w: np.ndarray) -> np.ndarray:
    """max |w| over each run of 64 consecutive elements of the flattened float32 weight."""
    w = np.asarray(w, dtype=np.float32).reshape(-1, BLOCK)
    return np.abs(w).max(axis=1)


def encode_numpy(w: np.ndarray, absmax: np.ndarray, chunk: int = 1 << 20) -> np.ndarray:
    """4-bit codes (uint8, one per element) of the flattened float32 weight against absmax."""
    w = np.asarray(w, dtype=np.float32).reshape(-1)
    a = np.repeat(np.asarray(absmax, dtype=np.float32), BLOCK)
    levels = _CODEBOOK.astype(np.float64)
    out = np.empty(w.size, dtype=np.uint8)
    for lo in range(0, w.size, chunk):
        wi, ai = w[lo:lo + chunk], a[lo:lo + chunk]
        zero = ai == 0
        with np.errstate(invalid="ignore", divide="ignore"):
            v = (wi / np.where(zero, np.float32(1), ai)).astype(np.float32)   # fl32(w / a)
        dist = np.abs(v.astype(np.float64)[:, None] - levels[None, :])     # exact in float64
        code = np.argmin(dist, axis=1)                                       # first = lower on ties
        code[zero] = 7
        out[lo:lo + chunk] = code
    return out


_HERE = os.path.dirname(os.path.abspath(__file__))
_C_SRC = os.path.join(_HERE, "nf4_encode.c")
_C_LIB = os.path.join(_HERE, "libnf4oracle.so")
_c = None


def build_c() -> str:
    """Compile the C twin of the encoder (plain loop, gcc -O2 -fopenmp, no fast-math)."""
    tmp = _C_LIB + ".tmp"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", _C_SRC, "-o", tmp, "-lm"],
                   check=True)
    os.replace(tmp, _C_LIB)
    return _C_LIB


def _c_lib():
    global _c
    if _c is None:
        if not os.path.exists(_C_LIB) or os.path.getmtime(_C_LIB) < os.path.getmtime(_C_SRC):
            build_c()
        lib = ctypes.CDLL(_C_LIB)
        lib.oracle_nf4_encode.restype = None
        lib.oracle_nf4_encode.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_void_p]
        _c = lib
    return _c


def encode_c(w: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """The same definition as encode_numpy, as a C loop (oracle/nf4_encode.c)."""
    w = np.ascontiguousarray(w, dtype=np.float32).reshape(-1)
    a = np.ascontiguousarray(absmax, dtype=np.float32).reshape(-1)
    if a.size * BLOCK != w.size:
        raise ValueError("absmax must hold one value per 64 elements")
    lv = np.ascontiguousarray(_CODEBOOK, dtype=np.float32)
    out = np.empty(w.size, dtype=np.uint8)
    _c_lib().oracle_nf4_encode(w.ctypes.data, a.ctypes.data, w.size, lv.ctypes.data,
                               out.ctypes.data)
    return out


def encode(w: np.ndarray, absmax: np.ndarray) -> np.ndarray:
    """4-bit codes of the flattened float32 weight: the C loop for large inputs, numpy else."""
    w = np.asarray(w, dtype=np.float32)
    if w.size >= (1 << 16):
        return encode_c(w, absmax)
    return encode_numpy(w, absmax)


def pack(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).reshape(-1)
    return ((c[0::2] << 4) | c[1::2]).astype(np.uint8)


def unpack(packed: np.ndarray) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8).reshape(-1)
    out = np.empty(p.size * 2, dtype=np.uint8)
    out[0::2] = p >> 4
    out[1::2] = p & 0x0F
    return out


def double_quant(absmax: np.ndarray, dq_block: int):
    """(int8 q [len], float32 S [runs]) for runs of dq_block consecutive absmax values."""
    a = np.asarray(absmax, dtype=np.float32).reshape(-1)
    runs = (a.size + dq_block - 1) // dq_block
    q = np.zeros(a.size, dtype=np.int8)
    S = np.zeros(runs, dtype=np.float32)
    for j in range(runs):
        seg = a[j * dq_block:(j + 1) * dq_block]
        s = np.float32(seg.max() / np.float32(127))
        S[j] = s
        if s == 0:
            continue
        ratio = (seg / s).astype(np.float32)
        q[j * dq_block:(j + 1) * dq_block] = np.clip(np.rint(ratio), 0, 127).astype(np.int8)
    return q, S


def decode_absmax(wq: NF4Weight) -> np.ndarray:
    """The float32 absmax each block is dequantised with: a itself, or fl32(q * S)."""
    if wq.dq_block == 0:
        return np.asarray(wq.absmax, dtype=np.float32)
    q = np.asarray(wq.absmax, dtype=np.int8).astype(np.float32)
    S = np.repeat(wq.scale, wq.dq_block)[: q.size]
    return (q * S).astype(np.float32)


def quantize(w: np.ndarray, dq_block: int = 0) -> NF4Weight:
    """Quantise a float32 weight [n, k] (k a multiple of 64) to NF4."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % BLOCK:
        raise ValueError("k must be a multiple of 64")
    a = block_absmax(w)
    codes = pack(encode(w, a))
    if dq_block == 0:
        return NF4Weight(n, k, 0, codes, a)
    q, S = double_quant(a, dq_block)
    return NF4Weight(n, k, dq_block, codes, q, S)


def dequantize_f32(wq: NF4Weight) -> np.ndarray:
    """w' = fl32(level[code] * a') as float32 [n, k]."""
    c = _CODEBOOK[unpack(wq.codes)]
    a = np.repeat(decode_absmax(wq), BLOCK)
    return (c * a).astype(np.float32).reshape(wq.n, wq.k)


def dequantize_bf16(wq: NF4Weight) -> np.ndarray:
    """bf16 bit patterns (uint16 [n, k]) of the dequantised weight."""
    return bf16_bits(dequantize_f32(wq))
