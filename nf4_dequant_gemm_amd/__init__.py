"""Python binding of libnf4qlora, the fused NF4 QLoRA linear layer for MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of the C-ABI library
(include/nf4qlora.h). torch provides device memory and the current stream. There is no CPU or
torch fallback: if the library is not built, every call raises.

    q = nf4_quantize(W_bf16, dq_block=256)          # NF4Tensor (frozen base weight)
    Y, T = qlora_fwd(X, q, A, B, s)                  # Y = X deq(W)^T + s (X A^T) B^T
    dX, dA, dB = qlora_bwd(dY, X, q, A, B, s, T)
    Y = QLoRALinearFunction.apply(X, q, A, B, s)     # autograd: gradients for X, A, B
    qgu = nf4_quantize(torch.cat([Wg, Wu]))           # gate/up pair, stacked [2n, k]
    H, Ygu, Tgu = qlora_swiglu_fwd(X, qgu, Agu, Bg, Bu, s)   # H = silu(Yg) * Yu
    dX, dAgu, dBg, dBu = qlora_swiglu_bwd(dH, X, qgu, Agu, Bg, Bu, s, Ygu, Tgu)
    W_merged = qlora_merge(q, A, B, s)                # bf16 deq(W) + s B A (requantize=256: NF4)
    Y, T = qlora_moe_fwd(X, counts, qe, Ae, Be, s)    # experts: rows grouped, tensors stacked
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Tuple

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libnf4qlora.so")
_lib = None

NF4_OK, NF4_EINVAL, NF4_EUNSUPPORTED, NF4_EHIP = 0, -1, -2, -3
NF4_BF16, NF4_F32 = 0, 1

EXPORTED = ("nf4_quantize", "nf4_dequantize", "nf4_codebook", "qlora_fwd_workspace_bytes",
            "qlora_fwd", "qlora_lora_down", "qlora_fwd_fused", "qlora_bwd_workspace_bytes",
            "qlora_bwd", "qlora_bwd_dx", "qlora_swiglu_workspace_bytes", "qlora_swiglu_fwd",
            "qlora_swiglu_fwd_fused",
            "qlora_swiglu_bwd", "qlora_merge", "qlora_moe_workspace_bytes", "qlora_moe_fwd",
            "qlora_moe_fwd_fused", "qlora_moe_bwd", "qlora_moe_workspace_bytes_dev", "qlora_moe_fwd_dev",
            "qlora_moe_bwd_dev", "qlora_fwd_noalloc", "nf4_last_error")


class NF4Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"status {status}: {msg}")
        self.status = status


class _NF4TensorC(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("k", ctypes.c_int64), ("block", ctypes.c_int32),
                ("dq_block", ctypes.c_int32), ("codes", ctypes.c_void_p),
                ("absmax", ctypes.c_void_p), ("absmax_scale", ctypes.c_void_p)]


def library() -> ctypes.CDLL:
    """Load libnf4qlora.so (built by nf4_dequant_gemm_amd.build); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run python -m nf4_dequant_gemm_amd.build")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, i32, f32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    P = ctypes.POINTER(_NF4TensorC)
    sig = {
        "nf4_quantize": (ctypes.c_int, [vp, ctypes.c_int, P, vp]),
        "nf4_dequantize": (ctypes.c_int, [P, vp, ctypes.c_int, vp]),
        "nf4_codebook": (ctypes.c_int, [ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float)]),
        "qlora_fwd_workspace_bytes": (sz, [i64, i64, i64, i32]),
        "qlora_fwd": (ctypes.c_int, [vp, i64, P, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "qlora_fwd_noalloc": (ctypes.c_int, [vp, i64, P, vp, vp, i32, f32, vp, vp, vp]),
        "qlora_lora_down": (ctypes.c_int, [vp, i64, i64, vp, i32, vp, vp, sz, vp]),
        "qlora_fwd_fused": (ctypes.c_int, [vp, i64, P, vp, vp, i32, f32, vp, vp]),
        "qlora_bwd_workspace_bytes": (sz, [i64, i64, i64, i32]),
        "qlora_bwd": (ctypes.c_int, [vp, vp, i64, P, vp, vp, i32, f32, vp, vp, vp, vp, vp, sz, vp]),
        "qlora_bwd_dx": (ctypes.c_int, [vp, i64, P, vp, vp, i32, f32, vp, vp]),
        "qlora_merge": (ctypes.c_int, [P, vp, vp, i32, f32, vp, vp]),
        "qlora_moe_workspace_bytes": (sz, [vp, i32, i64, i64, i32]),
        "qlora_moe_fwd": (ctypes.c_int, [vp, vp, i32, P, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "qlora_moe_fwd_fused": (ctypes.c_int, [vp, vp, i32, P, vp, vp, i32, f32, vp, vp]),
        "qlora_moe_bwd": (ctypes.c_int, [vp, vp, vp, i32, P, vp, vp, i32, f32, vp, vp, vp, vp, vp, sz, vp]),
        "qlora_moe_workspace_bytes_dev": (sz, [i64, i32, i64, i64, i32]),
        "qlora_moe_fwd_dev": (ctypes.c_int, [vp, i64, vp, i32, P, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "qlora_moe_bwd_dev": (ctypes.c_int, [vp, vp, i64, vp, i32, P, vp, vp, i32, f32, vp, vp, vp, vp, vp,
                                             sz, vp]),
        "qlora_swiglu_workspace_bytes": (sz, [i64, i64, i64, i32]),
        "qlora_swiglu_fwd": (ctypes.c_int, [vp, i64, P, vp, vp, vp, i32, f32, vp, vp, vp, vp, sz, vp]),
        "qlora_swiglu_fwd_fused": (ctypes.c_int, [vp, i64, P, vp, vp, vp, i32, f32, vp, vp, vp]),
        "qlora_swiglu_bwd": (ctypes.c_int, [vp, vp, i64, P, vp, vp, vp, i32, f32, vp, vp, vp, vp, vp, vp,
                                            vp, sz, vp]),
        "nf4_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != NF4_OK:
        raise NF4Error(status, library().nf4_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")


@dataclasses.dataclass
class NF4Tensor:
    """A 4-bit quantised weight [n, k]: packed codes, block constants and their scales.

    block 64 (NF4): absmax float32 [n*k/64] (dq_block 0) or int8 [n*k/64] with float32 run
    scales [ceil(n*k/64/256)] (dq_block 256). block 16 (E2M1): absmax holds the uint8 E4M3 group
    scales [n*k/16] and scale the float32 tensor scale [1]."""
    n: int
    k: int
    dq_block: int
    codes: torch.Tensor                   # uint8 [n*k/2]
    absmax: torch.Tensor                  # block constants (see above)
    scale: Optional[torch.Tensor] = None  # run scales or the tensor scale (see above)
    block: int = 64

    @property
    def device(self) -> torch.device:
        return self.codes.device

    def c_struct(self) -> _NF4TensorC:
        return _NF4TensorC(self.n, self.k, self.block, self.dq_block, self.codes.data_ptr(),
                           self.absmax.data_ptr(),
                           self.scale.data_ptr() if self.scale is not None else None)

    def clone(self) -> "NF4Tensor":
        """A copy in new device buffers (same values, different addresses)."""
        return NF4Tensor(self.n, self.k, self.dq_block, self.codes.clone(), self.absmax.clone(),
                         self.scale.clone() if self.scale is not None else None, self.block)

    @staticmethod
    def empty(n: int, k: int, dq_block: int, device) -> "NF4Tensor":
        nblk = n * k // 64
        codes = torch.empty(n * k // 2, dtype=torch.uint8, device=device)
        if dq_block:
            absmax = torch.empty(nblk, dtype=torch.int8, device=device)
            scale = torch.empty((nblk + dq_block - 1) // dq_block, dtype=torch.float32, device=device)
        else:
            absmax = torch.empty(nblk, dtype=torch.float32, device=device)
            scale = None
        return NF4Tensor(n, k, dq_block, codes, absmax, scale)


def nf4_codebook():
    """(levels[16], thresholds[15]) as float lists, read from the library (host only)."""
    lv = (ctypes.c_float * 16)()
    th = (ctypes.c_float * 15)()
    _check(library().nf4_codebook(lv, th))
    return list(lv), list(th)


def nf4_quantize(w: torch.Tensor, dq_block: int = 256) -> NF4Tensor:
    """Quantise a bf16 or float32 device weight [n, k] to NF4 (blocks of 64)."""
    if w.dim() != 2:
        raise ValueError("w must be 2-D [n, k]")
    if w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("w must be bfloat16 or float32")
    _need(w, "w", w.dtype)
    n, k = w.shape
    if k % 64:
        raise NF4Error(NF4_EUNSUPPORTED, "k must be a multiple of 64")
    q = NF4Tensor.empty(n, k, dq_block, w.device)
    st = q.c_struct()
    _check(library().nf4_quantize(_ptr(w), NF4_F32 if w.dtype == torch.float32 else NF4_BF16,
                                  ctypes.byref(st), _stream(w.device)))
    return q


def fp4_quantize(w: torch.Tensor) -> NF4Tensor:
    """Quantise a bf16 or float32 device weight [n, k] to the E2M1 format: 4-bit floats in groups
    of 16 with one E4M3 scale each and a float32 tensor scale (block 16 of the descriptor)."""
    if w.dim() != 2:
        raise ValueError("w must be 2-D [n, k]")
    if w.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("w must be bfloat16 or float32")
    _need(w, "w", w.dtype)
    n, k = w.shape
    if k % 64:
        raise NF4Error(NF4_EUNSUPPORTED, "k must be a multiple of 64")
    dev = w.device
    q = NF4Tensor(n, k, 0, torch.empty(n * k // 2, dtype=torch.uint8, device=dev),
                  torch.empty(n * k // 16, dtype=torch.uint8, device=dev),
                  torch.empty(4, dtype=torch.float32, device=dev), block=16)
    st = q.c_struct()
    _check(library().nf4_quantize(_ptr(w), NF4_F32 if w.dtype == torch.float32 else NF4_BF16,
                                  ctypes.byref(st), _stream(dev)))
    return q


def nf4_dequantize(q: NF4Tensor, dtype=torch.bfloat16) -> torch.Tensor:
    """deq(W) [n, k] as bfloat16 (rounded) or float32 (exact)."""
    if dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("dtype must be bfloat16 or float32")
    out = torch.empty(q.n, q.k, dtype=dtype, device=q.device)
    st = q.c_struct()
    _check(library().nf4_dequantize(ctypes.byref(st), _ptr(out),
                                    NF4_F32 if dtype == torch.float32 else NF4_BF16,
                                    _stream(q.device)))
    return out


def qlora_fwd(X: torch.Tensor, q: NF4Tensor, A: Optional[torch.Tensor], B: Optional[torch.Tensor],
              s: float) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """(Y, T): Y = X deq(W)^T + s T B^T with T = X A^T (T is None when r == 0)."""
    m = X.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(X, "X", torch.bfloat16, (m, q.k))
    if r:
        _need(A, "A", torch.bfloat16, (r, q.k))
        _need(B, "B", torch.bfloat16, (q.n, r))
    Y = torch.empty(m, q.n, dtype=torch.bfloat16, device=X.device)
    T = torch.empty(m, r, dtype=torch.bfloat16, device=X.device) if r else None
    lib = library()
    wsb = lib.qlora_fwd_workspace_bytes(m, q.n, q.k, r)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=X.device)
    st = q.c_struct()
    _check(lib.qlora_fwd(_ptr(X), m, ctypes.byref(st), _ptr(A), _ptr(B), r, float(s), _ptr(Y),
                         _ptr(T), _ptr(ws), wsb, _stream(X.device)))
    return Y, T


NOALLOC_SCRATCH_BYTES = 16 << 20   # NF4_NOALLOC_SCRATCH_BYTES of the header


def qlora_fwd_noalloc(X: torch.Tensor, q: NF4Tensor, A: Optional[torch.Tensor], B: Optional[torch.Tensor],
                      s: float, Y: torch.Tensor, T: Optional[torch.Tensor] = None) -> None:
    """qlora_fwd into caller-provided Y [m, n] and T [m, r] with no workspace: the library's
    static per-GPU scratch array holds the partial sums (calls on one GPU must not overlap)."""
    m = X.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(X, "X", torch.bfloat16, (m, q.k))
    _need(Y, "Y", torch.bfloat16, (m, q.n))
    if r:
        _need(A, "A", torch.bfloat16, (r, q.k))
        _need(B, "B", torch.bfloat16, (q.n, r))
        _need(T, "T", torch.bfloat16, (m, r))
    st = q.c_struct()
    _check(library().qlora_fwd_noalloc(_ptr(X), m, ctypes.byref(st), _ptr(A), _ptr(B), r, float(s),
                                       _ptr(Y), _ptr(T), _stream(X.device)))


def qlora_lora_down(X: torch.Tensor, A: torch.Tensor) -> torch.Tensor:
    """T = X A^T (bf16 [m, r])."""
    m, k = X.shape
    r = A.shape[0]
    _need(X, "X", torch.bfloat16, (m, k))
    _need(A, "A", torch.bfloat16, (r, k))
    T = torch.empty(m, r, dtype=torch.bfloat16, device=X.device)
    lib = library()
    wsb = lib.qlora_fwd_workspace_bytes(m, 0, k, r)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=X.device)
    _check(lib.qlora_lora_down(_ptr(X), m, k, _ptr(A), r, _ptr(T), _ptr(ws), wsb, _stream(X.device)))
    return T


def qlora_fwd_fused(X: torch.Tensor, q: NF4Tensor, T: Optional[torch.Tensor],
                    B: Optional[torch.Tensor], s: float) -> torch.Tensor:
    """Y = X deq(W)^T + s T B^T in one kernel launch, given T = X A^T."""
    m = X.shape[0]
    r = 0 if T is None else T.shape[1]
    _need(X, "X", torch.bfloat16, (m, q.k))
    if r:
        _need(T, "T", torch.bfloat16, (m, r))
        _need(B, "B", torch.bfloat16, (q.n, r))
    Y = torch.empty(m, q.n, dtype=torch.bfloat16, device=X.device)
    st = q.c_struct()
    _check(library().qlora_fwd_fused(_ptr(X), m, ctypes.byref(st), _ptr(T), _ptr(B), r, float(s),
                                     _ptr(Y), _stream(X.device)))
    return Y


def qlora_bwd(dY: torch.Tensor, X: torch.Tensor, q: NF4Tensor, A: Optional[torch.Tensor],
              B: Optional[torch.Tensor], s: float, T: Optional[torch.Tensor], need_dx: bool = True):
    """(dX, dA, dB) of the layer; dX is None when need_dx is False, dA/dB None when r == 0."""
    m = X.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(dY, "dY", torch.bfloat16, (m, q.n))
    _need(X, "X", torch.bfloat16, (m, q.k))
    if r:
        _need(A, "A", torch.bfloat16, (r, q.k))
        _need(B, "B", torch.bfloat16, (q.n, r))
        if T is not None:                 # None: the library recomputes T = X A^T
            _need(T, "T", torch.bfloat16, (m, r))
    dev = X.device
    dX = torch.empty(m, q.k, dtype=torch.bfloat16, device=dev) if need_dx else None
    dA = torch.empty(r, q.k, dtype=torch.bfloat16, device=dev) if r else None
    dB = torch.empty(q.n, r, dtype=torch.bfloat16, device=dev) if r else None
    lib = library()
    wsb = lib.qlora_bwd_workspace_bytes(m, q.n, q.k, r)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = q.c_struct()
    _check(lib.qlora_bwd(_ptr(dY), _ptr(X), m, ctypes.byref(st), _ptr(A), _ptr(B), r, float(s),
                         _ptr(T), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), wsb, _stream(dev)))
    return dX, dA, dB


def qlora_bwd_dx(dY: torch.Tensor, q: NF4Tensor, U: Optional[torch.Tensor], A: Optional[torch.Tensor],
                 s: float) -> torch.Tensor:
    """dX = bf16(dY deq(W) + s U A) in one launch; U = dY B as qlora_bwd computes it."""
    m = dY.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(dY, "dY", torch.bfloat16, (m, q.n))
    if r:
        _need(U, "U", torch.bfloat16, (m, r))
        _need(A, "A", torch.bfloat16, (r, q.k))
    dX = torch.empty(m, q.k, dtype=torch.bfloat16, device=dY.device)
    st = q.c_struct()
    _check(library().qlora_bwd_dx(_ptr(dY), m, ctypes.byref(st), _ptr(U), _ptr(A), r, float(s),
                                  _ptr(dX), _stream(dY.device)))
    return dX


def qlora_merge(q: NF4Tensor, A: Optional[torch.Tensor], B: Optional[torch.Tensor], s: float,
                requantize=None):
    """W' = bf16(deq(W) + s B A) [n, k] (NF4 or E2M1 base); with requantize = a dq_block (0, 256),
    nf4_quantize(W') instead, with requantize = "e2m1", fp4_quantize(W')."""
    r = 0 if A is None else A.shape[0]
    if r:
        _need(A, "A", torch.bfloat16, (r, q.k))
        _need(B, "B", torch.bfloat16, (q.n, r))
    out = torch.empty(q.n, q.k, dtype=torch.bfloat16, device=q.device)
    st = q.c_struct()
    _check(library().qlora_merge(ctypes.byref(st), _ptr(A), _ptr(B), r, float(s), _ptr(out),
                                 _stream(q.device)))
    if requantize is None:
        return out
    if requantize == "e2m1":
        return fp4_quantize(out)
    return nf4_quantize(out, requantize)


def _moe_args(X, counts, q: NF4Tensor, A, B):
    E = len(counts)
    if E < 1 or q.n % E:
        raise ValueError("the stacked weight must hold E*n rows for E = len(counts) experts")
    n = q.n // E
    r = 0 if A is None else A.shape[0] // E
    M = int(sum(counts))
    _need(X, "X", torch.bfloat16, (M, q.k))
    if r:
        _need(A, "A", torch.bfloat16, (E * r, q.k))
        _need(B, "B", torch.bfloat16, (E * n, r))
    c = (ctypes.c_int64 * E)(*[int(x) for x in counts])
    return E, n, r, M, c


def qlora_moe_fwd(X: torch.Tensor, counts, q: NF4Tensor, A: Optional[torch.Tensor],
                  B: Optional[torch.Tensor], s: float):
    """(Y, T) of the grouped layer: rows of X grouped by expert (counts[e] rows for expert e), q the
    stacked NF4 weight [E*n, k], A [E*r, k], B [E*n, r]; T is None when r == 0."""
    E, n, r, M, c = _moe_args(X, counts, q, A, B)
    dev = X.device
    Y = torch.empty(M, n, dtype=torch.bfloat16, device=dev)
    T = torch.empty(M, r, dtype=torch.bfloat16, device=dev) if r else None
    lib = library()
    wsb = lib.qlora_moe_workspace_bytes(c, E, n, q.k, r)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = q.c_struct()
    _check(lib.qlora_moe_fwd(_ptr(X), c, E, ctypes.byref(st), _ptr(A), _ptr(B), r, float(s), _ptr(Y),
                             _ptr(T), _ptr(ws), wsb, _stream(dev)))
    return Y, T


def qlora_moe_fwd_fused(X: torch.Tensor, counts, q: NF4Tensor, T: Optional[torch.Tensor],
                        B: Optional[torch.Tensor], s: float) -> torch.Tensor:
    """Y of the grouped layer in one launch, given T (the experts' X_e A_e^T, rows grouped)."""
    E = len(counts)
    if E < 1 or q.n % E:
        raise ValueError("the stacked weight must hold E*n rows for E = len(counts) experts")
    n, M = q.n // E, int(sum(counts))
    r = 0 if T is None else T.shape[1]
    _need(X, "X", torch.bfloat16, (M, q.k))
    if r:
        _need(T, "T", torch.bfloat16, (M, r))
        _need(B, "B", torch.bfloat16, (E * n, r))
    c = (ctypes.c_int64 * E)(*[int(x) for x in counts])
    Y = torch.empty(M, n, dtype=torch.bfloat16, device=X.device)
    st = q.c_struct()
    _check(library().qlora_moe_fwd_fused(_ptr(X), c, E, ctypes.byref(st), _ptr(T), _ptr(B), r, float(s),
                                         _ptr(Y), _stream(X.device)))
    return Y


def qlora_moe_bwd(dY: torch.Tensor, X: torch.Tensor, counts, q: NF4Tensor, A: Optional[torch.Tensor],
                  B: Optional[torch.Tensor], s: float, T: Optional[torch.Tensor], need_dx: bool = True):
    """(dX, dA, dB) of the grouped layer; dA [E*r, k], dB [E*n, r] (None when r == 0)."""
    E, n, r, M, c = _moe_args(X, counts, q, A, B)
    _need(dY, "dY", torch.bfloat16, (M, n))
    if r and T is not None:
        _need(T, "T", torch.bfloat16, (M, r))
    dev = X.device
    dX = torch.empty(M, q.k, dtype=torch.bfloat16, device=dev) if need_dx else None
    dA = torch.empty(E * r, q.k, dtype=torch.bfloat16, device=dev) if r else None
    dB = torch.empty(E * n, r, dtype=torch.bfloat16, device=dev) if r else None
    lib = library()
    wsb = lib.qlora_moe_workspace_bytes(c, E, n, q.k, r)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = q.c_struct()
    _check(lib.qlora_moe_bwd(_ptr(dY), _ptr(X), c, E, ctypes.byref(st), _ptr(A), _ptr(B), r, float(s),
                             _ptr(T), _ptr(dX), _ptr(dA), _ptr(dB), _ptr(ws), wsb, _stream(dev)))
    return dX, dA, dB


def moe_workspace_bytes_dev(m: int, E: int, n: int, k: int, r: int) -> int:
    """Workspace bytes of the device-routed grouped calls for m routed rows."""
    return int(library().qlora_moe_workspace_bytes_dev(m, E, n, k, r))


def qlora_moe_fwd_dev(X: torch.Tensor, counts: torch.Tensor, q: NF4Tensor, A: Optional[torch.Tensor],
                      B: Optional[torch.Tensor], s: float, Y: torch.Tensor, T: Optional[torch.Tensor],
                      ws: torch.Tensor) -> None:
    """The grouped forward with the routing on the device: counts int64 [E] device tensor; Y, T
    and the workspace ws (moe_workspace_bytes_dev bytes) are the caller's, so the call allocates
    nothing and can be captured in a graph."""
    E = counts.numel()
    if counts.dtype != torch.int64 or not counts.is_cuda or not counts.is_contiguous():
        raise ValueError("counts must be a contiguous int64 device tensor")
    if E < 1 or q.n % E:
        raise ValueError("the stacked weight must hold E*n rows for E = counts.numel() experts")
    M, n = X.shape[0], q.n // E
    r = 0 if A is None else A.shape[0] // E
    _need(X, "X", torch.bfloat16, (M, q.k))
    _need(Y, "Y", torch.bfloat16, (M, n))
    if r:
        _need(A, "A", torch.bfloat16, (E * r, q.k))
        _need(B, "B", torch.bfloat16, (E * n, r))
        _need(T, "T", torch.bfloat16, (M, r))
    st = q.c_struct()
    _check(library().qlora_moe_fwd_dev(_ptr(X), M, _ptr(counts), E, ctypes.byref(st), _ptr(A), _ptr(B), r,
                                       float(s), _ptr(Y), _ptr(T), _ptr(ws), ws.numel(), _stream(X.device)))


def qlora_moe_bwd_dev(dY: torch.Tensor, X: torch.Tensor, counts: torch.Tensor, q: NF4Tensor,
                      A: Optional[torch.Tensor], B: Optional[torch.Tensor], s: float,
                      T: Optional[torch.Tensor], dX: Optional[torch.Tensor], dA: Optional[torch.Tensor],
                      dB: Optional[torch.Tensor], ws: torch.Tensor) -> None:
    """The grouped backward with the routing on the device, into the caller's dX, dA, dB."""
    E = counts.numel()
    if counts.dtype != torch.int64 or not counts.is_cuda or not counts.is_contiguous():
        raise ValueError("counts must be a contiguous int64 device tensor")
    M, n = X.shape[0], q.n // E
    r = 0 if A is None else A.shape[0] // E
    _need(dY, "dY", torch.bfloat16, (M, n))
    st = q.c_struct()
    _check(library().qlora_moe_bwd_dev(_ptr(dY), _ptr(X), M, _ptr(counts), E, ctypes.byref(st), _ptr(A),
                                       _ptr(B), r, float(s), _ptr(T), _ptr(dX), _ptr(dA), _ptr(dB),
                                       _ptr(ws), ws.numel(), _stream(X.device)))


def _swiglu_args(X, q: NF4Tensor, Agu, Bg, Bu):
    if q.n % 2:
        raise ValueError("the gate/up weight must hold 2n rows (gate rows, then up rows)")
    m, n = X.shape[0], q.n // 2
    r = 0 if Agu is None else Agu.shape[0] // 2
    _need(X, "X", torch.bfloat16, (m, q.k))
    if r:
        _need(Agu, "Agu", torch.bfloat16, (2 * r, q.k))
        _need(Bg, "Bg", torch.bfloat16, (n, r))
        _need(Bu, "Bu", torch.bfloat16, (n, r))
    return m, n, r


def qlora_swiglu_fwd(X: torch.Tensor, q: NF4Tensor, Agu: Optional[torch.Tensor],
                     Bg: Optional[torch.Tensor], Bu: Optional[torch.Tensor], s: float):
    """(H, Ygu, Tgu) of the gate/up pair: q is the stacked NF4 weight [Wg; Wu] [2n, k], Agu the
    stacked [Ag; Au] [2r, k]; H = silu(Yg) * Yu [m, n], Ygu = [Yg | Yu] [m, 2n], Tgu [m, 2r]."""
    m, n, r = _swiglu_args(X, q, Agu, Bg, Bu)
    dev = X.device
    H = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    Ygu = torch.empty(m, 2 * n, dtype=torch.bfloat16, device=dev)
    Tgu = torch.empty(m, 2 * r, dtype=torch.bfloat16, device=dev) if r else None
    lib = library()
    wsb = lib.qlora_swiglu_workspace_bytes(m, n, q.k, r)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = q.c_struct()
    _check(lib.qlora_swiglu_fwd(_ptr(X), m, ctypes.byref(st), _ptr(Agu), _ptr(Bg), _ptr(Bu), r,
                                float(s), _ptr(H), _ptr(Ygu), _ptr(Tgu), _ptr(ws), wsb,
                                _stream(dev)))
    return H, Ygu, Tgu


def qlora_swiglu_fwd_fused(X: torch.Tensor, q: NF4Tensor, Tgu: Optional[torch.Tensor],
                           Bg: Optional[torch.Tensor], Bu: Optional[torch.Tensor], s: float):
    """(H, Ygu) of the gate/up pair in one kernel launch, given Tgu = [X Ag^T | X Au^T] [m, 2r]."""
    m = X.shape[0]
    if q.n % 2:
        raise ValueError(f"the stacked weight must have an even number of rows (got {q.n})")
    n = q.n // 2
    r = 0 if Tgu is None else Tgu.shape[1] // 2
    _need(X, "X", torch.bfloat16, (m, q.k))
    if r:
        _need(Tgu, "Tgu", torch.bfloat16, (m, 2 * r))
        _need(Bg, "Bg", torch.bfloat16, (n, r))
        _need(Bu, "Bu", torch.bfloat16, (n, r))
    dev = X.device
    H = torch.empty(m, n, dtype=torch.bfloat16, device=dev)
    Ygu = torch.empty(m, 2 * n, dtype=torch.bfloat16, device=dev)
    st = q.c_struct()
    _check(library().qlora_swiglu_fwd_fused(_ptr(X), m, ctypes.byref(st), _ptr(Tgu if r else None),
                                            _ptr(Bg if r else None), _ptr(Bu if r else None), r,
                                            float(s), _ptr(H), _ptr(Ygu), _stream(dev)))
    return H, Ygu


def qlora_swiglu_bwd(dH: torch.Tensor, X: torch.Tensor, q: NF4Tensor, Agu: Optional[torch.Tensor],
                     Bg: Optional[torch.Tensor], Bu: Optional[torch.Tensor], s: float,
                     Ygu: torch.Tensor, Tgu: Optional[torch.Tensor], need_dx: bool = True):
    """(dX, dAgu, dBg, dBu) of the gate/up pair for the upstream gradient dH [m, n]."""
    m, n, r = _swiglu_args(X, q, Agu, Bg, Bu)
    _need(dH, "dH", torch.bfloat16, (m, n))
    _need(Ygu, "Ygu", torch.bfloat16, (m, 2 * n))
    if r and Tgu is not None:
        _need(Tgu, "Tgu", torch.bfloat16, (m, 2 * r))
    dev = X.device
    dX = torch.empty(m, q.k, dtype=torch.bfloat16, device=dev) if need_dx else None
    dAgu = torch.empty(2 * r, q.k, dtype=torch.bfloat16, device=dev) if r else None
    dBg = torch.empty(n, r, dtype=torch.bfloat16, device=dev) if r else None
    dBu = torch.empty(n, r, dtype=torch.bfloat16, device=dev) if r else None
    lib = library()
    wsb = lib.qlora_swiglu_workspace_bytes(m, n, q.k, r)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)
    st = q.c_struct()
    _check(lib.qlora_swiglu_bwd(_ptr(dH), _ptr(X), m, ctypes.byref(st), _ptr(Agu), _ptr(Bg),
                                _ptr(Bu), r, float(s), _ptr(Ygu), _ptr(Tgu if r else None),
                                _ptr(dX), _ptr(dAgu), _ptr(dBg), _ptr(dBu), _ptr(ws), wsb,
                                _stream(dev)))
    return dX, dAgu, dBg, dBu


class QLoRALinearFunction(torch.autograd.Function):
    """Y = X deq(W)^T + s (X A^T) B^T with W frozen; gradients flow to X, A and B."""

    @staticmethod
    def forward(ctx, X, q: NF4Tensor, A, B, s: float):
        Y, T = qlora_fwd(X, q, A, B, s)
        ctx.q, ctx.s = q, s
        ctx.save_for_backward(X, A, B, T)
        return Y

    @staticmethod
    def backward(ctx, dY):
        X, A, B, T = ctx.saved_tensors
        dX, dA, dB = qlora_bwd(dY.contiguous(), X, ctx.q, A, B, ctx.s, T,
                               need_dx=ctx.needs_input_grad[0])
        return dX, None, dA, dB, None


class QLoRASwiGLUFunction(torch.autograd.Function):
    """H = silu(X deq(Wg)^T + s (X Ag^T) Bg^T) * (X deq(Wu)^T + s (X Au^T) Bu^T) with the bases frozen
    (q = stacked NF4 [Wg; Wu]); gradients flow to X, Agu = [Ag; Au], Bg and Bu."""

    @staticmethod
    def forward(ctx, X, q: NF4Tensor, Agu, Bg, Bu, s: float):
        H, Ygu, Tgu = qlora_swiglu_fwd(X, q, Agu, Bg, Bu, s)
        ctx.q, ctx.s = q, s
        ctx.save_for_backward(X, Agu, Bg, Bu, Ygu, Tgu)
        return H

    @staticmethod
    def backward(ctx, dH):
        X, Agu, Bg, Bu, Ygu, Tgu = ctx.saved_tensors
        dX, dAgu, dBg, dBu = qlora_swiglu_bwd(dH.contiguous(), X, ctx.q, Agu, Bg, Bu, ctx.s, Ygu, Tgu,
                                              need_dx=ctx.needs_input_grad[0])
        return dX, None, dAgu, dBg, dBu, None
