"""Bit-exact probes of the dequantisation inside every fused GEMM path, at every pipeline phase.

With one nonzero product per output (X or dY a row of the identity), the float32 sums of a GEMM
are exact, so the output shows the kernel's weight operand bit for bit:

* the large-M forward and dX kernels consume bf16(fl32(level * a')) (the layer's definition):
  X = I_K gives Y = bf16(deq(W))^T and dY = I_N gives dX = bf16(deq(W)), for both block-constant
  formats and for step counts of either parity, one step, and a ragged last step of dX;
* the decode-shaped kernels (at most 48 rows) multiply the bf16-rounded level by X and scale the
  float32 block partial by a': row i of X the unit vector e_k gives
  Y[i, n] = bf16(fl32(a'(n, k / 64) * bf16(level(code[n, k])))), which is the definition's
  bf16(fl32(level * a')) whenever a' is a power of two (both roundings then commute with the
  scaling). The probes run every stage count around the stream kernel's 8-stage loop and its
  4-stage code windows, and several workgroups (whose start stages are staggered), so that a
  copy that lands late (an LDS race between the DMA and its readers) changes some output's bits
  instead of hiding under the 1e-2 tolerance.

Expected values come from the oracle's quantisation (codes, a', levels) only.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from oracle import fp4, nf4
from tests.gpu_helpers import say, u16

pytestmark = pytest.mark.gpu

DEV = "cuda"


def probe_weight(n, k, dq, seed):
    """Weight whose block constants decode to powers of two: small normal values, one element per
    block of magnitude 2^e (e in {-6, -5, -4}); with double quantisation the first block of each
    run of 256 holds 127 * 2^-7, so S = 2^-7 and every other block's q is a power of two."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.002).astype(np.float32)
    nblk = n * k // 64
    b = np.arange(nblk)
    pos = b * 64 + (b * 7) % 64
    mag = 2.0 ** rng.integers(-6, -3, nblk)
    sign = np.where(rng.integers(0, 2, nblk) == 1, 1.0, -1.0)
    if dq:
        first = b % 256 == 0
        mag = np.where(first, 127 * 2.0 ** -7, mag)
    flat = w.reshape(-1)
    flat[pos] = (sign * mag).astype(np.float32)
    # bf16 storage rounds the small values; the planted block maxima are exact in bf16
    return torch.from_numpy(w).to(torch.bfloat16)


def scaled_level_probe(qo, cols):
    """bf16 bits of fl32(a'(n, k / 64) * bf16(level(code[n, k]))) for each probed column k (rows
    of the result follow cols), and whether a' is a power of two there."""
    n, k = qo.n, qo.k
    lv = nf4.codebook()
    lv_bf = nf4.bf16_value(nf4.bf16_bits(lv))
    codes = nf4.unpack(qo.codes).reshape(n, k)
    a = nf4.decode_absmax(qo).reshape(n, k // 64)
    out = np.empty((len(cols), n), np.uint16)
    pow2 = np.empty((len(cols), n), bool)
    for i, kk in enumerate(cols):
        ak = a[:, kk // 64]
        out[i] = nf4.bf16_bits((ak * lv_bf[codes[:, kk]]).astype(np.float32))
        m, _ = np.frexp(ak)
        pow2[i] = (m == 0.5) | (ak == 0)
    return out, pow2


def unit_rows(k, cols):
    X = torch.zeros(len(cols), k, dtype=torch.bfloat16)
    X[torch.arange(len(cols)), torch.as_tensor(cols)] = 1.0
    return X


def probe_columns(kblk, call, rows):
    """Row i of probe call c: a column of block (i + rows c) mod kblk, at a varying offset."""
    return [64 * ((i + rows * call) % kblk) + (37 * i + 11 * call) % 64 for i in range(rows)]


# ---------------------------------------------------------------- large-M forward and dX kernels
@pytest.mark.parametrize("K", [64, 320, 1088])
@pytest.mark.parametrize("dq", [0, 256])
def test_identity_probe_forward_steps(lib, K, dq):
    """X = I_K, r = 0: Y = bf16(deq(W))^T bit for bit (one, an odd and an even number of steps)."""
    N = 264
    say(f"forward identity probe K={K} dq={dq}")
    W = wl.normal_bf16(910 + K + dq, (N, K), 0.02)
    qg = lib.nf4_quantize(W.to(DEV), dq)
    X = torch.eye(K, dtype=torch.bfloat16, device=DEV)
    Yg, _ = lib.qlora_fwd(X, qg, None, None, 1.0)
    torch.cuda.synchronize()
    want = nf4.dequantize_bf16(nf4.quantize(W.float().numpy(), dq)).T
    assert np.array_equal(u16(Yg), want)


@pytest.mark.parametrize("N", [56, 264, 1032])
@pytest.mark.parametrize("dq", [0, 256])
def test_identity_probe_dx_steps(lib, N, dq):
    """dY = I_N, r = 0: dX = bf16(deq(W)) bit for bit through the transposed weight read, with
    double-quantised constants too; N = 56 and 264 end in a partial step, 1032 in a step of 8."""
    K = 320
    say(f"dX identity probe N={N} dq={dq}")
    W = wl.normal_bf16(920 + N + dq, (N, K), 0.02)
    qg = lib.nf4_quantize(W.to(DEV), dq)
    dY = torch.eye(N, dtype=torch.bfloat16, device=DEV)
    X = torch.zeros(N, K, dtype=torch.bfloat16, device=DEV)
    dXg, _, _ = lib.qlora_bwd(dY, X, qg, None, None, 1.0, None)
    torch.cuda.synchronize()
    want = nf4.dequantize_bf16(nf4.quantize(W.float().numpy(), dq))
    assert np.array_equal(u16(dXg), want)


# ---------------------------------------------------------------- decode-shaped kernels
# M <= 16 with double quantisation: the stream kernel (stages of 4 blocks, an 8-stage unrolled
# loop, code windows of 4 stages, staggered start stages when the stage count is a multiple of 4
# and at least 8). N = 336 is three workgroups of 112 rows; 296 leaves a ragged last workgroup.
STREAM_STAGES = [1, 2, 3, 4, 5, 7, 8, 9, 12, 15, 16, 17, 33]


def run_unit_probe(lib, qg, qo, K, rows, ncalls=None):
    kblk = K // 64
    calls = ncalls or -(-kblk // rows)
    for c in range(calls):
        cols = probe_columns(kblk, c, rows)
        Yg, _ = lib.qlora_fwd(unit_rows(K, cols).to(DEV), qg, None, None, 1.0)
        torch.cuda.synchronize()
        want, pow2 = scaled_level_probe(qo, cols)
        got = u16(Yg)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"call {c}: {len(bad)} outputs differ, first (row, n) {bad[:4].tolist()}"
        full = nf4.dequantize_bf16(qo)[:, cols].T
        assert np.array_equal(got[pow2], full[pow2]), "power-of-two a' must give bf16(deq(W))"
        assert pow2.mean() > 0.9


@pytest.mark.parametrize("nst", STREAM_STAGES)
@pytest.mark.parametrize("N", [336, 296])
def test_decode16_unit_probe(lib, nst, N):
    K = 256 * nst
    say(f"stream-kernel unit probe stages={nst} K={K} N={N}")
    W = probe_weight(N, K, 256, 930 + nst + N)
    qg = lib.nf4_quantize(W.to(DEV), 256)
    qo = nf4.quantize(W.float().numpy(), 256)
    run_unit_probe(lib, qg, qo, K, 16)


@pytest.mark.parametrize("M,dq,K", [(16, 0, 256), (16, 0, 2560), (40, 256, 768), (40, 256, 4352),
                                    (48, 0, 1280), (9, 0, 4352)])
def test_decode_unit_probe(lib, M, dq, K):
    """The other decode-shaped kernel (M <= 48 with float32 constants, 17..48 rows otherwise)."""
    N = 200
    say(f"decode-kernel unit probe M={M} dq={dq} K={K}")
    W = probe_weight(N, K, dq, 940 + M + K)
    qg = lib.nf4_quantize(W.to(DEV), dq)
    qo = nf4.quantize(W.float().numpy(), dq)
    run_unit_probe(lib, qg, qo, K, M)


@pytest.mark.parametrize("nst", [1, 2, 3, 4, 5, 7, 8, 9, 12, 17])
@pytest.mark.parametrize("N", [336, 200])
def test_decode_e2m1_unit_probe(lib, nst, N):
    """E2M1 weights on the stream kernel (M <= 16, K % 256 == 0; stages of 256 elements, a
    4-stage loop): a group's product e2m1 * s is exact in float32 and S multiplies the sum once,
    so Y = bf16(deq(W)) at any group scale (bit for bit up to the sign of zero), for every stage
    count around the loop and a ragged last workgroup (N = 200)."""
    K, M = 256 * nst, 16
    say(f"E2M1 stream-kernel unit probe stages={nst} K={K} N={N}")
    W = wl.normal_bf16(950 + K + N, (N, K), 0.02)
    qg = lib.fp4_quantize(W.to(DEV))
    want_full = nf4.bf16_bits(fp4.dequantize_f32(fp4.quantize(W.float().numpy())))
    kblk = K // 64
    for c in range(-(-kblk // M)):
        cols = probe_columns(kblk, c, M)
        Yg, _ = lib.qlora_fwd(unit_rows(K, cols).to(DEV), qg, None, None, 1.0)
        torch.cuda.synchronize()
        # equal values bit for bit; the E2M1 code for -0 dequantises to -0, which a sum of zero
        # products returns as +0
        got, want = nf4.bf16_value(u16(Yg)), nf4.bf16_value(want_full[:, cols].T)
        assert np.array_equal(got, want)


# ---------------------------------------------------------------- T and the LoRA term, exactly
# With the adapter A (r % 8 == 0, 8 <= r <= 64 for NF4, r <= 16 for E2M1) the stream kernel
# forms T = X A^T from the X slices it streams (NF4: A from registers on the 4-tile waves; E2M1:
# A's slice copied to LDS beside X's by the copying waves); above, qlora_fwd takes T's split
# partials or the separate row projection. With unit rows of X every entry of T is one product A[j, k_i], exact in
# any summation order, so T must equal A's probed columns bit for bit; with B the rank selector
# (B[n, j] = 1 for j = n mod r) and s = 2, output (i, n) is bf16(fl32(base + fl32(2 A[n mod r, k_i])))
# with base the decode's float32 value (fl32(a' * bf16(level)) for NF4, the E2M1 dequantisation
# for E2M1), so every workgroup's T shows in its own columns bit for bit, staggered start stages
# included. Stage counts run around the 8-stage (NF4) and 4-stage (E2M1) loops; ranks cover one,
# two and four rank tiles of 16.
LORA_PROBES = ([(nst, r, 336 if i % 2 == 0 else 296, "nf4")
                for i, (nst, r) in enumerate(zip(STREAM_STAGES, [8, 16, 24, 32, 40, 48, 56, 64, 16, 32, 64, 8, 24]))]
               + [(nst, r, 336 if i % 2 == 0 else 296, "e2m1")
                  for i, (nst, r) in enumerate(zip([1, 2, 3, 4, 5, 7, 8, 9, 12, 17], [8, 16, 24, 16, 8, 48, 16, 8, 16, 64]))])


@pytest.mark.parametrize("nst,r,N,fmt", LORA_PROBES)
def test_stream_kernel_lora_unit_probe(lib, nst, r, N, fmt):
    K, M, s = 256 * nst, 16, 2.0
    say(f"stream-kernel T probe {fmt} stages={nst} K={K} N={N} r={r}")
    kblk = K // 64
    if fmt == "nf4":
        W = probe_weight(N, K, 256, 960 + nst + N + r)
        qg = lib.nf4_quantize(W.to(DEV), 256)
        qo = nf4.quantize(W.float().numpy(), 256)
        lv_bf = nf4.bf16_value(nf4.bf16_bits(nf4.codebook()))
        codes = nf4.unpack(qo.codes).reshape(N, K)
        a = nf4.decode_absmax(qo).reshape(N, kblk).astype(np.float32)
    else:
        W = wl.normal_bf16(970 + nst + N + r, (N, K), 0.02)
        qg = lib.fp4_quantize(W.to(DEV))
        deq = fp4.dequantize_f32(fp4.quantize(W.float().numpy()))
    A = wl.normal_bf16(980 + nst + r, (r, K), 0.5)
    B = torch.zeros(N, r, dtype=torch.bfloat16)
    B[torch.arange(N), torch.arange(N) % r] = 1.0
    cols = probe_columns(kblk, 1, M)
    Yg, Tg = lib.qlora_fwd(unit_rows(K, cols).to(DEV), qg, A.to(DEV), B.to(DEV), s)
    torch.cuda.synchronize()
    Af = A.float().numpy()
    assert np.array_equal(u16(Tg), nf4.bf16_bits(Af[:, cols].T.astype(np.float32)))
    if fmt == "nf4":
        base = np.stack([(a[:, kk // 64] * lv_bf[codes[:, kk]]).astype(np.float32) for kk in cols])
    else:
        base = deq[:, cols].T.astype(np.float32)
    lora = (np.float32(s) * Af[np.arange(N) % r][:, cols].T).astype(np.float32)
    want = nf4.bf16_value(nf4.bf16_bits((base + lora).astype(np.float32)))
    got = nf4.bf16_value(u16(Yg))
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} outputs differ, first (row, n) {bad[:4].tolist()}"
