"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each case below patches one plausible mistake into the oracle (a dropped term, a wrong sign, a
wrong operand or index, a wrong rounding or nibble order, a wrong codebook constant) and runs the
pin tests of test_oracle_codebook/quant/gemm against it; at least one pin must fail. The patches
live only inside this test (pytest's monkeypatch undoes them).
"""
import numpy as np
import pytest

from oracle import fp4, merge, moe, nf4, qlora, swiglu
from tests import test_oracle_codebook as tc
from tests import test_oracle_fp4 as tf
from tests import test_oracle_gemm as tg
from tests import test_oracle_merge as tm
from tests import test_oracle_moe as to
from tests import test_oracle_quant as tq
from tests import test_oracle_swiglu as ts

PINS = [
    tc.test_codebook_structure,
    tc.test_levels_sit_at_evenly_spaced_probabilities,
    tc.test_codebook_golden_file,
    tc.test_bf16_rounding_matches_torch,
    tq.test_encode_brute_force_near_midpoints,
    tq.test_encode_brute_force_random,
    tq.test_encode_ties_go_to_lower_code,
    tq.test_special_blocks,
    tq.test_pack_known_pattern,
    tq.test_round_trip_exact_on_codebook_points,
    tq.test_double_quant_definition_and_bound,
    tq.test_dequantize_definition,
    lambda: tg.test_forward_backward_brute_force(3, 64, 5, 2, 0, 2.0),
    lambda: tg.test_forward_backward_brute_force(4, 128, 3, 3, 256, 0.5),
    lambda: tg.test_adjoint_identities(1),
    tg.test_finite_differences_are_exact_by_linearity,
    tg.test_rank_zero_equals_b_zero_equals_plain_gemm,
    tg.test_zero_base_leaves_lora_term,
    tg.test_identity_input_returns_dequantised_weight,
    ts.test_silu_matches_scipy_logistic,
    lambda: ts.test_forward_is_the_gated_composition(5, 128, 7, 3, 0, 1.5),
    lambda: ts.test_backward_matches_finite_differences(5, 2.0),
    ts.test_stacked_form_equals_the_pair,
    ts.test_zero_up_projection,
    tm.test_merged_layer_equals_the_qlora_layer,
    tm.test_merge_brute_force,
    tm.test_merge_special_cases,
    to.test_one_expert_is_the_single_layer,
    to.test_brute_force_rows,
    to.test_empty_expert,
    to.test_expert_reordering,
    tf.test_e2m1_codebook_matches_the_page,
    tf.test_e4m3_grid_matches_torch,
    tf.test_e4m3_rounding_matches_torch,
    tf.test_group_scales_match_torch,
    tf.test_encode_brute_force_random,
    tf.test_encode_brute_force_at_midpoints,
    tf.test_special_cases,
    tf.test_pack_known_pattern,
    tf.test_dequantize_definition_and_bound,
]

_fwd, _bwd = qlora.forward, qlora.backward
_f64 = qlora._f64


def fwd_no_lora(X, Wd, A, B, s):
    Y, T = _fwd(X, Wd, A, B, s)
    return Y - s * (T @ _f64(B).T), T


def fwd_wrong_sign(X, Wd, A, B, s):
    Y, T = _fwd(X, Wd, A, B, s)
    return Y - 2 * s * (T @ _f64(B).T), T


def fwd_s_twice(X, Wd, A, B, s):
    return _fwd(X, Wd, A, B, s * s) if s != 1 else _fwd(X, Wd, A, B, 2 * s)


def fwd_reversed_adapter_rows(X, Wd, A, B, s):
    return _fwd(X, Wd, _f64(A)[::-1], B, s)


def bwd_dx_no_lora(dY, X, Wd, A, B, s):
    dX, dA, dB = _bwd(dY, X, Wd, A, B, s)
    return dX - s * (_f64(dY) @ _f64(B)) @ _f64(A), dA, dB


def bwd_da_no_s(dY, X, Wd, A, B, s):
    dX, dA, dB = _bwd(dY, X, Wd, A, B, s)
    return dX, dA / s, dB


def bwd_db_uses_u(dY, X, Wd, A, B, s):
    dX, dA, _ = _bwd(dY, X, Wd, A, B, s)
    return dX, dA, s * (_f64(dY).T @ (_f64(dY) @ _f64(B)))


def bwd_da_uses_t(dY, X, Wd, A, B, s):
    dX, _, dB = _bwd(dY, X, Wd, A, B, s)
    return dX, s * ((_f64(X) @ _f64(A).T).T @ _f64(X)), dB


def bwd_dx_transposed_weight_rows(dY, X, Wd, A, B, s):
    dX, dA, dB = _bwd(dY, X, _f64(Wd)[::-1], A, B, s)
    return dX, dA, dB


_sfwd, _sbwd = swiglu.forward, swiglu.backward


def swiglu_gate_up_swapped(X, Wd_g, Wd_u, Ag, Au, Bg, Bu, s):
    H, Yg, Yu, Tg, Tu = _sfwd(X, Wd_g, Wd_u, Ag, Au, Bg, Bu, s)
    return swiglu.silu(Yu) * Yg, Yg, Yu, Tg, Tu


def swiglu_dyu_without_silu(dH, X, Wd_g, Wd_u, Ag, Au, Bg, Bu, s):
    Yg, _ = qlora.forward(X, Wd_g, Ag, Bg, s)
    Yu, _ = qlora.forward(X, Wd_u, Au, Bu, s)
    dYg = _f64(dH) * Yu * swiglu.silu_grad(Yg)
    dXg, dAg, dBg = qlora.backward(dYg, X, Wd_g, Ag, Bg, s)
    dXu, dAu, dBu = qlora.backward(_f64(dH) * Yg, X, Wd_u, Au, Bu, s)
    return dXg + dXu, dAg, dAu, dBg, dBu


def swiglu_dx_gate_only(dH, X, Wd_g, Wd_u, Ag, Au, Bg, Bu, s):
    dX, dAg, dAu, dBg, dBu = _sbwd(dH, X, Wd_g, Wd_u, Ag, Au, Bg, Bu, s)
    Yg, _ = qlora.forward(X, Wd_g, Ag, Bg, s)
    dXu, _, _ = qlora.backward(_f64(dH) * swiglu.silu(Yg), X, Wd_u, Au, Bu, s)
    return dX - dXu, dAg, dAu, dBg, dBu


_merge = merge.merge


def merge_transposed_product(Wd, A, B, s):
    return _f64(Wd) + s * (_f64(B)[:, ::-1] @ _f64(A))     # adapter ranks paired in reverse


def merge_without_s(Wd, A, B, s):
    return _merge(Wd, A, B, 1.0)


_mfwd, _mbwd = moe.forward, moe.backward


def moe_next_experts_weights(X, counts, Wd, A, B, s):
    E = len(counts)
    N = _f64(Wd).shape[0] // E
    return _mfwd(X, counts, np.roll(_f64(Wd), -N, axis=0), A, B, s)


def moe_offsets_shifted(counts):
    off = np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))])
    off[1:-1] += 1
    return np.minimum(off, off[-1])


def moe_db_over_all_rows(dY, X, counts, Wd, A, B, s):
    dX, dA, dB = _mbwd(dY, X, counts, Wd, A, B, s)
    E = len(counts)
    N, r = _f64(Wd).shape[0] // E, _f64(A).shape[0] // E
    T = _f64(X) @ _f64(A)[:r].T
    dB = dB.copy()
    dB[:N] = s * _f64(dY).T @ T
    return dX, dA, dB


_encode = nf4.encode
_double_quant = nf4.double_quant
_levels = nf4.nf4_levels_f64


def encode_ties_up(w, absmax):
    out = _encode(w, absmax)
    w = np.asarray(w, np.float32).reshape(-1)
    a = np.repeat(np.asarray(absmax, np.float32), 64)
    c = nf4._CODEBOOK.astype(np.float64)
    with np.errstate(invalid="ignore", divide="ignore"):
        v = (w / np.where(a == 0, 1, a)).astype(np.float32).astype(np.float64)
    for i in range(15):
        tie = (v - c[i]) == (c[i + 1] - v)
        out[tie & (a != 0)] = i + 1
    return out


def encode_rne_midpoints(w, absmax):
    w = np.asarray(w, np.float32).reshape(-1)
    a = np.repeat(np.asarray(absmax, np.float32), 64)
    c = nf4._CODEBOOK.astype(np.float64)
    mids = np.array([(c[i] + c[i + 1]) / 2 for i in range(15)]).astype(np.float32)
    with np.errstate(invalid="ignore", divide="ignore"):
        v = (w / np.where(a == 0, 1, a)).astype(np.float32)
    out = (v[:, None] > mids[None, :]).sum(axis=1).astype(np.uint8)
    out[a == 0] = 7
    return out


def pack_swapped(codes):
    c = np.asarray(codes, np.uint8).reshape(-1)
    return ((c[1::2] << 4) | c[0::2]).astype(np.uint8)


def unpack_swapped(packed):
    p = np.asarray(packed, np.uint8).reshape(-1)
    out = np.empty(p.size * 2, np.uint8)
    out[1::2] = p >> 4
    out[0::2] = p & 0x0F
    return out


def dq_by_128(absmax, dq_block):
    a = np.asarray(absmax, np.float32).reshape(-1)
    runs = (a.size + dq_block - 1) // dq_block
    q = np.zeros(a.size, np.int8)
    S = np.zeros(runs, np.float32)
    for j in range(runs):
        seg = a[j * dq_block:(j + 1) * dq_block]
        S[j] = np.float32(seg.max() / np.float32(128))
        if S[j]:
            q[j * dq_block:(j + 1) * dq_block] = np.clip(np.rint(seg / S[j]), 0, 127)
    return q, S


def dq_truncating(absmax, dq_block):
    q, S = _double_quant(absmax, dq_block)
    a = np.asarray(absmax, np.float32).reshape(-1)
    Sx = np.repeat(S, dq_block)[: a.size]
    with np.errstate(invalid="ignore", divide="ignore"):
        t = np.where(Sx > 0, np.floor((a / np.where(Sx > 0, Sx, 1)).astype(np.float32)), 0)
    return np.clip(t, 0, 127).astype(np.int8), S


def bf16_truncate(x):
    return (np.ascontiguousarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def deq_code_off_by_one(wq):
    c = nf4._CODEBOOK[np.minimum(nf4.unpack(wq.codes) + 1, 15)]
    a = np.repeat(nf4.decode_absmax(wq), 64)
    return (c * a).astype(np.float32).reshape(wq.n, wq.k)


def decode_absmax_next_run(wq):
    if wq.dq_block == 0:
        return np.asarray(wq.absmax, np.float32)
    q = np.asarray(wq.absmax, np.int8).astype(np.float32)
    S = np.repeat(np.roll(wq.scale, 1), wq.dq_block)[: q.size]
    return (q * S).astype(np.float32)


_fp4_round, _fp4_encode = fp4.round_to_grid, fp4.encode


def fp4_round_ties_up(x, grid):
    x = np.asarray(x, dtype=np.float64)
    mids = (grid[1:] + grid[:-1]) / 2.0
    return np.searchsorted(mids, x, side="right")


def fp4_encode_ties_up(w, scales, S):
    fp4.round_to_grid = fp4_round_ties_up
    try:
        return _fp4_encode(w, scales, S)
    finally:
        fp4.round_to_grid = _fp4_round


def fp4_scales_truncated(w, S):
    g = np.abs(w.astype(np.float32)).reshape(-1, fp4.GROUP).max(axis=1)
    if S == 0:
        return np.zeros(g.shape, np.uint8)
    t = (g / np.float32(np.float32(6.0) * S)).astype(np.float32)
    return np.clip(np.searchsorted(fp4.e4m3_grid(), t, side="right") - 1, 0, 126).astype(np.uint8)


def fp4_deq_without_tensor_scale(q):
    codes = fp4.unpack(q.codes).reshape(-1, fp4.GROUP)
    s = fp4.e4m3_grid()[q.scales].astype(np.float32)[:, None]
    return (fp4.e2m1_codebook()[codes].astype(np.float32) * s).astype(np.float32).reshape(q.n, q.k)


def fp4_value_bias_zero(code):
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = m / 2.0 if e == 0 else 2.0 ** e * (1.0 + m / 2.0)
    return -mag if s else mag


MUTATIONS = {
    "fp4: E2M1 ties go up": [(fp4, "encode", fp4_encode_ties_up)],
    "fp4: group scales truncated": [(fp4, "group_scales", fp4_scales_truncated)],
    "fp4: tensor scale divides by 448": [(fp4, "TSCALE_DIV", 448.0)],
    "fp4: dequant drops the tensor scale": [(fp4, "dequantize_f32", fp4_deq_without_tensor_scale)],
    "fp4: nibble order swapped": [(fp4, "pack", pack_swapped), (fp4, "unpack", unpack_swapped)],
    "fp4: exponent bias 0": [(fp4, "e2m1_value", fp4_value_bias_zero)],
    "fwd drops the LoRA term": [(qlora, "forward", fwd_no_lora)],
    "fwd flips the LoRA sign": [(qlora, "forward", fwd_wrong_sign)],
    "fwd applies s twice": [(qlora, "forward", fwd_s_twice)],
    "fwd reverses adapter rows": [(qlora, "forward", fwd_reversed_adapter_rows)],
    "bwd dX drops the LoRA term": [(qlora, "backward", bwd_dx_no_lora)],
    "bwd dA misses s": [(qlora, "backward", bwd_da_no_s)],
    "bwd dB uses U instead of T": [(qlora, "backward", bwd_db_uses_u)],
    "bwd dA uses T instead of U": [(qlora, "backward", bwd_da_uses_t)],
    "bwd dX reads weight rows reversed": [(qlora, "backward", bwd_dx_transposed_weight_rows)],
    "swiglu: silu derivative misses x (1 - sigma)": [(swiglu, "silu_grad", swiglu.sigmoid)],
    "swiglu: gate and up swapped": [(swiglu, "forward", swiglu_gate_up_swapped)],
    "swiglu: dYu uses Yg instead of silu(Yg)": [(swiglu, "backward", swiglu_dyu_without_silu)],
    "swiglu: dX drops the up projection": [(swiglu, "backward", swiglu_dx_gate_only)],
    "merge pairs ranks in reverse": [(merge, "merge", merge_transposed_product)],
    "merge drops s": [(merge, "merge", merge_without_s)],
    "moe: rows use the next expert's weight": [(moe, "forward", moe_next_experts_weights)],
    "moe: expert boundaries shifted by a row": [(moe, "offsets", moe_offsets_shifted)],
    "moe: dB summed over every row": [(moe, "backward", moe_db_over_all_rows)],
    "encode ties go up": [(nf4, "encode", encode_ties_up)],
    "encode by rounded-to-nearest midpoints": [(nf4, "encode", encode_rne_midpoints)],
    "nibble order swapped": [(nf4, "pack", pack_swapped), (nf4, "unpack", unpack_swapped)],
    "double quant divides by 128": [(nf4, "double_quant", dq_by_128)],
    "double quant truncates": [(nf4, "double_quant", dq_truncating)],
    "bf16 truncates": [(nf4, "bf16_bits", bf16_truncate)],
    "dequant code off by one": [(nf4, "dequantize_f32", deq_code_off_by_one)],
    "dequant uses the wrong run's scale": [(nf4, "decode_absmax", decode_absmax_next_run)],
    "codebook delta wrong": [(nf4, "DELTA", 1.0 - 1.0 / 32.0)],
    "codebook sides swapped": [(nf4, "nf4_levels_f64", lambda quantile=nf4.normal_quantile:
                                -_levels(quantile)[::-1])],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    for mod, attr, val in MUTATIONS[name]:
        monkeypatch.setattr(mod, attr, val)
    if any(attr in ("DELTA", "nf4_levels_f64") for _, attr, _ in MUTATIONS[name]):
        monkeypatch.setattr(nf4, "_CODEBOOK", nf4.codebook())
        monkeypatch.setattr(tq, "C", nf4.codebook())
        monkeypatch.setattr(tg, "C", nf4.codebook())
    caught = []
    for pin in PINS:
        try:
            pin()
        except AssertionError as e:
            caught.append((getattr(pin, "__name__", "pin"), type(e).__name__))
    assert caught, f"no pin catches: {name}"
