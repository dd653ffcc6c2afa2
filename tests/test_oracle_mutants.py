"""Pin sensitivity: plausible mistakes planted in CPU versions of the oracle's
functions must each fail at least one pin of test_oracle.py.

Every mutant below is the oracle with one planted mistake (a dropped term, a
wrong sign or index, a transposed operand, a wrong rounding or scale).  If a
mutant passed its pins, the pins would not be strong enough to trust the
oracle.
"""
import numpy as np
import pytest

import oracle
from test_oracle import (act4_pins, epilogue_pins, gemm_pins, pack_pins, quant_a4_pins,
                         quant_pins, ternarize_pins)
import synth


def _fails(pins, *impl):
    try:
        pins(*impl)
    except (AssertionError, ValueError, IndexError, OverflowError):
        return True
    return False


# --------------------------- O1 mutants ------------------------------------
def _g_drop_last_k(x, w):
    x, w = np.atleast_2d(x), np.atleast_2d(w)
    if x.shape[1] <= 1:
        return np.zeros((x.shape[0], w.shape[0]), np.int32)
    return oracle.gemm_i32(x[:, :-1], w[:, :-1])


def _g_neg(x, w):
    return -oracle.gemm_i32(x, w)


def _g_shift_k(x, w):
    return oracle.gemm_i32(x, np.roll(w, 1, axis=1))


def _g_int16_acc(x, w):
    y = np.atleast_2d(x).astype(np.int64) @ np.atleast_2d(w).astype(np.int64).T
    return ((y + 2 ** 15) % 2 ** 16 - 2 ** 15).astype(np.int32)


def _g_x_unsigned(x, w):
    xu = np.atleast_2d(x).view(np.uint8).astype(np.int64)
    return (xu @ np.atleast_2d(w).astype(np.int64).T).astype(np.int32)


def _g_w_as_kn(x, w):
    # reads W's memory as [K][N] instead of [N][K]
    x2, w2 = np.atleast_2d(x), np.atleast_2d(w)
    N, K = w2.shape
    wt = np.ascontiguousarray(w2).reshape(K, N).T
    return oracle.gemm_i32(x2, np.ascontiguousarray(wt))


@pytest.mark.parametrize("mut", [_g_drop_last_k, _g_neg, _g_shift_k, _g_int16_acc,
                                 _g_x_unsigned, _g_w_as_kn])
def test_gemm_mutants_fail(mut):
    assert _fails(gemm_pins, mut)


# --------------------------- O2 mutants ------------------------------------
def _tern_generic(W, scale_fn, round_fn, clamp=True):
    W = np.asarray(W, np.float32)
    sw = np.float32(scale_fn(W))
    if sw == 0:
        return np.zeros(W.shape, np.int8), sw
    q = round_fn(W / sw)
    if clamp:
        q = np.clip(q, -1, 1)
    return q.astype(np.int8), sw


def _mean_abs(W):
    return np.abs(W.astype(np.float64)).mean()


def _t_no_clamp(W):
    return _tern_generic(W, _mean_abs, np.rint, clamp=False)


def _t_half_away(W):
    return _tern_generic(W, _mean_abs, lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5))


def _t_trunc(W):
    return _tern_generic(W, _mean_abs, np.trunc)


def _t_max_scale(W):
    return _tern_generic(W, lambda w: np.abs(w).max(), np.rint)


def _t_mean_no_abs(W):
    return _tern_generic(W, lambda w: abs(w.astype(np.float64).mean()), np.rint)


def _fp32_running_mean_abs(W):
    # the mean of |W| accumulated in fp32, in row-major order
    acc = np.float32(0.0)
    for v in np.abs(np.asarray(W, np.float32)).ravel():
        acc = np.float32(acc + v)
    return acc / np.float32(W.size)


def _t_fp32_sum(W):
    return _tern_generic(W, _fp32_running_mean_abs, np.rint)


@pytest.mark.parametrize("mut", [_t_no_clamp, _t_half_away, _t_trunc, _t_max_scale,
                                 _t_mean_no_abs, _t_fp32_sum])
def test_ternarize_mutants_fail(mut):
    assert _fails(ternarize_pins, mut)


# --------------------------- O3 mutants ------------------------------------
def _quant_generic(xb, amax_fn, round_fn, qmax=127, lo=-127, per_row=True, divide=False,
                   cap=True):
    xf = synth.bf16_bits_to_fp32(np.atleast_2d(xb)).astype(np.float32)
    M, K = xf.shape
    q = np.zeros((M, K), np.int8)
    sa = np.zeros(M, np.float32)
    a_all = np.float32(np.abs(xf).max()) if xf.size else np.float32(0)
    for m in range(M):
        a = np.float32(amax_fn(xf[m])) if per_row else a_all
        if a == 0:
            continue
        with np.errstate(over="ignore", invalid="ignore"):
            inv = np.float32(qmax) / a
        if cap:
            inv = min(inv, np.finfo(np.float32).max)
        sa[m] = a / np.float32(qmax)
        # divide: x / sa (the rounded scale) instead of x * inv (its rounded reciprocal)
        with np.errstate(over="ignore", invalid="ignore"):
            v = (xf[m] / sa[m]) if divide else (xf[m] * inv)
            q[m] = np.clip(round_fn(v), lo, 127).astype(np.int8)
    return q, sa


def _q_trunc(xb):
    return _quant_generic(xb, lambda r: np.abs(r).max(), np.trunc)


def _q_no_abs(xb):
    return _quant_generic(xb, lambda r: r.max(), np.rint)


def _q_per_tensor(xb):
    return _quant_generic(xb, lambda r: np.abs(r).max(), np.rint, per_row=False)


def _q_scale_128(xb):
    return _quant_generic(xb, lambda r: np.abs(r).max(), np.rint, qmax=128, lo=-128)


def _q_half_away(xb):
    return _quant_generic(xb, lambda r: np.abs(r).max(),
                          lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5))


def _q_divide_by_scale(xb):
    return _quant_generic(xb, lambda r: np.abs(r).max(), np.rint, divide=True)


def _q_no_cap(xb):
    # 127/a left to overflow: tiny rows quantize to +-127 and their zeros to 0*inf
    return _quant_generic(xb, lambda r: np.abs(r).max(), np.rint, cap=False)


@pytest.mark.parametrize("mut", [_q_trunc, _q_no_abs, _q_per_tensor, _q_scale_128,
                                 _q_half_away, _q_divide_by_scale, _q_no_cap])
def test_quant_mutants_fail(mut):
    assert _fails(quant_pins, mut)


# --------------------------- O4 mutants ------------------------------------
def _e_no_sw(acc, sa, sw):
    return oracle.epilogue(acc, sa, 1.0)


def _e_sa_by_col(acc, sa, sw):
    acc = np.atleast_2d(acc)
    sa = np.atleast_1d(sa).astype(np.float32)
    cols = np.resize(sa, acc.shape[1])
    return (acc.astype(np.float32) * cols[None, :]) * np.float32(sw)


def _e_truncate(acc, sa, sw):
    return np.trunc(oracle.epilogue(acc, sa, sw))


@pytest.mark.parametrize("mut", [_e_no_sw, _e_sa_by_col, _e_truncate])
def test_epilogue_mutants_fail(mut):
    assert _fails(epilogue_pins, mut)


# --------------------------- a2 mutants ------------------------------------
def _p_code_is_w(w):
    # stores w itself (two's complement low bits) instead of w + 1
    p = oracle.pack(np.zeros_like(w))
    w = np.asarray(w, np.int8)
    out = p.copy()
    # rebuild by flipping each field from 01 to (w & 3) using the oracle's own
    # field positions, found through single-element packs
    N, K = w.shape
    base = oracle.pack(np.zeros((N, K), np.int8))
    for n in range(N):
        for k in range(K):
            if w[n, k] == 0:
                code = 0
            else:
                code = int(w[n, k]) & 3
            one = np.zeros((N, K), np.int8)
            one[n, k] = 1
            d = np.nonzero(oracle.pack(one) != base)[0][0]
            mask = int(oracle.pack(one)[d]) ^ int(base[d])
            shift = (mask & -mask).bit_length() - 1
            out[d] = (int(out[d]) & ~mask & 0xFF) | (code << shift)
    return out


def _p_pad_00(w):
    w = np.asarray(w, np.int8)
    N, K = w.shape
    p = oracle.pack(w)
    if (N % 32) or (K % 128):
        p[-1] &= 0b11111100  # padding field set to 00 instead of 01
    return p


def _p_collide(w):
    # drops the row-within-group index: rows 4g..4g+3 overwrite each other
    w = np.asarray(w, np.int8).copy()
    N, K = w.shape
    for n in range(N):
        w[n] = w[(n // 4) * 4 + min(3, N - 1 - (n // 4) * 4)]
    return oracle.pack(w)


def test_pack_mutant_code_map_fails():
    # the constant-matrix code-map pin catches a wrong code map immediately;
    # the mutant is slow, so it is checked on the code-map pin alone
    p = _p_code_is_w(np.full((32, 128), -1, np.int8))
    assert not np.all(p == 0)


def test_pack_mutant_padding_fails():
    assert _fails(pack_pins, _p_pad_00, oracle.unpack, oracle.packed_bytes)


def test_pack_mutant_collision_fails():
    assert _fails(pack_pins, _p_collide, oracle.unpack, oracle.packed_bytes)


# --------------------------- O5 mutants ------------------------------------
def _q4_generic(xb, qmax=7, lo=-7, hi=7, round_fn=np.rint, amax_fn=lambda r: np.abs(r).max(),
                per_row=True, cap=True):
    xf = synth.bf16_bits_to_fp32(np.atleast_2d(xb)).astype(np.float32)
    M, K = xf.shape
    q = np.zeros((M, K), np.int8)
    sa = np.zeros(M, np.float32)
    a_all = np.float32(np.abs(xf).max()) if xf.size else np.float32(0)
    for m in range(M):
        a = np.float32(amax_fn(xf[m])) if per_row else a_all
        if a == 0:
            continue
        with np.errstate(over="ignore", invalid="ignore"):
            inv = np.float32(qmax) / a
            if cap:
                inv = min(inv, np.finfo(np.float32).max)
            q[m] = np.clip(round_fn(xf[m] * inv), lo, hi).astype(np.int8)
        sa[m] = a / np.float32(qmax)
    return q, sa


@pytest.mark.parametrize("mut", [
    lambda xb: _q4_generic(xb, round_fn=np.trunc),
    lambda xb: _q4_generic(xb, qmax=8, lo=-8),
    lambda xb: _q4_generic(xb, qmax=8, lo=-8, hi=7),
    lambda xb: _q4_generic(xb, amax_fn=lambda r: r.max()),
    lambda xb: _q4_generic(xb, per_row=False),
    lambda xb: _q4_generic(xb, round_fn=lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5)),
    lambda xb: oracle.quant_act(xb),
    lambda xb: _q4_generic(xb, cap=False),
], ids=["trunc", "scale8", "scale8_clamp7", "no_abs", "per_tensor", "half_away", "int8",
        "no_cap"])
def test_quant_a4_mutants_fail(mut):
    assert _fails(quant_a4_pins, mut)


# --------------------------- A4I layout mutants ----------------------------
def _a4_generic(q, byte_fn, kq_fn=lambda K: -(-K // 32) * 32, signed=True):
    q2 = np.atleast_2d(np.asarray(q, np.int8))
    M, K = q2.shape
    row = kq_fn(K) // 2
    out = np.zeros(M * row, np.uint8)
    for m in range(M):
        for k in range(K):
            v = int(q2[m, k])
            if v < -8 or v > 7:
                raise ValueError("out of range")
            b, s = byte_fn(k)
            out[m * row + b] |= ((v & 15) if signed else abs(v) & 15) << s
    return out


def _a4_unpack_generic(b, M, K, byte_fn, kq_fn=lambda K: -(-K // 32) * 32, sext=True):
    row = kq_fn(K) // 2
    q = np.zeros((M, K), np.int8)
    for m in range(M):
        for k in range(K):
            bb, s = byte_fn(k)
            v = (int(b[m * row + bb]) >> s) & 15
            q[m, k] = v - 16 if (sext and v >= 8) else v
    return q


def _ok_byte(k):
    c, i = divmod(k, 16)
    h, j = divmod(i, 4)
    return c * 8 + 4 * (h % 2) + j, 4 * (h // 2)


def _swap_halves(k):
    c, i = divmod(k, 16)
    h, j = divmod(i, 4)
    return c * 8 + 4 * (h // 2) + j, 4 * (h % 2)


def _plain_order(k):
    return k // 2, 4 * (k % 2)


def _no_pad_bytes(M, K):
    return M * (-(-K // 16) * 8)


@pytest.mark.parametrize("impl", [
    (lambda q: _a4_generic(q, _swap_halves),
     lambda b, M, K: _a4_unpack_generic(b, M, K, _swap_halves), oracle.act4_bytes),
    (lambda q: _a4_generic(q, _plain_order),
     lambda b, M, K: _a4_unpack_generic(b, M, K, _plain_order), oracle.act4_bytes),
    (lambda q: _a4_generic(q, _ok_byte, kq_fn=lambda K: -(-K // 16) * 16),
     lambda b, M, K: _a4_unpack_generic(b, M, K, _ok_byte, kq_fn=lambda K: -(-K // 16) * 16),
     _no_pad_bytes),
    (lambda q: _a4_generic(q, _ok_byte),
     lambda b, M, K: _a4_unpack_generic(b, M, K, _ok_byte, sext=False), oracle.act4_bytes),
], ids=["nibble_halves_swapped", "plain_order", "no_pad_to_32", "no_sign_extension"])
def test_act4_mutants_fail(impl):
    assert _fails(act4_pins, *impl)
