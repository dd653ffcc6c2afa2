"""Pins for the oracle: each function is checked against what the pages and the
mathematics fix (worked examples derived by hand, closed forms, invariants,
brute force, library routines), never against a retyping of its own code.

The pin predicates take the implementation as an argument so that
test_oracle_mutants.py can show that plausible mistakes fail them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

from conftest import GOLDEN



def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# O1: integer product
# --------------------------------------------------------------------------

def gemm_pins(gemm):
    """Raise AssertionError if `gemm(x[M,K], w[N,K]) -> int32[M,N]` breaks a pin."""
    rng = np.random.default_rng(1234)
    # textbook: numpy int64 matmul, tiny to medium shapes incl. ragged and x = -128
    for M, N, K in [(1, 1, 1), (1, 7, 5), (3, 5, 97), (2, 33, 129), (5, 64, 300), (1, 97, 1)]:
        x = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
        w = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
        ref = x.astype(np.int64) @ w.astype(np.int64).T
        np.testing.assert_array_equal(gemm(x, w), ref)
    # pure-Python triple loop on tiny shapes
    for M, N, K in [(1, 3, 4), (2, 2, 3)]:
        x = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
        w = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
        ref = [[sum(int(x[m, k]) * int(w[n, k]) for k in range(K)) for n in range(N)]
               for m in range(M)]
        np.testing.assert_array_equal(gemm(x, w), np.array(ref))
    # worked example (hand-derived)
    ex = _load("worked_examples.json")["gemv"][0]
    y = gemm(np.array([ex["x"]], dtype=np.int8), np.array(ex["w"], dtype=np.int8))
    np.testing.assert_array_equal(y[0], ex["y"])
    # closed forms
    K = 129
    x = rng.integers(-128, 128, size=(3, K), dtype=np.int8)
    rs = x.astype(np.int64).sum(axis=1)
    np.testing.assert_array_equal(gemm(x, np.ones((4, K), np.int8)), np.repeat(rs[:, None], 4, 1))
    np.testing.assert_array_equal(gemm(x, -np.ones((4, K), np.int8)), -np.repeat(rs[:, None], 4, 1))
    np.testing.assert_array_equal(gemm(x, np.zeros((4, K), np.int8)), 0)
    # extremes at the largest K of the workloads: 127*K and 128*K
    Kmax = 27648
    assert gemm(np.full((1, Kmax), 127, np.int8), np.ones((1, Kmax), np.int8))[0, 0] == 127 * Kmax
    assert gemm(np.full((1, Kmax), -128, np.int8), -np.ones((1, Kmax), np.int8))[0, 0] == 128 * Kmax
    # one-hot activations recover columns of W (pins operand orientation)
    N, K = 6, 9
    w = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    for k in range(K):
        e = np.zeros((1, K), np.int8)
        e[0, k] = 1
        np.testing.assert_array_equal(gemm(e, w)[0], w[:, k])
    # symmetries: y(-W) = -y(W); joint permutation of k
    x = rng.integers(-127, 128, size=(2, 50), dtype=np.int8)
    w = rng.integers(-1, 2, size=(8, 50), dtype=np.int8)
    y = gemm(x, w)
    np.testing.assert_array_equal(gemm(x, -w), -y)
    perm = rng.permutation(50)
    np.testing.assert_array_equal(gemm(x[:, perm], w[:, perm]), y)


def test_gemm_pins():
    gemm_pins(oracle.gemm_i32)


def test_gemm_threads_equals_gemm():
    # the threaded caller splits the weight rows into blocks: same result for
    # more threads than rows, ragged blocks and M > 1
    rng = np.random.default_rng(99)
    for M, N, K, t in [(1, 5, 33, 8), (3, 97, 130, 4), (7, 64, 300, 3), (2, 1, 9, 2)]:
        x = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
        w = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
        np.testing.assert_array_equal(oracle.gemm_i32_threads(x, w, t), oracle.gemm_i32(x, w))
    np.testing.assert_array_equal(oracle.gemm_i32_threads(x[0], w, 2), oracle.gemm_i32(x[0], w))


def test_gemm_full_sweep_shape_vs_numpy():
    # one full-size workload shape at M = 1 against numpy's int64 matmul
    x, w = synth.gemv_case(2560, 2560, synth.SEED_SMALL)
    ref = w.astype(np.int64) @ x.astype(np.int64)
    np.testing.assert_array_equal(oracle.gemm_i32(x, w), ref)


# --------------------------------------------------------------------------
# O2: absmean ternarization
# --------------------------------------------------------------------------

def ternarize_pins(tern):
    for ex in _load("worked_examples.json")["ternarize"]:
        wq, sw = tern(np.array(ex["w"], dtype=np.float32))
        assert float(sw) == ex["sw"], ex
        np.testing.assert_array_equal(wq, ex["wq"])
    rng = np.random.default_rng(7)
    # all magnitudes equal c: scale c, weights = sign
    c = np.float32(0.375)
    sgn = rng.choice(np.array([-1, 1], np.int8), size=(5, 40))
    wq, sw = tern(sgn.astype(np.float32) * c)
    assert sw == c
    np.testing.assert_array_equal(wq, sgn)
    # sw is the mean of |W| (integer-valued matrix: exact rational mean)
    Wi = rng.integers(-9, 10, size=(7, 11)).astype(np.float32)
    wq, sw = tern(Wi)
    assert sw == np.float32(np.abs(Wi.astype(np.float64)).sum() / Wi.size)
    # outputs ternary
    assert set(np.unique(wq)).issubset({-1, 0, 1})
    # power-of-two scale invariance (exact in binary floating point)
    W = rng.normal(0, 0.02, size=(16, 64)).astype(np.float32)
    wq1, sw1 = tern(W)
    for e in (-3, 5):
        wq2, sw2 = tern(W * np.float32(2.0 ** e))
        np.testing.assert_array_equal(wq2, wq1)
        assert sw2 == sw1 * np.float32(2.0 ** e)
    # sign symmetry
    wq3, sw3 = tern(-W)
    np.testing.assert_array_equal(wq3, -wq1)
    assert sw3 == sw1
    # monotone in W for a fixed scale: the ordering of W is kept (non-strict)
    order = np.argsort(W.ravel(), kind="stable")
    assert np.all(np.diff(wq1.ravel()[order].astype(int)) >= 0)


def test_ternarize_pins():
    ternarize_pins(oracle.ternarize_absmean)


def test_ternarize_gaussian_zero_fraction():
    # For W ~ N(0, s^2): mean|W| -> s*sqrt(2/pi); W rounds to 0 iff |W| < mean/2,
    # so P(0) = erf(sqrt(2/pi)/2 / sqrt(2)) ~= 0.3101 and P(+1) = P(-1).
    _, W = synth.linear_case(1, 1024, 1024, seed=5)
    wq, sw = oracle.ternarize_absmean(W)
    p0 = float(np.mean(wq == 0))
    expect = math.erf(math.sqrt(2 / math.pi) / 2 / math.sqrt(2))
    assert abs(p0 - expect) < 0.003, (p0, expect)
    pp, pn = float(np.mean(wq == 1)), float(np.mean(wq == -1))
    assert abs(pp - pn) < 0.004
    assert abs(float(sw) - 0.02 * math.sqrt(2 / math.pi)) < 2e-4


# --------------------------------------------------------------------------
# O3: per-token absmax int8 quantization
# --------------------------------------------------------------------------

def _bf16(a):
    return synth.fp32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def quant_pins(quant):
    for ex in _load("worked_examples.json")["quant_act"]:
        q, sa = quant(_bf16([ex["x"]]))
        np.testing.assert_array_equal(q[0], ex["q"])
        assert sa[0] == np.float32(ex["sa_num"]) / np.float32(ex["sa_den"])
    # zero row
    q, sa = quant(_bf16(np.zeros((1, 33))))
    assert np.all(q == 0) and sa[0] == 0.0
    rng = np.random.default_rng(11)
    x = rng.standard_normal((6, 257)).astype(np.float32)
    x[2, 5] = 40.0  # an outlier row
    xb = _bf16(x)
    xf = synth.bf16_bits_to_fp32(xb)
    q, sa = quant(xb)
    # range, absmax element -> +-127, scale = absmax / 127
    assert q.min() >= -127 and q.max() <= 127
    for m in range(6):
        i = int(np.argmax(np.abs(xf[m])))
        assert abs(int(q[m, i])) == 127
        assert sa[m] == np.float32(np.abs(xf[m]).max()) / np.float32(127.0)
    # rows are independent (per-token)
    for m in range(6):
        qm, sam = quant(xb[m:m + 1])
        np.testing.assert_array_equal(qm[0], q[m])
        assert sam[0] == sa[m]
    # reconstruction error at most half a step (plus fp32 rounding slack)
    err = np.abs(xf - q.astype(np.float64) * sa[:, None].astype(np.float64))
    assert np.all(err <= sa[:, None] * (0.5 + 1e-5) + 1e-30)
    # monotone within a row; odd symmetry
    for m in range(6):
        o = np.argsort(xf[m], kind="stable")
        assert np.all(np.diff(q[m][o].astype(int)) >= 0)
    qn, san = quant(_bf16(-x))
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(san, sa)
    # power-of-two invariance: q(2^e x) == q(x), sa scales by 2^e
    for e in (-4, 3):
        q2, sa2 = quant(_bf16(x * np.float32(2.0 ** e)))
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(sa2, sa * np.float32(2.0 ** e))


def test_quant_pins():
    quant_pins(oracle.quant_act)


def test_bf16_generator_encodings():
    # the generator's fp32 -> bf16 conversion: known encodings and ties to even
    b = synth.fp32_to_bf16_bits(np.array([1.0, -2.0, 0.5, 0.0], np.float32))
    np.testing.assert_array_equal(b, [0x3F80, 0xC000, 0x3F00, 0x0000])
    # 1 + 2^-8 is halfway between bf16 1.0 and 1 + 2^-7: ties to even -> 1.0
    assert synth.fp32_to_bf16_bits(np.array([1.0 + 2.0 ** -8], np.float32))[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 (odd) and 1 + 2^-6 (even) -> up
    assert synth.fp32_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8], np.float32))[0] == 0x3F82


# --------------------------------------------------------------------------
# O4: epilogue
# --------------------------------------------------------------------------

def epilogue_pins(epi):
    acc = np.array([[0, 1, -1, 12345, -(2 ** 23), 2 ** 24 - 1]], dtype=np.int32)
    # zeros are exactly zero; unit scales give float(acc) exactly (|acc| < 2^24)
    y = epi(acc, np.array([1.0], np.float32), 1.0)
    np.testing.assert_array_equal(y, acc.astype(np.float32))
    assert epi(np.zeros((2, 3), np.int32), np.array([0.3, 7.0], np.float32), 0.1).tolist() == [[0.0] * 3] * 2
    # power-of-two scales are exact
    y = epi(acc, np.array([0.125], np.float32), 0.0625)
    np.testing.assert_array_equal(y, acc.astype(np.float64) / 128.0)
    # per-row scale: row m uses sa[m]
    y = epi(np.array([[3], [3]], np.int32), np.array([2.0, 4.0], np.float32), 0.5)
    np.testing.assert_array_equal(y[:, 0], [3.0, 6.0])
    # within two fp32 roundings of the exact product
    rng = np.random.default_rng(3)
    acc = rng.integers(-3_511_296, 3_511_297, size=(4, 100)).astype(np.int32)
    sa = rng.uniform(1e-3, 1.0, size=4).astype(np.float32)
    sw = np.float32(0.0159)
    y = epi(acc, sa, sw).astype(np.float64)
    exact = acc.astype(np.float64) * sa[:, None].astype(np.float64) * float(sw)
    nz = exact != 0
    rel = np.abs(y[nz] - exact[nz]) / np.abs(exact[nz])
    assert rel.max() <= 2 * 2.0 ** -24 * (1 + 1e-6)


def test_epilogue_pins():
    epilogue_pins(oracle.epilogue)


# --------------------------------------------------------------------------
# a2: 2-bit packing
# --------------------------------------------------------------------------

def pack_pins(pack, unpack, packed_bytes):
    cm = _load("code_map.json")
    code = {int(k): int(v, 2) for k, v in cm["codes"].items()}
    # density: 8 parameters per 2 bytes on aligned shapes
    for N, K in [(32, 128), (64, 256), (2560, 2560), (55296, 5120)]:
        assert packed_bytes(N, K) * cm["params_per_2_bytes"] == N * K * 2
    # code map: a constant matrix fills every byte with four copies of its code
    for v in (-1, 0, 1):
        p = pack(np.full((64, 256), v, np.int8))
        byte = code[v] | code[v] << 2 | code[v] << 4 | code[v] << 6
        assert np.all(p == byte), (v, hex(byte))
    # padding holds the weight-0 code: one -1 in a 1x1 matrix
    p = pack(np.array([[-1]], np.int8))
    assert p.size == packed_bytes(1, 1) == 32 * 128 // 4
    zero_byte = code[0] * 0x55
    diff = np.nonzero(p != zero_byte)[0]
    assert diff.size == 1
    fields = [(int(p[diff[0]]) >> s) & 3 for s in (0, 2, 4, 6)]
    assert sorted(fields) == [code[-1], code[0], code[0], code[0]]
    # bijection of positions onto 2-bit fields over one full tile
    seen = set()
    base = pack(np.zeros((32, 128), np.int8))
    for n in range(32):
        for k in range(128):
            w = np.zeros((32, 128), np.int8)
            w[n, k] = 1
            d = np.nonzero(pack(w) != base)[0]
            assert d.size == 1
            x = int(pack(w)[d[0]]) ^ int(base[d[0]])
            assert x in (0b11, 0b11 << 2, 0b11 << 4, 0b11 << 6)
            seen.add((int(d[0]), x))
    assert len(seen) == 32 * 128
    # round trip on random and ragged shapes
    rng = np.random.default_rng(9)
    for N, K in [(1, 1), (31, 127), (33, 129), (64, 384), (97, 300), (5, 1000)]:
        w = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
        p = pack(w)
        assert p.size == packed_bytes(N, K)
        np.testing.assert_array_equal(unpack(p, N, K), w)
        # code 11 never produced
        for s in (0, 2, 4, 6):
            assert not np.any(((p >> s) & 3) == 3)


def test_pack_pins():
    pack_pins(oracle.pack, oracle.unpack, oracle.packed_bytes)


def test_pack_rejects_non_ternary():
    with pytest.raises(ValueError):
        oracle.pack(np.array([[2]], np.int8))
    with pytest.raises(ValueError):
        oracle.pack(np.array([[-2]], np.int8))


def test_unpack_rejects_code_11():
    p = oracle.pack(np.zeros((1, 1), np.int8))
    p[0] |= 0b11
    with pytest.raises(ValueError):
        oracle.unpack(p, 1, 1)


# --------------------------------------------------------------------------
# O5: per-token absmax int4 quantization (W2A4 variant)
# --------------------------------------------------------------------------

def quant_a4_pins(quant):
    for ex in _load("worked_examples.json")["quant_act_a4"]:
        q, sa = quant(_bf16([ex["x"]]))
        np.testing.assert_array_equal(q[0], ex["q"])
        assert sa[0] == np.float32(ex["sa_num"]) / np.float32(ex["sa_den"])
    q, sa = quant(_bf16(np.zeros((1, 17))))
    assert np.all(q == 0) and sa[0] == 0.0
    rng = np.random.default_rng(21)
    x = rng.standard_normal((5, 301)).astype(np.float32)
    x[3, 7] = -25.0
    xb = _bf16(x)
    xf = synth.bf16_bits_to_fp32(xb)
    q, sa = quant(xb)
    assert q.min() >= -7 and q.max() <= 7
    for m in range(5):
        i = int(np.argmax(np.abs(xf[m])))
        assert abs(int(q[m, i])) == 7
        assert sa[m] == np.float32(np.abs(xf[m]).max()) / np.float32(7.0)
        qm, sam = quant(xb[m:m + 1])
        np.testing.assert_array_equal(qm[0], q[m])
        assert sam[0] == sa[m]
        o = np.argsort(xf[m], kind="stable")
        assert np.all(np.diff(q[m][o].astype(int)) >= 0)
    # at most half a step of reconstruction error
    err = np.abs(xf - q.astype(np.float64) * sa[:, None].astype(np.float64))
    assert np.all(err <= sa[:, None] * (0.5 + 1e-5) + 1e-30)
    qn, san = quant(_bf16(-x))
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(san, sa)
    for e in (-3, 5):
        q2, sa2 = quant(_bf16(x * np.float32(2.0 ** e)))
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(sa2, sa * np.float32(2.0 ** e))


def test_quant_a4_pins():
    quant_a4_pins(oracle.quant_act_a4)


def _sext4(v):
    v = v.astype(np.int64) & 15
    return np.where(v >= 8, v - 16, v)


def _dot8(a, b):
    """Signed 4-bit dot product of 8 nibble pairs, element-wise over uint32 arrays."""
    s = np.zeros(a.shape, np.int64)
    for p in range(8):
        s += _sext4(a >> (4 * p)) * _sext4(b >> (4 * p))
    return s


def act4_product(packed_w, act, N, K):
    """Sum_k w*x through the documented decode: masks 0x33333333 and
    (word >> 2) & 0x33333333 of each T32x128 weight word, paired nibble by
    nibble with the two words of the matching A4I activation chunk, minus
    sum_k x (codes are w + 1).  Pure numpy, from the two layout definitions."""
    KT = -(-K // 128)
    W32 = np.ascontiguousarray(packed_w).view("<u4").astype(np.int64)
    A32 = np.ascontiguousarray(act).view("<u4").astype(np.int64)
    nchunk = A32.size // 2
    xa = np.zeros(KT * 8, np.int64)
    xb = np.zeros(KT * 8, np.int64)
    xa[:nchunk], xb[:nchunk] = A32[0::2], A32[1::2]
    sumx = int((_dot8(xa, np.full_like(xa, 0x11111111)) +
                _dot8(xb, np.full_like(xb, 0x11111111))).sum())
    t = np.repeat(np.arange(KT), 8)
    kg = np.tile(np.arange(8), KT)
    y = np.zeros(N, np.int64)
    for n in range(N):
        s, r = divmod(n, 32)
        rg, q = divmod(r, 4)
        w = W32[(s * KT + t) * 256 + (8 * rg + kg) * 4 + q]
        y[n] = int((_dot8(w & 0x33333333, xa) + _dot8((w >> 2) & 0x33333333, xb)).sum()) - sumx
    return y


def act4_pins(pack, unpack, nbytes):
    ex = _load("worked_examples.json")["act4_layout"]
    b = pack(np.array([ex["q"]], np.int8))
    np.testing.assert_array_equal(b, np.array(ex["bytes"], np.uint8))
    # size: rows padded to 32 values, half a byte per value
    for M, K in [(1, 1), (1, 32), (2, 33), (3, 2560), (1, 27648)]:
        assert nbytes(M, K) == M * (-(-K // 32) * 16)
    # every value position is its own nibble, padding stays zero
    K = 48
    base = pack(np.zeros((1, K), np.int8))
    assert base.size == 32 and not base.any()
    seen = set()
    for k in range(K):
        e = np.zeros((1, K), np.int8)
        e[0, k] = 1
        d = np.nonzero(pack(e))[0]
        assert d.size == 1
        v = int(pack(e)[d[0]])
        assert v in (0x01, 0x10)
        seen.add((int(d[0]), v))
    assert len(seen) == K and max(i for i, _ in seen) < K // 2
    # round trip over the whole int4 range, ragged K, several rows
    rng = np.random.default_rng(17)
    for M, K in [(1, 1), (1, 15), (2, 33), (3, 300), (1, 2560)]:
        q = rng.integers(-8, 8, size=(M, K), dtype=np.int8)
        b = pack(q)
        assert b.size == nbytes(M, K)
        np.testing.assert_array_equal(unpack(b, M, K), q)
    # the layout pairs each activation with its weight code under the decode
    for N, K in [(5, 16), (40, 300), (33, 129), (7, 1000)]:
        w = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
        q = rng.integers(-8, 8, size=(1, K), dtype=np.int8)
        ref = q.astype(np.int64) @ w.astype(np.int64).T
        np.testing.assert_array_equal(act4_product(oracle.pack(w), pack(q), N, K), ref[0])


def test_act4_pins():
    act4_pins(oracle.pack_act4, oracle.unpack_act4, oracle.act4_bytes)


def test_pack_act4_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.pack_act4(np.array([[8]], np.int8))
    with pytest.raises(ValueError):
        oracle.pack_act4(np.array([[-9]], np.int8))


def test_synth_distributions():
    x, w = synth.gemv_case(256, 4096, seed=3)
    assert x.dtype == np.int8 and x.min() >= -127 and x.max() <= 127
    frac = [float(np.mean(w == v)) for v in (-1, 0, 1)]
    assert all(abs(f - 1 / 3) < 0.01 for f in frac)
    x, w = synth.gemv_case(256, 4096, seed=3, sparse=True)
    assert abs(float(np.mean(w == 0)) - 0.6) < 0.01
    assert abs(float(np.mean(w == 1)) - 0.2) < 0.01
    # same seed, same arrays
    x2, w2 = synth.gemv_case(256, 4096, seed=3, sparse=True)
    np.testing.assert_array_equal(w, w2)
    np.testing.assert_array_equal(x, x2)
