"""CPU-only tests of libw2a8.so: it loads, exports what include/*.h declares,
its size formulas and host steps agree with the oracle, and its argument
validation rejects bad calls before any device work.

No device computation is requested here: every device entry point is called
with exactly one invalid argument, which the library rejects before it makes
any HIP call (the fake pointers below are never dereferenced).
"""
import ctypes
import functools
import glob
import os
import re

import numpy as np
import pytest
import torch

import oracle
import synth
import w2a8_gemv_amd as w2a8

from conftest import ROOT

ST = {"OK": 0, "NULL": 1, "SHAPE": 2, "ALIGN": 3, "VALUE": 4, "BUFSIZE": 5, "NODEVICE": 6,
      "ARCH": 7, "SCRATCH": 9}
F = ctypes.c_float
FAKE = 0x10000          # 16-byte aligned stand-in, never dereferenced
FAKE_ODD = 0x10004      # 4-byte aligned only


def _declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M):
            names.append(m.group(1))
    return sorted(set(names))


def test_header_status_codes_match_library():
    text = open(os.path.join(ROOT, "include", "w2a8.h")).read()
    codes = dict((k, int(v)) for k, v in re.findall(r"W2A8_(?:ERR_)?(\w+)\s*=\s*(\d+)", text))
    assert codes["OK"] == 0 and len(codes) == 10
    L = w2a8.lib()
    for v in codes.values():
        assert L.w2a8_status_str(v) and L.w2a8_status_str(v) != b"unknown status"
    assert L.w2a8_status_str(99) == b"unknown status"


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    expected = {"w2a8_status_str", "w2a8_layout_version", "w2a8_packed_bytes",
                "w2a8_workspace_bytes", "w2a8_ternarize_absmean", "pack_ternary",
                "unpack_ternary", "quant_act_int8", "w2a8_gemv", "w2a8_gemm",
                "w2a8_tune_gemv", "w2a8_gemv_plan", "w2a8_linear_plan", "w2a8_tune_gemm",
                "w2a8_tune_gemv_force",
                "w2a8_tune_gemm_ring", "w2a8_tune_gemm_pipe",
                "w2a8_gemv_noalloc",
                "w2a8_linear_gemv", "w2a8_gemv_grouped", "w2a8_linear_gemv_grouped",
                "w2a4_act_bytes", "pack_act_int4", "quant_act_int4", "w2a4_gemv",
                "w2a4_linear_gemv"}
    assert expected.issubset(set(names)), set(names) ^ expected
    L = ctypes.CDLL(w2a8.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_layout_version():
    assert w2a8.layout_version() == 1


@pytest.mark.parametrize("N,K", [(1, 1), (31, 127), (32, 128), (33, 129), (2560, 2560),
                                 (55296, 5120), (5120, 27648), (3200, 3200)])
def test_packed_bytes_matches_oracle(N, K):
    assert w2a8.packed_bytes(N, K) == oracle.packed_bytes(N, K)


def test_packed_bytes_is_n_k_over_4_on_workload_shapes():
    for N, K in synth.SWEEP_SHAPES + synth.LARGE_SHAPES + synth.GEMM_SHAPES:
        assert w2a8.packed_bytes(N, K) == N * K // 4


def test_size_queries_reject_bad_shapes():
    L = w2a8.lib()
    assert L.w2a8_packed_bytes(0, 5) == -1
    assert L.w2a8_packed_bytes(5, 0) == -1
    assert L.w2a8_packed_bytes(5, 1048448 + 1) == -1
    assert L.w2a8_workspace_bytes(0, 5, 5) == -1
    assert L.w2a8_workspace_bytes(1, 5, 5) == 0 and L.w2a8_workspace_bytes(1, 5, 27648) > 0


# ---------------------------------------------------------------------------
# a2 parity: the library's packer is byte-identical to the oracle's
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,seed", [(1, 1, 0), (31, 127, 1), (33, 129, 2), (64, 384, 3),
                                      (97, 300, 4), (5, 1000, 5), (2560, 2560, 6)])
def test_pack_matches_oracle_bytes(N, K, seed):
    rng = np.random.default_rng(seed)
    w = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    mine = w2a8.pack_ternary(torch.from_numpy(w)).numpy()
    ref = oracle.pack(w)
    np.testing.assert_array_equal(mine, ref)
    back = w2a8.unpack_ternary(torch.from_numpy(ref), N, K).numpy()
    np.testing.assert_array_equal(back, w)


def test_pack_matches_oracle_on_sparse_workload_rows():
    # first 4096 rows of the 55296 x 5120 workload (P(0) = 0.6)
    x, w = synth.gemv_case(4096, 5120, synth.LARGE_SEEDS[1], sparse=True)
    np.testing.assert_array_equal(w2a8.pack_ternary(torch.from_numpy(w)).numpy(), oracle.pack(w))


def test_pack_rejects_non_ternary():
    w = torch.zeros((4, 4), dtype=torch.int8)
    w[2, 3] = 2
    with pytest.raises(w2a8.W2A8Error) as e:
        w2a8.pack_ternary(w)
    assert e.value.status == ST["VALUE"]
    w[2, 3] = -128
    with pytest.raises(w2a8.W2A8Error):
        w2a8.pack_ternary(w)


def test_unpack_rejects_code_11():
    p = w2a8.pack_ternary(torch.zeros((3, 3), dtype=torch.int8))
    p[0] = 0xFF
    with pytest.raises(w2a8.W2A8Error) as e:
        w2a8.unpack_ternary(p, 3, 3)
    assert e.value.status == ST["VALUE"]


def test_pack_bufsize_and_null():
    L = w2a8.lib()
    w = np.zeros((32, 128), np.int8)
    out = np.zeros(1024, np.uint8)
    pw, po = w.ctypes.data_as(ctypes.c_void_p), out.ctypes.data_as(ctypes.c_void_p)
    assert L.pack_ternary(pw, 32, 128, po, 1023) == ST["BUFSIZE"]
    assert L.pack_ternary(None, 32, 128, po, 1024) == ST["NULL"]
    assert L.pack_ternary(pw, 32, 128, None, 1024) == ST["NULL"]
    assert L.pack_ternary(pw, 0, 128, po, 1024) == ST["SHAPE"]
    assert L.pack_ternary(pw, 32, 128, po, 1024) == ST["OK"]
    assert L.unpack_ternary(po, 1023, 32, 128, pw) == ST["BUFSIZE"]


# ---------------------------------------------------------------------------
# a1 parity: the library's ternarizer is bit-identical to the oracle's
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("N,K,seed", [(1, 1, 0), (7, 300, 1), (64, 640, 2), (1024, 1024, 3)])
def test_ternarize_matches_oracle(N, K, seed):
    _, W = synth.linear_case(1, N, K, seed=seed)
    wq, sw = w2a8.ternarize_absmean(torch.from_numpy(W))
    owq, osw = oracle.ternarize_absmean(W)
    assert np.float32(sw) == osw
    np.testing.assert_array_equal(wq.numpy(), owq)


def test_ternarize_matches_oracle_full_linear_shape():
    _, W = synth.linear_case(1, 13824, 2560, seed=synth.LINEAR_SEEDS[1])
    wq, sw = w2a8.ternarize_absmean(torch.from_numpy(W))
    owq, osw = oracle.ternarize_absmean(W)
    assert np.float32(sw) == osw
    np.testing.assert_array_equal(wq.numpy(), owq)


def test_ternarize_worked_examples_and_zero():
    for W, sw_e, wq_e in [([[0.75, 0.25], [-0.25, -0.75]], 0.5, [[1, 0], [0, -1]]),
                          ([[0.0, 0.0]], 0.0, [[0, 0]])]:
        wq, sw = w2a8.ternarize_absmean(torch.tensor(W, dtype=torch.float32))
        assert sw == sw_e
        assert wq.tolist() == wq_e


# ---------------------------------------------------------------------------
# argument validation of the device entry points (rejected before any HIP call)
# ---------------------------------------------------------------------------
# K of 64 tiles: the plan may split the k-range, so the workspace is required
KS = 8192


def _gemv(**kw):
    a = dict(wp=FAKE, x=FAKE, N=64, K=KS, y=FAKE, sa=FAKE, sw=1.0, yf=FAKE, ws=FAKE,
             wsb=1 << 20)
    a.update(kw)
    return w2a8.lib().w2a8_gemv(a["wp"], a["x"], a["N"], a["K"], a["y"], a["sa"], F(a["sw"]),
                                a["yf"], a["ws"], a["wsb"], None)


def test_gemv_validation():
    assert _gemv(wp=None) == ST["NULL"]
    assert _gemv(x=None) == ST["NULL"]
    assert _gemv(ws=None) == ST["NULL"]
    assert _gemv(y=None, yf=None) == ST["NULL"]
    assert _gemv(sa=None) == ST["NULL"]            # y_f32 needs s_a
    assert _gemv(N=0) == ST["SHAPE"]
    assert _gemv(K=0) == ST["SHAPE"]
    assert _gemv(K=1048448 + 128) == ST["SHAPE"]
    assert _gemv(N=(1 << 30) + 1) == ST["SHAPE"]
    assert _gemv(wp=FAKE + 8) == ST["ALIGN"]
    assert _gemv(x=FAKE + 1) == ST["ALIGN"]
    assert _gemv(y=FAKE_ODD) == ST["ALIGN"]
    assert _gemv(yf=FAKE_ODD) == ST["ALIGN"]
    assert _gemv(sa=FAKE + 2) == ST["ALIGN"]
    assert _gemv(wsb=w2a8.workspace_bytes(1, 64, KS) - 1) == ST["BUFSIZE"]


def test_gemv_noalloc_validation():
    L = w2a8.lib()

    def g(**kw):
        a = dict(wp=FAKE, x=FAKE, N=64, K=KS, y=FAKE, sa=FAKE, sw=1.0, yf=FAKE)
        a.update(kw)
        return L.w2a8_gemv_noalloc(a["wp"], a["x"], a["N"], a["K"], a["y"], a["sa"], F(a["sw"]),
                                   a["yf"], None)
    assert g(wp=None) == ST["NULL"]
    assert g(x=None) == ST["NULL"]
    assert g(y=None, yf=None) == ST["NULL"]
    assert g(sa=None) == ST["NULL"]
    assert g(N=0) == ST["SHAPE"]
    assert g(K=1048448 + 1) == ST["SHAPE"]
    assert g(x=FAKE + 1) == ST["ALIGN"]
    assert g(yf=FAKE_ODD) == ST["ALIGN"]
    # scratch: 1 MiB of 8-byte words, one per padded row, needed when K splits
    assert g(N=131072) not in (ST["SCRATCH"], ST["NULL"], ST["ALIGN"], ST["SHAPE"])
    assert g(N=131073) == ST["SCRATCH"]
    assert g(N=131073, K=2560) not in (ST["SCRATCH"], ST["NULL"], ST["ALIGN"], ST["SHAPE"])
    assert L.w2a8_status_str(ST["SCRATCH"]) != b"unknown status"


def _gemm(**kw):
    a = dict(wp=FAKE, x=FAKE, M=8, N=64, K=256, y=FAKE, sa=FAKE, sw=1.0, yf=FAKE, ws=FAKE,
             wsb=1 << 24)
    a.update(kw)
    return w2a8.lib().w2a8_gemm(a["wp"], a["x"], a["M"], a["N"], a["K"], a["y"], a["sa"],
                                F(a["sw"]), a["yf"], a["ws"], a["wsb"], None)


def test_gemm_validation():
    assert _gemm(wp=None) == ST["NULL"]
    assert _gemm(x=None) == ST["NULL"]
    assert _gemm(y=None, yf=None) == ST["NULL"]
    assert _gemm(sa=None) == ST["NULL"]
    assert _gemm(ws=None) == ST["NULL"]            # this shape needs split-K scratch
    assert _gemm(M=0) == ST["SHAPE"]
    assert _gemm(M=(1 << 20) + 1) == ST["SHAPE"]
    assert _gemm(N=0) == ST["SHAPE"]
    assert _gemm(x=FAKE + 4) == ST["ALIGN"]
    assert _gemm(y=FAKE_ODD) == ST["ALIGN"]
    assert _gemm(wsb=w2a8.workspace_bytes(8, 64, 256) - 1) == ST["BUFSIZE"]


def _linear(entry="w2a8_linear_gemv", **kw):
    a = dict(wp=FAKE, xb=FAKE, N=64, K=KS, sw=1.0, yf=FAKE, y=FAKE, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    return getattr(w2a8.lib(), entry)(a["wp"], a["xb"], a["N"], a["K"], F(a["sw"]), a["yf"],
                                      a["y"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("entry", ["w2a8_linear_gemv", "w2a4_linear_gemv"])
def test_linear_gemv_validation(entry):
    _linear = functools.partial(globals()["_linear"], entry)
    assert _linear(wp=None) == ST["NULL"]
    assert _linear(xb=None) == ST["NULL"]
    assert _linear(yf=None) == ST["NULL"]          # the fp32 output is required
    assert _linear(ws=None) == ST["NULL"]
    assert _linear(N=0) == ST["SHAPE"]
    assert _linear(K=1048448 + 1) == ST["SHAPE"]
    assert _linear(xb=FAKE + 2) == ST["ALIGN"]
    assert _linear(yf=FAKE_ODD) == ST["ALIGN"]
    assert _linear(y=FAKE_ODD) == ST["ALIGN"]
    assert _linear(wsb=w2a8.workspace_bytes(1, 64, KS) - 1) == ST["BUFSIZE"]


def _arr(ctype, vals):
    return None if vals is None else (ctype * len(vals))(*vals)


def _grouped(linear=False, **kw):
    Ns = kw.pop("Ns", [64, 33, 100])
    G = len(Ns)
    a = dict(G=G, wp=[FAKE] * G, x=FAKE, K=KS, sa=FAKE, sw=[1.0] * G, y=[FAKE] * G,
             yf=[FAKE] * G, ws=FAKE, wsb=1 << 20)
    a.update(kw)
    L = w2a8.lib()
    V, I64A = ctypes.c_void_p, ctypes.c_int64
    args = (a["G"], _arr(V, a["wp"]), _arr(I64A, Ns), a["K"])
    if linear:
        return L.w2a8_linear_gemv_grouped(*args, a["x"], _arr(F, a["sw"]), _arr(V, a["yf"]),
                                          _arr(V, a["y"]), a["ws"], a["wsb"], None)
    return L.w2a8_gemv_grouped(*args, a["x"], a["sa"], _arr(F, a["sw"]), _arr(V, a["y"]),
                               _arr(V, a["yf"]), a["ws"], a["wsb"], None)


@pytest.mark.parametrize("linear", [False, True], ids=["gemv", "linear"])
def test_grouped_validation(linear):
    g = lambda **kw: _grouped(linear, **kw)                      # noqa: E731
    assert g(G=0) == ST["SHAPE"]
    assert g(G=9, Ns=[64] * 9) == ST["SHAPE"]                    # more than W2A8_MAX_GROUPS
    assert g(Ns=[64, 0, 100]) == ST["SHAPE"]
    assert g(K=0) == ST["SHAPE"]
    assert g(Ns=[1 << 30, 32]) == ST["SHAPE"]                    # padded rows above 2^30
    assert g(wp=None) == ST["NULL"]
    assert g(wp=[FAKE, None, FAKE]) == ST["NULL"]
    assert g(sw=None) == ST["NULL"]
    assert g(x=None) == ST["NULL"]
    assert g(ws=None) == ST["NULL"]
    if linear:
        assert g(yf=None) == ST["NULL"]
    assert g(wp=[FAKE, FAKE + 8, FAKE]) == ST["ALIGN"]
    assert g(yf=[FAKE, FAKE, FAKE_ODD]) == ST["ALIGN"]
    assert g(y=[FAKE_ODD, FAKE, FAKE]) == ST["ALIGN"]
    assert g(x=FAKE + 2) == ST["ALIGN"]
    need = sum(w2a8.workspace_bytes(1, n, KS) for n in (64, 33, 100))
    assert g(wsb=need - 1) == ST["BUFSIZE"]
    assert g(K=256, ws=None, wsb=0) not in (ST["NULL"], ST["ALIGN"], ST["BUFSIZE"])
    if linear:
        assert g(yf=[FAKE, None, FAKE]) == ST["NULL"]          # every fp32 output required
    else:
        assert g(y=[FAKE, None, FAKE], yf=[FAKE, None, FAKE]) == ST["NULL"]   # no output
        assert g(sa=None) == ST["NULL"]                          # y_f32 needs s_a
        assert g(sa=FAKE + 2) == ST["ALIGN"]


def test_act4_bytes_and_host_packer_match_oracle():
    for M, K in [(1, 1), (1, 31), (1, 32), (2, 33), (3, 2560), (1, 27648)]:
        assert w2a8.act4_bytes(M, K) == oracle.act4_bytes(M, K)
    L = w2a8.lib()
    assert L.w2a4_act_bytes(0, 16) == -1 and L.w2a4_act_bytes(1, 0) == -1
    rng = np.random.default_rng(4)
    for M, K in [(1, 1), (1, 15), (2, 33), (3, 300), (1, 2560), (2, 1000)]:
        q = rng.integers(-8, 8, size=(M, K), dtype=np.int8)
        np.testing.assert_array_equal(w2a8.pack_act_int4(torch.from_numpy(q)).numpy(),
                                      oracle.pack_act4(q))


def test_pack_act_int4_validation():
    L = w2a8.lib()
    q = np.zeros((1, 40), np.int8)
    out = np.zeros(64, np.uint8)
    qp, op = q.ctypes.data, out.ctypes.data
    assert L.pack_act_int4(None, 1, 40, op, 64) == ST["NULL"]
    assert L.pack_act_int4(qp, 1, 40, None, 64) == ST["NULL"]
    assert L.pack_act_int4(qp, 0, 40, op, 64) == ST["SHAPE"]
    assert L.pack_act_int4(qp, 1, 40, op, 31) == ST["BUFSIZE"]
    for bad in (8, -9, 127):
        q[0, 17] = bad
        assert L.pack_act_int4(qp, 1, 40, op, 64) == ST["VALUE"]
    q[0, 17] = -8
    assert L.pack_act_int4(qp, 1, 40, op, 64) == ST["OK"]


def test_w2a4_validation():
    L = w2a8.lib()
    assert L.quant_act_int4(None, 1, 16, FAKE, FAKE, None) == ST["NULL"]
    assert L.quant_act_int4(FAKE, 1, 16, None, FAKE, None) == ST["NULL"]
    assert L.quant_act_int4(FAKE, 0, 16, FAKE, FAKE, None) == ST["SHAPE"]
    assert L.quant_act_int4(FAKE, 1, 0, FAKE, FAKE, None) == ST["SHAPE"]
    assert L.quant_act_int4(FAKE + 2, 1, 16, FAKE, FAKE, None) == ST["ALIGN"]
    assert L.quant_act_int4(FAKE, 1, 16, FAKE + 8, FAKE, None) == ST["ALIGN"]

    def g(**kw):
        a = dict(wp=FAKE, x=FAKE, N=64, K=KS, y=FAKE, sa=FAKE, sw=1.0, yf=FAKE, ws=FAKE,
                 wsb=1 << 20)
        a.update(kw)
        return L.w2a4_gemv(a["wp"], a["x"], a["N"], a["K"], a["y"], a["sa"], F(a["sw"]),
                           a["yf"], a["ws"], a["wsb"], None)
    assert g(wp=None) == ST["NULL"]
    assert g(x=None) == ST["NULL"]
    assert g(ws=None) == ST["NULL"]
    assert g(y=None, yf=None) == ST["NULL"]
    assert g(sa=None) == ST["NULL"]
    assert g(N=0) == ST["SHAPE"]
    assert g(K=1048448 + 1) == ST["SHAPE"]
    assert g(x=FAKE + 8) == ST["ALIGN"]
    assert g(yf=FAKE_ODD) == ST["ALIGN"]
    assert g(wsb=w2a8.workspace_bytes(1, 64, KS) - 1) == ST["BUFSIZE"]


def test_quant_validation():
    L = w2a8.lib()
    assert L.quant_act_int8(None, 1, 16, FAKE, FAKE, None) == ST["NULL"]
    assert L.quant_act_int8(FAKE, 1, 16, None, FAKE, None) == ST["NULL"]
    assert L.quant_act_int8(FAKE, 1, 16, FAKE, None, None) == ST["NULL"]
    assert L.quant_act_int8(FAKE, 0, 16, FAKE, FAKE, None) == ST["SHAPE"]
    assert L.quant_act_int8(FAKE, 1, 0, FAKE, FAKE, None) == ST["SHAPE"]
    assert L.quant_act_int8(FAKE + 2, 1, 16, FAKE, FAKE, None) == ST["ALIGN"]
    assert L.quant_act_int8(FAKE, 1, 16, FAKE + 8, FAKE, None) == ST["ALIGN"]
    assert L.quant_act_int8(FAKE, 1, 16, FAKE, FAKE + 1, None) == ST["ALIGN"]


def test_workspace_formula():
    # GEMV: one 8-byte combining word per padded row, rounded up to 256 bytes,
    # when a plan may split the k-range (K >= 48 tiles with the default knobs)
    for N in (1, 31, 32, 2560, 55296):
        Np = -(-N // 32) * 32
        assert w2a8.workspace_bytes(1, N, 6017) == -(-(8 * Np) // 256) * 256
        assert w2a8.workspace_bytes(1, N, 27648) == -(-(8 * Np) // 256) * 256
        # no plan splits K <= 47 tiles: no workspace
        for K in (1, 1000, 2560, 6016):
            assert w2a8.workspace_bytes(1, N, K) == 0
    # large batched outputs never split K: no workspace needed
    assert w2a8.workspace_bytes(512, 13824, 2560) == 0


def test_workspace_rule_matches_the_plans():
    # w2a8_workspace_bytes(1, N, K) is 0 exactly when no device's plan splits
    # a strip, under the default knobs and others
    pols = [w2a8.DEFAULT_GEMV_POLICY, (4, 4, 4, 3, 1), (1, 32, 8, 256, 10 ** 6), (8, 6, 8, 20, 100)]
    try:
        for pol in pols:
            w2a8.tune_gemv(*pol)
            for N in (1, 2560, 55296):
                for K in (1, 128, 385, 2560, 6016, 6017, 27648, 40000):
                    ws = w2a8.workspace_bytes(1, N, K)
                    # (kernel 3's 8 workgroups per strip are row slices, not k-ranges)
                    splits = [p[2] > 1 and p[0] != 3
                              for p in (w2a8.gemv_plan(N, K, cus) for cus in (1, 80, 256, 304))]
                    if ws == 0:
                        assert not any(splits), (pol, N, K)
                    kt = -(-K // 128)
                    assert (ws > 0) == (kt >= pol[4] or kt > pol[3]), (pol, N, K)
    finally:
        w2a8.tune_gemv(*w2a8.DEFAULT_GEMV_POLICY)


def test_gemv_accepts_null_workspace_only_when_unsplit():
    # Validation order: a NULL workspace is an error only when the k-range
    # may be split; otherwise validation passes on to the device query
    # (NODEVICE on this host without a GPU).
    L = w2a8.lib()
    nodev = (ST["NODEVICE"], ST["ARCH"], ST["OK"])
    assert L.w2a8_gemv(FAKE, FAKE, 64, 2560, FAKE, None, 1.0, None, None, 0, None) in nodev
    assert L.w2a8_gemv(FAKE, FAKE, 64, 27648, FAKE, None, 1.0, None, None, 0, None) == ST["NULL"]
    assert L.w2a8_linear_gemv(FAKE, FAKE, 64, 2560, 1.0, FAKE, None, None, 0, None) in nodev
    assert L.w2a8_linear_gemv(FAKE, FAKE, 64, 27648, 1.0, FAKE, None, None, 0, None) == ST["NULL"]
    assert L.w2a4_gemv(FAKE, FAKE, 64, 2560, FAKE, None, 1.0, None, None, 0, None) in nodev
    assert L.w2a4_gemv(FAKE, FAKE, 64, 27648, FAKE, None, 1.0, None, None, 0, None) == ST["NULL"]


def test_tuning_knobs_are_thread_safe():
    # Knob changes from one thread while others read plans and sizes: every
    # plan read must be one of the two policies' plans, never a mix.
    import threading
    a, b = w2a8.DEFAULT_GEMV_POLICY, (1, 32, 2, 3, 1)
    shapes = [(2560, 2560), (5120, 27648), (55296, 5120)]
    plans = {}
    try:
        for pol in (a, b):
            w2a8.tune_gemv(*pol)
            for nk in shapes:
                plans.setdefault(nk, set()).add(tuple(w2a8.gemv_plan(*nk, 256)))
        stop = threading.Event()
        bad = []

        def flip():
            i = 0
            while not stop.is_set():
                w2a8.tune_gemv(*(a if i % 2 else b))
                w2a8.tune_gemm(i % 4)
                i += 1

        def read():
            for _ in range(3000):
                for nk in shapes:
                    p = tuple(w2a8.gemv_plan(*nk, 256))
                    if p not in plans[nk]:
                        bad.append((nk, p))
        t = threading.Thread(target=flip)
        t.start()
        rs = [threading.Thread(target=read) for _ in range(3)]
        for r in rs:
            r.start()
        for r in rs:
            r.join()
        stop.set()
        t.join()
        assert not bad, bad[:5]
    finally:
        w2a8.tune_gemv(*a)
        w2a8.tune_gemm(0)


def test_tuning_knobs_validate():
    for bad in [(0, 8, 4, 256, 64), (4, 0, 4, 256, 64), (4, 33, 4, 256, 64), (4, 8, 3, 256, 64),
                (4, 8, 4, 257, 64), (4, 8, 4, 0, 64), (4, 8, 4, 256, 0), (65, 8, 4, 256, 64)]:
        with pytest.raises(w2a8.W2A8Error):
            w2a8.tune_gemv(*bad)
    with pytest.raises(w2a8.W2A8Error):
        w2a8.gemv_plan(0, 2560, 256)
    for bad in [(-1,), (5,)]:
        with pytest.raises(w2a8.W2A8Error):
            w2a8.tune_gemm(*bad)
    for bad in [(0, 1, 4), (17, 1, 4), (4, 0, 4), (4, 4097, 4), (4, 3, 3), (4, 3, 12), (1, 1, 0)]:
        with pytest.raises(w2a8.W2A8Error):
            w2a8.tune_gemm_ring(*bad)
    for ok in [(1, 1, 2), (16, 4096, 8), (0, 0, 0)]:
        w2a8.tune_gemm_ring(*ok)
    for bad in (-2, 10):
        with pytest.raises(w2a8.W2A8Error):
            w2a8.tune_gemm_pipe(bad)
    for ok in (0, 9, -1):
        w2a8.tune_gemm_pipe(ok)
    for bad in [(3, 1, 1, 4, 1), (2, 4, 1, 4, 0), (1, 4, 1, 8, 1), (2, 4, 1, 3, 1), (8, 1, 1, 4, 1),
                (3, 1, 8, 12, 1), (3, 2, 8, 4, 1), (3, 1, 8, 4, 0), (4, 1, 8, 4, 1)]:
        with pytest.raises(w2a8.W2A8Error):
            w2a8.tune_gemv_force(*bad)
    w2a8.tune_gemv_force(3, 1, 8, 6, 1)
    assert w2a8.workspace_bytes(1, 2560, 2560) == 0      # the row-slice kernel never splits
    w2a8.tune_gemv_force(0)


def test_linear_plan_properties():
    """The fused layers' plans keep every LDS region, run and workgroup within
    the kernels' bounds, split strips only where the workspace exists, and
    pick the shared ring kernel exactly where the ring plan has one wave per
    strip (int8)."""
    pols = [w2a8.DEFAULT_GEMV_POLICY, (1, 32, 8, 256, 10 ** 6), (64, 1, 8, 256, 1),
            (4, 4, 4, 3, 1), (16, 32, 2, 1, 1)]
    try:
        for pol in pols:
            w2a8.tune_gemv(*pol)
            for N in (1, 31, 2560, 2600, 16448, 55296, 400000):
                for K in (1, 127, 2560, 6912, 27648, 70000, 140000, 1048448):
                    ws = w2a8.workspace_bytes(1, N, K)
                    kt, ns = -(-K // 128), -(-N // 32)
                    for cus in (1, 80, 256, 304):
                        for int4 in (False, True):
                            kern, wk, sg, run, d = w2a8.linear_plan(N, K, cus, int4)
                            assert 1 <= wk <= 16 and 1 <= sg <= kt
                            assert sg == 1 or ws > 0, (pol, N, K, cus, int4)
                            ktw = -(-kt // sg)
                            if kern == 3:                 # shared k-ranges
                                assert wk <= ns and run == ktw and d in (2, 4, 6, 8, 12)
                                assert run * (64 if int4 else 128) <= 64 * 1024
                            elif kern == 4:               # per-wave runs (int4)
                                assert int4 and run <= 64 and run >= -(-ktw // wk)
                                assert wk * run * 64 <= 64 * 1024 and d in (2, 4, 6, 8, 12)
                            else:                         # workgroup kernel (int8)
                                assert kern == 1 and not int4
                            gp = w2a8.gemv_plan(N, K, cus)
                            if not int4 and gp[0] == 2:
                                # the ring plan's shape, where the plain GEMV takes it
                                assert (kern == 3) == (gp[1] == 1), (pol, N, K, cus)
    finally:
        w2a8.tune_gemv(*w2a8.DEFAULT_GEMV_POLICY)
    # the measured choices on a 256-CU device
    assert w2a8.linear_plan(5120, 27648, 256)[:4] == (3, 8, 12, 18)
    assert w2a8.linear_plan(55296, 5120, 256)[:4] == (3, 8, 1, 40)
    assert w2a8.linear_plan(20480, 3200, 256)[:4] == (3, 4, 1, 25)
    assert w2a8.linear_plan(13824, 2560, 256)[0] == 1
    assert w2a8.linear_plan(13824, 2560, 256, int4=True)[:4] == (4, 8, 1, 3)
    with pytest.raises(w2a8.W2A8Error):
        w2a8.linear_plan(0, 2560, 256)


def test_gemv_plan_properties():
    """The launch plan keeps every wave/workgroup within its documented bounds."""
    pols = [w2a8.DEFAULT_GEMV_POLICY, (1, 32, 8, 256, 10 ** 6), (1, 1, 4, 256, 10 ** 6),
            (64, 1, 8, 256, 1), (4, 4, 4, 3, 1), (16, 32, 2, 1, 1)]
    try:
        for pol in pols:
            w2a8.tune_gemv(*pol)
            for N in (1, 31, 2560, 55296):
                for K in (1, 127, 128, 2560, 27648, 100000, 1048448):
                    for cus in (1, 80, 256):
                        kern, wk, sg, u = w2a8.gemv_plan(N, K, cus)
                        assert kern in ((2, 3) if K % 16 == 0 else (1,))
                        if kern == 3:
                            # 8 row slices per strip: at most 4 waves per CU, or
                            # up to 8 on strips of 48-64 tiles
                            kt, ns = -(-K // 128), -(-N // 32)
                            assert (wk, sg) == (1, 8) and u in (4, 6)
                            assert kt <= 96 and (2 * ns <= cus or (ns <= cus and 48 <= kt <= 64))
                            continue
                        if kern == 2:
                            kt = -(-K // 128)
                            assert 1 <= sg <= kt and 1 <= wk <= 16 and u in (4, 6, 8, 12)
                            if sg > 1:
                                assert kt >= pol[4] and wk == 1
                            if -(-N // 32) >= 2 * cus:
                                assert (wk, sg) == (1, 1)
                            continue
                        kt = -(-K // 128)
                        ktw = -(-kt // sg)
                        run = -(-ktw // wk)
                        assert 1 <= sg <= kt and ktw <= pol[3]
                        assert 1 <= wk <= 16 and wk <= ktw
                        assert run <= 32                              # <= 4 staged chunks per lane
                        assert wk * run * 128 + wk * 128 + 16 <= 64 * 1024  # LDS per workgroup
                        assert u in (2, 4, 8) and u <= pol[2]
                        if kt < pol[4] and kt <= pol[3]:
                            assert sg == 1
    finally:
        w2a8.tune_gemv(*w2a8.DEFAULT_GEMV_POLICY)


def test_gemv_default_plans_of_the_measured_shapes():
    """The default plans (kernel, waves per workgroup, workgroups per strip,
    depth) on a 256-CU device for the shapes the rules were measured on.

    Ring kernel (K a multiple of 16): one wave per whole strip from two
    strips per CU up, the ring deeper the fewer strips per CU; single-wave
    workgroups with the k-range split to at most 4 waves per CU for strips
    of 48 tiles or more; 8-wave workgroups otherwise.  Batch kernel (ragged K; the same tile counts as the workload
    shapes, K one less): twice the waves with half-length runs in unsplit
    strips while there are no more strips than CUs, 4-wave workgroups above
    that, and a split over workgroups for strips of 48 k-tiles or more, into
    equal k-ranges where one of the two smaller counts gives them."""
    assert w2a8.DEFAULT_GEMV_POLICY == (4, 6, 8, 256, 48)
    ring = {(4800, 3200): (8, 1, 4), (13824, 2560): (8, 1, 4), (20480, 3200): (1, 1, 8),
            (5120, 27648): (1, 6, 8), (55296, 5120): (1, 1, 4), (6912, 5120): (8, 1, 6),
            (5120, 3456): (8, 1, 4)}
    for (N, K), plan in ring.items():
        assert tuple(w2a8.gemv_plan(N, K, 256)) == (2,) + plan, (N, K)
    # Row-slice kernel: at most 128 strips (4 single-wave workgroups per CU)
    # with strips of at most 64 tiles, or 96 from 64 strips, depth 6 above 40
    # tiles; and up to 256 strips of 48-64 tiles (where the ring plan would
    # split them), depth 4
    slices = {(2560, 2560): 4, (3840, 2560): 4, (3200, 3200): 4, (2560, 6912): 6,
              (3200, 10240): 6, (512, 4096): 4, (2048, 6912): 6, (2048, 10240): 6,
              (3840, 10240): 6, (32, 16): 4, (4096, 4096): 4, (4096, 11008): 6,
              (4800, 6912): 4, (8192, 6144): 4, (8192, 8192): 4, (8192, 6912): 4}
    for (N, K), d in slices.items():
        assert tuple(w2a8.gemv_plan(N, K, 256)) == (3, 1, 8, d), (N, K)
    for N, K in ((1536, 10240), (512, 14336), (4128, 2560), (2560, 12416), (10240, 6144),
                 (5120, 10240), (8224, 6144), (6912, 5120)):
        assert w2a8.gemv_plan(N, K, 256)[0] == 2, (N, K)
    # one wave per strip: ring depth by strips per CU (12 below 2.5, 8 up to 4,
    # 6 up to 5.5, then 4), from the depth sweep on many-strip shapes
    for N, d in ((16384, 12), (18432, 12), (20480, 8), (24576, 8), (27648, 8), (32768, 8), (41472, 6),
                 (55296, 4), (73728, 4)):
        for K in (2560, 5120):
            assert tuple(w2a8.gemv_plan(N, K, 256)) == (2, 1, 1, d), (N, K)
    # long strips below two strips per CU: floor(4 cus / NS) k-ranges (at most
    # 4 waves on every CU), depth 8 unless the runs are at most 5 tiles
    for (N, K), plan in {(12288, 14336): (1, 2, 8), (12288, 6912): (1, 2, 8),
                         (6144, 10240): (1, 5, 8), (4096, 27648): (1, 8, 8),
                         (1024, 14336): (1, 28, 4), (2048, 27648): (1, 16, 8)}.items():
        assert tuple(w2a8.gemv_plan(N, K, 256)) == (2,) + plan, (N, K)
    batch = {(2560, 2560): (8, 1, 2), (3840, 2560): (8, 1, 2), (3200, 3200): (8, 1, 2),
             (4800, 3200): (8, 1, 2), (1024, 1024): (4, 1, 2), (13824, 2560): (4, 1, 4),
             (20480, 3200): (4, 1, 4), (2560, 6912): (1, 9, 4), (3200, 10240): (1, 10, 4),
             (5120, 27648): (3, 12, 4), (55296, 5120): (8, 1, 4), (2560, 27648): (3, 12, 4),
             (8192, 8192): (1, 11, 4)}
    for (N, K), plan in batch.items():
        assert tuple(w2a8.gemv_plan(N, K - 1, 256)) == (1,) + plan, (N, K)
    # The same 80-strip matrix on a 64-CU device has more strips than CUs.
    assert tuple(w2a8.gemv_plan(2560, 2559, 64)) == (1, 4, 1, 4)


def test_binding_refuses_host_tensors_for_device_calls():
    with pytest.raises(ValueError):
        w2a8.quant_act_int8(torch.zeros((1, 16), dtype=torch.bfloat16))
