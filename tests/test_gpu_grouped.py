"""GPU parity of the grouped GEMV: several projections sharing one activation
row and K in one launch (w2a8_gemv_grouped, w2a8_linear_gemv_grouped).

Each projection's int32 output is compared bit-exactly with the oracle's
integer product, its fp32 output with the oracle's epilogue (the same two
correctly rounded products, so bit-identical); every output has a guard band.
The sets cover decode projections of a 2560-wide model (query/key/value
2560 + 640 + 640, gate/up 2 x 6912), ragged N and K, one to eight
projections, long K (strips split over workgroups, so the split-k combining
words of different projections share the workspace) and missing outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import w2a8_gemv_amd as w2a8

from gpu_util import CANARY_I32, GUARD, check_guard, dev, packed_on_device, to_dev

pytestmark = pytest.mark.gpu

GROUPS = [
    ([2560, 640, 640], 2560),
    ([6912, 6912], 2560),
    ([1], 1),
    ([31, 33, 1, 64], 129),
    ([100, 7, 300], 1000),
    ([1, 2, 3, 31, 32, 33, 63, 65], 15),
    ([31, 33, 1, 64, 97], 2000),     # row-slice kernel: ragged rows, a ragged last tile
    ([200, 33], 8192),               # row-slice kernel at depth 6
    ([5120], 27648),
    ([96, 40, 200], 27648),
    ([250, 1, 77, 129, 64, 32, 500, 3], 4000),
    ([2560, 2560], 6912),
]


def _case(Ns, K, seed):
    x, _ = synth.gemv_case(1, K, seed=seed)
    ws = [synth.gemv_case(n, K, seed=seed + 1 + g, sparse=g % 2 == 1)[1] for g, n in enumerate(Ns)]
    return x, ws


def _outputs(Ns, kinds):
    yi, yf = [], []
    for n, kind in zip(Ns, kinds):
        yi.append(torch.full((n + GUARD,), CANARY_I32, dtype=torch.int32, device=dev())
                  if "i" in kind else None)
        yf.append(torch.full((n + GUARD,), float("nan"), dtype=torch.float32, device=dev())
                  if "f" in kind else None)
    return yi, yf


def _run_grouped(Ns, K, x, ws, sw, sa, kinds, workspace=None):
    wps = [packed_on_device(w) for w in ws]
    yi, yf = _outputs(Ns, kinds)
    w2a8.w2a8_gemv_grouped(wps, to_dev(x), Ns, K, list(map(float, sw)),
                           y_i32=[None if y is None else y[:n] for y, n in zip(yi, Ns)],
                           y_f32=[None if y is None else y[:n] for y, n in zip(yf, Ns)],
                           s_a=to_dev(np.array([sa], np.float32)), workspace=workspace)
    torch.cuda.synchronize()
    return yi, yf


def _check(Ns, x, ws, sw, sa, yi, yf):
    for g, n in enumerate(Ns):
        acc = oracle.gemm_i32(x.reshape(1, -1), ws[g])
        if yi[g] is not None:
            check_guard(yi[g], n)
            np.testing.assert_array_equal(yi[g][:n].cpu().numpy(), acc[0], err_msg=f"proj {g}")
        if yf[g] is not None:
            check_guard(yf[g], n)
            ref = oracle.epilogue(acc, np.array([sa], np.float32), np.float32(sw[g]))
            np.testing.assert_array_equal(yf[g][:n].cpu().numpy(), ref[0], err_msg=f"proj {g}")


@pytest.mark.parametrize("Ns,K", GROUPS, ids=[f"{len(n)}x{K}" for n, K in GROUPS])
def test_grouped_gemv_matches_oracle(Ns, K):
    x, ws = _case(Ns, K, seed=sum(Ns) + K)
    sw = (np.arange(1, len(Ns) + 1, dtype=np.float32) * np.float32(0.0071)).astype(np.float32)
    sa = np.float32(0.0213)
    yi, yf = _run_grouped(Ns, K, x, ws, sw, sa, ["if"] * len(Ns))
    _check(Ns, x, ws, sw, sa, yi, yf)


def test_grouped_gemv_missing_outputs():
    Ns, K = [100, 64, 33, 300], 2560
    x, ws = _case(Ns, K, seed=5)
    sw = np.full(4, 0.5, np.float32)
    yi, yf = _run_grouped(Ns, K, x, ws, sw, np.float32(0.25), ["i", "f", "if", "i"])
    _check(Ns, x, ws, sw, np.float32(0.25), yi, yf)


def test_grouped_gemv_int32_only_without_scale():
    Ns, K = [64, 96], 512
    x, ws = _case(Ns, K, seed=6)
    wps = [packed_on_device(w) for w in ws]
    yi, _ = _outputs(Ns, ["i", "i"])
    w2a8.w2a8_gemv_grouped(wps, to_dev(x), Ns, K, [1.0, 1.0],
                           y_i32=[y[:n] for y, n in zip(yi, Ns)])
    torch.cuda.synchronize()
    _check(Ns, x, ws, [1.0, 1.0], np.float32(1), yi, [None, None])


@pytest.mark.parametrize("policy", [(1, 32, 8, 256, 10 ** 6), (64, 1, 8, 256, 1),
                                    (2, 2, 8, 7, 1), (16, 32, 4, 1, 1)])
def test_grouped_gemv_forced_splits(policy):
    try:
        w2a8.tune_gemv(*policy)
        for Ns, K in [([200, 33, 1], 3200), ([96, 40], 27648), ([33, 64, 31, 5], 1000)]:
            x, ws = _case(Ns, K, seed=K + len(Ns))
            sw = np.full(len(Ns), 0.03, np.float32)
            yi, yf = _run_grouped(Ns, K, x, ws, sw, np.float32(0.5), ["if"] * len(Ns))
            _check(Ns, x, ws, sw, np.float32(0.5), yi, yf)
    finally:
        w2a8.tune_gemv(*w2a8.DEFAULT_GEMV_POLICY)


def test_grouped_gemv_workspace_left_zeroed():
    """Three calls on one workspace (strips split over workgroups): every call
    exact, and the workspace all zero afterwards."""
    Ns, K = [700, 96, 33], 27648
    x, ws = _case(Ns, K, seed=9)
    need = sum(w2a8.workspace_bytes(1, n, K) for n in Ns)
    wsb = torch.zeros(need, dtype=torch.uint8, device=dev())
    sw = np.full(3, 0.01, np.float32)
    for _ in range(3):
        yi, yf = _run_grouped(Ns, K, x, ws, sw, np.float32(0.1), ["if"] * 3, workspace=wsb)
        _check(Ns, x, ws, sw, np.float32(0.1), yi, yf)
    assert int(wsb.count_nonzero()) == 0


def test_grouped_equals_separate_calls():
    """The grouped launch and one w2a8_gemv per projection agree bit for bit."""
    Ns, K = [2560, 640, 640], 2560
    x, ws = _case(Ns, K, seed=12)
    sw = np.array([0.01, 0.02, 0.03], np.float32)
    sa = to_dev(np.array([0.3], np.float32))
    yi, yf = _run_grouped(Ns, K, x, ws, sw, np.float32(0.3), ["if"] * 3)
    xd = to_dev(x)
    for g, n in enumerate(Ns):
        a = torch.empty(n, dtype=torch.int32, device=dev())
        b = torch.empty(n, dtype=torch.float32, device=dev())
        w2a8.w2a8_gemv(packed_on_device(ws[g]), xd, n, K, y_i32=a, s_a=sa, s_w=float(sw[g]),
                       y_f32=b)
        torch.cuda.synchronize()
        assert torch.equal(a, yi[g][:n]) and torch.equal(b, yf[g][:n])


# ---------------------------------------------------------------------------
# Grouped linear GEMV: quantize the bf16 token, then every projection
# ---------------------------------------------------------------------------
def _bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(bits.astype(np.uint16)).view(torch.bfloat16)


LINEAR_GROUPS = [([2560, 640, 640], 2560), ([6912, 6912], 2560), ([33, 1, 100], 7),
                 ([96, 40, 200], 27648), ([1, 2, 3, 31, 32, 33, 63, 65], 1000)]


@pytest.mark.parametrize("Ns,K", LINEAR_GROUPS, ids=[f"{len(n)}x{K}" for n, K in LINEAR_GROUPS])
def test_grouped_linear_matches_oracle(Ns, K):
    xb, _ = synth.linear_case(1, 1, K, seed=K + 1)
    ws = [synth.gemv_case(n, K, seed=n + g)[1] for g, n in enumerate(Ns)]
    sw = (np.arange(1, len(Ns) + 1, dtype=np.float32) * np.float32(0.013)).astype(np.float32)
    wps = [packed_on_device(w) for w in ws]
    yi, yf = _outputs(Ns, ["if"] * len(Ns))
    w2a8.w2a8_linear_gemv_grouped(wps, _bf16_dev(xb.reshape(-1)), Ns, K, list(map(float, sw)),
                                  [y[:n] for y, n in zip(yf, Ns)],
                                  y_i32=[y[:n] for y, n in zip(yi, Ns)])
    torch.cuda.synchronize()
    xq, sa = oracle.quant_act(xb)
    for g, n in enumerate(Ns):
        acc = oracle.gemm_i32(xq, ws[g])
        check_guard(yi[g], n)
        check_guard(yf[g], n)
        np.testing.assert_array_equal(yi[g][:n].cpu().numpy(), acc[0])
        np.testing.assert_array_equal(yf[g][:n].cpu().numpy(),
                                      oracle.epilogue(acc, sa, sw[g])[0])


def test_grouped_linear_equals_single_linear_calls():
    Ns, K = [6912, 6912], 2560
    xb, W = synth.linear_case(1, 1, K, seed=31)
    ws = [synth.gemv_case(n, K, seed=40 + g)[1] for g, n in enumerate(Ns)]
    wps = [packed_on_device(w) for w in ws]
    x = _bf16_dev(xb.reshape(-1))
    ys = w2a8.linear_grouped(x, wps, [0.02, 0.03], Ns, K)
    for g, n in enumerate(Ns):
        y1 = w2a8.linear(x, wps[g], [0.02, 0.03][g], n, K)
        torch.cuda.synchronize()
        assert torch.equal(ys[g], y1)
