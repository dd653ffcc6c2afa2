"""GPU parity of the W2A4 variant (int4 activations, A4I layout).

Quantizer: the packed bytes and per-token scales are bit-identical to the
oracle's int4 quantizer followed by its A4I packer (both take every decision
with the same correctly rounded fp32 operations).
GEMV: the int32 output is bit-exact against the oracle's integer product of
the int4 values with the ternary weights; the fp32 epilogue is bit-identical
to the oracle's.  Activations span the whole int4 range -8..7; shapes cover
ragged N and K (K % 32 != 0 exercises the row padding), several tiles,
strips split over workgroups, the sweep shapes and the two large shapes.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import w2a8_gemv_amd as w2a8

from gpu_util import check_guard, dev, guarded, packed_on_device, to_dev

pytestmark = pytest.mark.gpu


def _bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(bits.astype(np.uint16)).view(torch.bfloat16)


# K % 16 == 0 up to 32768 takes the one-read kernel (an odd number of 16-value
# chunks leaves the last granule's second half to the lane after the last);
# other K the two-pass kernel.
@pytest.mark.parametrize("M,K", [(1, 1), (1, 7), (1, 15), (1, 16), (1, 31), (2, 33), (3, 100),
                                 (1, 2560), (4, 4000), (1, 27648), (17, 64), (3, 48),
                                 (2, 8192), (5, 8176), (1, 8208), (128, 2560),
                                 # 2 to 4 chunks per lane up to K = 32768 (odd chunk
                                 # counts among them), then the two-pass kernel
                                 (1, 16400), (2, 24576), (1, 32752), (3, 32768), (1, 32784)])
def test_quant_int4_matches_oracle(M, K):
    xb, _ = synth.linear_case(M, 1, K, seed=3 * M + K)
    nbytes = w2a8.act4_bytes(M, K)
    out = torch.full((nbytes + 64,), 0xA5, dtype=torch.uint8, device=dev())
    xq4, sa = w2a8.quant_act_int4(_bf16_dev(xb), x_q4=out)
    torch.cuda.synchronize()
    q, osa = oracle.quant_act_a4(xb)
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got[:nbytes], oracle.pack_act4(q))
    assert (got[nbytes:] == 0xA5).all(), "write past the end of the A4I rows"
    np.testing.assert_array_equal(sa.cpu().numpy(), osa)


def test_quant_int4_worked_examples_and_zero_rows():
    rows = [[1.0, -0.5, 0.25, 0.0], [2.0, 1.0, -1.0, 0.5], [1.75, 0.625, -0.375, 0.125],
            [0.0, 0.0, 0.0, 0.0], [-3.0, -3.0, -3.0, -3.0]]
    bits = synth.fp32_to_bf16_bits(np.array(rows, np.float32))
    xq4, sa = w2a8.quant_act_int4(_bf16_dev(bits))
    torch.cuda.synchronize()
    q = oracle.unpack_act4(xq4.cpu().numpy(), 5, 4)
    assert q[0].tolist() == [7, -4, 2, 0]
    assert q[1].tolist() == [7, 4, -4, 2]
    assert q[2].tolist() == [7, 2, -2, 0]
    assert q[3].tolist() == [0, 0, 0, 0] and sa.cpu().numpy()[3] == 0.0
    oq, osa = oracle.quant_act_a4(bits)
    np.testing.assert_array_equal(q, oq)
    np.testing.assert_array_equal(sa.cpu().numpy(), osa)


def _gemv_a4(q, w, N, K, sa=None, sw=1.0, want_f32=False, workspace=None):
    xq4 = to_dev(oracle.pack_act4(q.reshape(1, -1)))
    y = guarded(N, torch.int32)
    yf = guarded(N, torch.float32) if want_f32 else None
    w2a8.w2a4_gemv(packed_on_device(w), xq4, N, K, y_i32=y[:N], s_a=sa, s_w=sw,
                   y_f32=None if yf is None else yf[:N], workspace=workspace)
    torch.cuda.synchronize()
    check_guard(y, N)
    if yf is None:
        return y[:N].cpu().numpy()
    check_guard(yf, N)
    return y[:N].cpu().numpy(), yf[:N].cpu().numpy()


SHAPES = [(1, 1), (1, 16), (33, 7), (64, 31), (97, 100), (32, 128), (100, 129), (300, 1000),
          (2560, 2560), (3840, 2560), (13824, 2560), (2560, 6912), (3200, 3200), (4800, 3200),
          (3200, 10240), (20480, 3200), (96, 27648), (130, 4000)]


@pytest.mark.parametrize("N,K", SHAPES)
def test_w2a4_gemv_matches_oracle(N, K):
    q, w = synth.gemv_a4_case(N, K, seed=N + 7 * K, sparse=N % 2 == 1)
    y = _gemv_a4(q, w, N, K)
    np.testing.assert_array_equal(y, oracle.gemm_i32(q.reshape(1, -1), w)[0])


@pytest.mark.parametrize("N,K", [(5120, 27648), (55296, 5120)])
def test_w2a4_gemv_large_shapes(N, K):
    q, w = synth.gemv_a4_case(N, K, seed=N, sparse=True)
    y = _gemv_a4(q, w, N, K)
    np.testing.assert_array_equal(y, oracle.gemm_i32(q.reshape(1, -1), w)[0])


def test_w2a4_gemv_extremes():
    """-8 everywhere against all -1 and all +1 weights: +-8K, the largest magnitudes."""
    for N, K in [(40, 3000), (64, 27648)]:
        q = np.full(K, -8, np.int8)
        for v in (-1, 1):
            w = np.full((N, K), v, np.int8)
            y = _gemv_a4(q, w, N, K)
            assert np.all(y == -8 * K * v)


def test_w2a4_gemv_fp32_epilogue():
    N, K = 700, 2560
    q, w = synth.gemv_a4_case(N, K, seed=5)
    sa = np.array([0.0371], np.float32)
    sw = np.float32(0.0213)
    yi, yf = _gemv_a4(q, w, N, K, sa=to_dev(sa), sw=float(sw), want_f32=True)
    acc = oracle.gemm_i32(q.reshape(1, -1), w)
    np.testing.assert_array_equal(yi, acc[0])
    np.testing.assert_array_equal(yf, oracle.epilogue(acc, sa, sw)[0])


@pytest.mark.parametrize("policy", [(1, 32, 8, 256, 10 ** 6), (64, 1, 8, 256, 1),
                                    (2, 2, 8, 7, 1), (16, 32, 4, 1, 1)])
def test_w2a4_gemv_forced_splits(policy):
    try:
        w2a8.tune_gemv(*policy)
        for N, K in [(200, 3200), (96, 27648), (33, 1000), (64, 100)]:
            q, w = synth.gemv_a4_case(N, K, seed=K)
            np.testing.assert_array_equal(_gemv_a4(q, w, N, K),
                                          oracle.gemm_i32(q.reshape(1, -1), w)[0])
    finally:
        w2a8.tune_gemv(*w2a8.DEFAULT_GEMV_POLICY)


def test_w2a4_workspace_left_zeroed():
    N, K = 500, 27648                       # strips split over workgroups
    q, w = synth.gemv_a4_case(N, K, seed=8)
    ws = torch.zeros(w2a8.workspace_bytes(1, N, K), dtype=torch.uint8, device=dev())
    ref = oracle.gemm_i32(q.reshape(1, -1), w)[0]
    for _ in range(3):
        np.testing.assert_array_equal(_gemv_a4(q, w, N, K, workspace=ws), ref)
    assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("N,K", [(13824, 2560), (300, 1000), (64, 33)])
def test_linear_a4_layer(N, K):
    """bf16 token -> int4 quantizer -> W2A4 GEMV -> fp32, against the oracle's
    chain of the same steps (bit-identical)."""
    xb, W = synth.linear_case(1, N, K, seed=N + K)
    wq, sw = oracle.ternarize_absmean(W)
    y = w2a8.linear_a4(_bf16_dev(xb.reshape(-1)), packed_on_device(wq), float(sw), N, K)
    torch.cuda.synchronize()
    q, sa = oracle.quant_act_a4(xb)
    ref = oracle.epilogue(oracle.gemm_i32(q, wq), sa, sw)
    np.testing.assert_array_equal(y.cpu().numpy(), ref)


# ---------------------------------------------------------------------------
# fused int4 linear layer (w2a4_linear_gemv): bit-identical to the oracle's
# int4 quantizer, integer product and epilogue, and to the two-launch path
# ---------------------------------------------------------------------------
def _fused_a4(xb, wq, N, K, sw, workspace=None):
    wp = packed_on_device(wq)
    yf = guarded(N, torch.float32)
    yi = guarded(N, torch.int32)
    w2a8.w2a4_linear_gemv(wp, _bf16_dev(xb.reshape(-1)), N, K, float(sw), yf[:N],
                          y_i32=yi[:N], workspace=workspace)
    torch.cuda.synchronize()
    check_guard(yf, N)
    check_guard(yi, N)
    return yf[:N].cpu().numpy(), yi[:N].cpu().numpy()


def _a4_ref(xb, wq, sw):
    q, sa = oracle.quant_act_a4(xb.reshape(1, -1))
    acc = oracle.gemm_i32(q, wq)
    return oracle.epilogue(acc, sa, sw)[0], acc[0]


# K < 8 and K % 8 != 0 (the row maximum's scalar tail), K % 16 != 0 (the last
# chunk of a run read value by value), K % 32 != 0 (padding), strips split over
# workgroups (K = 27648, 10240), per-wave runs and shared k-ranges (one wave
# per strip; 2600 x 6912 and 16448 x 9000 leave the last workgroup with strips
# past N).
FUSED_A4_SHAPES = [(5, 1), (33, 7), (64, 15), (300, 16), (97, 100), (129, 129), (2, 130),
                   (40, 4000), (1000, 2560), (2560, 6912), (2600, 6912), (3200, 10240),
                   (5120, 27648), (96, 27648), (700, 8195), (13824, 2560), (55296, 5120)]


@pytest.mark.parametrize("N,K", FUSED_A4_SHAPES)
def test_w2a4_linear_gemv_matches_oracle(N, K):
    xb, _ = synth.linear_case(1, 1, K, seed=N + 5 * K)
    _, wq = synth.gemv_case(N, K, seed=N + K, sparse=N % 2 == 1)
    sw = np.float32(0.0137)
    yf, yi = _fused_a4(xb, wq, N, K, sw)
    ref, acc = _a4_ref(xb, wq, sw)
    np.testing.assert_array_equal(yi, acc)
    np.testing.assert_array_equal(yf, ref)


def test_w2a4_linear_gemv_zero_and_single_value_rows():
    N, K = 300, 1000
    _, wq = synth.gemv_case(N, K, seed=4)
    for row in (np.zeros(K, np.float32), np.eye(1, K, 517, dtype=np.float32)[0] * -3.5,
                np.full(K, 2.0, np.float32)):
        xb = synth.fp32_to_bf16_bits(row.reshape(1, K))
        yf, yi = _fused_a4(xb, wq, N, K, np.float32(0.5))
        ref, acc = _a4_ref(xb, wq, np.float32(0.5))
        np.testing.assert_array_equal(yi, acc)
        np.testing.assert_array_equal(yf, ref)


# Runs longer than the fused kernel's LDS regions hold (64 tiles): more waves
# (unsplit long strips: 600 tiles; one wave per strip on 514 strips: 71
# tiles), and more workgroups per strip beyond 1024 tiles.
@pytest.mark.parametrize("policy,N,K", [((1, 32, 8, 256, 10 ** 6), 64, 76800),
                                        ((1, 32, 8, 256, 10 ** 6), 40, 140000),
                                        (None, 16448, 9000)])
def test_w2a4_linear_gemv_long_runs(policy, N, K):
    try:
        if policy is not None:
            w2a8.tune_gemv(*policy)
        xb, _ = synth.linear_case(1, 1, K, seed=K)
        _, wq = synth.gemv_case(N, K, seed=N)
        yf, yi = _fused_a4(xb, wq, N, K, np.float32(0.02))
        ref, acc = _a4_ref(xb, wq, np.float32(0.02))
        np.testing.assert_array_equal(yi, acc)
        np.testing.assert_array_equal(yf, ref)
    finally:
        w2a8.tune_gemv(*w2a8.DEFAULT_GEMV_POLICY)


@pytest.mark.parametrize("policy", [(1, 32, 8, 256, 10 ** 6), (64, 1, 8, 256, 1),
                                    (2, 2, 8, 7, 1), (16, 32, 4, 1, 1)])
def test_w2a4_linear_gemv_forced_splits(policy):
    try:
        w2a8.tune_gemv(*policy)
        for N, K in [(200, 3200), (96, 27648), (33, 1000)]:
            xb, _ = synth.linear_case(1, 1, K, seed=K + 1)
            _, wq = synth.gemv_case(N, K, seed=N + 1)
            yf, yi = _fused_a4(xb, wq, N, K, np.float32(0.02))
            ref, acc = _a4_ref(xb, wq, np.float32(0.02))
            np.testing.assert_array_equal(yi, acc)
            np.testing.assert_array_equal(yf, ref)
    finally:
        w2a8.tune_gemv(*w2a8.DEFAULT_GEMV_POLICY)


def test_w2a4_linear_gemv_workspace_left_zeroed():
    N, K = 500, 27648
    xb, _ = synth.linear_case(1, 1, K, seed=12)
    _, wq = synth.gemv_case(N, K, seed=13)
    ws = torch.zeros(w2a8.workspace_bytes(1, N, K), dtype=torch.uint8, device=dev())
    ref, acc = _a4_ref(xb, wq, np.float32(0.25))
    for _ in range(3):
        yf, yi = _fused_a4(xb, wq, N, K, np.float32(0.25), workspace=ws)
        np.testing.assert_array_equal(yi, acc)
        np.testing.assert_array_equal(yf, ref)
    assert int(ws.count_nonzero()) == 0


@pytest.mark.parametrize("N,K", [(13824, 2560), (5120, 27648), (64, 33)])
def test_w2a4_fused_equals_two_launch_path(N, K):
    xb, W = synth.linear_case(1, N, K, seed=N * 3 + K)
    wq, sw = oracle.ternarize_absmean(W)
    wp = packed_on_device(wq)
    x = _bf16_dev(xb.reshape(-1))
    a = w2a8.linear_a4(x, wp, float(sw), N, K, fused=True)
    b = w2a8.linear_a4(x, wp, float(sw), N, K, fused=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())
