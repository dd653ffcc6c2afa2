"""GPU parity of the activation quantizer and of the full W2A8 linear layer.

Quantizer: int8 codes and per-token scales bit-identical to the oracle (both
take every decision with the same correctly rounded fp32 operations).
Linear layer: quantize -> integer product -> fp32 epilogue, against the
oracle's chain of the same steps; the epilogue bar is max relative error
1e-6 (expected bit-identical), zeros exactly zero.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import w2a8_gemv_amd as w2a8

from gpu_util import dev, to_dev

pytestmark = pytest.mark.gpu


def _bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(bits.astype(np.uint16)).view(torch.bfloat16)


def _quant_dev(bits):
    xq, sa = w2a8.quant_act_int8(_bf16_dev(bits))
    torch.cuda.synchronize()
    return xq.cpu().numpy(), sa.cpu().numpy()


@pytest.mark.parametrize("M,K", [(1, 2560), (128, 2560), (1, 27648), (3, 100), (5, 1),
                                 (2, 7), (4, 4000), (1, 8), (17, 16)])
def test_quant_matches_oracle(M, K):
    xb, _ = synth.linear_case(M, 1, K, seed=M * 7 + K)
    q, sa = _quant_dev(xb)
    oq, osa = oracle.quant_act(xb)
    np.testing.assert_array_equal(q, oq)
    np.testing.assert_array_equal(sa, osa)


def test_quant_worked_examples_and_zero_rows():
    rows = [[1.0, -0.5, 0.25, 0.0], [2.0, 1.0, -1.0, 0.5],
            [1.984375, 0.9765625, -0.9765625, 0.5078125], [0.0, 0.0, 0.0, 0.0],
            [-4.0, -4.0, -4.0, -4.0]]
    bits = synth.fp32_to_bf16_bits(np.array(rows, np.float32))
    q, sa = _quant_dev(bits)
    oq, osa = oracle.quant_act(bits)
    np.testing.assert_array_equal(q, oq)
    np.testing.assert_array_equal(sa, osa)
    assert q[0].tolist() == [127, -64, 32, 0]
    assert q[2].tolist() == [127, 62, -62, 32]
    assert q[3].tolist() == [0, 0, 0, 0] and sa[3] == 0.0


def _linear_ref(xb, wq, sw):
    xq, sa = oracle.quant_act(xb)
    acc = oracle.gemm_i32(xq, wq)
    return oracle.epilogue(acc, sa, sw), acc


def _check_f32(y, ref):
    nz = ref != 0
    assert np.all(y[~nz] == 0)
    rel = np.abs(y[nz].astype(np.float64) - ref[nz]) / np.abs(ref[nz].astype(np.float64))
    assert rel.max() <= 1e-6, rel.max()
    np.testing.assert_array_equal(y, ref)


@pytest.mark.parametrize("M,fused", [(1, True), (1, False), (128, False)],
                         ids=["M1-fused", "M1-two-launch", "M128"])
def test_full_linear_layer(M, fused):
    N, K = 13824, 2560
    xb, W = synth.linear_case(M, N, K, seed=synth.LINEAR_SEEDS[M])
    wq, sw = oracle.ternarize_absmean(W)
    wp = w2a8.pack_ternary(torch.from_numpy(wq)).to(dev())
    y = w2a8.linear(_bf16_dev(xb), wp, float(sw), N, K, fused=fused)
    torch.cuda.synchronize()
    ref, _ = _linear_ref(xb, wq, sw)
    _check_f32(y.cpu().numpy(), ref)


# ---------------------------------------------------------------------------
# Fused linear GEMV (quantize + product + epilogue in one launch)
# ---------------------------------------------------------------------------
def _fused_dev(xb, wq, N, K, sw):
    wp = w2a8.pack_ternary(torch.from_numpy(wq)).to(dev())
    yf = torch.full((N,), float("nan"), dtype=torch.float32, device=dev())
    yi = torch.full((N,), -7, dtype=torch.int32, device=dev())
    w2a8.w2a8_linear_gemv(wp, _bf16_dev(xb.reshape(-1)), N, K, float(sw), yf, y_i32=yi)
    torch.cuda.synchronize()
    return yf.cpu().numpy(), yi.cpu().numpy()


# ragged K (K % 16 != 0, K < 16, K = 1), split strips (K = 27648, 10240),
# several workgroup shapes
FUSED_SHAPES = [(1000, 2560), (97, 100), (33, 7), (5, 1), (64, 15), (300, 16), (129, 129),
                (2560, 6912), (3200, 10240), (5120, 27648), (40, 4000), (2, 130)]


@pytest.mark.parametrize("N,K", FUSED_SHAPES)
def test_fused_linear_gemv_matches_oracle(N, K):
    xb, _ = synth.linear_case(1, 1, K, seed=N + 3 * K)
    _, wq = synth.gemv_case(N, K, seed=N + K, sparse=True)
    sw = np.float32(0.0137)
    yf, yi = _fused_dev(xb, wq, N, K, sw)
    ref, acc = _linear_ref(xb, wq, sw)
    np.testing.assert_array_equal(yi, acc[0])
    _check_f32(yf, ref[0])


def test_fused_linear_gemv_zero_and_single_value_rows():
    N, K = 300, 1000
    _, wq = synth.gemv_case(N, K, seed=4)
    for row in (np.zeros(K, np.float32), np.eye(1, K, 517, dtype=np.float32)[0] * -3.5):
        xb = synth.fp32_to_bf16_bits(row.reshape(1, K))
        yf, yi = _fused_dev(xb, wq, N, K, np.float32(0.5))
        ref, acc = _linear_ref(xb, wq, np.float32(0.5))
        np.testing.assert_array_equal(yi, acc[0])
        np.testing.assert_array_equal(yf, ref[0])


@pytest.mark.parametrize("policy", [(1, 32, 8, 256, 10 ** 6), (1, 1, 4, 256, 10 ** 6),
                                    (64, 1, 8, 256, 1), (2, 2, 8, 7, 1), (16, 32, 4, 1, 1)])
def test_fused_linear_gemv_forced_splits(policy):
    try:
        w2a8.tune_gemv(*policy)
        for N, K in [(200, 3200), (96, 27648), (33, 1000)]:
            xb, _ = synth.linear_case(1, 1, K, seed=K)
            _, wq = synth.gemv_case(N, K, seed=N)
            yf, yi = _fused_dev(xb, wq, N, K, np.float32(0.02))
            ref, acc = _linear_ref(xb, wq, np.float32(0.02))
            np.testing.assert_array_equal(yi, acc[0])
            np.testing.assert_array_equal(yf, ref[0])
    finally:
        w2a8.tune_gemv(*w2a8.DEFAULT_GEMV_POLICY)


def test_fused_equals_two_launch_path():
    N, K = 13824, 2560
    xb, W = synth.linear_case(1, N, K, seed=synth.LINEAR_SEEDS[1])
    wq, sw = oracle.ternarize_absmean(W)
    wp = w2a8.pack_ternary(torch.from_numpy(wq)).to(dev())
    a = w2a8.linear(_bf16_dev(xb), wp, float(sw), N, K, fused=True)
    b = w2a8.linear(_bf16_dev(xb), wp, float(sw), N, K, fused=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())


def test_full_linear_uses_library_ternarizer_identically():
    N, K = 1024, 2560
    xb, W = synth.linear_case(1, N, K, seed=9)
    wq, sw = w2a8.ternarize_absmean(torch.from_numpy(W))
    owq, osw = oracle.ternarize_absmean(W)
    assert np.float32(sw) == osw
    np.testing.assert_array_equal(wq.numpy(), owq)
    y = w2a8.linear(_bf16_dev(xb), w2a8.pack_ternary(wq).to(dev()), sw, N, K)
    torch.cuda.synchronize()
    ref, _ = _linear_ref(xb, owq, osw)
    _check_f32(y.cpu().numpy(), ref)


def test_full_linear_reports_error_vs_unquantized():
    """Not a pass/fail parity bar: the quantized layer's error against the
    unquantized fp64 product is reported and must merely be finite and small
    relative to the output scale (the page defines no accuracy target)."""
    N, K = 2048, 2560
    xb, W = synth.linear_case(1, N, K, seed=10)
    wq, sw = oracle.ternarize_absmean(W)
    y = w2a8.linear(_bf16_dev(xb), w2a8.pack_ternary(torch.from_numpy(wq)).to(dev()), float(sw),
                    N, K)
    torch.cuda.synchronize()
    xf = synth.bf16_bits_to_fp32(xb).astype(np.float64)
    ref = xf @ W.astype(np.float64).T
    err = np.linalg.norm(y.cpu().numpy() - ref) / np.linalg.norm(ref)
    print(f"relative L2 error of the quantized layer vs fp64: {err:.4f}")
    assert np.isfinite(err) and err < 1.0
