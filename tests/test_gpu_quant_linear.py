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

from gpu_util import check_guard, dev, guarded, to_dev

pytestmark = pytest.mark.gpu


def _bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return to_dev(bits.astype(np.uint16)).view(torch.bfloat16)


def _quant_dev(bits):
    xq, sa = w2a8.quant_act_int8(_bf16_dev(bits))
    torch.cuda.synchronize()
    return xq.cpu().numpy(), sa.cpu().numpy()


@pytest.mark.parametrize("M,K", [(1, 2560), (128, 2560), (1, 27648), (3, 100), (5, 1),
                                 (2, 7), (4, 4000), (1, 8), (17, 16),
                                 # one workgroup per row, one chunk of 8 per lane: 1..16
                                 # waves (the last partly idle), and K just past the limit
                                 (1, 8192), (9, 520), (7, 512), (600, 4096), (1100, 1024),
                                 (33, 8200), (3, 6912), (512, 2560), (4, 8184), (2, 504)])
def test_quant_matches_oracle(M, K):
    xb, _ = synth.linear_case(M, 1, K, seed=M * 7 + K)
    q, sa = _quant_dev(xb)
    oq, osa = oracle.quant_act(xb)
    np.testing.assert_array_equal(q, oq)
    np.testing.assert_array_equal(sa, osa)


# Rows past 8192 values: 2 to 4 chunks of 8 per lane (K up to 32768), and K
# just past that limit (the two-pass kernel); the output sits between guard
# bands that must stay untouched.
@pytest.mark.parametrize("M,K", [(1, 8200), (1, 16384), (2, 24576), (1, 27648), (3, 32768),
                                 (1, 32776), (2, 10248)])
def test_quant_long_rows_with_guards(M, K):
    xb, _ = synth.linear_case(M, 1, K, seed=M * 11 + K)
    buf = torch.full((M * K + 128,), -91, dtype=torch.int8, device=dev())
    sab = torch.full((M + 16,), float("nan"), dtype=torch.float32, device=dev())
    w2a8.quant_act_int8(_bf16_dev(xb), x_q=buf[64:64 + M * K], s_a=sab[:M])
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    oq, osa = oracle.quant_act(xb)
    np.testing.assert_array_equal(got[64:64 + M * K].reshape(M, K), oq)
    assert (got[:64] == -91).all() and (got[64 + M * K:] == -91).all()
    np.testing.assert_array_equal(sab[:M].cpu().numpy(), osa)
    assert bool(torch.isnan(sab[M:]).all())


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


def test_quant_zero_rows_register_path():
    # zero rows between nonzero ones, K a multiple of 8 (one chunk per lane)
    xb, _ = synth.linear_case(6, 1, 48, seed=5)
    xb[1] = 0
    xb[4] = 0x8000          # negative zeros
    q, sa = _quant_dev(xb)
    oq, osa = oracle.quant_act(xb)
    np.testing.assert_array_equal(q, oq)
    np.testing.assert_array_equal(sa, osa)
    assert np.all(q[1] == 0) and np.all(q[4] == 0) and sa[1] == 0.0 and sa[4] == 0.0


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
    yf = guarded(N, torch.float32)
    yi = guarded(N, torch.int32)
    w2a8.w2a8_linear_gemv(wp, _bf16_dev(xb.reshape(-1)), N, K, float(sw), yf[:N], y_i32=yi[:N])
    torch.cuda.synchronize()
    check_guard(yf, N)
    check_guard(yi, N)
    return yf[:N].cpu().numpy(), yi[:N].cpu().numpy()


# ragged K (K % 16 != 0, K < 16, K = 1, K % 8 != 0), split strips (K = 27648,
# 10240), per-wave runs and shared k-ranges (one wave per strip: split strips
# and many strips; 2600 x 6912 and 16448 x 3000 leave the last workgroup with
# strips past N)
FUSED_SHAPES = [(1000, 2560), (97, 100), (33, 7), (5, 1), (64, 15), (300, 16), (129, 129),
                (2560, 6912), (2600, 6912), (3200, 10240), (5120, 27648), (40, 4000), (2, 130),
                (700, 8195), (13824, 2560), (55296, 5120), (16448, 3000), (20480, 3200)]


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


# Runs longer than the fused kernel's LDS regions hold (32 tiles per wave):
# more waves (unsplit long strips: 600 tiles), and more workgroups per strip
# beyond 512 tiles (shared k-ranges: 1094 tiles over 2 or more workgroups).
@pytest.mark.parametrize("policy,N,K", [((1, 32, 8, 256, 10 ** 6), 64, 76800),
                                        ((1, 32, 8, 256, 10 ** 6), 40, 140000),
                                        (None, 16448, 70000)])
def test_fused_linear_gemv_long_runs(policy, N, K):
    try:
        if policy is not None:
            w2a8.tune_gemv(*policy)
        xb, _ = synth.linear_case(1, 1, K, seed=K)
        _, wq = synth.gemv_case(N, K, seed=N)
        yf, yi = _fused_dev(xb, wq, N, K, np.float32(0.02))
        ref, acc = _linear_ref(xb, wq, np.float32(0.02))
        np.testing.assert_array_equal(yi, acc[0])
        np.testing.assert_array_equal(yf, ref[0])
    finally:
        w2a8.tune_gemv(*w2a8.DEFAULT_GEMV_POLICY)


@pytest.mark.parametrize("N,K", [(13824, 2560), (5120, 27648), (55296, 5120), (64, 33)])
def test_fused_equals_two_launch_shapes(N, K):
    xb, W = synth.linear_case(1, N, K, seed=N * 5 + K)
    wq, sw = oracle.ternarize_absmean(W)
    wp = w2a8.pack_ternary(torch.from_numpy(wq)).to(dev())
    x = _bf16_dev(xb)
    a = w2a8.linear(x, wp, float(sw), N, K, fused=True)
    b = w2a8.linear(x, wp, float(sw), N, K, fused=False)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())


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


@pytest.mark.parametrize("entry", ["w2a8_linear_gemv", "w2a4_linear_gemv"])
def test_fused_layers_graph_replays_match_eager(entry):
    """The fused layers on a split plan with shared k-ranges, captured in a
    graph: every replay (with eager work between them) equals the eager call,
    and the combining words are left zeroed."""
    N, K = 5120, 27648
    xb, _ = synth.linear_case(1, 1, K, seed=91)
    _, wq = synth.gemv_case(N, K, seed=92, sparse=True)
    wp = w2a8.pack_ternary(torch.from_numpy(wq)).to(dev())
    x = _bf16_dev(xb.reshape(-1))
    fn = getattr(w2a8, entry)
    ws = torch.zeros(w2a8.workspace_bytes(1, N, K), dtype=torch.uint8, device=dev())
    s = torch.cuda.Stream()
    eager = torch.empty(N, dtype=torch.float32, device=dev())
    fn(wp, x, N, K, 0.03, eager, workspace=ws, stream=s)
    torch.cuda.synchronize()
    y = torch.empty(N, dtype=torch.float32, device=dev())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn(wp, x, N, K, 0.03, y, workspace=ws, stream=s)
    for _ in range(4):
        y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, eager)
        other = torch.empty(N, dtype=torch.float32, device=dev())
        fn(wp, x, N, K, 0.03, other, workspace=ws, stream=s)
        torch.cuda.synchronize()
        assert torch.equal(other, eager)
    assert int(ws.count_nonzero()) == 0


def _tiny_rows(K, seed):
    """Rows whose maximum is below 127 / FLT_MAX (subnormal-scale bf16): the
    quantizers' reciprocal overflows and is capped, zeros must stay zero."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((3, K)) * 2.0 ** -130).astype(np.float32)
    x[0, :4] = [2.0 ** -126, 0.0, -2.0 ** -127, 2.0 ** -128][:K]
    x[1, ::7] = 0.0
    x[2] = 0.0
    x[2, K // 2] = -2.0 ** -133                  # the least bf16 subnormal, alone
    return synth.fp32_to_bf16_bits(x)


@pytest.mark.parametrize("K", [4, 100, 2560, 27648])
def test_quantizers_tiny_rows(K):
    xb = _tiny_rows(K, seed=K)
    q, sa = _quant_dev(xb)
    oq, osa = oracle.quant_act(xb)
    np.testing.assert_array_equal(q, oq)
    np.testing.assert_array_equal(sa, osa)
    assert np.all(q[xb == 0] == 0)
    xq4, sa4 = w2a8.quant_act_int4(_bf16_dev(xb))
    torch.cuda.synchronize()
    q4, osa4 = oracle.quant_act_a4(xb)
    np.testing.assert_array_equal(xq4.cpu().numpy(), oracle.pack_act4(q4))
    np.testing.assert_array_equal(sa4.cpu().numpy(), osa4)


@pytest.mark.parametrize("N,K", [(300, 100), (2560, 2560), (55296, 5120), (5120, 27648)])
def test_fused_layers_tiny_rows(N, K):
    """Both fused layers (workgroup and ring kernels) on rows of subnormal
    scale, bit-identical to the oracle chain (subnormal scales and outputs
    included)."""
    xb = _tiny_rows(K, seed=N + K)
    _, wq = synth.gemv_case(N, K, seed=N, sparse=True)
    wp = w2a8.pack_ternary(torch.from_numpy(wq)).to(dev())
    sw = np.float32(0.75)
    for m in range(xb.shape[0]):
        row = xb[m:m + 1]
        yf = torch.empty(N, dtype=torch.float32, device=dev())
        yi = torch.empty(N, dtype=torch.int32, device=dev())
        w2a8.w2a8_linear_gemv(wp, _bf16_dev(row.reshape(-1)), N, K, float(sw), yf, y_i32=yi)
        ref, acc = _linear_ref(row, wq, sw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(yi.cpu().numpy(), acc[0])
        np.testing.assert_array_equal(yf.cpu().numpy(), ref[0])
        w2a8.w2a4_linear_gemv(wp, _bf16_dev(row.reshape(-1)), N, K, float(sw), yf, y_i32=yi)
        q4, sa4 = oracle.quant_act_a4(row)
        acc4 = oracle.gemm_i32(q4, wq)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(yi.cpu().numpy(), acc4[0])
        np.testing.assert_array_equal(yf.cpu().numpy(), oracle.epilogue(acc4, sa4, sw)[0])
