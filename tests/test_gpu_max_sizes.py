"""GPU parity at the largest K the library accepts (W2A8_MAX_K = 1048448,
8191 k-tiles), for every device path, with ragged N.

At this K a strip is split over hundreds of workgroups (GEMV), the pipelined
product runs 8191 ring steps, and |y| reaches 128*K = 134 201 344 for the
extreme inputs, the largest magnitude the int8 paths can produce.  The bar
is the same as everywhere: int32 bit-exact against the oracle, fp32
bit-identical.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import w2a8_gemv_amd as w2a8

from gpu_util import check_guard, dev, guarded, packed_on_device, to_dev

pytestmark = pytest.mark.gpu

KMAX = 1048448
N = 33


@pytest.fixture(scope="module")
def case():
    x, w = synth.gemv_case(N, KMAX, seed=77)
    return x, w, packed_on_device(w), oracle.gemm_i32(x.reshape(1, -1), w)[0]


def test_gemv_max_k(case):
    x, w, wp, ref = case
    y = guarded(N, torch.int32)
    w2a8.w2a8_gemv(wp, to_dev(x), N, KMAX, y_i32=y[:N])
    torch.cuda.synchronize()
    check_guard(y, N)
    np.testing.assert_array_equal(y[:N].cpu().numpy(), ref)


def test_gemv_max_k_extremes():
    x = np.full(KMAX, -128, np.int8)
    for v in (-1, 1):
        wp = packed_on_device(np.full((N, KMAX), v, np.int8))
        y = w2a8.gemv(wp, to_dev(x), N, KMAX)
        torch.cuda.synchronize()
        assert np.all(y.cpu().numpy() == -128 * KMAX * v)


def test_w2a4_gemv_max_k(case):
    _, w, wp, _ = case
    q, _ = synth.gemv_a4_case(1, KMAX, seed=78)
    y = torch.empty(N, dtype=torch.int32, device=dev())
    w2a8.w2a4_gemv(wp, to_dev(oracle.pack_act4(q.reshape(1, -1))), N, KMAX, y_i32=y)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.gemm_i32(q.reshape(1, -1), w)[0])


@pytest.mark.parametrize("kernel,M", [(0, 3), (1, 40), (2, 40)],
                         ids=["few-row", "pipelined", "general"])
def test_gemm_max_k(kernel, M, case):
    _, w, wp, _ = case
    x, _ = synth.gemm_case(M, 1, KMAX, seed=79)
    try:
        w2a8.tune_gemm(kernel)
        y = w2a8.gemm(wp, to_dev(x), N, KMAX)
        torch.cuda.synchronize()
    finally:
        w2a8.tune_gemm(0)
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.gemm_i32(x, w))


def test_quantizer_and_fused_linear_max_k():
    xb, W = synth.linear_case(2, N, KMAX, seed=80)
    wq, sw = oracle.ternarize_absmean(W)
    del W
    xq, sa = w2a8.quant_act_int8(to_dev(xb).view(torch.bfloat16))
    torch.cuda.synchronize()
    oq, osa = oracle.quant_act(xb)
    np.testing.assert_array_equal(xq.cpu().numpy(), oq)
    np.testing.assert_array_equal(sa.cpu().numpy(), osa)
    # fused layer on the first token
    y = w2a8.linear(to_dev(xb[0]).view(torch.bfloat16), packed_on_device(wq), float(sw), N, KMAX)
    torch.cuda.synchronize()
    ref = oracle.epilogue(oracle.gemm_i32(oq[:1], wq), osa[:1], sw)
    np.testing.assert_array_equal(y.cpu().numpy(), ref)
