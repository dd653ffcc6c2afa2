"""The allocation-free GEMV entry point (w2a8_gemv_noalloc), called through
the C ABI, against w2a8_gemv with a workspace on the same inputs: bit-identical
int32 and fp32 outputs, on two calls in a row (the second smaller, so it
reuses the static scratch the first left), on shapes whose plans combine
split strips through that scratch, and its refusal of shapes beyond it."""
import ctypes

import numpy as np
import pytest
import torch

import synth
import w2a8_gemv_amd as w2a8

from gpu_util import CANARY_I32, GUARD, check_guard, dev, packed_on_device, to_dev

pytestmark = pytest.mark.gpu


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _noalloc(wp, xd, N, K, sa, sw):
    """y_i32 and y_f32 of the C entry point, each with a canary guard band."""
    yi = torch.full((N + GUARD,), CANARY_I32, dtype=torch.int32, device=dev())
    yf = torch.full((N + GUARD,), float("nan"), dtype=torch.float32, device=dev())
    rc = w2a8.lib().w2a8_gemv_noalloc(wp.data_ptr(), xd.data_ptr(), N, K, yi.data_ptr(),
                                       sa.data_ptr(), ctypes.c_float(sw), yf.data_ptr(), _stream())
    assert rc == 0, w2a8.lib().w2a8_status_str(rc)
    torch.cuda.synchronize()
    check_guard(yi, N)
    check_guard(yf, N)
    return yi[:N].cpu().numpy(), yf[:N].cpu().numpy()


def _with_workspace(wp, xd, N, K, sa, sw):
    yi = torch.empty(N, dtype=torch.int32, device=dev())
    yf = torch.empty(N, dtype=torch.float32, device=dev())
    ws = torch.zeros(max(16, w2a8.workspace_bytes(1, N, K)), dtype=torch.uint8, device=dev())
    w2a8.w2a8_gemv(wp, xd, N, K, y_i32=yi, s_a=sa, s_w=sw, y_f32=yf, workspace=ws)
    torch.cuda.synchronize()
    return yi.cpu().numpy(), yf.cpu().numpy()


# (N, K, seed): first call, then a smaller one.  Every shape's default plan
# splits strips over workgroups (the path that uses the scratch): the ring
# kernel on strips of more than 96 tiles, the batch kernel for K not a
# multiple of 16 (40000 x 7000).  The row-slice kernel, which shorter strips
# on few rows get, never splits and so never touches the scratch.
CASES = [((3000, 13824, 61), (700, 12800, 62)),
         ((5120, 27648, 63), (96, 13312, 64)),
         ((40000, 7000, 65), (33, 12416, 66))]


@pytest.mark.parametrize("first,second", CASES, ids=["3000x13824", "5120x27648", "40000x7000"])
def test_noalloc_matches_gemv_twice(first, second):
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for N, K, seed in (first, second):
        assert w2a8.workspace_bytes(1, N, K) > 0
        kern, _, sg, _ = w2a8.gemv_plan(N, K, cus)
        assert kern in (1, 2) and sg > 1, (N, K)      # the plan combines through the scratch
        x, w = synth.gemv_case(N, K, seed)
        wp, xd = packed_on_device(w), to_dev(x)
        sa = to_dev(np.array([0.0137], np.float32))
        sw = 0.0211
        yi, yf = _noalloc(wp, xd, N, K, sa, sw)
        ri, rf = _with_workspace(wp, xd, N, K, sa, sw)
        np.testing.assert_array_equal(yi, ri)
        np.testing.assert_array_equal(yf, rf)


def test_noalloc_unsplit_and_ragged():
    # 2560 x 2560: the row-slice kernel (no scratch used); 300 x 1000: a short
    # ragged K (batch kernel, unsplit); 64 x 7001: a long ragged K (batch
    # kernel, split through the scratch)
    for N, K, seed in ((2560, 2560, 67), (300, 1000, 68), (64, 7001, 69)):
        x, w = synth.gemv_case(N, K, seed)
        wp, xd = packed_on_device(w), to_dev(x)
        sa = to_dev(np.array([0.5], np.float32))
        yi, yf = _noalloc(wp, xd, N, K, sa, 0.25)
        ri, rf = _with_workspace(wp, xd, N, K, sa, 0.25)
        np.testing.assert_array_equal(yi, ri)
        np.testing.assert_array_equal(yf, rf)


def test_noalloc_rejects_shapes_beyond_its_scratch():
    L = w2a8.lib()
    fake = 0x10000
    # 131072 padded rows fit; one more strip does not (when K splits)
    assert L.w2a8_gemv_noalloc(fake, fake, 131073, 8192, fake, None, ctypes.c_float(1.0), None,
                               _stream()) == 9
    # without a split no scratch is needed, so the same N is not refused for it
    x, w = synth.gemv_case(1, 16, 70)
    N = 131073
    wp = torch.zeros(w2a8.packed_bytes(N, 16), dtype=torch.uint8, device=dev())
    wp.fill_(0x55)                     # code 01 everywhere: all weights 0
    y = torch.full((N,), 7, dtype=torch.int32, device=dev())
    rc = L.w2a8_gemv_noalloc(wp.data_ptr(), to_dev(np.zeros(16, np.int8)).data_ptr(), N, 16,
                             y.data_ptr(), None, ctypes.c_float(1.0), None, _stream())
    assert rc == 0
    torch.cuda.synchronize()
    assert int(y.abs().sum()) == 0
