"""GPU parity of the W2A8 GEMV (M = 1) against the oracle: bit-exact int32.

The page's own test compares the kernel's output with numpy's int32 matmul
element by element ("如何编译 BitNet W2A8 CUDA 内核并用 test.py 运行 GEMV 加速测试？",
section "如何判断结果"); here the comparison is with the CPU oracle, on the
same seeded arrays, at small ragged sizes, at every full workload shape in the
launch configuration the benchmark times, and under forced k-splits.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
import w2a8_gemv_amd as w2a8

from gpu_util import dev, gemv_dev, packed_on_device, to_dev

pytestmark = pytest.mark.gpu

DEFAULT_POLICY = w2a8.DEFAULT_GEMV_POLICY


@pytest.fixture(autouse=True)
def _restore_policy():
    yield
    w2a8.tune_gemv(*DEFAULT_POLICY)
    w2a8.tune_gemv_force(0)


def _case(N, K, seed, sparse=False):
    x, w = synth.gemv_case(N, K, seed, sparse=sparse)
    return x, w, packed_on_device(w), to_dev(x)


SMALL = [(1, 1), (1, 16), (7, 5), (32, 128), (33, 129), (31, 127), (64, 256), (97, 97),
         (100, 300), (257, 1000), (96, 4000), (1000, 130), (3, 2600)]


@pytest.mark.parametrize("N,K", SMALL)
def test_gemv_small_ragged(N, K):
    x, w, wp, xd = _case(N, K, seed=N * 1000 + K)
    np.testing.assert_array_equal(gemv_dev(wp, xd, N, K), oracle.gemm_i32(x, w))


# (wg_per_cu, tiles_per_wave, unroll, krange_tiles, split_min_tiles): one
# workgroup per strip with long multi-batch runs, one tile per wave, the
# default, and strips split over 2..KT workgroups (the atomic path).
NOSPLIT = 10 ** 6
POLICIES = [(1, 32, 8, 256, NOSPLIT), (1, 32, 2, 256, NOSPLIT), (1, 1, 4, 256, NOSPLIT),
            w2a8.DEFAULT_GEMV_POLICY, (64, 1, 8, 256, 1), (4, 4, 4, 3, NOSPLIT),
            (2, 2, 8, 7, 1), (16, 32, 4, 1, 1), (8, 16, 8, 256, 1)]


@pytest.mark.parametrize("policy", POLICIES)
@pytest.mark.parametrize("N,K", [(33, 1000), (64, 2560), (200, 3200), (96, 27648)])
def test_gemv_forced_splits(policy, N, K):
    """Every way of splitting a strip's k-range over waves and workgroups."""
    w2a8.tune_gemv(*policy)
    x, w, wp, xd = _case(N, K, seed=7 + N + K)
    np.testing.assert_array_equal(gemv_dev(wp, xd, N, K), oracle.gemm_i32(x, w))


# Forced plans: (kernel, waves per workgroup, workgroups per strip, depth,
# direct activations).  Kernel 2 (ring) at every depth, single-wave and
# multi-wave workgroups, split and unsplit strips; kernel 1 (batch) with its
# staged and its direct activation path.
FORCED = [(2, 1, 1, 2, 1), (2, 1, 1, 12, 1), (2, 4, 1, 4, 1), (2, 3, 2, 6, 1), (2, 8, 3, 8, 1),
          (2, 16, 1, 12, 1), (2, 2, 5, 8, 1), (2, 4, 1, 8, 1), (2, 3, 4, 12, 1), (2, 6, 2, 6, 1),
          (2, 16, 8, 4, 1), (1, 4, 1, 4, 1), (1, 2, 3, 2, 1), (1, 1, 1, 2, 0), (1, 8, 2, 8, 0),
          (1, 3, 4, 4, 0), (3, 1, 8, 2, 1), (3, 1, 8, 4, 1), (3, 1, 8, 6, 1), (3, 1, 8, 8, 1)]


@pytest.mark.parametrize("force", FORCED, ids=[".".join(map(str, f)) for f in FORCED])
@pytest.mark.parametrize("N,K", [(33, 1000), (64, 2560), (200, 3200), (96, 27648), (31, 129),
                                 (70, 2000), (1, 16)])
def test_gemv_forced_plans(force, N, K):
    """Every kernel and ring depth, on ragged N and K (runs past K, empty runs)."""
    kt = -(-K // 128)
    sg = min(force[2], kt)
    if force[0] == 1 and -(-(-(-kt // sg)) // min(force[1], -(-kt // sg))) > 32:
        pytest.skip("run longer than the batch kernel stages")
    if force[0] in (2, 3) and K % 16:
        pytest.skip("the ring and row-slice kernels need K a multiple of 16")
    w2a8.tune_gemv_force(*force)
    try:
        x, w, wp, xd = _case(N, K, seed=11 + N + 3 * K)
        ws = torch.zeros(max(1, w2a8.workspace_bytes(1, N, K)), dtype=torch.uint8, device=dev())
        ref = oracle.gemm_i32(x, w)
        for _ in range(2):     # the split path leaves the workspace zeroed
            np.testing.assert_array_equal(gemv_dev(wp, xd, N, K, workspace=ws), ref)
            assert int(ws.count_nonzero()) == 0
        sa = np.array([0.0173], np.float32)
        yi, yf = gemv_dev(wp, xd, N, K, sa=to_dev(sa), sw=0.031, want_f32=True, workspace=ws)
        np.testing.assert_array_equal(yf, oracle.epilogue(ref, sa, np.float32(0.031)))
    finally:
        w2a8.tune_gemv_force(0)


@pytest.mark.parametrize("idx", range(len(synth.LARGE_SHAPES)))
@pytest.mark.parametrize("force", [(2, 6, 1, 12, 1), (2, 2, 2, 8, 1), (2, 1, 1, 12, 1),
                                   (2, 1, 6, 8, 1), (2, 4, 3, 4, 1), (2, 1, 12, 2, 1),
                                   (3, 1, 8, 4, 1), (3, 1, 8, 8, 1)])
def test_gemv_forced_ring_large_shapes(force, idx):
    N, K = synth.LARGE_SHAPES[idx]
    w2a8.tune_gemv_force(*force)
    try:
        x, w, wp, xd = _case(N, K, synth.LARGE_SEEDS[idx], sparse=True)
        np.testing.assert_array_equal(gemv_dev(wp, xd, N, K), oracle.gemm_i32(x, w))
    finally:
        w2a8.tune_gemv_force(0)


@pytest.mark.parametrize("N,K", [(33, 1000), (2560, 2560), (100, 6016)])
def test_gemv_without_workspace_when_unsplit(N, K):
    """No workspace is needed (nor passed) when no plan splits the k-range."""
    assert w2a8.workspace_bytes(1, N, K) == 0
    x, w, wp, xd = _case(N, K, seed=5 + N + K)
    y = torch.empty(N, dtype=torch.int32, device=dev())
    rc = w2a8.lib().w2a8_gemv(wp.data_ptr(), xd.data_ptr(), N, K, y.data_ptr(), None,
                              ctypes.c_float(1.0), None, None, 0,
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.gemm_i32(x, w))


@pytest.mark.parametrize("idx", range(len(synth.SWEEP_SHAPES)))
def test_gemv_sweep_shapes_full(idx):
    N, K = synth.SWEEP_SHAPES[idx]
    x, w, wp, xd = _case(N, K, synth.SWEEP_SEEDS[idx])
    np.testing.assert_array_equal(gemv_dev(wp, xd, N, K), oracle.gemm_i32(x, w))


# One wave per strip with every automatic ring depth (12 below 2.5 strips per
# CU, 8 up to 4, 6 up to 5.5, then 4 on a 256-CU device), ragged N and a K
# that is not a multiple of the depth's tile groups.
@pytest.mark.parametrize("N,K", [(16400, 2560), (20000, 1040), (26000, 1552), (41472, 1024),
                                 (57000, 656)])
def test_gemv_many_strip_depths_full(N, K):
    x, w, wp, xd = _case(N, K, seed=N % 1000 + K)
    np.testing.assert_array_equal(gemv_dev(wp, xd, N, K), oracle.gemm_i32(x, w))


def test_gemv_small_config_full():
    x, w, wp, xd = _case(2560, 2560, synth.SEED_SMALL)
    np.testing.assert_array_equal(gemv_dev(wp, xd, 2560, 2560), oracle.gemm_i32(x, w))


@pytest.mark.parametrize("idx", range(len(synth.LARGE_SHAPES)))
def test_gemv_large_shapes_full(idx):
    N, K = synth.LARGE_SHAPES[idx]
    x, w, wp, xd = _case(N, K, synth.LARGE_SEEDS[idx], sparse=True)
    np.testing.assert_array_equal(gemv_dev(wp, xd, N, K), oracle.gemm_i32(x, w))


@pytest.mark.parametrize("K", [128, 27648])
def test_gemv_extremes(K):
    N = 64
    for xv, wv, expect in [(127, 1, 127 * K), (-128, -1, 128 * K), (-128, 1, -128 * K),
                           (127, 0, 0)]:
        x = np.full(K, xv, np.int8)
        w = np.full((N, K), wv, np.int8)
        y = gemv_dev(packed_on_device(w), to_dev(x), N, K)
        assert np.all(y == expect), (xv, wv, y[:4])


def test_gemv_full_int8_range_activations():
    # the quantizer never emits -128, but the GEMV must be exact for it too
    rng = np.random.default_rng(5)
    N, K = 160, 1500
    x = rng.integers(-128, 128, size=K, dtype=np.int8)
    w = rng.integers(-1, 2, size=(N, K), dtype=np.int8)
    np.testing.assert_array_equal(gemv_dev(packed_on_device(w), to_dev(x), N, K),
                                  oracle.gemm_i32(x, w))


def test_gemv_one_hot_probe_recovers_weights():
    """x = e_k returns column k of W: pins every position of the layout."""
    N, K = 64, 300
    _, w, wp, _ = _case(N, K, seed=99)
    for k in range(K):
        e = np.zeros(K, np.int8)
        e[k] = 1
        y = gemv_dev(wp, to_dev(e), N, K)
        assert np.array_equal(y, w[:, k]), k


def test_gemv_balanced_ternary_probe():
    """x = 1, 3, 9, 27, 81 on 5 consecutive k decodes those 5 weights per row."""
    N, K = 96, 256
    _, w, wp, _ = _case(N, K, seed=123)
    for k0 in range(0, K - 4, 5):
        x = np.zeros(K, np.int8)
        x[k0:k0 + 5] = [1, 3, 9, 27, 81]
        y = gemv_dev(wp, to_dev(x), N, K).astype(np.int64)
        dec = np.zeros((N, 5), np.int64)
        r = y.copy()
        for i in range(5):           # balanced-ternary digits, least significant first
            d = ((r + 1) % 3) - 1
            dec[:, i] = d
            r = (r - d) // 3
        np.testing.assert_array_equal(dec, w[:, k0:k0 + 5])


def test_gemv_fp32_epilogue():
    N, K = 13824, 2560
    x, w, wp, xd = _case(N, K, seed=77)
    sa = np.array([0.0173], np.float32)
    sw = np.float32(0.0159)
    yi, yf = gemv_dev(wp, xd, N, K, sa=to_dev(sa), sw=float(sw), want_f32=True)
    acc = oracle.gemm_i32(x, w)
    np.testing.assert_array_equal(yi, acc)
    ref = oracle.epilogue(acc, sa, sw)
    nz = ref != 0
    assert np.all(yf[~nz] == 0)
    rel = np.abs(yf[nz].astype(np.float64) - ref[nz]) / np.abs(ref[nz].astype(np.float64))
    assert rel.max() <= 1e-6
    # same IEEE operations in the same order: expected bit-identical
    np.testing.assert_array_equal(yf, ref)


def test_gemv_f32_only_output():
    N, K = 200, 640
    x, w, wp, xd = _case(N, K, seed=4)
    sa = to_dev(np.array([0.5], np.float32))
    yf = torch.empty(N, dtype=torch.float32, device=dev())
    w2a8.w2a8_gemv(wp, xd, N, K, y_i32=None, s_a=sa, s_w=0.25, y_f32=yf)
    torch.cuda.synchronize()
    ref = oracle.epilogue(oracle.gemm_i32(x, w), np.array([0.5], np.float32), 0.25)
    np.testing.assert_array_equal(yf.cpu().numpy(), ref)


def test_gemv_repeat_deterministic_and_workspace_reset():
    N, K = 4800, 6912
    w2a8.tune_gemv(8, 4, 4, 256, 1)   # strips split over workgroups: exercises the atomics
    assert w2a8.gemv_plan(N, K, torch.cuda.get_device_properties(0).multi_processor_count)[2] > 1
    x, w, wp, xd = _case(N, K, seed=31)
    ws = torch.zeros(w2a8.workspace_bytes(1, N, K), dtype=torch.uint8, device=dev())
    ref = oracle.gemm_i32(x, w)
    for _ in range(5):
        np.testing.assert_array_equal(gemv_dev(wp, xd, N, K, workspace=ws), ref)
        assert int(ws.count_nonzero()) == 0, "workspace not left zeroed"


def test_gemv_non_default_stream():
    N, K = 3840, 2560
    x, w, wp, xd = _case(N, K, seed=8)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y = torch.empty(N, dtype=torch.int32, device=dev())
        w2a8.w2a8_gemv(wp, xd, N, K, y_i32=y, stream=s)
    s.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), oracle.gemm_i32(x, w))


def test_gemv_graph_replays_match_eager():
    N, K = 2560, 2560
    x, w, wp, xd = _case(N, K, seed=55)
    ref = oracle.gemm_i32(x, w)
    y = torch.empty(N, dtype=torch.int32, device=dev())
    w2a8.tune_gemv(8, 4, 4, 256, 1)   # split path: workspace must be reset between replays
    s = torch.cuda.Stream()
    ws = torch.zeros(w2a8.workspace_bytes(1, N, K), dtype=torch.uint8, device=dev())
    torch.cuda.synchronize()
    w2a8.w2a8_gemv(wp, xd, N, K, y_i32=y, workspace=ws, stream=s)   # eager warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        w2a8.w2a8_gemv(wp, xd, N, K, y_i32=y, workspace=ws, stream=s)
    for i in range(4):
        y.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), ref)
        # eager work between replays
        np.testing.assert_array_equal(gemv_dev(wp, xd, N, K), ref)


@pytest.mark.parametrize("N,K", [(4096, 4096), (4096, 11008), (11008, 4096), (8192, 8192),
                                 (4800, 6912)])
def test_gemv_automatic_plan_on_projection_shapes(N, K):
    """Common projection shapes on both sides of the row-slice rule (the
    automatic plan, whichever kernel it picks), every output against the
    oracle, int32 and fp32."""
    x, w, wp, xd = _case(N, K, seed=N + 3 * K)
    ref = oracle.gemm_i32(x, w)
    ws = torch.zeros(max(1, w2a8.workspace_bytes(1, N, K)), dtype=torch.uint8, device=dev())
    np.testing.assert_array_equal(gemv_dev(wp, xd, N, K, workspace=ws), ref)
    sa = np.array([0.0119], np.float32)
    yi, yf = gemv_dev(wp, xd, N, K, sa=to_dev(sa), sw=0.027, want_f32=True, workspace=ws)
    np.testing.assert_array_equal(yi, ref)
    np.testing.assert_array_equal(yf, oracle.epilogue(ref, sa, np.float32(0.027)))
    assert int(ws.count_nonzero()) == 0
