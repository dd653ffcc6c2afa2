"""GPU parity of the batched W2A8 product (M > 1, int8 MFMA): bit-exact int32.

Every shape is compared in full, the prefill workload shapes (M in
{8, 128, 512} at 13824x2560 and 2560x6912) included; the oracle runs those over
several host threads (each thread the same C product on its own block of
weight rows).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import w2a8_gemv_amd as w2a8

from gpu_util import CANARY_I32, GUARD, check_guard, dev, packed_on_device, to_dev

pytestmark = pytest.mark.gpu

# host threads for the oracle on the prefill shapes (a one-GPU machine's CPU share)
ORACLE_THREADS = max(1, min(16, os.cpu_count() or 1))


@pytest.fixture(autouse=True)
def _restore_gemm_kernel():
    yield
    w2a8.tune_gemm(0)
    w2a8.tune_gemm_ring(0, 0, 0)


def _gemm_dev(wp, xd, M, N, K, sa=None, sw=1.0, want_f32=False):
    y = torch.full((M * N + GUARD,), CANARY_I32, dtype=torch.int32, device=dev())
    yf = None
    if want_f32:
        yf = torch.full((M * N + GUARD,), float("nan"), dtype=torch.float32, device=dev())
    w2a8.w2a8_gemm(wp, xd, M, N, K, y_i32=y[:M * N], s_a=sa, s_w=sw,
                   y_f32=None if yf is None else yf[:M * N])
    torch.cuda.synchronize()
    check_guard(y, M * N)
    out = y[:M * N].cpu().numpy().reshape(M, N)
    if yf is None:
        return out
    check_guard(yf, M * N)
    return out, yf[:M * N].cpu().numpy().reshape(M, N)


SMALL = [(2, 1, 1), (2, 32, 128), (3, 33, 129), (16, 64, 256), (17, 100, 300),
         (31, 97, 97), (33, 128, 512), (64, 256, 1000), (65, 130, 2560), (128, 160, 640),
         (129, 64, 384), (200, 96, 1024), (8, 2560, 6912), (300, 33, 16)]


@pytest.mark.parametrize("M,N,K", SMALL)
def test_gemm_small_ragged(M, N, K):
    x, w = synth.gemm_case(M, N, K, seed=M + 10 * N + 100 * K)
    y = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K)
    np.testing.assert_array_equal(y, oracle.gemm_i32(x, w))


# Each kernel forced onto ragged shapes: every pipelined configuration
# (M <= 32, above, M > 448 over >= 256 strips, whose 128 x 256 tile is
# ragged in M, N and K at 460 x 8230 x 272, and the small-grid ones whose
# 2 or 4 wave groups split K: k-tile counts 9 and 20 for 2 groups and
# 40, 41, 43 for 4, so that the last group may have fewer tiles, with 32-row
# tiles and, for M <= 16, 16-row tiles whose activation tile is loaded by
# two waves each; the workgroups of one strip with 8 groups of 16-row tiles
# on 20 to 54 k-tiles, and those of 2 strips with 8 groups of 16-row tiles
# or 4 groups of 32-row tiles, on 21, 40 and 43 k-tiles with ragged M and N),
# K below one
# ring of tiles (K = 16, 144), a k-tile remainder (KT % 4 = 1, 2, 3), a
# partial last tile (K = 1040, 2608, 5200) and ragged N (strips past the
# matrix, rows past N in the last strip).
FORCED = [(8, 1000, 1040), (33, 100, 16), (64, 2560, 144), (100, 97, 2560), (128, 200, 384),
          (200, 1000, 1040), (257, 33, 3200), (2, 4096, 896), (17, 130, 640),
          (333, 8230, 1040), (256, 8192, 64), (40, 300, 5248), (96, 200, 5504),
          (129, 520, 5200), (48, 640, 5120), (12, 1000, 2560), (16, 300, 5248), (9, 2600, 1040),
          (3, 97, 5504), (24, 300, 5248), (100, 700, 6912), (129, 2600, 5120), (40, 97, 5504),
          (12, 20000, 5504), (100, 1500, 2608), (300, 1000, 2608), (460, 8230, 272),
          (200, 3000, 2560), (200, 3000, 5248), (41, 5000, 5504)]


@pytest.mark.parametrize("kernel", [1, 2], ids=["pipelined", "general"])
@pytest.mark.parametrize("M,N,K", FORCED + [s for s in SMALL if s[2] % 16 == 0])
def test_gemm_forced_kernel(kernel, M, N, K):
    w2a8.tune_gemm(kernel)
    x, w = synth.gemm_case(M, N, K, seed=7 * M + 3 * N + K)
    y = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K)
    np.testing.assert_array_equal(y, oracle.gemm_i32(x, w))


@pytest.mark.parametrize("cfg", range(10))
@pytest.mark.parametrize("M,N,K", [(100, 700, 1040), (17, 3000, 5248), (460, 520, 272)])
def test_gemm_every_pipelined_configuration(cfg, M, N, K):
    """Each configuration of the pipelined kernel's table forced on ragged M,
    N and K (the automatic choice picks them by shape)."""
    w2a8.tune_gemm(1)
    w2a8.tune_gemm_pipe(cfg)
    try:
        x, w = synth.gemm_case(M, N, K, seed=cfg + M + N)
        y = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K)
        np.testing.assert_array_equal(y, oracle.gemm_i32(x, w))
    finally:
        w2a8.tune_gemm_pipe(-1)


@pytest.mark.parametrize("M,N,K", [(150, 700, 1024), (200, 3000, 5120), (10, 300, 2432),
                                   (13, 2600, 1040), (50, 400, 5120), (100, 1500, 2608),
                                   (129, 2600, 5120)],
                         ids=["2-groups", "4-groups", "16-rows-2-groups", "16-rows-2-groups-b",
                              "1-strip-8-groups", "2-strips-8-groups", "2-strips-4-groups"])
@pytest.mark.parametrize("kernel", [1, 2], ids=["pipelined", "general"])
def test_gemm_forced_kernel_fp32_epilogue(kernel, M, N, K):
    w2a8.tune_gemm(kernel)
    x, w = synth.gemm_case(M, N, K, seed=99)
    rng = np.random.default_rng(5)
    sa = (rng.random(M, dtype=np.float32) * 0.05 + 1e-3).astype(np.float32)
    sw = np.float32(0.0173)
    yi, yf = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K, sa=to_dev(sa), sw=float(sw),
                       want_f32=True)
    acc = oracle.gemm_i32(x, w)
    np.testing.assert_array_equal(yi, acc)
    np.testing.assert_array_equal(yf, oracle.epilogue(acc, sa, sw))


# Automatic choice on small output grids, where the k-range is split over
# wave groups inside a workgroup (8 groups in workgroups of one strip:
# 9 x 2560 x 6912, 16 x 100 x 5248; of 2 strips: 16 x 13824 x 2560; 4 groups
# in workgroups of 2 strips: 32 x 13824 x 2560; 2 groups: 100 x 13824 x 2176,
# 32 x 2560 x 1040), with odd tile counts.
@pytest.mark.parametrize("M,N,K", [(9, 2560, 6912), (16, 100, 5248), (16, 13824, 2560),
                                   (32, 13824, 2560), (100, 13824, 2176), (32, 2560, 1040)])
def test_gemm_wave_group_split_auto(M, N, K):
    x, w = synth.gemm_case(M, N, K, seed=M * N + K)
    y = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K)
    np.testing.assert_array_equal(y, oracle.gemm_i32(x, w))


# Few-row kernel (M <= 8) forced: every M, ragged N and K (K % 16 != 0 takes
# the byte-wise activation path), long K (strips split over workgroups).
FEW = [(2, 1, 1), (2, 33, 129), (3, 100, 300), (4, 257, 1000), (5, 64, 2560), (6, 97, 15),
       (7, 1000, 4000), (8, 2560, 6912), (8, 13824, 2560), (3, 96, 27648), (8, 200, 10240)]


@pytest.mark.parametrize("M,N,K", FEW)
def test_gemm_few_rows_kernel(M, N, K):
    w2a8.tune_gemm(3)
    x, w = synth.gemm_case(M, N, K, seed=11 * M + N + 5 * K)
    y = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K)
    np.testing.assert_array_equal(y, oracle.gemm_i32(x, w))


@pytest.mark.parametrize("policy", [(1, 32, 8, 256, 10 ** 6), (64, 1, 8, 256, 1),
                                    (2, 2, 8, 7, 1), (16, 32, 4, 1, 1)])
def test_gemm_few_rows_forced_splits(policy):
    try:
        w2a8.tune_gemm(3)
        w2a8.tune_gemv(*policy)
        for M, N, K in [(4, 200, 3200), (8, 96, 27648), (2, 33, 1000)]:
            x, w = synth.gemm_case(M, N, K, seed=M + N + K)
            y = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K)
            np.testing.assert_array_equal(y, oracle.gemm_i32(x, w))
    finally:
        w2a8.tune_gemv(*w2a8.DEFAULT_GEMV_POLICY)


def test_gemm_few_rows_fp32_epilogue_and_workspace_reset():
    w2a8.tune_gemm(3)
    M, N, K = 6, 700, 27648                 # strips split over workgroups
    x, w = synth.gemm_case(M, N, K, seed=77)
    rng = np.random.default_rng(3)
    sa = (rng.random(M, dtype=np.float32) * 0.05 + 1e-3).astype(np.float32)
    sw = np.float32(0.011)
    wp, xd = packed_on_device(w), to_dev(x)
    ws = torch.zeros(w2a8.workspace_bytes(M, N, K), dtype=torch.uint8, device=dev())
    acc = oracle.gemm_i32(x, w)
    for _ in range(3):
        yi = torch.empty(M * N, dtype=torch.int32, device=dev())
        yf = torch.empty(M * N, dtype=torch.float32, device=dev())
        w2a8.w2a8_gemm(wp, xd, M, N, K, y_i32=yi, s_a=to_dev(sa), s_w=float(sw), y_f32=yf,
                       workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(yi.cpu().numpy().reshape(M, N), acc)
        np.testing.assert_array_equal(yf.cpu().numpy().reshape(M, N), oracle.epilogue(acc, sa, sw))
        assert int(ws.count_nonzero()) == 0, "workspace not left zeroed"


# Short-batch MFMA ring kernel (2 <= M <= 32, K a multiple of 16) forced:
# both activation tile heights (M <= 8 and 9..16), ragged N, k-tile
# remainders, runs shorter and longer than the ring, split strips.
RING = [(2, 1, 16), (2, 33, 144), (3, 100, 1040), (5, 64, 2560), (7, 257, 4000), (8, 2560, 6912),
        (8, 13824, 2560), (9, 31, 272), (12, 200, 10240), (16, 96, 27648), (16, 2560, 2560),
        (4, 5000, 3200), (11, 640, 128), (17, 300, 2560), (24, 2560, 6912), (32, 700, 10240),
        (32, 13824, 2560), (20, 64, 27648), (29, 100, 1040), (31, 33, 144)]


@pytest.mark.parametrize("M,N,K", RING)
def test_gemm_ring_kernel(M, N, K):
    w2a8.tune_gemm(4)
    x, w = synth.gemm_case(M, N, K, seed=13 * M + N + 7 * K)
    y = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K)
    np.testing.assert_array_equal(y, oracle.gemm_i32(x, w))


# The automatic choice for short batches, one shape per branch of the
# short-batch plan rule on a 256-CU device (strips = ceil(N/32), k-tiles =
# ceil(K/128)): one wave per strip from 1024 strips; 4 waves per strip for
# K under 40 tiles or from 192 strips; 4 workgroups per strip for 64-127
# k-tiles; 3 otherwise; for 9 <= M <= 16 the pipelined kernel from 768
# strips (the first of each pair below) against the ring kernel just under;
# for 17 <= M <= 32 the ring kernel (32-row tiles) only from 192 k-tiles
# under 256 strips (the last four: ring, ring, pipelined, pipelined).
AUTO_SHORT = [(4, 32800, 256), (8, 20000, 3200), (8, 6900, 5120), (9, 3100, 10000),
              (12, 2500, 6900), (16, 5000, 16400), (12, 24570, 384), (12, 24500, 384),
              (16, 24600, 640), (16, 24530, 640), (20, 3000, 24576), (32, 8160, 24600),
              (24, 8200, 24600), (20, 3000, 24448),
              # two waves per strip from three strips per CU, one from six;
              # depth 4 on strips of 32 tiles or more
              (8, 27648, 1040), (6, 55296, 528), (8, 8192, 8192), (5, 16400, 4096)]


@pytest.mark.parametrize("M,N,K", AUTO_SHORT)
def test_gemm_automatic_short_batches(M, N, K):
    x, w = synth.gemm_case(M, N, K, seed=3 * M + N + K)
    y = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K)
    np.testing.assert_array_equal(y, oracle.gemm_i32_threads(x, w, ORACLE_THREADS))


@pytest.mark.parametrize("plan", [(1, 1, 2), (1, 7, 8), (4, 3, 4), (8, 1, 6), (16, 2, 2),
                                  (2, 40, 4), (3, 5, 6), (8, 12, 8)])
def test_gemm_ring_kernel_plans(plan):
    """Forced plans: single- and many-wave workgroups, strips split over many
    workgroups (runs of one tile, empty runs), every depth."""
    try:
        w2a8.tune_gemm(4)
        w2a8.tune_gemm_ring(*plan)
        for M, N, K in [(4, 200, 3200), (8, 96, 27648), (2, 33, 1008), (16, 64, 6912),
                        (13, 700, 2560), (32, 200, 3200), (24, 96, 27648)]:
            x, w = synth.gemm_case(M, N, K, seed=M + N + K)
            ws = torch.zeros(max(256, w2a8.workspace_bytes(M, N, K)), dtype=torch.uint8,
                             device=dev())
            wp, xd = packed_on_device(w), to_dev(x)
            lds = plan[0] * plan[2] * 1024 * (2 if M <= 8 else 3 if M <= 16 else 5)
            if lds > torch.cuda.get_device_properties(dev()).shared_memory_per_block:
                # the rings do not fit a workgroup's LDS: refused, nothing launched
                y = torch.empty(M * N, dtype=torch.int32, device=dev())
                with pytest.raises(w2a8.W2A8Error):
                    w2a8.w2a8_gemm(wp, xd, M, N, K, y_i32=y, workspace=ws)
                continue
            ref = oracle.gemm_i32(x, w)
            for _ in range(2):
                y = torch.empty(M * N, dtype=torch.int32, device=dev())
                w2a8.w2a8_gemm(wp, xd, M, N, K, y_i32=y, workspace=ws)
                torch.cuda.synchronize()
                np.testing.assert_array_equal(y.cpu().numpy().reshape(M, N), ref)
                assert int(ws.count_nonzero()) == 0, "workspace not left zeroed"
    finally:
        w2a8.tune_gemm_ring(0, 0, 0)


@pytest.mark.parametrize("M,N,K", [(8, 700, 27648), (15, 333, 3200)])
def test_gemm_ring_kernel_fp32_epilogue(M, N, K):
    w2a8.tune_gemm(4)
    x, w = synth.gemm_case(M, N, K, seed=5 * M + K)
    rng = np.random.default_rng(8)
    sa = (rng.random(M, dtype=np.float32) * 0.05 + 1e-3).astype(np.float32)
    sw = np.float32(0.021)
    yi, yf = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K, sa=to_dev(sa), sw=float(sw),
                       want_f32=True)
    acc = oracle.gemm_i32(x, w)
    np.testing.assert_array_equal(yi, acc)
    np.testing.assert_array_equal(yf, oracle.epilogue(acc, sa, sw))


@pytest.mark.parametrize("key", list(synth.GEMM_SEEDS.keys()),
                         ids=[f"{n}x{k}_M{m}" for (n, k), m in synth.GEMM_SEEDS.keys()])
def test_gemm_prefill_shapes(key):
    (N, K), M = key
    x, w = synth.gemm_case(M, N, K, seed=synth.GEMM_SEEDS[key])
    y = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K)
    # every output element, M = 512 included (the oracle over host threads)
    np.testing.assert_array_equal(y, oracle.gemm_i32_threads(x, w, ORACLE_THREADS))


def test_gemm_extremes():
    M, N, K = 20, 64, 27648
    x = np.full((M, K), -128, np.int8)
    x[1::2] = 127
    w = -np.ones((N, K), np.int8)
    y = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K)
    assert np.all(y[0::2] == 128 * K) and np.all(y[1::2] == -127 * K)


def test_gemm_fp32_epilogue_per_row_scales():
    M, N, K = 40, 2560, 2560
    x, w = synth.gemm_case(M, N, K, seed=3)
    rng = np.random.default_rng(4)
    sa = rng.uniform(0.001, 0.1, size=M).astype(np.float32)
    sw = np.float32(0.0159)
    yi, yf = _gemm_dev(packed_on_device(w), to_dev(x), M, N, K, sa=to_dev(sa), sw=float(sw),
                       want_f32=True)
    acc = oracle.gemm_i32(x, w)
    np.testing.assert_array_equal(yi, acc)
    np.testing.assert_array_equal(yf, oracle.epilogue(acc, sa, sw))


def test_gemm_rows_match_gemv():
    """Row m of the batched product equals the GEMV of row m."""
    M, N, K = 24, 2560, 2560
    x, w = synth.gemm_case(M, N, K, seed=12)
    wp = packed_on_device(w)
    y = _gemm_dev(wp, to_dev(x), M, N, K)
    for m in (0, 7, 23):
        yv = torch.empty(N, dtype=torch.int32, device=dev())
        w2a8.w2a8_gemv(wp, to_dev(x[m]), N, K, y_i32=yv)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y[m], yv.cpu().numpy())


def test_gemm_repeat_deterministic_and_workspace_reset():
    M, N, K = 8, 2560, 6912
    x, w = synth.gemm_case(M, N, K, seed=41)
    wp, xd = packed_on_device(w), to_dev(x)
    nb = w2a8.workspace_bytes(M, N, K)
    assert nb > 0
    ws = torch.zeros(nb, dtype=torch.uint8, device=dev())
    ref = oracle.gemm_i32(x, w)
    for _ in range(4):
        y = torch.empty((M, N), dtype=torch.int32, device=dev())
        w2a8.w2a8_gemm(wp, xd, M, N, K, y_i32=y, workspace=ws)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(y.cpu().numpy(), ref)
        assert int(ws.count_nonzero()) == 0
