"""The benchmark script's contract: one GPU only, and the JSON line it prints
(exact step counts, the roofline and context objects)."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _run(*args, timeout=600):
    return subprocess.run([sys.executable, BENCH, *args], cwd=ROOT, capture_output=True,
                          text=True, timeout=timeout)


@pytest.mark.parametrize("gpus", ["2", "8"])
def test_more_than_one_gpu_is_refused(gpus):
    r = _run("--gpus", gpus, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


@pytest.mark.gpu
def test_json_line_contract():
    """Small run: 3 timed steps after 2 warm-up steps, in graphs of 2 steps (so
    the last timed graph holds one step)."""
    r = _run("--steps", "3", "--warmup", "2", "--steps-per-graph", "2", "--no-extra",
             "--no-detail", "--no-cpu-baseline")
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1
    out = json.loads(lines[0])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "roofline"):
        assert key in out, key
    assert out["n_gpus"] == 1 and out["steps"] == 3 and out["warmup"] == 2
    assert out["value"] > 0 and out["ms_per_step"] > 0 and out["higher_is_better"] is True
    assert out["config"]["launch"].startswith("hipGraphs of up to 2 steps")
    rf = out["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert 0 < rf["frac"] < 1 and abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    # per launch: the step's device time over the 8 launches of a step
    assert abs(rf["avg_launch_us"] * 8 - rf["step_device_us"]) < 0.01 * rf["step_device_us"] + 0.01


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_under_test", BENCH)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


TRACE_HEADER = ('"Kind","Kernel_Name","Start_Timestamp","End_Timestamp","LDS_Block_Size",'
                '"VGPR_Count","Accum_VGPR_Count","Workgroup_Size_X","Workgroup_Size_Y",'
                '"Workgroup_Size_Z","Grid_Size_X","Grid_Size_Y","Grid_Size_Z"')


def test_kernel_names_are_shortened():
    b = _bench_module()
    assert b._short_kernel_name(
        "void w2a8::(anonymous namespace)::gemm_pipe_kernel<32, 1, 4, 1, 3, 2>(w2a8::GemmArgs)"
    ) == "gemm_pipe_kernel<32, 1, 4, 1, 3, 2>"
    assert b._short_kernel_name("w2a8::(anonymous namespace)::quant_rows_kernel(unsigned short "
                                "const*, int)") == "quant_rows_kernel"
    assert b._short_kernel_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_trace_summary_by_grid_and_by_kernel(tmp_path):
    # two grids of one kernel, durations 1, 2, 3 us and 10 us
    rows = [("k<2>(int)", 0, 1000, 512, 1024), ("k<2>(int)", 0, 2000, 512, 1024),
            ("k<2>(int)", 0, 3000, 512, 1024), ("k<2>(int)", 0, 10000, 512, 2048)]
    p = tmp_path / "t_kernel_trace.csv"
    with open(p, "w") as f:
        f.write(TRACE_HEADER + "\n")
        for name, t0, t1, wg, grid in rows:
            f.write(f'"KERNEL_DISPATCH","void {name}",{t0},{t1},2048,32,0,{wg},1,1,{grid},1,1\n')
    b = _bench_module()
    by_grid = b.trace_summary(str(p))
    assert [(r["grid"], r["launches"], r["median_us"], r["min_us"]) for r in by_grid] == [
        (1024, 3, 2.0, 1.0), (2048, 1, 10.0, 10.0)]
    assert by_grid[0]["workgroups"] == 2
    (k,) = b.trace_summary(str(p), "kernel")
    assert (k["kernel"], k["launches"], k["mean_us"], k["vgpr"], k["lds_bytes"]) == (
        "k<2>", 4, 4.0, 32, 2048)


def test_gemm_counter_summary(tmp_path):
    # one dispatch shape: 8 us, 1000 MFMAs of 16 busy cycles each, 5000 VALU
    trace = tmp_path / "g_kernel_trace.csv"
    with open(trace, "w") as f:
        f.write(TRACE_HEADER + "\n")
        f.write('"KERNEL_DISPATCH","void gemm_x<1>(int)",0,8000,0,40,0,256,1,1,2560,1,1\n')
    head = '"Kernel_Name","Grid_Size","Workgroup_Size","Counter_Name","Counter_Value"\n'
    a = tmp_path / "a.csv"
    b_ = tmp_path / "b.csv"
    with open(a, "w") as f:
        f.write(head)
        for n, v in (("SQ_INSTS_VALU_MFMA_I8", 1000), ("SQ_VALU_MFMA_BUSY_CYCLES", 16000),
                     ("SQ_INSTS_VALU", 5000), ("SQ_INSTS_LDS", 500), ("SQ_WAVES", 40)):
            f.write(f'"void gemm_x<1>(int)",2560,256,"{n}",{v}\n')
    with open(b_, "w") as f:
        f.write(head)
        for n, v in (("SQ_INSTS_SALU", 2000), ("SQ_LDS_BANK_CONFLICT", 7)):
            f.write(f'"void gemm_x<1>(int)",2560,256,"{n}",{v}\n')
    b = _bench_module()
    (r,) = b.gemm_counter_summary(str(trace), str(a), str(b_))
    assert r["kernel"] == "gemm_x<1>" and r["median_us"] == 8.0 and r["mfma"] == 1000
    assert r["busy_cycles_per_mfma"] == 16.0 and r["other_valu_per_mfma"] == 4.0
    assert r["lds_per_mfma"] == 0.5 and r["salu_per_mfma"] == 2.0
    # 16000 busy cycles over 1024 SIMDs x 8 us x 2.4 GHz
    assert abs(r["mfma_busy"] - round(16000 / (1024 * 8 * 2400), 4)) < 1e-12


def test_gemv_dispatch_keys_are_distinct_per_sweep_shape():
    """The counter summaries match GEMV dispatches to sweep shapes by kernel
    with its depth, grid and workgroup size: every sweep shape's key must be
    its own, and a counter row of that dispatch must map back to it."""
    sys.path.insert(0, ROOT)
    import bench
    import synth
    import w2a8_gemv_amd as w2a8
    keys = [bench.gemv_dispatch_key(w2a8, n, k, 256) for n, k in synth.SWEEP_SHAPES]
    assert len(set(keys)) == len(keys)
    for (n, k), key in zip(synth.SWEEP_SHAPES, keys):
        kern = w2a8.gemv_plan(n, k, 256)[0]
        assert key[0].startswith(bench.GEMV_KERNELS[kern] + "<")
        row = {"Kernel_Name": f"void w2a8::(anonymous namespace)::{key[0]}(w2a8::GemvLaunch)",
               "Grid_Size": str(key[1]), "Workgroup_Size": str(key[2])}
        assert bench._gemv_row_key(row) == key
    assert bench._gemv_row_key({"Kernel_Name": "void w2a8::(anonymous namespace)::"
                                "gemv_ring_grouped_kernel<4>(w2a8::GemvLaunch, w2a8::GemvGroups)",
                                "Grid_Size": "1", "Workgroup_Size": "64"}) is None
