"""Host logic of bench.py: the clock reading parser, the sample window filter, the traffic
figure's source-hash gate, the one-GPU rule and the CPU baseline leg."""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _amdsmi_json(mhz, gpu=0):
    clock = {f"gfx_{i}": {"clk": {"value": v, "unit": "MHz"}, "max_clk": {"value": 2400, "unit": "MHz"}}
             for i, v in enumerate(mhz)}
    clock["mem_0"] = {"clk": {"value": 2000, "unit": "MHz"}}
    clock["fclk_0"] = {"clk": {"value": 2100, "unit": "MHz"}}
    return {"gpu": gpu, "clock": clock}


def test_parse_gfx_clocks_takes_only_gpu0_xcd_clocks():
    text = json.dumps({"gpu_data": [_amdsmi_json([1900, 1950, 1880]), _amdsmi_json([100, 100], gpu=1)]})
    assert bench.parse_gfx_clocks(text) == [1900.0, 1950.0, 1880.0]


def test_parse_gfx_clocks_list_form_and_missing_values():
    entry = _amdsmi_json([1800, 1850])
    entry["clock"]["gfx_1"]["clk"]["value"] = "N/A"
    assert bench.parse_gfx_clocks(json.dumps([entry])) == [1800.0]
    assert bench.parse_gfx_clocks(json.dumps({"gpu_data": []})) == []


def test_read_clock_samples_keeps_readings_inside_the_window(tmp_path):
    p = tmp_path / "clk.txt"
    p.write_text("10.0 10.4 1000 2000\n"
                 "11.0 11.5 1900 1900\n"
                 "12.0 12.2 1800 2000\n"
                 "13.9 14.1 1500 1500\n"
                 "garbage\n")
    assert bench.read_clock_samples(str(p), 10.5, 14.0) == [1900.0, 1900.0]
    assert bench.read_clock_samples(str(tmp_path / "missing.txt"), 0, 1e9) == []


def test_under_profiler_detects_the_profiler_environment():
    assert bench.under_profiler({"LD_PRELOAD": "/opt/rocm/lib/rocprofiler-sdk/librocprofiler-sdk-tool.so"})
    assert bench.under_profiler({"ROCPROF_KERNEL_TRACE": "1"})
    assert not bench.under_profiler({"LD_PRELOAD": "/usr/lib/libother.so", "PATH": "/usr/bin"})
    assert not bench.under_profiler({})


def test_measured_traffic_is_gated_by_the_kernel_source_hash(tmp_path):
    """The traffic figure is reported only while the kernel source is the one profiled."""
    import hashlib
    src = tmp_path / "gemm.hip"
    src.write_text("// kernel source\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    prof = tmp_path / "traffic.md"
    prof.write_text(f"traffic_bytes_per_launch: 123456\nkernel_source_sha256_prefix: {digest[:16]}\n")
    assert bench.measured_traffic(str(prof), str(src)) == 123456
    src.write_text("// kernel source, changed\n")
    assert bench.measured_traffic(str(prof), str(src)) is None
    assert bench.measured_traffic(str(tmp_path / "missing.md"), str(src)) is None
    prof.write_text("no machine-readable lines\n")
    assert bench.measured_traffic(str(prof), str(src)) is None


def test_more_than_one_gpu_is_refused():
    """bench.py measures one GPU; --gpus above 1 exits with status 2 and says so."""
    import subprocess
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_on_the_small_workload():
    """The CPU leg runs the oracle on the whole small workload and reports its figures."""
    import workloads
    wl = workloads.WORKLOADS["c1"]
    cb = bench.cpu_baseline(wl, workloads.weights(wl), workloads.activations(wl))
    assert cb["kind"] == "oracle" and cb["unit"] == "TFLOP/s (dense-equivalent)"
    assert cb["value"] > 0 and cb["cores"] >= 1
    assert cb["sample"].startswith(f"{wl.M} of {wl.M} output rows of c1")
    assert cb["prune_compress_s"] >= 0 and cb["gemm_and_bound_s"] >= 0
    assert set(cb) >= {"cpu_model", "blas"}


def test_spmm24_kernel_label_follows_the_tile_rule():
    """The roofline's kernel name is the instantiation the library's tile rule picks."""
    import workloads
    want = {"c1": "64x128", "c2": "192x256", "c3a": "128x128", "c3b": "64x128", "c4": "256x256",
            "c4n8": "128x256", "c4m8": "128x256"}
    for key, tile in want.items():
        wl = workloads.WORKLOADS[key]
        bm, bn = tile.split("x")
        assert bench.spmm24_kernel(wl.M, wl.N, env={}).startswith(f"k_gemm<{bm},{bn},"), key
    assert bench.spmm24_kernel(8192, 8192, env={}) == "k_gemm<256,256,2,4,sparse,X_KN> (spmm24)"
    assert bench.spmm24_kernel(8192, 8192, env={"P24_TILE": "128x128"}).startswith("k_gemm<128,128,2,4,")
    assert bench.spmm24_kernel(8192, 8192, env={"P24_TILE": "192x256"}).startswith("k_gemm<192,256,2,4,")
    assert bench.spmm24_kernel(8192, 8192, env={"P24_TILE": "bogus"}).startswith("k_gemm<256,256,")


def test_traffic_source_says_where_the_figure_comes_from():
    assert bench.traffic_source(None).startswith("null")
    assert bench.traffic_source(123).startswith(bench.TRAFFIC_PROFILE)


def test_gfx_clocks_from_metrics_and_sampler_header(tmp_path):
    m = {"current_gfxclks": [1850, 1860, 65535, 0, "N/A", 1870, 1880, 1890], "other": 1}
    assert bench.gfx_clocks_from_metrics(m) == [1850.0, 1860.0, 1870.0, 1880.0, 1890.0]
    assert bench.gfx_clocks_from_metrics({"current_gfxclks": "N/A"}) == []
    assert bench.gfx_clocks_from_metrics(None) == []
    p = tmp_path / "clk.txt"
    p.write_text("# source amdsmi gpu metrics\n1.0 1.1 1800 1900\n")
    assert bench.clock_source(str(p)) == "amdsmi gpu metrics"
    assert bench.read_clock_samples(str(p), 0.0, 2.0) == [1850.0]
    assert bench.clock_source(str(tmp_path / "none.txt")) is None


def test_refresh_estimate_counts_changes_of_the_reading(tmp_path):
    p = tmp_path / "clk.txt"
    p.write_text("# source amdsmi gpu metrics\n" +
                 "".join(f"{0.005 * i:.4f} {0.005 * i + 0.001:.4f} {1800 + 10 * (i // 10)}\n" for i in range(100)))
    timed = bench.read_clock_samples(str(p), 0.0, 1.0, with_time=True)
    assert len(timed) == 100 and timed[0] == (0.0, 1800.0)
    assert bench.refresh_ms_est(timed) == 50.0          # the value changes every 10 readings of 5 ms
    assert bench.refresh_ms_est(timed[:5]) is None
