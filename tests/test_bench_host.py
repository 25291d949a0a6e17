"""Host logic of bench.py: the clock reading parser and the sample window filter."""
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
