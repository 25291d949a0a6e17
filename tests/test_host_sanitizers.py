"""The library's host code (argument validation and dispatch of every entry point)
under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

`build.py --sanitize` builds a copy of the library whose host pass carries both
sanitizers (the device code has none); the host-side ABI and binding tests then
run against that copy in a child process with the shared ASan runtime preloaded.
A sanitizer report aborts the child, so any finding fails this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.join(ROOT, "structured_sparse_gemm_prune24_amd"))

pytestmark = pytest.mark.slow

HOST_TESTS = ["tests/test_abi_host.py", "tests/test_binding_host.py", "tests/test_c_abi.py"]


def test_host_code_under_asan_and_ubsan():
    import build
    try:
        build.hipcc()
        runtime = build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(f"no ROCm toolchain here: {e}")
    lib = build.build_sanitized()
    out = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in out and "__ubsan_handle" in out, "the copy carries no sanitizer hooks"
    env = build.sanitizer_env()
    assert env["LD_PRELOAD"] == runtime and env["P24_LIBRARY"] == lib
    probe = subprocess.run([sys.executable, "-c", "import structured_sparse_gemm_prune24_amd as p; "
                            "print(p.LIB_PATH); print(p.lib().prune24_abi_version())"],
                           env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0, probe.stderr[-2000:]
    assert probe.stdout.split() == [lib, "1"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        *HOST_TESTS], env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, (r.stdout[-3000:], r.stderr[-3000:])
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
