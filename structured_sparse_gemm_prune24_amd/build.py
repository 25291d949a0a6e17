"""Build libprune24.so (HIP for gfx950) in-tree, next to this file.

Each .hip source is compiled to an object under <repo>/_build, then linked into
the shared library.  Always recompiles (a build is the "does it build" check).
The device assembly kept by -save-temps is checked by isa_check.

`python build.py --sanitize` builds a second copy, _build/sanitize/libprune24.so,
whose host code (argument validation and dispatch) carries AddressSanitizer and
UndefinedBehaviorSanitizer; the device code is built as usual, without any
sanitizer.  It is for CPU test runs: the library links the shared ASan runtime,
so the Python process needs that runtime preloaded (`sanitizer_env()` gives the
environment), and the binding loads it when P24_LIBRARY names it.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

try:
    from . import isa_check
except ImportError:          # run as a script
    import isa_check

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libprune24.so"
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # keep hipcc from emitting packed fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    f"-I{INCLUDE}",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libprune24.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def device_asm(src: str) -> str:
    """The gfx950 assembly that -save-temps leaves next to the object of `src`."""
    stem = os.path.splitext(os.path.basename(src))[0]
    return os.path.join(BUILD_DIR, f"{stem}-hip-amdgcn-amd-amdhsa-{ARCH}.s")


# host-only sanitizers: each -fsanitize applies to the host pass alone
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-g", "-shared-libasan"]
SANITIZE_DIR = os.path.join(BUILD_DIR, "sanitize")


def asan_runtime() -> str:
    """The shared ASan runtime of the compiler hipcc drives."""
    r = subprocess.run([os.path.join(os.path.dirname(os.path.realpath(hipcc())), "..", "llvm", "bin", "clang"),
                        "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    if r.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        import glob
        hits = glob.glob("/opt/rocm/llvm/lib/clang/*/lib/*/libclang_rt.asan-x86_64.so")
        if not hits:
            raise RuntimeError("the shared ASan runtime was not found")
        path = hits[0]
    return path


def sanitizer_env(base=None) -> dict:
    """Environment for a CPU test run against the sanitized library."""
    env = dict(os.environ if base is None else base)
    env["LD_PRELOAD"] = asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"    # the interpreter's own allocations are not ours
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["P24_LIBRARY"] = os.path.join(SANITIZE_DIR, LIB_NAME)
    return env


def _compile(src: str, verbose: bool, sanitize: bool = False) -> str:
    out_dir = SANITIZE_DIR if sanitize else BUILD_DIR
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    extra = SANITIZE_FLAGS if sanitize else ["-save-temps=obj"]
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    return obj


def build_sanitized(verbose: bool = False) -> str:
    """The host-sanitized copy of the library (see the module docstring)."""
    os.makedirs(SANITIZE_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, sanitize=True), srcs))
    out = os.path.join(SANITIZE_DIR, LIB_NAME)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", *objs, "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed\n{r.stdout}\n{r.stderr}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    out = os.path.join(PKG, LIB_NAME)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    # every kernel's final assembly: no LDS read result used before its wait
    for src in srcs:
        isa_check.check_file(device_asm(src))
    return out


if __name__ == "__main__":
    if "--sanitize" in sys.argv:
        print(build_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
