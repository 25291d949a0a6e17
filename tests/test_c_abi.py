"""The C ABI seen from a C99 program (tests/c_abi/abi_caller.c) that includes only
include/prune24.h and the HIP runtime API, allocates its own device buffers, workspace
and stream, and hands its results back in host buffers.

CPU: the caller links and its argument checks return the documented statuses.
GPU: its compression and TVW selection are bit-exact and its products are within
tolerance against the oracle, on ragged shapes.
"""
import ctypes
import os

import numpy as np
import pytest

import workloads
from oracle import prune24 as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CALLER = os.path.join(ROOT, "tests", "c_abi", "libp24_c_caller.so")

_vp, _i64 = ctypes.c_void_p, ctypes.c_int64


@pytest.fixture(scope="module")
def C():
    # Bind the caller to the HIP runtime this process already uses.  torch opens its own
    # copy of the runtime by path; a second copy loaded first (the caller's link-time
    # /opt/rocm one) would sit beside it in the process, and a copy that is not the one
    # the process initialised reports no device.
    import torch  # noqa: F401
    if not os.path.exists(CALLER):
        pytest.fail(f"{CALLER} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(CALLER)
    L.p24c_run_24.restype = ctypes.c_int
    L.p24c_run_24.argtypes = [_vp, _i64, _i64, _vp, _i64, _vp, _vp, _vp]
    L.p24c_run_tvw.restype = ctypes.c_int
    L.p24c_run_tvw.argtypes = [_vp, _i64, _i64, _i64, _i64, _vp, _i64, _vp, _vp]
    L.p24c_error_paths.restype = ctypes.c_int
    L.p24c_error_paths.argtypes = [_vp]
    return L


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(_vp)


def test_c_caller_argument_checks(C):
    codes = np.zeros(6, dtype=np.int32)
    assert C.p24c_error_paths(_ptr(codes)) == 1          # ABI version
    # K % 64 for spmm24; canonical layout refused by spmm24; K % 4; NULL W; M == 0 is a no-op; bad dtype
    assert codes.tolist() == [-5, -8, -2, -1, 0, -4]


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,N", [(300, 256, 200), (256, 768, 64), (33, 128, 8)])
def test_c_caller_24(C, M, K, N):
    from gpu_util import need_gpu
    need_gpu()
    W = workloads.random_matrix((M, K), seed=M * 7 + K, sigma=0.02)
    X = workloads.random_bf16((K, N), seed=N + 1)
    values = np.zeros((M, K // 2), dtype=np.uint16)
    meta = np.zeros((M, (K + 31) // 32), dtype=np.uint32)
    Y = np.zeros((M, N), dtype=np.float32)
    rc = C.p24c_run_24(_ptr(W), M, K, _ptr(X), N, _ptr(values), _ptr(meta), _ptr(Y))
    assert rc == 0, rc
    ov, om = O.compress_24(W, "f32")
    assert np.array_equal(values, ov)
    assert np.array_equal(meta, om)
    y_ref, bnd = O.gemm_ref(O.decompress_24(ov, om, K), X)
    ok, worst = O.check(Y.astype(np.float64), y_ref, bnd, "f32")
    assert ok, worst


@pytest.mark.gpu
@pytest.mark.parametrize("M,K,tile,keep,N", [(384, 512, 128, 256, 136), (300, 256, 128, 128, 96)])
def test_c_caller_tvw(C, M, K, tile, keep, N):
    from gpu_util import need_gpu
    need_gpu()
    W = workloads.random_matrix((M, K), seed=M + K + keep, sigma=0.02)
    X = workloads.random_bf16((K, N), seed=N + 2)
    tiles = (M + tile - 1) // tile
    kept = np.zeros((tiles, keep), dtype=np.int32)
    Y = np.zeros((M, N), dtype=np.float32)
    rc = C.p24c_run_tvw(_ptr(W), M, K, tile, keep, _ptr(X), N, _ptr(kept), _ptr(Y))
    assert rc == 0, rc
    okept, tv, tm = O.tvw_compress(W, tile, keep)
    assert np.array_equal(kept, okept)
    y_ref, bnd = O.gemm_ref(O.tvw_decompress(okept, tv, tm, M, K, tile), X)
    ok, worst = O.check(Y.astype(np.float64), y_ref, bnd, "f32")
    assert ok, worst
