"""GPU parity: spmm24 (sparse MFMA) and gemm_bf16 (dense MFMA baseline) against the oracle.

Tolerance: |y - y_ref| <= 1e-3 * (|W|.|X|)_ij on fp32 output; a bf16 output
also gets the half-ulp of its final rounding (see oracle.prune24.tolerance).
Exact pins: integer data (every partial sum exact in fp32) and X = I.
Full-size workloads run in the launch configuration the benchmark uses and
are checked on every output element.
"""
import os

import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import (DEV, bf16_dev, cached_ref, check_full, f32_dev, need_gpu, pruned_workload_ref, torch,
                      u16_host, y_host)

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu

TILES = ["256x256", "192x256", "128x256", "128x128", "64x128"]


def _run_sparse(W, Xb, out_dtype, x_pad=0):
    Wt = f32_dev(W)
    Xt = bf16_dev(Xb, pad_cols=x_pad)
    c = p24.compress(Wt, layout="device")
    Y = p24.spmm24(c, Xt, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return c, Y


def _check(Y, W, Xb, out):
    values, meta = O.compress_24(W, "f32")
    K = W.shape[1]
    y_ref, bnd = O.gemm_ref(O.decompress_24(values, meta, K), Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, out)
    assert ok, f"worst err/tol {worst}"
    return worst


@pytest.mark.parametrize("M,K,N,x_pad", [
    (96, 128, 72, 0),        # sub-tile everything, N tail inside one chunk row
    (300, 256, 200, 0),      # several tiles, ragged M and N
    (257, 192, 1001, 7),     # N not a multiple of 8 (strided X), ragged M
    (1024, 512, 640, 0),
    (64, 64, 8, 0),          # one K step, tiny N
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_parity_ragged(M, K, N, x_pad, out):
    need_gpu()
    print(f"[spmm24] {M}x{K}x{N} pad {x_pad} {out}", flush=True)
    W = workloads.random_matrix((M, K), seed=M * 7 + K, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N)
    _, Y = _run_sparse(W, Xb, torch.float32 if out == "f32" else torch.bfloat16, x_pad)
    _check(Y, W, Xb, out)


@pytest.mark.parametrize("tile", TILES)
def test_every_tile_config(tile, monkeypatch):
    need_gpu()
    monkeypatch.setenv("P24_TILE", tile)
    M, K, N = 544, 320, 600
    W = workloads.random_matrix((M, K), seed=11, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=12)
    _, Y = _run_sparse(W, Xb, torch.float32)
    _check(Y, W, Xb, "f32")


def test_192_row_tiles(monkeypatch):
    """192-row blocks start on a metadata-group boundary (even block rows) or in the middle of
    a group (odd ones); several of each, a ragged last block row, ragged N."""
    need_gpu()
    monkeypatch.setenv("P24_TILE", "192x256")
    M, K, N = 1000, 384, 696
    print(f"[spmm24] 192x256 tiles {M}x{K}x{N}", flush=True)
    W = workloads.random_matrix((M, K), seed=21, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=22)
    for out_dtype, out in ((torch.float32, "f32"), (torch.bfloat16, "bf16")):
        _, Y = _run_sparse(W, Xb, out_dtype)
        _check(Y, W, Xb, out)


def test_integer_exact_and_identity():
    need_gpu()
    M, K, N = 160, 256, 96
    W = workloads.small_int_matrix((M, K), seed=31)
    X = workloads.small_int_matrix((K, N), seed=32)
    Xb = workloads.truncate_to_bf16_bits(X)
    _, Y = _run_sparse(W, Xb, torch.float32)
    exact = O.prune_24(W, "f32").astype(np.int64) @ X.astype(np.int64)
    assert np.array_equal(y_host(Y), exact.astype(np.float64))
    # X = I returns the decompressed matrix bit for bit (pins the metadata semantics)
    W2 = workloads.random_matrix((96, 128), seed=33)
    I = workloads.truncate_to_bf16_bits(np.eye(128, dtype=np.float32))
    _, Y = _run_sparse(W2, I, torch.float32)
    v, m = O.compress_24(W2, "f32")
    assert np.array_equal(y_host(Y), O.bf16_to_f64(O.decompress_24(v, m, 128)))


@pytest.mark.parametrize("key", ["c1", "c2", "c3a", "c3b", "c4", "c4n8", "c4m8"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_workloads_full_size(key, out):
    need_gpu()
    wl = workloads.WORKLOADS[key]
    print(f"[spmm24] {key} {out}", flush=True)
    W = workloads.weights(wl)
    Xb = workloads.activations(wl)
    _, Y = _run_sparse(W, Xb, torch.float32 if out == "f32" else torch.bfloat16)
    check_full(Y, *pruned_workload_ref(key), out)


def test_deterministic():
    need_gpu()
    wl = workloads.WORKLOADS["c2"]
    W = workloads.weights(wl)
    Xb = workloads.activations(wl)
    c, Y1 = _run_sparse(W, Xb, torch.bfloat16)
    Y2 = p24.spmm24(c, bf16_dev(Xb), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))


# ---------------------------------------------------------------------------
# dense baseline
# ---------------------------------------------------------------------------
def _run_dense(Wb, Xb, out_dtype):
    Wt = bf16_dev(Wb)
    Wp = p24.pack_dense(Wt)
    Y = p24.gemm_bf16(Wp, Wb.shape[0], Wb.shape[1], bf16_dev(Xb), out_dtype=out_dtype)
    torch.cuda.synchronize()
    return Y


@pytest.mark.parametrize("M,K,N", [(96, 128, 72), (300, 256, 200), (1024, 512, 640)])
def test_dense_parity(M, K, N):
    need_gpu()
    Wb = workloads.random_bf16((M, K), seed=M, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N + 1)
    Y = _run_dense(Wb, Xb, torch.float32)
    y_ref, bnd = O.gemm_ref(Wb, Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, "f32")
    assert ok, worst


@pytest.mark.parametrize("key", ["c2", "c4"])
def test_dense_workloads(key):
    need_gpu()
    wl = workloads.WORKLOADS[key]
    Wb = workloads.truncate_to_bf16_bits(workloads.weights(wl))
    Xb = workloads.activations(wl)
    Y = _run_dense(Wb, Xb, torch.bfloat16)
    check_full(Y, *cached_ref(("dense", key), lambda: O.gemm_ref(Wb, Xb)), "bf16")


def test_zero_sized_noop():
    need_gpu()
    L = p24.lib()
    assert L.spmm24(None, None, 1, 0, 128, None, 64, 64, None, 0, 64, 0, None) == p24.P24_OK
    assert L.gemm_bf16(None, 64, 128, None, 0, 0, None, 0, 0, None) == p24.P24_OK


@pytest.mark.parametrize("pad", [3, 8])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_strided_outputs(pad, out):
    """Y as a column slice of a wider buffer (row stride N + pad): pad = 3 leaves the rows
    unaligned, so the epilogue stores element by element; pad = 8 keeps 16-byte row pieces.
    The products match the oracle and no write lands in the padding."""
    need_gpu()
    M, K, N = 300, 256, 200
    print(f"[spmm] strided Y pad={pad} {out}", flush=True)
    W = workloads.random_matrix((M, K), seed=21, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=22)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = p24.compress(f32_dev(W), layout="device")
    X = bf16_dev(Xb)
    XT = bf16_dev(np.ascontiguousarray(Xb.T))
    Wp = p24.pack_dense(bf16_dev(O.decompress_24(*O.compress_24(W, "f32"), K)))
    t = p24.tvw_compress(f32_dev(W), tile_m=128, keep_k=128)
    calls = {
        "spmm24": lambda Y: p24.spmm24(c, X, out=Y),
        "spmm24_xt": lambda Y: p24.spmm24_xt(c, XT, out=Y),
        "spmm24_fused": lambda Y: p24.spmm24(c, X, out=Y, act="relu"),
        "gemm_bf16": lambda Y: p24.gemm_bf16(Wp, M, K, X, out=Y),
        "spmm_tvw": lambda Y: p24.spmm_tvw(t, X, out=Y),
    }
    values, meta = O.compress_24(W, "f32")
    y24, b24 = O.gemm_ref(O.decompress_24(values, meta, K), Xb)
    kept, tv, tm = O.tvw_compress(W, 128, 128)
    ytvw, btvw = O.gemm_ref(O.tvw_decompress(kept, tv, tm, M, K, 128), Xb)
    for name, call in calls.items():
        full = torch.full((M, N + pad), 7.0, dtype=dt, device=DEV)
        Y = full[:, :N]
        call(Y)
        torch.cuda.synchronize()
        assert torch.all(full[:, N:] == 7.0), f"{name} wrote into the padding"
        y_ref, bnd = (ytvw, btvw) if name == "spmm_tvw" else (y24, b24)
        if name == "spmm24_fused":
            y_ref = np.maximum(y_ref, 0.0)
        ok, worst = O.check(y_host(Y), y_ref, bnd, out)
        assert ok, f"{name}: worst err/tol {worst}"


@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_non_finite_x_where_w_is_pruned(out):
    """X rows that meet only pruned weights: the sparse MFMA never multiplies them (the
    result is the product without those terms), while the expanded-tile path multiplies the
    explicit zeros (0 * Inf = NaN), as the header states."""
    need_gpu()
    M, K, N, g = 256, 256, 136, 5
    print(f"[spmm] non-finite X rows {out}", flush=True)
    W = workloads.random_matrix((M, K), seed=41, sigma=0.05)
    W[:, 4 * g + 0:4 * g + 2] += np.float32(10.0)       # positions 0 and 1 win in every row
    Xb = workloads.random_bf16((K, N), seed=42)
    Xb[4 * g + 2, :] = 0x7F80                            # +Inf
    Xb[4 * g + 3, ::3] = 0x7FC0                          # NaN in every third column
    values, meta = O.compress_24(W, "f32")
    Wd = O.decompress_24(values, meta, K)
    assert not Wd[:, 4 * g + 2:4 * g + 4].any()          # both rows pruned everywhere
    X0 = Xb.copy()
    X0[4 * g + 2:4 * g + 4, :] = 0                       # the terms the sparse MFMA skips
    y_ref, bnd = O.gemm_ref(Wd, X0)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = p24.compress(f32_dev(W))
    X = bf16_dev(Xb)
    Y = p24.spmm24(c, X, out_dtype=dt)
    Yd = p24.spmm24(c, X, out_dtype=dt, algo="decomp_mfma")
    torch.cuda.synchronize()
    assert torch.isfinite(Y).all().item()
    ok, worst = O.check(y_host(Y), y_ref, bnd, out)
    assert ok, f"worst err/tol {worst}"
    assert torch.isnan(Yd).all().item()
