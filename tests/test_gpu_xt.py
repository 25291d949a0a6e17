"""GPU parity for the transposed-X entry points (spmm24_xt, gemm_bf16_xt) and transpose_bf16.

spmm24_xt consumes the same fragments in the same order as spmm24, only read
from a K-contiguous copy of X, so for the same inputs the two must agree bit for
bit; both are also held to the oracle's elementwise bound.
"""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import bf16_dev, check_full, f32_dev, need_gpu, pruned_workload_ref, torch, u16_host, y_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("R,C", [(1, 1), (64, 64), (100, 37), (513, 1000), (768, 4096)])
def test_transpose_exact(R, C):
    need_gpu()
    a = workloads.random_bf16((R, C), seed=R * 31 + C)
    t = p24.transpose(bf16_dev(a))
    torch.cuda.synchronize()
    assert np.array_equal(u16_host(t), a.T)


def test_transpose_strided():
    need_gpu()
    a = workloads.random_bf16((70, 90), seed=3)
    src = bf16_dev(a, pad_cols=6)                       # ld 96
    out = torch.zeros((90, 80), dtype=torch.bfloat16, device=src.device)[:, :70]
    p24.transpose(src, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(u16_host(out), a.T)


@pytest.mark.parametrize("M,K,N", [(96, 128, 72), (300, 256, 200), (257, 192, 1001), (1024, 512, 640),
                                   (64, 64, 8), (544, 320, 600)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_spmm24_xt_matches_kn_path_and_oracle(M, K, N, out):
    need_gpu()
    print(f"[spmm24_xt] {M}x{K}x{N} {out}", flush=True)
    W = workloads.random_matrix((M, K), seed=M * 5 + K, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N + 7)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    c = p24.compress(f32_dev(W))
    Y1 = p24.spmm24(c, bf16_dev(Xb, pad_cols=(-N) % 8), out_dtype=dt)   # K x N path needs ldx % 8 == 0
    Y2 = p24.spmm24_xt(c, bf16_dev(np.ascontiguousarray(Xb.T)), out_dtype=dt)
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16 if out == "bf16" else torch.int32),
                       Y2.view(torch.int16 if out == "bf16" else torch.int32))
    v, m = O.compress_24(W, "f32")
    y_ref, bnd = O.gemm_ref(O.decompress_24(v, m, K), Xb)
    ok, worst = O.check(y_host(Y2), y_ref, bnd, out)
    assert ok, worst


@pytest.mark.parametrize("tile", ["256x256", "192x256", "128x256", "128x128", "64x128"])
def test_spmm24_xt_every_tile(tile, monkeypatch):
    need_gpu()
    monkeypatch.setenv("P24_TILE", tile)
    M, K, N = 544, 320, 600
    W = workloads.random_matrix((M, K), seed=19, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=20)
    c = p24.compress(f32_dev(W))
    Y = p24.spmm24_xt(c, bf16_dev(np.ascontiguousarray(Xb.T)), out_dtype=torch.float32)
    torch.cuda.synchronize()
    v, m = O.compress_24(W, "f32")
    y_ref, bnd = O.gemm_ref(O.decompress_24(v, m, K), Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, "f32")
    assert ok, worst


@pytest.mark.parametrize("key", ["c2", "c4"])
def test_spmm24_xt_workloads(key):
    need_gpu()
    wl = workloads.WORKLOADS[key]
    print(f"[spmm24_xt] {key}", flush=True)
    W = workloads.weights(wl)
    Xb = workloads.activations(wl)
    c = p24.compress(f32_dev(W))
    Xt = bf16_dev(Xb)
    XT = p24.transpose(Xt)
    Y = p24.spmm24_xt(c, XT, out_dtype=torch.bfloat16)
    Yk = p24.spmm24(c, Xt, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Yk.view(torch.int16))
    check_full(Y, *pruned_workload_ref(key), "bf16")


@pytest.mark.parametrize("M,K,N", [(96, 128, 72), (300, 256, 200), (1024, 512, 640)])
def test_gemm_bf16_xt(M, K, N):
    need_gpu()
    Wb = workloads.random_bf16((M, K), seed=M + 1, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N + 2)
    Wp = p24.pack_dense(bf16_dev(Wb))
    Y1 = p24.gemm_bf16(Wp, M, K, bf16_dev(Xb), out_dtype=torch.float32)
    Y2 = p24.gemm_bf16_xt(Wp, M, K, bf16_dev(np.ascontiguousarray(Xb.T)), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(Y1, Y2)
    y_ref, bnd = O.gemm_ref(Wb, Xb)
    ok, worst = O.check(y_host(Y2), y_ref, bnd, "f32")
    assert ok, worst
