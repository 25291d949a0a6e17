"""GPU parity for spmm24's second algorithm, P24_ALGO_DECOMP_MFMA: the compressed
operand is expanded block-wide into a dense LDS tile (zeros in the pruned slots)
and multiplied on the dense MFMA.

It must meet the same elementwise bound against the oracle as the sparse-MFMA
path.  On integer data every partial sum is exact in fp32, so there both
algorithms return the exact product, bit for bit; X = I returns the decompressed
matrix, which pins the expansion's reading of the metadata.
"""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import bf16_dev, check_full, f32_dev, need_gpu, pruned_workload_ref, torch, y_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu


def _check(Y, W, Xb, out):
    v, m = O.compress_24(W, "f32")
    y_ref, bnd = O.gemm_ref(O.decompress_24(v, m, W.shape[1]), Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, out)
    assert ok, f"worst err/tol {worst}"


@pytest.mark.parametrize("M,K,N,x_pad", [
    (96, 128, 72, 0),
    (300, 256, 200, 0),
    (257, 192, 1001, 7),
    (1024, 512, 640, 0),
    (64, 64, 8, 0),
    (544, 2304, 520, 0),
])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_decomp_parity_ragged(M, K, N, x_pad, out):
    need_gpu()
    print(f"[spmm24 decomp] {M}x{K}x{N} pad {x_pad} {out}", flush=True)
    W = workloads.random_matrix((M, K), seed=M * 3 + K, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N + 5)
    c = p24.compress(f32_dev(W))
    Y = p24.spmm24(c, bf16_dev(Xb, pad_cols=x_pad), out_dtype=torch.float32 if out == "f32" else torch.bfloat16,
                   algo="decomp_mfma")
    torch.cuda.synchronize()
    _check(Y, W, Xb, out)


@pytest.mark.parametrize("tile", ["256x256", "128x256", "128x128", "64x128"])
def test_decomp_every_tile(tile, monkeypatch):
    need_gpu()
    monkeypatch.setenv("P24_TILE", tile)
    M, K, N = 544, 320, 600
    W = workloads.random_matrix((M, K), seed=23, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=24)
    c = p24.compress(f32_dev(W))
    Y = p24.spmm24(c, bf16_dev(Xb), out_dtype=torch.float32, algo="decomp_mfma")
    torch.cuda.synchronize()
    _check(Y, W, Xb, "f32")


@pytest.mark.parametrize("tile", ["256x256", "64x128"])
def test_decomp_integer_exact_matches_smfmac(tile, monkeypatch):
    need_gpu()
    monkeypatch.setenv("P24_TILE", tile)
    M, K, N = 288, 384, 200
    W = workloads.small_int_matrix((M, K), seed=41)
    X = workloads.small_int_matrix((K, N), seed=42)
    Xb = workloads.truncate_to_bf16_bits(X)
    c = p24.compress(f32_dev(W))
    Xd = bf16_dev(Xb)
    Yd = p24.spmm24(c, Xd, out_dtype=torch.float32, algo="decomp_mfma")
    Ys = p24.spmm24(c, Xd, out_dtype=torch.float32, algo="smfmac")
    torch.cuda.synchronize()
    exact = O.prune_24(W, "f32").astype(np.int64) @ X.astype(np.int64)
    assert np.array_equal(y_host(Yd), exact.astype(np.float64))
    assert torch.equal(Yd, Ys)


def test_decomp_identity_returns_decompressed():
    need_gpu()
    W = workloads.random_matrix((160, 192), seed=43)
    I = workloads.truncate_to_bf16_bits(np.eye(192, dtype=np.float32))
    c = p24.compress(f32_dev(W))
    Y = p24.spmm24(c, bf16_dev(I), out_dtype=torch.float32, algo="decomp_mfma")
    torch.cuda.synchronize()
    v, m = O.compress_24(W, "f32")
    assert np.array_equal(y_host(Y), O.bf16_to_f64(O.decompress_24(v, m, 192)))


@pytest.mark.parametrize("key", ["c2", "c3b", "c4"])
def test_decomp_workloads(key):
    need_gpu()
    wl = workloads.WORKLOADS[key]
    print(f"[spmm24 decomp] {key}", flush=True)
    W = workloads.weights(wl)
    Xb = workloads.activations(wl)
    c = p24.compress(f32_dev(W))
    Y = p24.spmm24(c, bf16_dev(Xb), out_dtype=torch.bfloat16, algo="decomp_mfma")
    torch.cuda.synchronize()
    check_full(Y, *pruned_workload_ref(key), "bf16")


def test_decomp_deterministic():
    need_gpu()
    wl = workloads.WORKLOADS["c2"]
    W = workloads.weights(wl)
    Xb = workloads.activations(wl)
    c = p24.compress(f32_dev(W))
    Xd = bf16_dev(Xb)
    Y1 = p24.spmm24(c, Xd, out_dtype=torch.bfloat16, algo="decomp_mfma")
    Y2 = p24.spmm24(c, Xd, out_dtype=torch.bfloat16, algo="decomp_mfma")
    torch.cuda.synchronize()
    assert torch.equal(Y1.view(torch.int16), Y2.view(torch.int16))


def test_bad_algo_name():
    need_gpu()
    c = p24.compress(f32_dev(workloads.random_matrix((32, 64), seed=1)))
    with pytest.raises(ValueError):
        p24.spmm24(c, bf16_dev(workloads.random_bf16((64, 8), seed=2)), algo="dense")
