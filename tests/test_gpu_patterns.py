"""GPU parity for the comparison patterns: block-wise (bw_compress + spmm_tw)
and unstructured (ew_compress + spmm_ew), compression bit-exact against the
oracle, products within the GEMM tolerance."""
import numpy as np
import pytest

import workloads
from oracle import prune24 as O
from gpu_util import bf16_dev, f32_dev, need_gpu, torch, u16_host, y_host

p24 = pytest.importorskip("structured_sparse_gemm_prune24_amd")
pytestmark = pytest.mark.gpu


def _bw(W, keep_blocks):
    M, K = W.shape
    print(f"[bw] compress {M}x{K} keep {keep_blocks} blocks", flush=True)
    t = p24.bw_compress(f32_dev(W), keep_blocks)
    torch.cuda.synchronize()
    kept, Wc = O.bw_compress(W, keep_blocks)
    assert np.array_equal(t.kept.cpu().numpy(), kept)
    dv = O.dense_device_layout(Wc, -(-M // 32) * 32)
    assert np.array_equal(u16_host(t.Wp)[:dv.size], dv)
    Wd = O.tw_decompress(list(kept), [Wc[128 * i:128 * i + 128] for i in range(kept.shape[0])], M, K, 128)
    return t, Wd


def _ew(W, keep):
    M, K = W.shape
    print(f"[ew] compress {M}x{K} keep {keep}", flush=True)
    t = p24.ew_compress(f32_dev(W), keep)
    torch.cuda.synchronize()
    rp, cols, vals = O.ew_compress(W, keep)
    assert np.array_equal(t.row_ptr.cpu().numpy(), rp)
    assert np.array_equal(t.cols.cpu().numpy()[:keep], cols)
    assert np.array_equal(u16_host(t.vals)[:keep], vals)
    return t, O.ew_decompress(rp, cols, vals, M, K)


@pytest.mark.parametrize("M,K,keep", [(256, 256, 2), (300, 320, 3), (128, 2304, 9), (200, 192, 3)])
def test_bw_compress(M, K, keep):
    need_gpu()
    _bw(workloads.random_matrix((M, K), seed=M + K + keep, sigma=0.02), keep)


def test_bw_ties():
    need_gpu()
    W = workloads.small_int_matrix((256, 256), seed=81, lo=-2, hi=2)
    W[:, 128:192] = W[:, 0:64]
    _bw(W, 2)


@pytest.mark.parametrize("M,K,N,keep", [(256, 256, 200, 2), (300, 512, 1000, 3)])
def test_bw_spmm(M, K, N, keep):
    need_gpu()
    W = workloads.random_matrix((M, K), seed=N, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N + 1)
    t, Wd = _bw(W, keep)
    Y = p24.spmm_tw(t, bf16_dev(Xb), out_dtype=torch.float32)
    torch.cuda.synchronize()
    y_ref, bnd = O.gemm_ref(Wd, Xb)
    ok, worst = O.check(y_host(Y), y_ref, bnd, "f32")
    assert ok, worst


@pytest.mark.parametrize("M,K,keep", [(64, 64, 1), (64, 64, 1000), (100, 300, 7500), (37, 520, 37 * 520),
                                      (1000, 96, 20000)])
def test_ew_compress(M, K, keep):
    need_gpu()
    _ew(workloads.random_matrix((M, K), seed=M + K, sigma=0.05), keep)


@pytest.mark.parametrize("fill", [0.5, 0.0])
def test_ew_all_tied(fill):
    """Every magnitude equal (zeros included): the first keep_total entries in row-major order."""
    need_gpu()
    W = np.full((50, 70), fill, dtype=np.float32)
    W[::3, ::2] *= -1.0
    _ew(W, 1234)


def test_ew_tie_at_cut():
    need_gpu()
    W = workloads.random_matrix((80, 128), seed=82, sigma=0.02)
    W[10:30, 5:60] = 0.5                  # 1100 equal magnitudes straddling the cut
    W[40:45, :] = 2.0                     # 640 entries above everything else
    _ew(W, 1000)


@pytest.mark.parametrize("M,K,N,frac,out", [(64, 128, 512, 0.3, "f32"), (100, 300, 77, 0.25, "f32"),
                                            (130, 256, 1000, 0.5, "bf16"), (40, 64, 5, 0.6, "f32")])
def test_ew_spmm(M, K, N, frac, out):
    need_gpu()
    W = workloads.random_matrix((M, K), seed=M * N, sigma=0.05)
    Xb = workloads.random_bf16((K, N), seed=N)
    t, Wd = _ew(W, int(frac * M * K))
    print(f"[ew] spmm {M}x{K}x{N} {out}", flush=True)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    X = bf16_dev(Xb, pad_cols=(-N) % 8)                                  # ldx % 8 == 0
    Y = p24.spmm_ew(t, X, out_dtype=dt)
    Ys = torch.zeros((M, N + 3), dtype=dt, device=Y.device)[:, :N]       # strided output rows
    p24.spmm_ew(t, X, out=Ys)
    torch.cuda.synchronize()
    y_ref, bnd = O.gemm_ref(Wd, Xb)
    for y in (Y, Ys):
        ok, worst = O.check(y_host(y), y_ref, bnd, out)
        assert ok, worst


def test_c5_shape_75pct():
    """The TVW workload's shape at its 75 % sparsity, block-wise (16 of 64 blocks per tile) and
    unstructured (a quarter of all weights)."""
    need_gpu()
    wl = workloads.WORKLOADS["c5"]
    W = workloads.weights(wl)
    Xb = workloads.activations(wl)
    X = bf16_dev(Xb)
    tb, Wdb = _bw(W, 16)
    te, Wde = _ew(W, wl.M * wl.K // 4)
    for name, run, Wd in (("bw", lambda: p24.spmm_tw(tb, X, out_dtype=torch.bfloat16), Wdb),
                          ("ew", lambda: p24.spmm_ew(te, X, out_dtype=torch.bfloat16), Wde)):
        print(f"[patterns] c5 {name}", flush=True)
        Y = run()
        torch.cuda.synchronize()
        y_ref, bnd = O.gemm_ref(Wd, Xb)
        ok, worst = O.check(y_host(Y), y_ref, bnd, "bf16")
        assert ok, worst
